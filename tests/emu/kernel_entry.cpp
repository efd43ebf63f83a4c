// Direct entry points into single kernel families of the emulated library,
// for tests that check one kernel at a size the whole step could not reach
// in emulation.  TEST INFRASTRUCTURE ONLY: compiled into the emulator build,
// never into libgpt2mi.so.
#include <hip/hip_runtime.h>

#include "kernels.h"

#define EMU_API extern "C" __attribute__((visibility("default")))

EMU_API int emu_gemm(int M, int N, int K, const void* A, int lda, int a_t, const void* B, int ldb, int b_t,
                     int kind, void* out, int ldo, void* out2, const void* aux, const float* bias,
                     float alpha, float beta, int dt, float* ws, size_t ws_elems) {
  gk::GemmArgs a;
  a.M = M; a.N = N; a.K = K;
  a.A = A; a.lda = lda; a.a_t = a_t != 0;
  a.B = B; a.ldb = ldb; a.b_t = b_t != 0;
  a.kind = kind; a.out = out; a.ldo = ldo; a.out2 = out2; a.aux = aux; a.bias = bias;
  a.alpha = alpha; a.beta = beta; a.dt = dt;
  a.splitk_ws = ws; a.splitk_ws_elems = ws_elems;
  return (int)gk::gemm(a, nullptr);
}

// Weight gradient out = alpha A^T B + beta out (A [K][M], B [K][N]) with the
// bias gradient dbias = beta dbias + sum_k A[k][:] (alpha must be 1 then).
EMU_API int emu_gemm_wgrad_bias(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* out,
                                int ldo, float alpha, float beta, int dt, float* ws, size_t ws_elems,
                                float* dbias, float* colsum_ws) {
  gk::GemmArgs a;
  a.M = M; a.N = N; a.K = K;
  a.A = A; a.lda = lda; a.a_t = true;
  a.B = B; a.ldb = ldb; a.b_t = true;
  a.kind = gk::EPI_WGRAD; a.out = out; a.ldo = ldo; a.out2 = nullptr; a.aux = nullptr; a.bias = nullptr;
  a.alpha = alpha; a.beta = beta; a.dt = dt;
  a.splitk_ws = ws; a.splitk_ws_elems = ws_elems;
  a.dbias = dbias; a.colsum_ws = colsum_ws;
  return (int)gk::gemm(a, nullptr);
}

EMU_API size_t emu_gemm_splitk_ws_elems(int M, int N, int K) { return gk::gemm_splitk_ws_elems(M, N, K); }

EMU_API int emu_attn_fwd(const void* qkv, void* o, float* lse, int B, int T, int H, int hd, int dt) {
  return (int)gk::attn_fwd(qkv, o, lse, B, T, H, hd, dt, nullptr);
}

EMU_API size_t emu_attn_bwd_ws(int B, int T, int H) { return gk::attn_bwd_workspace(B, T, H); }

EMU_API int emu_attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse, void* dqkv,
                         float* ws, int B, int T, int H, int hd, int dt) {
  return (int)gk::attn_bwd(qkv, o, dout, lse, dqkv, ws, B, T, H, hd, dt, nullptr);
}

EMU_API int emu_xent(void* logits, int dt, int ld, int V, int vt, const int32_t* tgt, float* losses,
                     float scale, int want_grad, int M, int* flag) {
  return (int)gk::xent(logits, dt, ld, V, vt, tgt, losses, scale, want_grad != 0, M, flag, nullptr, nullptr);
}

EMU_API size_t emu_embed_bwd_ws(int M, int C) { return gk::embed_bwd_workspace(M, C); }

EMU_API int emu_embed_bwd(const int32_t* tok, const float* dh, float* dwte, float* dwpe, int B, int T, int C,
                          int V, int block_size, float beta, void* ws) {
  return (int)gk::embed_bwd(tok, dh, dwte, dwpe, B, T, C, V, block_size, beta, ws, nullptr);
}

EMU_API int emu_ln_fwd(const float* x, const float* w, const float* b, void* y, int dt, float* mean,
                       float* rstd, int M, int C, float eps) {
  return (int)gk::ln_fwd(x, w, b, y, dt, mean, rstd, M, C, eps, nullptr);
}

EMU_API int emu_ln_bwd_part_floats(int M, int C) { return gk::ln_bwd_part_floats(M, C); }

EMU_API int emu_ln_bwd(const float* x, const float* mean, const float* rstd, const float* w, const void* dy,
                       int dt, float* dres, void* dres_act, int accum, float* part, int M, int C,
                       float* dw, float* db, float beta) {
  hipError_t e = gk::ln_bwd(x, mean, rstd, w, dy, dt, dres, dres_act, accum != 0, part, M, C, nullptr);
  if (e != hipSuccess) return (int)e;
  return (int)gk::ln_param_grad_reduce(part, gk::ln_bwd_blocks(M), dw, db, C, beta, nullptr);
}

EMU_API size_t emu_colsum_part_floats(int M, int N) { return gk::colsum_part_floats(M, N); }

EMU_API int emu_colsum(const void* X, int dt, int M, int N, int ldx, float* db, float beta, float* part) {
  return (int)gk::colsum(X, dt, M, N, ldx, db, beta, part, nullptr);
}

