// Host-side launch functions of the HIP kernels (internal to the library).
// Every function enqueues on `st` and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gk {

// Storage type of activations and GEMM / attention operands.
enum ActType { ACT_F32 = 0, ACT_BF16 = 1, ACT_F16 = 2 };

// ---------------------------------------------------------------- elementwise
// h[m, :] = wte[clamp(tok[m]), :] + wpe[pos0 + m % T, :]; flags bad ids in *flag.
hipError_t embed_fwd(const int32_t* tok, const float* wte, const float* wpe, float* h, int M, int T,
                     int C, int V, int* flag, hipStream_t st, int pos0 = 0);
// LayerNorm forward of fp32 rows; y in the activation type dt (ActType);
// mean / rstd per row.
hipError_t ln_fwd(const float* x, const float* w, const float* b, void* y, int dt, float* mean,
                  float* rstd, int M, int C, float eps, hipStream_t st);
// LayerNorm backward: dres = (accum ? dres : 0) + dx; dres_act = copy of
// dres in the activation type; per-block dw/db partials into part
// ([nblk, 2, C]); then ln_param_grad_reduce folds them into dw/db.
int ln_bwd_blocks(int M);
int ln_bwd_part_floats(int M, int C);  // workspace floats for part (+ reduction slices)
hipError_t ln_bwd(const float* x, const float* mean, const float* rstd, const float* w,
                  const void* dy, int dt, float* dres, void* dres_act, bool accum,
                  float* part, int M, int C, hipStream_t st);
hipError_t ln_param_grad_reduce(const float* part, int nblk, float* dw, float* db, int C,
                                float beta, hipStream_t st);
// Column sums of an activation matrix X[M, N] (row stride ldx): db = beta *
// db + sum_m X[m, :], deterministic two-stage reduction through `part`.
size_t colsum_part_floats(int M, int N);  // partials buffer of colsum for an M x N input
hipError_t colsum(const void* X, int dt, int M, int N, int ldx, float* db, float beta,
                  float* part, hipStream_t st);
// Fused softmax cross-entropy over the first V columns: per-row loss into
// losses[m]; when want_grad, logits row m is overwritten by
// (softmax - onehot) * scale (* dev_scale[0] when dev_scale is given: fp16
// only) and columns [V, ld) by 0.  Targets outside [0, vt) set *flag and
// are clamped.
hipError_t xent(void* logits, int dt, int ld, int V, int vt, const int32_t* tgt, float* losses, float scale,
                bool want_grad, int M, int* flag, const float* dev_scale, hipStream_t st);
// loss_out[0] = sum(losses) / M (float64 accumulation, fixed order);
// nonfinite -> flag bit 2.
hipError_t loss_reduce(const float* losses, int M, float* loss_out, int* flag, hipStream_t st);
// Embedding backward: dwte[id] += sum of dh rows with that id (sorted,
// deterministic), dwpe[t] = beta * dwpe[t] + sum_b dh[b, t] for t < T and
// beta * dwpe[t] for T <= t < block_size.
size_t embed_bwd_workspace(int M, int C);
hipError_t embed_bwd(const int32_t* tok, const float* dh, float* dwte, float* dwpe, int B, int T,
                     int C, int V, int block_size, float beta, void* ws, hipStream_t st);
// Sum of squares of n fp32 values into per-block float64 partials, then
// finalize: scal = {norm, coef, bc1, bc2, skip, t} (see adamw); with
// loss_scaling, the dynamic loss scale scal[10] and its step counter
// scal[11] are updated (elementwise.hip).
int sumsq_blocks();
hipError_t sumsq(const float* g, size_t n, double* part, hipStream_t st);
hipError_t norm_finalize(const double* part, int nblk, float clip, float beta1, float beta2,
                         float* scal, int* flag, bool loss_scaling, int growth_interval, hipStream_t st);
// Multi-tensor AdamW over chunk table entries {start, count, flags}.
struct AdamChunk {
  uint64_t start;
  uint32_t count;
  uint32_t flags;  // bit0 decay, bit1 write bf16 copy
};
// shadow_dt: type of the 16-bit weight copy (ACT_BF16 or ACT_F16).
hipError_t adamw(float* p, const float* g, float* m, float* v, uint16_t* shadow, int shadow_dt,
                 const AdamChunk* chunks, int nchunks, const float* scal, float lr, float beta1,
                 float beta2, float eps, float wd, hipStream_t st);
// 16-bit copy (bf16 or fp16 per dt, round to nearest even) of n fp32 values.
hipError_t to_h16(const float* x, uint16_t* y, size_t n, int dt, hipStream_t st);
hipError_t fill_f32(float* x, size_t n, float v, hipStream_t st);
hipError_t copy_f32_to_act(const float* x, void* y, int dt, size_t n, hipStream_t st);

// ---------------------------------------------------------------- GEMM
// C[m, n] = sum_k A(m, k) * B(n, k) with
//   A(m, k) = a_t ? A[k * lda + m] : A[m * lda + k]
//   B(n, k) = b_t ? B[k * ldb + n] : B[n * ldb + k]
// followed by an epilogue.  bf16 operands use MFMA with fp32 accumulation;
// fp32 operands use an FMA kernel.
enum EpiKind {
  EPI_STORE = 0,       // out(act) = alpha * acc + bias
  EPI_LOGITS = 1,      // out(act) = acc (classifier)
  EPI_GELU = 2,        // u = acc + bias -> out(act); gelu(u) -> out2(act)
  EPI_RESID = 3,       // outf(fp32) = resid(fp32) + acc + bias
  EPI_DGELU = 4,       // out(act) = acc * gelu'(aux(act))
  EPI_WGRAD = 5        // outf(fp32) = alpha * acc + beta * outf
};
struct GemmArgs {
  int M, N, K;
  const void* A; int lda; bool a_t;
  const void* B; int ldb; bool b_t;
  int kind;
  void* out; int ldo;
  void* out2;            // EPI_GELU: gelu output (same ld)
  const void* aux;       // EPI_DGELU: pre-activation u (same ld); EPI_RESID: residual in (fp32)
  const float* bias;
  float alpha, beta;
  int dt;                // operand / activation storage type (ActType)
  float* splitk_ws;      // EPI_WGRAD split-K partials (may be null -> no split)
  size_t splitk_ws_elems;
  // EPI_WGRAD only, alpha == 1: also dbias[r] = beta dbias[r] + sum_k A[k][r]
  // (the bias gradient: column sums of dY).  The TN kernel forms it from
  // the A fragments it holds; other paths run colsum on A with colsum_ws
  // (colsum_part_floats(K, M) floats).  Null: no bias gradient.
  float* dbias = nullptr;
  float* colsum_ws = nullptr;
};
hipError_t gemm(const GemmArgs& a, hipStream_t st);
// Workspace floats that EPI_WGRAD may use for split-K at this size (the
// bias-gradient partials included).
size_t gemm_splitk_ws_elems(int M, int N, int K);

// ---------------------------------------------------------------- attention
// Causal multi-head attention on the packed qkv buffer [B*T, 3C] (q, k, v
// thirds, heads contiguous hd-wide).  Forward writes o [B*T, C] and
// lse [B, H, T] (log2 units).  Backward writes dqkv [B*T, 3C]; needs a
// workspace of attn_bwd_workspace floats.
hipError_t attn_fwd(const void* qkv, void* o, float* lse, int B, int T, int H, int hd, int dt,
                    hipStream_t st);
size_t attn_bwd_workspace(int B, int T, int H);
hipError_t attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse, void* dqkv,
                    float* ws, int B, int T, int H, int hd, int dt, hipStream_t st);

// ---------------------------------------------------------------- sampling with a key/value cache
// cache[b][t0 + i][0:2C] = qkv[b * n + i][C:3C] (keys and values of n new
// positions of B sequences; cache rows of max_seq positions).
hipError_t kv_store(const void* qkv, void* cache, int B, int n, int t0, int Tmax, int C, int dt,
                    hipStream_t st);
// out[b] = attention of query qkv[b][0:C] over the keys / values of cache
// positions 0 .. nkeys-1 of sequence b.
hipError_t attn_decode(const void* qkv, const void* cache, void* out, int B, int H, int hd, int Tmax, int nkeys,
                       int dt, hipStream_t st);
// tok[b * tok_stride] = inverse-CDF sample of softmax(z[0:V]) at u[b * u_stride]
// for the logits row b * row_stride + row0; logprob (nullable) gets its
// log-probability.
hipError_t sample(const void* logits, int dt, int ld, int row_stride, int row0, int V, int B, const float* u,
                  int u_stride, int32_t* tok, int tok_stride, float* logprob, int lp_stride, hipStream_t st);

}  // namespace gk
