// Bandwidth-bound kernels of the training step: embeddings, LayerNorm,
// fused softmax cross-entropy, bias-gradient column sums, global gradient
// norm and the multi-tensor AdamW.  One wavefront (64 lanes) per row for the
// row-wise kernels; all reductions are in a fixed order (no float atomics),
// so results are bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace gk {



// ------------------------------------------------------------------ helpers
template <typename T> struct Vec4;
// Raw / load_raw / cvt split a load from its conversion, so a load can be
// issued ahead (a prefetch) without waiting for its data.
template <> struct Vec4<float> {
  typedef float4 Raw;
  static __device__ __forceinline__ Raw load_raw(const float* p) { return *(const float4*)p; }
  static __device__ __forceinline__ float4 cvt(Raw u) { return u; }
  static __device__ __forceinline__ float4 load(const float* p) { return *(const float4*)p; }
  static __device__ __forceinline__ void store(float* p, float a, float b, float c, float d) {
    *(float4*)p = make_float4(a, b, c, d);
  }
};
template <> struct Vec4<bf16> {
  typedef uint2 Raw;
  static __device__ __forceinline__ Raw load_raw(const bf16* p) { return *(const uint2*)p; }
  static __device__ __forceinline__ float4 cvt(Raw u) {
    return make_float4(bfbits2f(u.x & 0xffffu), bfbits2f(u.x >> 16), bfbits2f(u.y & 0xffffu),
                       bfbits2f(u.y >> 16));
  }
  static __device__ __forceinline__ float4 load(const bf16* p) {
    uint2 u = *(const uint2*)p;
    return make_float4(bfbits2f(u.x & 0xffffu), bfbits2f(u.x >> 16), bfbits2f(u.y & 0xffffu),
                       bfbits2f(u.y >> 16));
  }
  static __device__ __forceinline__ void store(bf16* p, float a, float b, float c, float d) {
    *(uint2*)p = make_uint2(pack_bf2(a, b), pack_bf2(c, d));
  }
};
template <> struct Vec4<f16> {
  typedef uint2 Raw;
  static __device__ __forceinline__ Raw load_raw(const f16* p) { return *(const uint2*)p; }
  static __device__ __forceinline__ float4 cvt(Raw u) {
    return make_float4(H16<f16>::lo(u.x), H16<f16>::hi(u.x), H16<f16>::lo(u.y), H16<f16>::hi(u.y));
  }
  static __device__ __forceinline__ float4 load(const f16* p) {
    uint2 u = *(const uint2*)p;
    return make_float4(H16<f16>::lo(u.x), H16<f16>::hi(u.x), H16<f16>::lo(u.y), H16<f16>::hi(u.y));
  }
  static __device__ __forceinline__ void store(f16* p, float a, float b, float c, float d) {
    *(uint2*)p = make_uint2(H16<f16>::pack2(a, b), H16<f16>::pack2(c, d));
  }
};

// flag bits
enum { FLAG_TOKEN = 1, FLAG_TARGET = 2, FLAG_LOSS = 4, FLAG_NORM = 8, FLAG_OVERFLOW = 16 };

// ------------------------------------------------------------------ embedding forward
// "From Scratch: Building GPT-2 ...", Key Features: token and positional
// embeddings, summed.
__global__ __launch_bounds__(256) void k_embed_fwd(const int32_t* __restrict__ tok,
                                                   const float* __restrict__ wte,
                                                   const float* __restrict__ wpe,
                                                   float* __restrict__ h, int M, int T, int C,
                                                   int V, int* flag, int pos0) {
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= M) return;
  int id = tok[row];
  if (id < 0 || id >= V) {
    if (lane == 0) atomicOr(flag, FLAG_TOKEN);
    id = id < 0 ? 0 : V - 1;
  }
  int t = pos0 + row % T;
  const float4* a = (const float4*)(wte + (size_t)id * C);
  const float4* b = (const float4*)(wpe + (size_t)t * C);
  float4* o = (float4*)(h + (size_t)row * C);
  for (int c = lane; c < C / 4; c += 64) {
    float4 x = a[c], y = b[c];
    o[c] = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
  }
}

hipError_t embed_fwd(const int32_t* tok, const float* wte, const float* wpe, float* h, int M, int T,
                     int C, int V, int* flag, hipStream_t st, int pos0) {
  k_embed_fwd<<<cdiv(M, 4), 256, 0, st>>>(tok, wte, wpe, h, M, T, C, V, flag, pos0);
  return hipGetLastError();
}

// ------------------------------------------------------------------ LayerNorm forward
// FULL: C is exactly 256 NV (each lane's NV float4 columns all exist), so the
// per-chunk column tests go away; other widths take NV = 4 with the tests.
template <bool FULL>
__device__ __forceinline__ bool ln_in(int c, int C) { return FULL || c < C; }

// y = (x - mean) * rstd * w + b, biased variance, one wave per row.  The row
// stays in registers (NV float4 per lane, C <= 256 * NV).  Each wave walks
// the rows wave_id, wave_id + nwaves, ... with w and b held in registers
// and the next row's loads issued before the current row's reductions.
constexpr int LN_FWD_BLOCKS = 1024;

template <typename TO, int NV, bool FULL>
__global__ __launch_bounds__(256) void k_ln_fwd(const float* __restrict__ x,
                                                const float* __restrict__ w,
                                                const float* __restrict__ b, TO* __restrict__ y,
                                                float* __restrict__ mean, float* __restrict__ rstd,
                                                int M, int C, float eps) {
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x * 4;
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  float4 ww[NV], bb[NV], v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int c = (lane + i * 64) * 4;
    ww[i] = ln_in<FULL>(c, C) ? *(const float4*)(w + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    bb[i] = ln_in<FULL>(c, C) ? *(const float4*)(b + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    v[i] = ln_in<FULL>(c, C) ? *(const float4*)(x + (size_t)row * C + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float invC = 1.0f / (float)C;
  for (; row < M; row += stride) {
    const bool more = row + stride < M;
    // The next row's loads, issued before this row's reductions and without
    // a branch around them (the last row reloads itself): loads under a
    // branch leave a register copy at the join that waits for them, and the
    // prefetch would then overlap nothing.
    const int rn = more ? row + stride : row;
    float4 vn[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int c = (lane + i * 64) * 4;
      vn[i] = ln_in<FULL>(c, C) ? *(const float4*)(x + (size_t)rn * C + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    const float mu = wave_sum(s) * invC;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int c = (lane + i * 64) * 4;
      if (ln_in<FULL>(c, C)) {
        float a0 = v[i].x - mu, a1 = v[i].y - mu, a2 = v[i].z - mu, a3 = v[i].w - mu;
        q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
      }
    }
    const float rs = rsqrtf(wave_sum(q) * invC + eps);
    TO* yr = y + (size_t)row * C;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int c = (lane + i * 64) * 4;
      if (ln_in<FULL>(c, C))
        Vec4<TO>::store(yr + c, (v[i].x - mu) * rs * ww[i].x + bb[i].x, (v[i].y - mu) * rs * ww[i].y + bb[i].y,
                        (v[i].z - mu) * rs * ww[i].z + bb[i].z, (v[i].w - mu) * rs * ww[i].w + bb[i].w);
    }
    if (lane == 0) {
      mean[row] = mu;
      rstd[row] = rs;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = vn[i];
  }
}

template <typename TO, int NV, bool FULL>
static void ln_fwd_launch(int g, hipStream_t st, const float* x, const float* w, const float* b, void* y,
                          float* mean, float* rstd, int M, int C, float eps) {
  k_ln_fwd<TO, NV, FULL><<<g, 256, 0, st>>>(x, w, b, (TO*)y, mean, rstd, M, C, eps);
}
// the exact-width variant for C = 256, 512, 768, 1024, else NV = 4 with tests
template <typename TO>
static void ln_fwd_width(int g, hipStream_t st, const float* x, const float* w, const float* b, void* y,
                         float* mean, float* rstd, int M, int C, float eps) {
  if (C == 256) ln_fwd_launch<TO, 1, true>(g, st, x, w, b, y, mean, rstd, M, C, eps);
  else if (C == 512) ln_fwd_launch<TO, 2, true>(g, st, x, w, b, y, mean, rstd, M, C, eps);
  else if (C == 768) ln_fwd_launch<TO, 3, true>(g, st, x, w, b, y, mean, rstd, M, C, eps);
  else if (C == 1024) ln_fwd_launch<TO, 4, true>(g, st, x, w, b, y, mean, rstd, M, C, eps);
  else ln_fwd_launch<TO, 4, false>(g, st, x, w, b, y, mean, rstd, M, C, eps);
}

hipError_t ln_fwd(const float* x, const float* w, const float* b, void* y, int dt, float* mean,
                  float* rstd, int M, int C, float eps, hipStream_t st) {
  if (C % 4 || C > 1024) return hipErrorInvalidValue;
  int g = min(cdiv(M, 4), LN_FWD_BLOCKS);
  if (dt == ACT_BF16) ln_fwd_width<bf16>(g, st, x, w, b, y, mean, rstd, M, C, eps);
  else if (dt == ACT_F16) ln_fwd_width<f16>(g, st, x, w, b, y, mean, rstd, M, C, eps);
  else ln_fwd_width<float>(g, st, x, w, b, y, mean, rstd, M, C, eps);
  return hipGetLastError();
}

// ------------------------------------------------------------------ LayerNorm backward
// With g = dy * w and xhat = (x - mean) * rstd:
//   dx = rstd * (g - mean_c(g) - xhat * mean_c(g * xhat))
//   dw = sum_rows dy * xhat, db = sum_rows dy.
// Each block handles a contiguous run of rows (4 waves interleaved) and
// writes one partial row of dw and db.
int ln_bwd_blocks(int M) {
  int nb = cdiv(M, 4);
  return nb < 512 ? nb : 512;
}

// ACC: add to the residual gradient already in dres (a template parameter:
// as a run-time flag, the compiler sank part of that load into the branch
// that uses it, where its wait drained the next row's prefetch).
template <typename TA, int NV, bool FULL, bool ACC>
__global__ __launch_bounds__(256) void k_ln_bwd(const float* __restrict__ x,
                                                const float* __restrict__ mean,
                                                const float* __restrict__ rstd,
                                                const float* __restrict__ w,
                                                const TA* __restrict__ dy, float* __restrict__ dres,
                                                TA* __restrict__ dres_act,
                                                float* __restrict__ part, int M, int C, int rpb) {
  __shared__ float red[2][4][1024];
  int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int r0 = blockIdx.x * rpb, r1 = min(r0 + rpb, M);
  float4 wr[NV], dwa[NV], dba[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int c = (lane + i * 64) * 4;
    wr[i] = ln_in<FULL>(c, C) ? *(const float4*)(w + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    dwa[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    dba[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float invC = 1.0f / (float)C;
  typedef typename Vec4<TA>::Raw Raw;
  // The wave's rows are row, row + 4, ...: the next row's x, dy, mean and
  // rstd are loaded before the current row's reductions, so each wave keeps
  // two rows of loads in flight.
  float4 xc[NV];
  Raw dc[NV];
  float mu = 0.f, rs = 0.f;
  auto load_row = [&](int r, float4 (&xo)[NV], Raw (&d_o)[NV], float& mu_o, float& rs_o) {
    mu_o = mean[r];
    rs_o = rstd[r];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int c = (lane + i * 64) * 4;
      if (ln_in<FULL>(c, C)) {
        xo[i] = *(const float4*)(x + (size_t)r * C + c);
        d_o[i] = Vec4<TA>::load_raw(dy + (size_t)r * C + c);
      }
    }
  };
  int row = r0 + wv;
  if (row < r1) load_row(row, xc, dc, mu, rs);
  for (; row < r1; row += 4) {
    const bool more = row + 4 < r1;
    float4 xn[NV];
    Raw dn[NV];
    float mun = 0.f, rsn = 0.f;
    // Unconditional, as in the forward (the last row reloads itself): loads
    // under a branch are waited for where the paths join, before this row's
    // reductions.
    load_row(more ? row + 4 : row, xn, dn, mun, rsn);
    float* dr = dres + (size_t)row * C;
    TA* da = dres_act + (size_t)row * C;
    float4 prev[NV];
    if constexpr (ACC) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        int c = (lane + i * 64) * 4;
        if (ln_in<FULL>(c, C)) prev[i] = *(const float4*)(dr + c);
      }
    }
    float4 xh[NV], gg[NV];
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int c = (lane + i * 64) * 4;
      if (ln_in<FULL>(c, C)) {
        const float4 xv = xc[i];
        const float4 d = Vec4<TA>::cvt(dc[i]);
        xh[i] = make_float4((xv.x - mu) * rs, (xv.y - mu) * rs, (xv.z - mu) * rs, (xv.w - mu) * rs);
        gg[i] = make_float4(d.x * wr[i].x, d.y * wr[i].y, d.z * wr[i].z, d.w * wr[i].w);
        sg += (gg[i].x + gg[i].y) + (gg[i].z + gg[i].w);
        sgx += (gg[i].x * xh[i].x + gg[i].y * xh[i].y) + (gg[i].z * xh[i].z + gg[i].w * xh[i].w);
        dwa[i].x += d.x * xh[i].x; dwa[i].y += d.y * xh[i].y;
        dwa[i].z += d.z * xh[i].z; dwa[i].w += d.w * xh[i].w;
        dba[i].x += d.x; dba[i].y += d.y; dba[i].z += d.z; dba[i].w += d.w;
      }
    }
    float mg = wave_sum(sg) * invC, mgx = wave_sum(sgx) * invC;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int c = (lane + i * 64) * 4;
      if (ln_in<FULL>(c, C)) {
        float4 o = make_float4(rs * (gg[i].x - mg - xh[i].x * mgx), rs * (gg[i].y - mg - xh[i].y * mgx),
                               rs * (gg[i].z - mg - xh[i].z * mgx), rs * (gg[i].w - mg - xh[i].w * mgx));
        if constexpr (ACC) {
          o.x += prev[i].x; o.y += prev[i].y; o.z += prev[i].z; o.w += prev[i].w;
        }
        *(float4*)(dr + c) = o;
        Vec4<TA>::store(da + c, o.x, o.y, o.z, o.w);
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      xc[i] = xn[i];
      dc[i] = dn[i];
    }
    mu = mun;
    rs = rsn;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int c = (lane + i * 64) * 4;
    if (ln_in<FULL>(c, C)) {
      *(float4*)&red[0][wv][c] = dwa[i];
      *(float4*)&red[1][wv][c] = dba[i];
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += 256) {
    float a = (red[0][0][c] + red[0][1][c]) + (red[0][2][c] + red[0][3][c]);
    float b = (red[1][0][c] + red[1][1][c]) + (red[1][2][c] + red[1][3][c]);
    part[((size_t)blockIdx.x * 2 + 0) * C + c] = a;
    part[((size_t)blockIdx.x * 2 + 1) * C + c] = b;
  }
}

template <typename TA, int NV, bool FULL>
static void ln_bwd_launch(int nb, hipStream_t st, const float* x, const float* mean, const float* rstd,
                          const float* w, const void* dy, float* dres, void* dres_act, bool accum, float* part,
                          int M, int C, int rpb) {
  if (accum)
    k_ln_bwd<TA, NV, FULL, true><<<nb, 256, 0, st>>>(x, mean, rstd, w, (const TA*)dy, dres, (TA*)dres_act,
                                                     part, M, C, rpb);
  else
    k_ln_bwd<TA, NV, FULL, false><<<nb, 256, 0, st>>>(x, mean, rstd, w, (const TA*)dy, dres, (TA*)dres_act,
                                                      part, M, C, rpb);
}
template <typename TA>
static void ln_bwd_width(int nb, hipStream_t st, const float* x, const float* mean, const float* rstd,
                         const float* w, const void* dy, float* dres, void* dres_act, bool accum, float* part,
                         int M, int C, int rpb) {
  if (C == 256) ln_bwd_launch<TA, 1, true>(nb, st, x, mean, rstd, w, dy, dres, dres_act, accum, part, M, C, rpb);
  else if (C == 512) ln_bwd_launch<TA, 2, true>(nb, st, x, mean, rstd, w, dy, dres, dres_act, accum, part, M, C, rpb);
  else if (C == 768) ln_bwd_launch<TA, 3, true>(nb, st, x, mean, rstd, w, dy, dres, dres_act, accum, part, M, C, rpb);
  else if (C == 1024) ln_bwd_launch<TA, 4, true>(nb, st, x, mean, rstd, w, dy, dres, dres_act, accum, part, M, C, rpb);
  else ln_bwd_launch<TA, 4, false>(nb, st, x, mean, rstd, w, dy, dres, dres_act, accum, part, M, C, rpb);
}

hipError_t ln_bwd(const float* x, const float* mean, const float* rstd, const float* w,
                  const void* dy, int dt, float* dres, void* dres_act, bool accum,
                  float* part, int M, int C, hipStream_t st) {
  if (C % 4 || C > 1024) return hipErrorInvalidValue;
  int nb = ln_bwd_blocks(M);
  int rpb = cdiv(M, nb);
  if (dt == ACT_BF16) ln_bwd_width<bf16>(nb, st, x, mean, rstd, w, dy, dres, dres_act, accum, part, M, C, rpb);
  else if (dt == ACT_F16) ln_bwd_width<f16>(nb, st, x, mean, rstd, w, dy, dres, dres_act, accum, part, M, C, rpb);
  else ln_bwd_width<float>(nb, st, x, mean, rstd, w, dy, dres, dres_act, accum, part, M, C, rpb);
  return hipGetLastError();
}

// dw[c] = beta * dw[c] + sum_b part[b][0][c]; db likewise.  Stage 1: blocks
// of 64 columns x 4 row groups sum a slice of the partial rows; stage 2 sums
// the slices (fixed order, so deterministic).
constexpr int LNR_SLICES = 16;

__global__ __launch_bounds__(256) void k_ln_param_reduce1(const float* __restrict__ part, int nblk,
                                                          int C, float* __restrict__ part2) {
  __shared__ float red[4][64];
  int c = blockIdx.x * 64 + (threadIdx.x & 63);
  int wb = blockIdx.y;                  // 0: dw, 1: db
  int grp = threadIdx.x >> 6;
  int per = (nblk + LNR_SLICES - 1) / LNR_SLICES;
  int r0 = blockIdx.z * per, r1 = min(r0 + per, nblk);
  float s = 0.f;
  if (c < C) {  // rows r0 + grp, + 4, ... in order; four loads in flight at a time
    int r = r0 + grp;
    for (; r + 12 < r1; r += 16) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = part[((size_t)(r + 4 * u) * 2 + wb) * C + c];
#pragma unroll
      for (int u = 0; u < 4; ++u) s += v[u];
    }
    for (; r < r1; r += 4) s += part[((size_t)r * 2 + wb) * C + c];
  }
  red[grp][threadIdx.x & 63] = s;
  __syncthreads();
  if (grp == 0 && c < C) {
    int l = threadIdx.x & 63;
    part2[((size_t)blockIdx.z * 2 + wb) * C + c] = (red[0][l] + red[1][l]) + (red[2][l] + red[3][l]);
  }
}

__global__ __launch_bounds__(256) void k_ln_param_reduce2(const float* __restrict__ part2, int C,
                                                          float* dw, float* db, float beta) {
  int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  float* out = blockIdx.y == 0 ? dw : db;
  float s = 0.f;
  for (int z = 0; z < LNR_SLICES; ++z) s += part2[((size_t)z * 2 + blockIdx.y) * C + c];
  out[c] = (beta != 0.f ? beta * out[c] : 0.f) + s;
}

hipError_t ln_param_grad_reduce(const float* part, int nblk, float* dw, float* db, int C,
                                float beta, hipStream_t st) {
  // part2 lives right after the nblk partial rows in the same workspace
  float* part2 = const_cast<float*>(part) + (size_t)nblk * 2 * C;
  k_ln_param_reduce1<<<dim3(cdiv(C, 64), 2, LNR_SLICES), 256, 0, st>>>(part, nblk, C, part2);
  k_ln_param_reduce2<<<dim3(cdiv(C, 256), 2), 256, 0, st>>>(part2, C, dw, db, beta);
  return hipGetLastError();
}

int ln_bwd_part_floats(int M, int C) { return (ln_bwd_blocks(M) + LNR_SLICES) * 2 * C; }

// ------------------------------------------------------------------ bias-gradient column sums
// db[n] = beta db[n] + sum_m X[m][n] in two deterministic stages.  Stage 1
// splits the rows into R slices so that the grid has about 1024 blocks
// whatever N is (a block covers 256 columns of one slice: 32 threads x 8
// columns, 16-byte loads, 8 row groups); stage 2 has 16 row groups per 16
// columns walk the R partial rows, four loads in flight each, and combines
// the groups in a fixed order.  R * N <= 1024 * 256 floats.
constexpr int COLSUM_BLOCKS = 1024;

static int colsum_slices(int M, int N) {
  const int nb = cdiv(N, 256);
  int r = COLSUM_BLOCKS / nb;
  r = r < 1 ? 1 : r;
  const int rmax = cdiv(M, 16);  // at least 16 rows per slice
  return r < rmax ? r : rmax;
}

size_t colsum_part_floats(int M, int N) { return (size_t)colsum_slices(M, N) * N; }

template <typename T>
__global__ __launch_bounds__(256) void k_colsum_part(const T* __restrict__ X, int M, int N, int ldx,
                                                     int rows_per, float* __restrict__ part) {
  constexpr int E = 16 / sizeof(T);           // columns per 16-byte load
  constexpr int TPR = 256 / 8;                // threads across one row segment
  __shared__ float red[8][TPR * 8];
  const int tc = threadIdx.x % TPR, g = threadIdx.x / TPR;
  const int n0 = blockIdx.x * (TPR * 8);
  const int r0 = blockIdx.y * rows_per, r1 = min(r0 + rows_per, M);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c8 = 0; c8 < 8; c8 += E) {
    int n = n0 + tc * 8 + c8;
    if (n >= N) break;
    for (int m = r0 + g; m < r1; m += 8) {
      uint4 u = *(const uint4*)(X + (size_t)m * ldx + n);
      if constexpr (E == 8) {
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[c8 + j] += (j & 1) ? H16<T>::hi(w[j >> 1]) : H16<T>::lo(w[j >> 1]);
      } else {
        acc[c8 + 0] += __uint_as_float(u.x); acc[c8 + 1] += __uint_as_float(u.y);
        acc[c8 + 2] += __uint_as_float(u.z); acc[c8 + 3] += __uint_as_float(u.w);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[g][tc * 8 + j] = acc[j];
  __syncthreads();
  int col = threadIdx.x;  // 256 columns of this block
  int n = n0 + col;
  if (n < N) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += red[k][col];
    part[(size_t)blockIdx.y * N + n] = s;
  }
}

__global__ __launch_bounds__(256) void k_colsum_final(const float* __restrict__ part, int R, int N,
                                                      float* db, float beta) {
  __shared__ float red[16][16];
  const int c = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int n = blockIdx.x * 16 + c;
  float s = 0.f;
  if (n < N) {  // rows grp, grp + 16, ... in order
    int r = grp;
    for (; r + 48 < R; r += 64) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = part[(size_t)(r + 16 * u) * N + n];
#pragma unroll
      for (int u = 0; u < 4; ++u) s += v[u];
    }
    for (; r < R; r += 16) s += part[(size_t)r * N + n];
  }
  red[grp][c] = s;
  __syncthreads();
  if (grp == 0 && n < N) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += red[k][c];
    db[n] = (beta != 0.f ? beta * db[n] : 0.f) + t;
  }
}

hipError_t colsum(const void* X, int dt, int M, int N, int ldx, float* db, float beta,
                  float* part, hipStream_t st) {
  if (N % 8 || ldx % 8 || M < 1) return hipErrorInvalidValue;
  int R = colsum_slices(M, N);
  int rows_per = cdiv(M, R);
  R = cdiv(M, rows_per);  // slices that hold rows
  dim3 g(cdiv(N, 256), R);
  if (dt == ACT_BF16)
    k_colsum_part<bf16><<<g, 256, 0, st>>>((const bf16*)X, M, N, ldx, rows_per, part);
  else if (dt == ACT_F16)
    k_colsum_part<f16><<<g, 256, 0, st>>>((const f16*)X, M, N, ldx, rows_per, part);
  else
    k_colsum_part<float><<<g, 256, 0, st>>>((const float*)X, M, N, ldx, rows_per, part);
  k_colsum_final<<<cdiv(N, 16), 256, 0, st>>>(part, R, N, db, beta);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fused softmax cross-entropy
// "Let's reproduce GPT-2 (124M)" chapter "cross entropy loss": per row
// loss = logsumexp(z) - z[y]; gradient (softmax(z) - onehot(y)) * scale
// written over the logits.  One 256-thread block per row; the row is held
// in registers (NCH 16-byte chunks per thread) so HBM sees one read and one
// write of it.
__device__ __forceinline__ float block_reduce_max(float v, float* sh) {
  v = wave_max(v);
  int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[wv] = v;
  __syncthreads();
  return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}
__device__ __forceinline__ float block_reduce_sum(float v, float* sh) {
  v = wave_sum(v);
  int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[wv] = v;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

template <typename T> struct Chunk16 {
  static constexpr int E = 16 / sizeof(T);
};

template <typename T>
__device__ __forceinline__ float chunk_elem(const uint4& u, int j);
template <>
__device__ __forceinline__ float chunk_elem<float>(const uint4& u, int j) {
  uint32_t w = j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w;
  return __uint_as_float(w);
}
template <>
__device__ __forceinline__ float chunk_elem<bf16>(const uint4& u, int j) {
  uint32_t w = (j >> 1) == 0 ? u.x : (j >> 1) == 1 ? u.y : (j >> 1) == 2 ? u.z : u.w;
  return bfbits2f((j & 1) ? (w >> 16) : (w & 0xffffu));
}
template <>
__device__ __forceinline__ float chunk_elem<f16>(const uint4& u, int j) {
  uint32_t w = (j >> 1) == 0 ? u.x : (j >> 1) == 1 ? u.y : (j >> 1) == 2 ? u.z : u.w;
  return (j & 1) ? H16<f16>::hi(w) : H16<f16>::lo(w);
}

// Element j of a chunk through shift and mask amounts the compiler cannot
// see as constants (read from LDS after a barrier).  The cross-entropy
// converts its register-held row afresh in each pass this way: otherwise
// the compiler keeps all 200 converted values of the first pass live for
// the later ones, which takes the kernel to 256 registers and one wave
// per SIMD.  `sh` is 16 and `mask` 0xffff0000.
struct Opaque {
  uint32_t sh, mask;
};
template <typename T>
__device__ __forceinline__ float chunk_elem_o(const uint4& u, int j, Opaque o);
template <>
__device__ __forceinline__ float chunk_elem_o<float>(const uint4& u, int j, Opaque) {
  return chunk_elem<float>(u, j);
}
template <>
__device__ __forceinline__ float chunk_elem_o<bf16>(const uint4& u, int j, Opaque o) {
  uint32_t w = (j >> 1) == 0 ? u.x : (j >> 1) == 1 ? u.y : (j >> 1) == 2 ? u.z : u.w;
  return __uint_as_float((j & 1) ? (w & o.mask) : (w << o.sh));
}
template <>
__device__ __forceinline__ float chunk_elem_o<f16>(const uint4& u, int j, Opaque o) {
  uint32_t w = (j >> 1) == 0 ? u.x : (j >> 1) == 1 ? u.y : (j >> 1) == 2 ? u.z : u.w;
  return (j & 1) ? H16<f16>::lo(w >> o.sh) : H16<f16>::lo(w & ~o.mask);
}

template <typename T>
__device__ __forceinline__ uint4 chunk_pack(const float* f);
template <>
__device__ __forceinline__ uint4 chunk_pack<float>(const float* f) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                    __float_as_uint(f[3]));
}
template <>
__device__ __forceinline__ uint4 chunk_pack<bf16>(const float* f) {
  return make_uint4(pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]), pack_bf2(f[4], f[5]),
                    pack_bf2(f[6], f[7]));
}
template <>
__device__ __forceinline__ uint4 chunk_pack<f16>(const float* f) {
  return make_uint4(H16<f16>::pack2(f[0], f[1]), H16<f16>::pack2(f[2], f[3]), H16<f16>::pack2(f[4], f[5]),
                    H16<f16>::pack2(f[6], f[7]));
}

constexpr float LOG2E = 1.4426950408889634f;

// A chunk of -inf values (the padding of a row past its V logits: it drops
// out of the max and the sum, and its gradient comes out as exp2(-inf) = 0).
template <typename T>
__device__ __forceinline__ uint4 chunk_neginf();
template <>
__device__ __forceinline__ uint4 chunk_neginf<float>() {
  return make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u);
}
template <>
__device__ __forceinline__ uint4 chunk_neginf<bf16>() {
  return make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
}
template <>
__device__ __forceinline__ uint4 chunk_neginf<f16>() {
  return make_uint4(0xfc00fc00u, 0xfc00fc00u, 0xfc00fc00u, 0xfc00fc00u);
}

// u with its elements n .. E-1 replaced by -inf (all of them for n <= 0).
template <typename T>
__device__ __forceinline__ uint4 chunk_keep(uint4 u, int n) {
  constexpr int E = Chunk16<T>::E;
  const uint4 ninf = chunk_neginf<T>();
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
  const uint32_t m[4] = {ninf.x, ninf.y, ninf.z, ninf.w};
  constexpr int PW = E / 4;  // elements per 32-bit word
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < PW; ++h)
      if (i * PW + h >= n) {
        const uint32_t mask = PW == 1 ? 0xffffffffu : (h ? 0xffff0000u : 0x0000ffffu);
        w[i] = (w[i] & ~mask) | (m[i] & mask);
      }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// DS: the gradient scale is also multiplied by *dev_scale (the dynamic
// loss scale of the fp16 workload, which lives on the device).
//
// The element loops carry no per-element tests: the one chunk that
// straddles V is padded with -inf at its load and chunks past V are all
// -inf, so the max, the sum and the gradient need no bounds checks.  The
// thread that owns the target's chunk reads the target logit itself before
// the first barrier (nobody else writes that chunk, and it writes it only
// after the reductions), skips that chunk in the gradient loop, and then
// reloads it and writes its gradient with the "- 1" applied.
template <typename T, int NCH, bool DS>
__global__ __launch_bounds__(256) void k_xent(T* __restrict__ logits, int ld, int V, int vt,
                                              const int32_t* __restrict__ tgt,
                                              float* __restrict__ losses, float scale,
                                              int want_grad, int* flag, const float* dev_scale) {
  constexpr int E = Chunk16<T>::E;
  __shared__ float sh[4];
  __shared__ float sh_zy;
  __shared__ Opaque sh_opq;
  int row = blockIdx.x;
  T* z = logits + (size_t)row * ld;
  int y = tgt[row];
  if (y < 0 || y >= vt) {
    if (threadIdx.x == 0) atomicOr(flag, FLAG_TARGET);
    y = y < 0 ? 0 : vt - 1;
  }
  if (threadIdx.x == 0) sh_opq = Opaque{16u, 0xffff0000u};
  const int ych = y / E;
  const int kown = ych / 256, town = ych % 256, yo = y - ych * E;  // the target's chunk: pass, thread, slot
  if ((int)threadIdx.x == town) sh_zy = to_f(z[y]);
  uint4 buf[NCH];
  // Every load first, without branches, so that the row's loads are all in
  // flight together: a load under a branch leaves a register copy where the
  // paths join, and that copy waits for the load before the next one is
  // issued.  A chunk at or past ld reads the row's first chunk instead (in
  // bounds) and is replaced below.  The tests on k alone are uniform
  // (scalar branches): only the last passes, whose chunks can reach ld or
  // V, pay for the per-thread tests.
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int e0 = (threadIdx.x + k * 256) * E;
    buf[k] = *(const uint4*)(z + (e0 < ld ? e0 : 0));
  }
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int e0 = (threadIdx.x + k * 256) * E;
    if ((k + 1) * 256 * E > ld && e0 >= ld) buf[k] = chunk_neginf<T>();
    if ((k + 1) * 256 * E > V && e0 + E > V) buf[k] = chunk_keep<T>(buf[k], V - e0);  // n <= 0: all -inf
  }
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < NCH; ++k)
#pragma unroll
    for (int j = 0; j < E; ++j) mx = fmaxf(mx, chunk_elem<T>(buf[k], j));
  mx = block_reduce_max(mx, sh);
  const float zy = sh_zy;
  const float mx2 = mx * LOG2E;
  float s = 0.f;
  const Opaque o2 = sh_opq;  // read after the reduction's barriers
#pragma unroll
  for (int k = 0; k < NCH; ++k)
#pragma unroll
    for (int j = 0; j < E; ++j) s += __builtin_amdgcn_exp2f(fmaf(chunk_elem_o<T>(buf[k], j, o2), LOG2E, -mx2));
  s = block_reduce_sum(s, sh);
  float lse = mx + __logf(s);
  if (threadIdx.x == 0) losses[row] = lse - zy;
  if (!want_grad) return;
  if constexpr (DS) scale *= dev_scale[0];
  const float lse2 = lse * LOG2E;
  const Opaque o3 = sh_opq;  // read after the second reduction's barriers
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int e0 = (threadIdx.x + k * 256) * E;
    if ((k + 1) * 256 * E <= ld || e0 < ld) {
      float f[E];
#pragma unroll
      for (int j = 0; j < E; ++j)
        f[j] = __builtin_amdgcn_exp2f(fmaf(chunk_elem_o<T>(buf[k], j, o3), LOG2E, -lse2)) * scale;
      if (!(k == kown && (int)threadIdx.x == town)) *(uint4*)(z + e0) = chunk_pack<T>(f);
    }
  }
  if ((int)threadIdx.x == town) {  // the target's chunk, untouched so far
    const int e0 = ych * E;
    uint4 u = *(const uint4*)(z + e0);
    if (e0 + E > V) u = chunk_keep<T>(u, V - e0);
    float f[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const float v = chunk_elem<T>(u, j);
      f[j] = (__builtin_amdgcn_exp2f(fmaf(v, LOG2E, -lse2)) - (j == yo ? 1.0f : 0.0f)) * scale;
    }
    *(uint4*)(z + e0) = chunk_pack<T>(f);
  }
}

// Streaming variant (row too long for registers): three passes over HBM.
template <typename T, bool DS>
__global__ __launch_bounds__(256) void k_xent_stream(T* __restrict__ logits, int ld, int V, int vt,
                                                     const int32_t* __restrict__ tgt,
                                                     float* __restrict__ losses, float scale,
                                                     int want_grad, int* flag, const float* dev_scale) {
  __shared__ float sh[4];
  int row = blockIdx.x;
  T* z = logits + (size_t)row * ld;
  int y = tgt[row];
  if (y < 0 || y >= vt) {
    if (threadIdx.x == 0) atomicOr(flag, FLAG_TARGET);
    y = y < 0 ? 0 : vt - 1;
  }
  __shared__ float sh_zy;
  float mx = -INFINITY;
  for (int e = threadIdx.x; e < V; e += 256) {
    float v = to_f(z[e]);
    mx = fmaxf(mx, v);
    if (e == y) sh_zy = v;
  }
  mx = block_reduce_max(mx, sh);
  const float zy = sh_zy;
  float s = 0.f;
  for (int e = threadIdx.x; e < V; e += 256)
    s += __builtin_amdgcn_exp2f((to_f(z[e]) - mx) * LOG2E);
  s = block_reduce_sum(s, sh);
  float lse = mx + __logf(s);
  if (threadIdx.x == 0) losses[row] = lse - zy;
  if (!want_grad) return;
  if constexpr (DS) scale *= dev_scale[0];
  __syncthreads();
  float lse2 = lse * LOG2E;
  for (int e = threadIdx.x; e < ld; e += 256) {
    float g = 0.f;
    if (e < V) {
      g = __builtin_amdgcn_exp2f(to_f(z[e]) * LOG2E - lse2);
      if (e == y) g -= 1.0f;
      g *= scale;
    }
    z[e] = from_f<T>(g);
  }
}

template <typename T, bool DS>
static hipError_t xent_t(T* logits, int ld, int V, int vt, const int32_t* tgt, float* losses, float scale,
                         bool want_grad, int M, int* flag, const float* ds, hipStream_t st) {
  constexpr int E = Chunk16<T>::E;
  int nch = cdiv(cdiv(ld, E), 256);
  int g = want_grad ? 1 : 0;
  if (nch <= 1)
    k_xent<T, 1, DS><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag, ds);
  else if (nch <= 2)
    k_xent<T, 2, DS><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag, ds);
  else if (nch <= 4)
    k_xent<T, 4, DS><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag, ds);
  else if (nch <= 8)
    k_xent<T, 8, DS><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag, ds);
  else if (nch <= 16)
    k_xent<T, 16, DS><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag, ds);
  else if (nch <= 25)
    k_xent<T, 25, DS><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag, ds);
  else
    k_xent_stream<T, DS><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag, ds);
  return hipGetLastError();
}

hipError_t xent(void* logits, int dt, int ld, int V, int vt, const int32_t* tgt, float* losses, float scale,
                bool want_grad, int M, int* flag, const float* dev_scale, hipStream_t st) {
  if (V < 1 || V > ld || vt < 1 || vt > V) return hipErrorInvalidValue;
  if (dt == ACT_F16) {
    if (ld % 8) return hipErrorInvalidValue;
    if (dev_scale)
      return xent_t<f16, true>((f16*)logits, ld, V, vt, tgt, losses, scale, want_grad, M, flag, dev_scale, st);
    return xent_t<f16, false>((f16*)logits, ld, V, vt, tgt, losses, scale, want_grad, M, flag, nullptr, st);
  }
  if (dev_scale) return hipErrorInvalidValue;  // dynamic loss scaling is the fp16 workload's
  if (dt == ACT_BF16) {
    if (ld % 8) return hipErrorInvalidValue;
    return xent_t<bf16, false>((bf16*)logits, ld, V, vt, tgt, losses, scale, want_grad, M, flag, nullptr, st);
  }
  if (ld % 4) return hipErrorInvalidValue;
  return xent_t<float, false>((float*)logits, ld, V, vt, tgt, losses, scale, want_grad, M, flag, nullptr, st);
}

// mean loss, float64 accumulation in a fixed order
__global__ __launch_bounds__(256) void k_loss_reduce(const float* __restrict__ losses, int M,
                                                     float* out, int* flag) {
  __shared__ double sh[4];
  double s = 0.0;
  for (int i = threadIdx.x; i < M; i += 256) s += losses[i];
  s = wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = ((sh[0] + sh[1]) + (sh[2] + sh[3])) / (double)M;
    out[0] = (float)t;
    if (!isfinite(t)) atomicOr(flag, FLAG_LOSS);
  }
}

hipError_t loss_reduce(const float* losses, int M, float* loss_out, int* flag, hipStream_t st) {
  k_loss_reduce<<<1, 256, 0, st>>>(losses, M, loss_out, flag);
  return hipGetLastError();
}

// ------------------------------------------------------------------ embedding backward
// Tied embedding ("parameter sharing wte and lm_head"): dwte[id] gains the
// sum of the residual-gradient rows of every position holding id.  The
// positions are sorted by (id, position) as 32-bit keys id << 15 | pos,
// then summed per id in sorted order: each chunk of 32 sorted entries sums
// its runs; runs that cross chunk borders are combined by a second kernel
// in chunk order.  No atomics, so the result is deterministic.
//
// The sort runs on the whole chip: blocks of 512 threads sort runs of 1024
// keys with a bitonic network in LDS, then merge passes double the run
// length until one run is left.  A merge pass places every key at its
// index within its run plus the number of keys of the partner run below it
// (a binary search; keys are distinct since positions are), so it needs no
// partitioning step and every thread works independently.
constexpr int SORT_MAX = 32768;  // positions per call (15 position bits)
constexpr int SORT_RUN = 1024;   // keys per block in the first stage
constexpr int SEG = 32;

size_t embed_bwd_workspace(int M, int C) {
  size_t nch = (size_t)cdiv(M, SEG);
  size_t mr = (size_t)cdiv(M, SORT_RUN) * SORT_RUN;
  return 2 * mr * 4 + 2 * nch * (size_t)C * 4 + 256;
}

__global__ __launch_bounds__(512) void k_sort_runs(const int32_t* __restrict__ tok, int M, int V,
                                                   uint32_t* __restrict__ out) {
  __shared__ uint32_t sk[SORT_RUN];
  const int base = blockIdx.x * SORT_RUN;
  for (int i = threadIdx.x; i < SORT_RUN; i += 512) {
    uint32_t key = 0xffffffffu;  // above every real key: ids < 65536, positions < 32768
    if (base + i < M) {
      int id = tok[base + i];
      id = id < 0 ? 0 : (id >= V ? V - 1 : id);
      key = ((uint32_t)id << 15) | (uint32_t)(base + i);
    }
    sk[i] = key;
  }
  __syncthreads();
  const int t = threadIdx.x;
  for (int k = 2; k <= SORT_RUN; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int i = (t / j) * 2 * j + (t % j), ixj = i + j;  // pair t of this stage
      const uint32_t a = sk[i], b = sk[ixj];
      const bool up = (i & k) == 0;
      if ((a > b) == up) {
        sk[i] = b;
        sk[ixj] = a;
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < SORT_RUN && base + i < M; i += 512) out[base + i] = sk[i];
}

// Sorted runs [a0, a0 + L) and [a0 + L, a0 + 2L) of `in` (clipped at M)
// merged into out[a0 ..): key x of one run lands at its offset in its run
// plus the count of keys below x in the other run.
__global__ __launch_bounds__(256) void k_merge_runs(const uint32_t* __restrict__ in, uint32_t* __restrict__ out,
                                                    int M, int L) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M) return;
  const uint32_t x = in[i];
  const int a0 = (i / (2 * L)) * 2 * L;
  const bool first = i < a0 + L;
  const int o0 = first ? a0 + L : a0;               // the other run
  const int o1 = first ? min(a0 + 2 * L, M) : a0 + L;
  int lo = o0, hi = o1;                              // first index in [o0, o1) with key > x
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (in[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  const int own = first ? i - a0 : i - (a0 + L);
  out[a0 + own + (lo - o0)] = x;
}

__device__ __forceinline__ int key_id(uint32_t k) { return (int)(k >> 15); }
__device__ __forceinline__ int key_pos(uint32_t k) { return (int)(k & 0x7fffu); }

// pass 1: per chunk of SEG sorted entries
__global__ __launch_bounds__(256) void k_emb_seg1(const uint32_t* __restrict__ keys,
                                                  const float* __restrict__ dh, float* dwte, int M,
                                                  int C, float* __restrict__ pfirst,
                                                  float* __restrict__ plast) {
  __shared__ uint32_t ks[SEG];
  int ch = blockIdx.x;
  int i0 = ch * SEG, i1 = min(i0 + SEG, M);
  if (threadIdx.x < i1 - i0) ks[threadIdx.x] = keys[i0 + threadIdx.x];
  __syncthreads();
  int prev_id = i0 > 0 ? key_id(keys[i0 - 1]) : -1;
  int next_id = i1 < M ? key_id(keys[i1]) : -1;
  const int n = i1 - i0;
  for (int c = threadIdx.x; c < C; c += 256) {
    // the chunk's SEG rows are loaded before any is summed, so their
    // latencies overlap; the sums below keep the sorted order
    float v[SEG];
#pragma unroll
    for (int i = 0; i < SEG; ++i) v[i] = i < n ? dh[(size_t)key_pos(ks[i]) * C + c] : 0.f;
    float acc = 0.f;
    bool at_start = true;  // the current run began at this chunk's first entry
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      if (i >= n) break;
      acc += v[i];
      const int id = key_id(ks[i]);
      const bool last = i == n - 1;
      const bool end = last || key_id(ks[i + 1]) != id;
      if (end) {
        const bool from_prev = at_start && prev_id == id;
        const bool to_next = last && next_id == id;
        if (!from_prev && !to_next) {
          dwte[(size_t)id * C + c] += acc;
        } else if (from_prev) {
          pfirst[(size_t)ch * C + c] = acc;  // continues a run from earlier chunks
        } else {
          plast[(size_t)ch * C + c] = acc;   // starts a run that continues
        }
        acc = 0.f;
        at_start = false;
      }
    }
  }
}

// pass 2: one block per chunk whose last run starts there and continues
__global__ __launch_bounds__(256) void k_emb_seg2(const uint32_t* __restrict__ keys,
                                                  float* dwte, int M, int C,
                                                  const float* __restrict__ pfirst,
                                                  const float* __restrict__ plast) {
  int ch = blockIdx.x;
  int nch = (M + SEG - 1) / SEG;
  int i0 = ch * SEG, i1 = min(i0 + SEG, M);
  int id = key_id(keys[i1 - 1]);
  if (i1 >= M || key_id(keys[i1]) != id) return;                       // does not continue
  if (i0 > 0 && key_id(keys[i0]) == id && key_id(keys[i0 - 1]) == id) return;  // not its start
  // The run's last chunk kend first: the block tests 256 chunk borders at a
  // time and keeps the smallest chunk where the run stops (the early returns
  // above depend on the chunk alone, so every thread reaches the barriers).
  // Then the sum over chunks ch + 1 .. kend, in order, four loads in flight.
  __shared__ int s_end;
  if (threadIdx.x == 0) s_end = nch;
  __syncthreads();
  for (int base = ch + 1; base < nch; base += 256) {
    const int k = base + (int)threadIdx.x;
    if (k < nch) {
      const int e = min((k + 1) * SEG, M);
      if (e >= M || key_id(keys[e]) != id || key_id(keys[e - 1]) != id) atomicMin(&s_end, k);
    }
    __syncthreads();
    const int found = s_end;
    __syncthreads();  // every thread has read s_end before the next round's updates
    if (found < nch) break;
  }
  const int kend = s_end;
  for (int c = threadIdx.x; c < C; c += 256) {
    float acc = plast[(size_t)ch * C + c];
    int k = ch + 1;
    for (; k + 3 <= kend; k += 4) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = pfirst[(size_t)(k + u) * C + c];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += v[u];
    }
    for (; k <= kend; ++k) acc += pfirst[(size_t)k * C + c];
    dwte[(size_t)id * C + c] += acc;
  }
}

// dwpe[t] = beta * dwpe[t] + sum_b dh[b, t]  (t < T), beta * dwpe[t] beyond T
__global__ __launch_bounds__(256) void k_dwpe(const float* __restrict__ dh, float* dwpe, int B,
                                              int T, int C, int block_size, float beta) {
  int c = blockIdx.x * 256 + threadIdx.x;
  int t = blockIdx.y;
  if (c >= C) return;
  float s = 0.f;
  if (t < T) {  // rows b = 0, 1, ... in order, four loads in flight
    int b = 0;
    for (; b + 4 <= B; b += 4) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = dh[((size_t)(b + u) * T + t) * C + c];
#pragma unroll
      for (int u = 0; u < 4; ++u) s += v[u];
    }
    for (; b < B; ++b) s += dh[((size_t)b * T + t) * C + c];
  }
  float* p = dwpe + (size_t)t * C + c;
  *p = (beta != 0.f ? beta * *p : 0.f) + s;
}

hipError_t embed_bwd(const int32_t* tok, const float* dh, float* dwte, float* dwpe, int B, int T,
                     int C, int V, int block_size, float beta, void* ws, hipStream_t st) {
  int M = B * T;
  if (M < 1 || M > SORT_MAX || V > 65536) return hipErrorInvalidValue;
  const size_t mr = (size_t)cdiv(M, SORT_RUN) * SORT_RUN;
  uint32_t* kb[2] = {(uint32_t*)ws, (uint32_t*)ws + mr};
  int nch = cdiv(M, SEG);
  float* pfirst = (float*)(kb[1] + mr);
  float* plast = pfirst + (size_t)nch * C;
  k_sort_runs<<<cdiv(M, SORT_RUN), 512, 0, st>>>(tok, M, V, kb[0]);
  int cur = 0;
  for (int L = SORT_RUN; L < M; L *= 2, cur ^= 1)
    k_merge_runs<<<cdiv(M, 256), 256, 0, st>>>(kb[cur], kb[cur ^ 1], M, L);
  const uint32_t* keys = kb[cur];
  k_emb_seg1<<<nch, 256, 0, st>>>(keys, dh, dwte, M, C, pfirst, plast);
  k_emb_seg2<<<nch, 256, 0, st>>>(keys, dwte, M, C, pfirst, plast);
  k_dwpe<<<dim3(cdiv(C, 256), block_size), 256, 0, st>>>(dh, dwpe, B, T, C, block_size, beta);
  return hipGetLastError();
}

// ------------------------------------------------------------------ gradient norm
// "Optimization Hyperparameters": clip the global gradient norm at 1.0.
int sumsq_blocks() { return 1024; }

__global__ __launch_bounds__(256) void k_sumsq(const float* __restrict__ g, size_t n,
                                               double* __restrict__ part) {
  __shared__ double sh[4];
  size_t n4 = n / 4;
  float s = 0.f;
  const float4* g4 = (const float4*)g;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  // four grid-strided loads in flight at a time, summed in the same order
  for (; i + 3 * stride < n4; i += 4 * stride) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = g4[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) s += (v[u].x * v[u].x + v[u].y * v[u].y) + (v[u].z * v[u].z + v[u].w * v[u].w);
  }
  for (; i < n4; i += stride) {
    float4 v = g4[i];
    s += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
  }
  if (blockIdx.x == 0)
    for (size_t i = n4 * 4 + threadIdx.x; i < n; i += 256) s += g[i] * g[i];
  double d = wave_sum_d((double)s);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = d;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

hipError_t sumsq(const float* g, size_t n, double* part, hipStream_t st) {
  k_sumsq<<<sumsq_blocks(), 256, 0, st>>>(g, n, part);
  return hipGetLastError();
}

// scal: [0] norm, [1] clip coefficient min(1, clip / (norm + 1e-6)),
// [2] 1 - beta1^t, [3] 1 - beta2^t, [4] skip flag, [5] step count t.
// LS (dynamic loss scaling, "Let's reproduce GPT-2 (124M)" chapter
// "float16, gradient scalers"): the gradients carry the loss scale
// S = scal[10]; the norm reported is theirs divided by S, and [1] becomes
// the clip coefficient divided by S, so AdamW sees unscaled clipped
// gradients.  A non-finite norm (an fp16 overflow) skips the update and
// halves S; otherwise [11] counts the steps since the last change of S and
// S doubles when it reaches growth_interval.
template <bool LS>
__global__ __launch_bounds__(256) void k_norm_finalize(const double* __restrict__ part, int nblk,
                                                       float clip, float beta1, float beta2,
                                                       float* scal, int* flag, int growth_interval) {
  __shared__ double sh[4];
  double s = 0.0;
  for (int i = threadIdx.x; i < nblk; i += 256) s += part[i];
  s = wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double nrm = sqrt((sh[0] + sh[1]) + (sh[2] + sh[3]));
    const float S = LS ? scal[10] : 1.f;
    if constexpr (LS) nrm /= (double)S;
    scal[0] = (float)nrm;
    if (isfinite(nrm)) {
      double c = (double)clip / (nrm + 1e-6);
      c = c < 1.0 ? c : 1.0;
      scal[1] = LS ? (float)(c / (double)S) : (float)c;
      float t = scal[5] + 1.0f;
      scal[5] = t;
      scal[2] = (float)(1.0 - pow((double)beta1, (double)t));
      scal[3] = (float)(1.0 - pow((double)beta2, (double)t));
      scal[4] = 0.f;
      if constexpr (LS) {
        const float good = scal[11] + 1.f;
        if (good >= (float)growth_interval) {
          scal[10] = S * 2.f;
          scal[11] = 0.f;
        } else {
          scal[11] = good;
        }
      }
    } else {
      scal[1] = 0.f;
      scal[4] = 1.f;
      if constexpr (LS) {
        scal[10] = S * 0.5f;
        scal[11] = 0.f;
        atomicOr(flag, FLAG_OVERFLOW);
      } else {
        atomicOr(flag, FLAG_NORM);
      }
    }
  }
}

hipError_t norm_finalize(const double* part, int nblk, float clip, float beta1, float beta2,
                         float* scal, int* flag, bool loss_scaling, int growth_interval, hipStream_t st) {
  if (loss_scaling)
    k_norm_finalize<true><<<1, 256, 0, st>>>(part, nblk, clip, beta1, beta2, scal, flag, growth_interval);
  else
    k_norm_finalize<false><<<1, 256, 0, st>>>(part, nblk, clip, beta1, beta2, scal, flag, growth_interval);
  return hipGetLastError();
}

// ------------------------------------------------------------------ AdamW
// "Optimization Hyperparameters": AdamW with betas (0.9, 0.95), eps 1e-8,
// decoupled decay on 2-D tensors only; gradients pre-scaled by the clip
// coefficient.  One block per table chunk; float4 vectorized.
template <typename TS>
__global__ __launch_bounds__(256) void k_adamw(float* __restrict__ p, const float* __restrict__ g,
                                               float* __restrict__ m, float* __restrict__ v,
                                               uint16_t* __restrict__ shadow,
                                               const AdamChunk* __restrict__ chunks,
                                               const float* __restrict__ scal, float lr,
                                               float beta1, float beta2, float eps, float wd) {
  if (scal[4] != 0.f) return;  // non-finite norm: skip the update
  AdamChunk ck = chunks[blockIdx.x];
  float coef = scal[1];
  float inv_bc1 = 1.0f / scal[2], inv_bc2 = 1.0f / scal[3];
  float wdl = (ck.flags & 1) ? wd : 0.f;
  bool wsh = (ck.flags & 2) != 0;
  size_t end = ck.start + ck.count;
  // two groups of 4 elements per thread and iteration (the second 1024
  // elements further on), all eight loads issued before any update
  for (size_t i0 = ck.start + (size_t)threadIdx.x * 4; i0 < end; i0 += 2 * 256 * 4) {
    const bool two = i0 + 256 * 4 < end;
    float4 pp[2], gg[2], mm[2], vv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1 && !two) break;
      const size_t i = i0 + (size_t)h * 256 * 4;
      pp[h] = *(float4*)(p + i);
      gg[h] = *(const float4*)(g + i);
      mm[h] = *(float4*)(m + i);
      vv[h] = *(float4*)(v + i);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1 && !two) break;
      const size_t i = i0 + (size_t)h * 256 * 4;
      float pa[4] = {pp[h].x, pp[h].y, pp[h].z, pp[h].w}, ga[4] = {gg[h].x, gg[h].y, gg[h].z, gg[h].w};
      float ma[4] = {mm[h].x, mm[h].y, mm[h].z, mm[h].w}, va[4] = {vv[h].x, vv[h].y, vv[h].z, vv[h].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float gj = ga[j] * coef;
        ma[j] = beta1 * ma[j] + (1.0f - beta1) * gj;
        va[j] = beta2 * va[j] + (1.0f - beta2) * gj * gj;
        float mh = ma[j] * inv_bc1, vh = va[j] * inv_bc2;
        pa[j] = pa[j] - lr * (mh / (sqrtf(vh) + eps) + wdl * pa[j]);
      }
      *(float4*)(p + i) = make_float4(pa[0], pa[1], pa[2], pa[3]);
      *(float4*)(m + i) = make_float4(ma[0], ma[1], ma[2], ma[3]);
      *(float4*)(v + i) = make_float4(va[0], va[1], va[2], va[3]);
      if (wsh) *(uint2*)(shadow + i) = make_uint2(H16<TS>::pack2(pa[0], pa[1]), H16<TS>::pack2(pa[2], pa[3]));
    }
  }
}

hipError_t adamw(float* p, const float* g, float* m, float* v, uint16_t* shadow, int shadow_dt,
                 const AdamChunk* chunks, int nchunks, const float* scal, float lr, float beta1,
                 float beta2, float eps, float wd, hipStream_t st) {
  if (shadow_dt == ACT_F16)
    k_adamw<f16><<<nchunks, 256, 0, st>>>(p, g, m, v, shadow, chunks, scal, lr, beta1, beta2, eps, wd);
  else
    k_adamw<bf16><<<nchunks, 256, 0, st>>>(p, g, m, v, shadow, chunks, scal, lr, beta1, beta2, eps, wd);
  return hipGetLastError();
}

// ------------------------------------------------------------------ misc
__global__ void k_to_bf16(const float* __restrict__ x, uint16_t* __restrict__ y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = f2bf_bits(x[i]);
}
__global__ void k_to_f16(const float* __restrict__ x, uint16_t* __restrict__ y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = __builtin_bit_cast(uint16_t, (f16)x[i]);
}
hipError_t to_h16(const float* x, uint16_t* y, size_t n, int dt, hipStream_t st) {
  if (dt == ACT_F16)
    k_to_f16<<<2048, 256, 0, st>>>(x, y, n);
  else
    k_to_bf16<<<2048, 256, 0, st>>>(x, y, n);
  return hipGetLastError();
}
__global__ void k_fill(float* x, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    x[i] = v;
}
hipError_t fill_f32(float* x, size_t n, float v, hipStream_t st) {
  k_fill<<<2048, 256, 0, st>>>(x, n, v);
  return hipGetLastError();
}
template <typename T>
__global__ void k_copy_act(const float* __restrict__ x, T* __restrict__ y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = from_f<T>(x[i]);
}
hipError_t copy_f32_to_act(const float* x, void* y, int dt, size_t n, hipStream_t st) {
  if (dt == ACT_BF16)
    k_copy_act<bf16><<<2048, 256, 0, st>>>(x, (bf16*)y, n);
  else if (dt == ACT_F16)
    k_copy_act<f16><<<2048, 256, 0, st>>>(x, (f16*)y, n);
  else
    k_copy_act<float><<<2048, 256, 0, st>>>(x, (float*)y, n);
  return hipGetLastError();
}

}  // namespace gk
