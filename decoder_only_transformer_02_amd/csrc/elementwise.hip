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
template <> struct Vec4<float> {
  static __device__ __forceinline__ float4 load(const float* p) { return *(const float4*)p; }
  static __device__ __forceinline__ void store(float* p, float a, float b, float c, float d) {
    *(float4*)p = make_float4(a, b, c, d);
  }
};
template <> struct Vec4<bf16> {
  static __device__ __forceinline__ float4 load(const bf16* p) {
    uint2 u = *(const uint2*)p;
    return make_float4(bfbits2f(u.x & 0xffffu), bfbits2f(u.x >> 16), bfbits2f(u.y & 0xffffu),
                       bfbits2f(u.y >> 16));
  }
  static __device__ __forceinline__ void store(bf16* p, float a, float b, float c, float d) {
    *(uint2*)p = make_uint2(pack_bf2(a, b), pack_bf2(c, d));
  }
};

// flag bits
enum { FLAG_TOKEN = 1, FLAG_TARGET = 2, FLAG_LOSS = 4, FLAG_NORM = 8 };

// ------------------------------------------------------------------ embedding forward
// "From Scratch: Building GPT-2 ...", Key Features: token and positional
// embeddings, summed.
__global__ __launch_bounds__(256) void k_embed_fwd(const int32_t* __restrict__ tok,
                                                   const float* __restrict__ wte,
                                                   const float* __restrict__ wpe,
                                                   float* __restrict__ h, int M, int T, int C,
                                                   int V, int* flag) {
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= M) return;
  int id = tok[row];
  if (id < 0 || id >= V) {
    if (lane == 0) atomicOr(flag, FLAG_TOKEN);
    id = id < 0 ? 0 : V - 1;
  }
  int t = row % T;
  const float4* a = (const float4*)(wte + (size_t)id * C);
  const float4* b = (const float4*)(wpe + (size_t)t * C);
  float4* o = (float4*)(h + (size_t)row * C);
  for (int c = lane; c < C / 4; c += 64) {
    float4 x = a[c], y = b[c];
    o[c] = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
  }
}

hipError_t embed_fwd(const int32_t* tok, const float* wte, const float* wpe, float* h, int M, int T,
                     int C, int V, int* flag, hipStream_t st) {
  k_embed_fwd<<<cdiv(M, 4), 256, 0, st>>>(tok, wte, wpe, h, M, T, C, V, flag);
  return hipGetLastError();
}

// ------------------------------------------------------------------ LayerNorm forward
// y = (x - mean) * rstd * w + b, biased variance, one wave per row.  The row
// stays in registers (NV float4 per lane, C <= 256 * NV).
template <typename TO, int NV>
__global__ __launch_bounds__(256) void k_ln_fwd(const float* __restrict__ x,
                                                const float* __restrict__ w,
                                                const float* __restrict__ b, TO* __restrict__ y,
                                                float* __restrict__ mean, float* __restrict__ rstd,
                                                int M, int C, float eps) {
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= M) return;
  const float* xr = x + (size_t)row * C;
  float4 v[NV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int c = (lane + i * 64) * 4;
    if (c < C) {
      v[i] = *(const float4*)(xr + c);
      s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    } else {
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  float mu = wave_sum(s) / (float)C;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int c = (lane + i * 64) * 4;
    if (c < C) {
      float a0 = v[i].x - mu, a1 = v[i].y - mu, a2 = v[i].z - mu, a3 = v[i].w - mu;
      q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  float rs = rsqrtf(wave_sum(q) / (float)C + eps);
  TO* yr = y + (size_t)row * C;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int c = (lane + i * 64) * 4;
    if (c < C) {
      float4 ww = *(const float4*)(w + c), bb = *(const float4*)(b + c);
      Vec4<TO>::store(yr + c, (v[i].x - mu) * rs * ww.x + bb.x, (v[i].y - mu) * rs * ww.y + bb.y,
                      (v[i].z - mu) * rs * ww.z + bb.z, (v[i].w - mu) * rs * ww.w + bb.w);
    }
  }
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

hipError_t ln_fwd(const float* x, const float* w, const float* b, void* y, bool y_bf16, float* mean,
                  float* rstd, int M, int C, float eps, hipStream_t st) {
  if (C % 4 || C > 1024) return hipErrorInvalidValue;
  int g = cdiv(M, 4);
  if (y_bf16)
    k_ln_fwd<bf16, 4><<<g, 256, 0, st>>>(x, w, b, (bf16*)y, mean, rstd, M, C, eps);
  else
    k_ln_fwd<float, 4><<<g, 256, 0, st>>>(x, w, b, (float*)y, mean, rstd, M, C, eps);
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

template <typename TA, int NV>
__global__ __launch_bounds__(256) void k_ln_bwd(const float* __restrict__ x,
                                                const float* __restrict__ mean,
                                                const float* __restrict__ rstd,
                                                const float* __restrict__ w,
                                                const TA* __restrict__ dy, float* __restrict__ dres,
                                                TA* __restrict__ dres_act, int accum,
                                                float* __restrict__ part, int M, int C, int rpb) {
  __shared__ float red[2][4][1024];
  int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int r0 = blockIdx.x * rpb, r1 = min(r0 + rpb, M);
  float4 wr[NV], dwa[NV], dba[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int c = (lane + i * 64) * 4;
    wr[i] = c < C ? *(const float4*)(w + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    dwa[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    dba[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float invC = 1.0f / (float)C;
  for (int row = r0 + wv; row < r1; row += 4) {
    float mu = mean[row], rs = rstd[row];
    const float* xr = x + (size_t)row * C;
    const TA* dyr = dy + (size_t)row * C;
    float4 xh[NV], gg[NV];
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int c = (lane + i * 64) * 4;
      if (c < C) {
        float4 xv = *(const float4*)(xr + c);
        float4 d = Vec4<TA>::load(dyr + c);
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
    float* dr = dres + (size_t)row * C;
    TA* da = dres_act + (size_t)row * C;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int c = (lane + i * 64) * 4;
      if (c < C) {
        float4 o = make_float4(rs * (gg[i].x - mg - xh[i].x * mgx), rs * (gg[i].y - mg - xh[i].y * mgx),
                               rs * (gg[i].z - mg - xh[i].z * mgx), rs * (gg[i].w - mg - xh[i].w * mgx));
        if (accum) {
          float4 p = *(const float4*)(dr + c);
          o.x += p.x; o.y += p.y; o.z += p.z; o.w += p.w;
        }
        *(float4*)(dr + c) = o;
        Vec4<TA>::store(da + c, o.x, o.y, o.z, o.w);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int c = (lane + i * 64) * 4;
    if (c < C) {
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

hipError_t ln_bwd(const float* x, const float* mean, const float* rstd, const float* w,
                  const void* dy, bool act_bf16, float* dres, void* dres_act, bool accum,
                  float* part, int M, int C, hipStream_t st) {
  if (C % 4 || C > 1024) return hipErrorInvalidValue;
  int nb = ln_bwd_blocks(M);
  int rpb = cdiv(M, nb);
  if (act_bf16)
    k_ln_bwd<bf16, 4><<<nb, 256, 0, st>>>(x, mean, rstd, w, (const bf16*)dy, dres, (bf16*)dres_act,
                                          accum, part, M, C, rpb);
  else
    k_ln_bwd<float, 4><<<nb, 256, 0, st>>>(x, mean, rstd, w, (const float*)dy, dres,
                                           (float*)dres_act, accum, part, M, C, rpb);
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
  if (c < C)
    for (int r = r0 + grp; r < r1; r += 4) s += part[((size_t)r * 2 + wb) * C + c];
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
int colsum_parts(int M) {
  int r = cdiv(M, 256);
  return r < 64 ? r : 64;
}

// Stage 1: a block covers 256 columns (32 threads x 8 columns, 16-byte
// loads) and 8 row groups over one slice of rows; stage 2 sums the slices.
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
        for (int j = 0; j < 8; ++j) acc[c8 + j] += bfbits2f((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu));
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
  int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
  for (int r = 0; r < R; ++r) s += part[(size_t)r * N + n];
  db[n] = (beta != 0.f ? beta * db[n] : 0.f) + s;
}

hipError_t colsum(const void* X, bool x_bf16, int M, int N, int ldx, float* db, float beta,
                  float* part, hipStream_t st) {
  if (N % 8 || ldx % 8) return hipErrorInvalidValue;
  int R = colsum_parts(M);
  int rows_per = cdiv(M, R);
  dim3 g(cdiv(N, 256), R);
  if (x_bf16)
    k_colsum_part<bf16><<<g, 256, 0, st>>>((const bf16*)X, M, N, ldx, rows_per, part);
  else
    k_colsum_part<float><<<g, 256, 0, st>>>((const float*)X, M, N, ldx, rows_per, part);
  k_colsum_final<<<cdiv(N, 256), 256, 0, st>>>(part, R, N, db, beta);
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

constexpr float LOG2E = 1.4426950408889634f;

template <typename T, int NCH>
__global__ __launch_bounds__(256) void k_xent(T* __restrict__ logits, int ld, int V, int vt,
                                              const int32_t* __restrict__ tgt,
                                              float* __restrict__ losses, float scale,
                                              int want_grad, int* flag) {
  constexpr int E = Chunk16<T>::E;
  __shared__ float sh[4];
  int row = blockIdx.x;
  T* z = logits + (size_t)row * ld;
  int y = tgt[row];
  if (y < 0 || y >= vt) {
    if (threadIdx.x == 0) atomicOr(flag, FLAG_TARGET);
    y = y < 0 ? 0 : vt - 1;
  }
  // The target logit is taken from the registers of the thread that loaded
  // it (a separate global read could still be in flight when another wave
  // overwrites the row with the gradient).
  __shared__ float sh_zy;
  uint4 buf[NCH];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    int e0 = (threadIdx.x + k * 256) * E;
    if (e0 < V) {
      buf[k] = *(const uint4*)(z + e0);
#pragma unroll
      for (int j = 0; j < E; ++j) {
        float v = chunk_elem<T>(buf[k], j);
        if (e0 + j < V) mx = fmaxf(mx, v);
        if (e0 + j == y) sh_zy = v;
      }
    }
  }
  mx = block_reduce_max(mx, sh);
  const float zy = sh_zy;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    int e0 = (threadIdx.x + k * 256) * E;
    if (e0 < V) {
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (e0 + j < V) s += __builtin_amdgcn_exp2f((chunk_elem<T>(buf[k], j) - mx) * LOG2E);
    }
  }
  s = block_reduce_sum(s, sh);
  float lse = mx + __logf(s);
  if (threadIdx.x == 0) losses[row] = lse - zy;
  if (!want_grad) return;
  float lse2 = lse * LOG2E;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    int e0 = (threadIdx.x + k * 256) * E;
    if (e0 < ld) {
      float f[E];
#pragma unroll
      for (int j = 0; j < E; ++j) {
        int e = e0 + j;
        float g = 0.f;
        if (e < V) {
          g = __builtin_amdgcn_exp2f(chunk_elem<T>(buf[k], j) * LOG2E - lse2);
          if (e == y) g -= 1.0f;
          g *= scale;
        }
        f[j] = g;
      }
      *(uint4*)(z + e0) = chunk_pack<T>(f);
    }
  }
}

// Streaming variant (row too long for registers): three passes over HBM.
template <typename T>
__global__ __launch_bounds__(256) void k_xent_stream(T* __restrict__ logits, int ld, int V, int vt,
                                                     const int32_t* __restrict__ tgt,
                                                     float* __restrict__ losses, float scale,
                                                     int want_grad, int* flag) {
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

template <typename T>
static hipError_t xent_t(T* logits, int ld, int V, int vt, const int32_t* tgt, float* losses, float scale,
                         bool want_grad, int M, int* flag, hipStream_t st) {
  constexpr int E = Chunk16<T>::E;
  int nch = cdiv(cdiv(ld, E), 256);
  int g = want_grad ? 1 : 0;
  if (nch <= 1)
    k_xent<T, 1><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag);
  else if (nch <= 2)
    k_xent<T, 2><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag);
  else if (nch <= 4)
    k_xent<T, 4><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag);
  else if (nch <= 8)
    k_xent<T, 8><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag);
  else if (nch <= 16)
    k_xent<T, 16><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag);
  else if (nch <= 25)
    k_xent<T, 25><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag);
  else
    k_xent_stream<T><<<M, 256, 0, st>>>(logits, ld, V, vt, tgt, losses, scale, g, flag);
  return hipGetLastError();
}

hipError_t xent(void* logits, bool bf16_logits, int ld, int V, int vt, const int32_t* tgt,
                float* losses, float scale, bool want_grad, int M, int* flag, hipStream_t st) {
  if (bf16_logits) {
    if (ld % 8) return hipErrorInvalidValue;
    return xent_t<bf16>((bf16*)logits, ld, V, vt, tgt, losses, scale, want_grad, M, flag, st);
  }
  if (ld % 4) return hipErrorInvalidValue;
  return xent_t<float>((float*)logits, ld, V, vt, tgt, losses, scale, want_grad, M, flag, st);
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
// positions are sorted by (id, position) with a bitonic sort in LDS, then
// summed per id in sorted order: each chunk of 32 sorted entries sums its
// runs; runs that cross chunk borders are combined by a second kernel in
// chunk order.  No atomics, so the result is deterministic.
constexpr int SORT_MAX = 32768;  // positions per call (keys: id << 15 | pos)
constexpr int SEG = 32;

size_t embed_bwd_workspace(int M, int C) {
  size_t nch = (size_t)cdiv(M, SEG);
  return (size_t)SORT_MAX * 4 + 2 * nch * (size_t)C * 4 + 256;
}

__global__ __launch_bounds__(1024) void k_sort_keys(const int32_t* __restrict__ tok, int M, int V,
                                                    uint32_t* __restrict__ out) {
  extern __shared__ uint32_t sk[];
  int N = 1;
  while (N < M) N <<= 1;
  for (int i = threadIdx.x; i < N; i += 1024) {
    uint32_t key = 0xffffffffu;
    if (i < M) {
      int id = tok[i];
      id = id < 0 ? 0 : (id >= V ? V - 1 : id);
      key = ((uint32_t)id << 15) | (uint32_t)i;
    }
    sk[i] = key;
  }
  __syncthreads();
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < N; i += 1024) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint32_t a = sk[i], b = sk[ixj];
          bool up = (i & k) == 0;
          if ((a > b) == up) {
            sk[i] = b;
            sk[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < M; i += 1024) out[i] = sk[i];
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
  for (int c = threadIdx.x; c < C; c += 256) {
    float acc = 0.f;
    int run_start = i0;
    for (int i = i0; i < i1; ++i) {
      uint32_t k = ks[i - i0];
      acc += dh[(size_t)key_pos(k) * C + c];
      int id = key_id(k);
      bool end = (i == i1 - 1) || key_id(ks[i + 1 - i0]) != id;
      if (end) {
        bool from_prev = (run_start == i0) && prev_id == id;
        bool to_next = (i == i1 - 1) && next_id == id;
        if (!from_prev && !to_next) {
          dwte[(size_t)id * C + c] += acc;
        } else if (from_prev) {
          pfirst[(size_t)ch * C + c] = acc;  // continues a run from earlier chunks
        } else {
          plast[(size_t)ch * C + c] = acc;   // starts a run that continues
        }
        acc = 0.f;
        run_start = i + 1;
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
  for (int c = threadIdx.x; c < C; c += 256) {
    float acc = plast[(size_t)ch * C + c];
    for (int k = ch + 1; k < nch; ++k) {
      acc += pfirst[(size_t)k * C + c];
      int e = min((k + 1) * SEG, M);
      if (e >= M || key_id(keys[e]) != id || key_id(keys[e - 1]) != id) break;
    }
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
  if (t < T)
    for (int b = 0; b < B; ++b) s += dh[((size_t)b * T + t) * C + c];
  float* p = dwpe + (size_t)t * C + c;
  *p = (beta != 0.f ? beta * *p : 0.f) + s;
}

hipError_t embed_bwd(const int32_t* tok, const float* dh, float* dwte, float* dwpe, int B, int T,
                     int C, int V, int block_size, float beta, void* ws, hipStream_t st) {
  int M = B * T;
  if (M > SORT_MAX || V > 65536) return hipErrorInvalidValue;
  uint32_t* keys = (uint32_t*)ws;
  int nch = cdiv(M, SEG);
  float* pfirst = (float*)((char*)ws + (size_t)SORT_MAX * 4);
  float* plast = pfirst + (size_t)nch * C;
  int N = 1;
  while (N < M) N <<= 1;
  if ((size_t)N * 4 > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k_sort_keys,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, N * 4);
    if (e != hipSuccess) return e;
  }
  k_sort_keys<<<1, 1024, (size_t)N * 4, st>>>(tok, M, V, keys);
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
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
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
__global__ __launch_bounds__(256) void k_norm_finalize(const double* __restrict__ part, int nblk,
                                                       float clip, float beta1, float beta2,
                                                       float* scal, int* flag) {
  __shared__ double sh[4];
  double s = 0.0;
  for (int i = threadIdx.x; i < nblk; i += 256) s += part[i];
  s = wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double nrm = sqrt((sh[0] + sh[1]) + (sh[2] + sh[3]));
    scal[0] = (float)nrm;
    if (isfinite(nrm)) {
      double c = (double)clip / (nrm + 1e-6);
      scal[1] = (float)(c < 1.0 ? c : 1.0);
      float t = scal[5] + 1.0f;
      scal[5] = t;
      scal[2] = (float)(1.0 - pow((double)beta1, (double)t));
      scal[3] = (float)(1.0 - pow((double)beta2, (double)t));
      scal[4] = 0.f;
    } else {
      scal[1] = 0.f;
      scal[4] = 1.f;
      atomicOr(flag, FLAG_NORM);
    }
  }
}

hipError_t norm_finalize(const double* part, int nblk, float clip, float beta1, float beta2,
                         float* scal, int* flag, hipStream_t st) {
  k_norm_finalize<<<1, 256, 0, st>>>(part, nblk, clip, beta1, beta2, scal, flag);
  return hipGetLastError();
}

// ------------------------------------------------------------------ AdamW
// "Optimization Hyperparameters": AdamW with betas (0.9, 0.95), eps 1e-8,
// decoupled decay on 2-D tensors only; gradients pre-scaled by the clip
// coefficient.  One block per table chunk; float4 vectorized.
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
  for (size_t i = ck.start + (size_t)threadIdx.x * 4; i < end; i += 256 * 4) {
    float4 pp = *(float4*)(p + i), gg = *(const float4*)(g + i);
    float4 mm = *(float4*)(m + i), vv = *(float4*)(v + i);
    float pa[4] = {pp.x, pp.y, pp.z, pp.w}, ga[4] = {gg.x, gg.y, gg.z, gg.w};
    float ma[4] = {mm.x, mm.y, mm.z, mm.w}, va[4] = {vv.x, vv.y, vv.z, vv.w};
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
    if (wsh) *(uint2*)(shadow + i) = make_uint2(pack_bf2(pa[0], pa[1]), pack_bf2(pa[2], pa[3]));
  }
}

hipError_t adamw(float* p, const float* g, float* m, float* v, uint16_t* shadow,
                 const AdamChunk* chunks, int nchunks, const float* scal, float lr, float beta1,
                 float beta2, float eps, float wd, hipStream_t st) {
  k_adamw<<<nchunks, 256, 0, st>>>(p, g, m, v, shadow, chunks, scal, lr, beta1, beta2, eps, wd);
  return hipGetLastError();
}

// ------------------------------------------------------------------ weight transpose
// dst[c * ldt + r] = src[r * C + c] for a bf16 matrix src [R, C]: 64 x 64
// tiles through LDS so both the reads and the writes are row-contiguous.
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ src, int R,
                                                        int C, uint16_t* __restrict__ dst, int ldt) {
  __shared__ uint16_t t[64][66];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int i = ty; i < 64; i += 8) {
    int r = r0 + i, c = c0 + 2 * tx;
    uint32_t v = 0;
    if (r < R && c + 1 < C) v = *(const uint32_t*)(src + (size_t)r * C + c);
    else if (r < R && c < C) v = src[(size_t)r * C + c];
    t[i][2 * tx] = (uint16_t)(v & 0xffffu);
    t[i][2 * tx + 1] = (uint16_t)(v >> 16);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 8) {
    int c = c0 + i, r = r0 + 2 * tx;
    if (c >= C) continue;
    if (r + 1 < R) {
      *(uint32_t*)(dst + (size_t)c * ldt + r) = (uint32_t)t[2 * tx][i] | ((uint32_t)t[2 * tx + 1][i] << 16);
    } else if (r < R) {
      dst[(size_t)c * ldt + r] = t[2 * tx][i];
    }
  }
}

hipError_t transpose_bf16(const uint16_t* src, int R, int C, uint16_t* dst, int ldt, hipStream_t st) {
  if (ldt % 2) return hipErrorInvalidValue;
  k_transpose_bf16<<<dim3(cdiv(C, 64), cdiv(R, 64)), 256, 0, st>>>(src, R, C, dst, ldt);
  return hipGetLastError();
}

// ------------------------------------------------------------------ misc
__global__ void k_to_bf16(const float* __restrict__ x, uint16_t* __restrict__ y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = f2bf_bits(x[i]);
}
hipError_t to_bf16(const float* x, uint16_t* y, size_t n, hipStream_t st) {
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
hipError_t copy_f32_to_act(const float* x, void* y, bool bf, size_t n, hipStream_t st) {
  if (bf)
    k_copy_act<bf16><<<2048, 256, 0, st>>>(x, (bf16*)y, n);
  else
    k_copy_act<float><<<2048, 256, 0, st>>>(x, (float*)y, n);
  return hipGetLastError();
}

}  // namespace gk
