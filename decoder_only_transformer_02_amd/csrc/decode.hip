// Kernels of autoregressive sampling with a key/value cache ("Let's
// reproduce GPT-2 (124M)" chapters "sampling init, prefix tokens" and
// "sampling loop"): the new positions' keys and values appended to the
// cache, causal attention of the new positions' queries over the cached
// keys, and the sampling of the next token from the classifier's logits.
//
// Cache layout, per layer: [max_batch][max_seq][2][C] in the activation type
// (keys then values of a position, heads contiguous hd-wide), so one
// position's 2C values are contiguous and sequence b's keys are a strided
// run of max_seq rows.
#include "common.h"
#include "kernels.h"

namespace gk {

// cache[b][t0 + i][0:2C] = qkv[b * n + i][C:3C] for b < B, i < n (16-byte
// chunks; 2C elements are a multiple of 16 bytes).
__global__ __launch_bounds__(256) void k_kv_store(const uint8_t* __restrict__ qkv, uint8_t* __restrict__ cache,
                                                  int B, int n, int t0, int Tmax, int C, int es) {
  const long row = blockIdx.x;  // b * n + i
  const int b = (int)(row / n), i = (int)(row % n);
  const int chunks = 2 * C * es / 16;
  const uint4* src = (const uint4*)(qkv + (row * 3 * C + C) * es);
  uint4* dst = (uint4*)(cache + (((long)b * Tmax + t0 + i) * 2 * C) * es);
  for (int k = threadIdx.x; k < chunks; k += 256) dst[k] = src[k];
}

hipError_t kv_store(const void* qkv, void* cache, int B, int n, int t0, int Tmax, int C, int dt,
                    hipStream_t st) {
  const int es = dt == ACT_F32 ? 4 : 2;
  if ((2 * C * es) % 16 || B < 1 || n < 1 || t0 < 0 || t0 + n > Tmax) return hipErrorInvalidValue;
  k_kv_store<<<B * n, 256, 0, st>>>((const uint8_t*)qkv, (uint8_t*)cache, B, n, t0, Tmax, C, es);
  return hipGetLastError();
}

// One query per sequence (the newest position t, keys 0..t from the cache):
// one 256-thread block per (sequence, head).  Wave w walks keys w, w + 4,
// ...; a key's score is a wave-wide dot product (lane l holds dimensions l
// and l + 64), the online softmax runs per wave, and the four waves' (max,
// sum, output) triples are merged in LDS in wave order.  exp2 with the
// scale folded into log2 units.
template <typename TA>
__global__ __launch_bounds__(256) void k_attn_decode(const TA* __restrict__ qkv, const TA* __restrict__ cache,
                                                     TA* __restrict__ out, int H, int hd, int Tmax,
                                                     int nkeys, float sl2) {
  __shared__ float red_m[4], red_l[4];
  __shared__ float red_o[4][128];
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int C = H * hd;
  // the wave index through readfirstlane: uniform to the compiler, so the
  // key loop below stays a scalar loop
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const TA* qrow = qkv + (size_t)b * 3 * C + h * hd;
  const float q0 = lane < hd ? to_f(qrow[lane]) : 0.f;
  const float q1 = lane + 64 < hd ? to_f(qrow[lane + 64]) : 0.f;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  const TA* kb = cache + (size_t)b * Tmax * 2 * C + h * hd;
  // Each wave's keys j = w, w + 4, ...: the next key's K and V elements are
  // loaded before this key's reduction, so one load latency per key
  // overlaps the previous key's work instead of adding to it.  The loads
  // carry no lane test (a lane past hd reads element 0, whose product with
  // q = 0 adds nothing, and whose output slot is never read): loads under
  // a test are waited for where the paths join.
  // Two register sets alternate (keys j and j + 4), so the loop carries no
  // copy of a loaded register, which would wait for its load.
  const int i0 = lane < hd ? lane : 0, i1 = lane + 64 < hd ? lane + 64 : 0;
  struct KV { float k0, k1, v0, v1; };
  auto load_key = [&](int j) {
    const TA* kr = kb + (size_t)(j < nkeys ? j : nkeys - 1) * 2 * C;  // past the last key: reload it
    return KV{to_f(kr[i0]), to_f(kr[i1]), to_f(kr[C + i0]), to_f(kr[C + i1])};
  };
  auto use_key = [&](const KV& kv) {
    const float s = wave_sum(q0 * kv.k0 + q1 * kv.k1) * sl2;
    const float mn = fmaxf(m, s);
    const float a = __builtin_amdgcn_exp2f(m - mn), p = __builtin_amdgcn_exp2f(s - mn);
    l = l * a + p;
    o0 = o0 * a + p * kv.v0;
    o1 = o1 * a + p * kv.v1;
    m = mn;
  };
  KV ka = load_key(w);
  for (int j = w; j < nkeys; j += 8) {
    const KV kb2 = load_key(j + 4);
    __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of the use
    use_key(ka);
    if (j + 4 >= nkeys) break;
    ka = load_key(j + 8);
    __builtin_amdgcn_sched_barrier(0);
    use_key(kb2);
  }
  if (lane == 0) {
    red_m[w] = m;
    red_l[w] = l;
  }
  red_o[w][lane] = o0;
  red_o[w][lane + 64] = o1;
  __syncthreads();
  if (w == 0) {
    float M = red_m[0];
    for (int k = 1; k < 4; ++k) M = fmaxf(M, red_m[k]);
    float L = 0.f, A0 = 0.f, A1 = 0.f;
    for (int k = 0; k < 4; ++k) {
      if (red_m[k] == -INFINITY) continue;  // a wave that saw no key
      const float f = __builtin_amdgcn_exp2f(red_m[k] - M);
      L += red_l[k] * f;
      A0 += red_o[k][lane] * f;
      A1 += red_o[k][lane + 64] * f;
    }
    TA* orow = out + (size_t)b * C + h * hd;
    if (lane < hd) orow[lane] = from_f<TA>(A0 / L);
    if (lane + 64 < hd) orow[lane + 64] = from_f<TA>(A1 / L);
  }
}

hipError_t attn_decode(const void* qkv, const void* cache, void* out, int B, int H, int hd, int Tmax, int nkeys,
                       int dt, hipStream_t st) {
  if (hd > 128 || nkeys < 1 || nkeys > Tmax) return hipErrorInvalidValue;
  const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
  if (dt == ACT_F16)
    k_attn_decode<f16><<<B * H, 256, 0, st>>>((const f16*)qkv, (const f16*)cache, (f16*)out, H, hd, Tmax, nkeys,
                                               sl2);
  else if (dt == ACT_BF16)
    k_attn_decode<bf16><<<B * H, 256, 0, st>>>((const bf16*)qkv, (const bf16*)cache, (bf16*)out, H, hd, Tmax,
                                                nkeys, sl2);
  else
    k_attn_decode<float><<<B * H, 256, 0, st>>>((const float*)qkv, (const float*)cache, (float*)out, H, hd,
                                                 Tmax, nkeys, sl2);
  return hipGetLastError();
}

// Next token of sequence b from its logits row z (row b * row_stride + row0
// of a [*, ld] matrix): with e_v = exp(z_v - max) over the vocabulary ids
// v < V (padding ids are never tokens), the smallest v whose running sum
// e_0 + ... + e_v exceeds u_b * (e_0 + ... + e_{V-1}), i.e. the inverse
// of the softmax's cumulative distribution in id order at the caller's
// uniform u_b.  Thread i owns the contiguous ids [i * per, (i + 1) * per);
// running sums are float64, prefix sums over the 256 owners are taken in
// owner order.  Writes the token and its log-probability z_v - max - log S.
template <typename TL>
__global__ __launch_bounds__(256) void k_sample(const TL* __restrict__ logits, int ld, int row_stride,
                                                int row0, int V, const float* __restrict__ u, int u_stride,
                                                int32_t* __restrict__ tok, int tok_stride,
                                                float* __restrict__ logprob, int lp_stride) {
  __shared__ float smax[4];
  __shared__ double part[256];
  __shared__ int pick_owner;
  __shared__ double pick_base, total;
  const int b = blockIdx.x;
  const TL* z = logits + ((size_t)b * row_stride + row0) * ld;
  const int per = (V + 255) / 256;
  const int v0 = min(V, (int)threadIdx.x * per), v1 = min(V, v0 + per);
  float mx = -INFINITY;
  for (int v = v0; v < v1; ++v) mx = fmaxf(mx, to_f(z[v]));
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) smax[threadIdx.x >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  double s = 0.0;
  for (int v = v0; v < v1; ++v) s += (double)__builtin_amdgcn_exp2f((to_f(z[v]) - M) * 1.4426950408889634f);
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double S = 0.0;
    for (int i = 0; i < 256; ++i) S += part[i];
    float uu = u[(size_t)b * u_stride];
    uu = uu < 0.f ? 0.f : (uu >= 1.f ? 0.99999994f : uu);
    const double target = (double)uu * S;
    double run = 0.0;
    int owner = -1;
    for (int i = 0; i < 256; ++i) {
      if (part[i] > 0.0) owner = i;  // last owner with mass, for a target at the very top
      if (run + part[i] > target && part[i] > 0.0) {
        owner = i;
        break;
      }
      run += part[i];
    }
    double base = 0.0;
    for (int i = 0; i < owner; ++i) base += part[i];
    pick_owner = owner;
    pick_base = base;
    total = S;
  }
  __syncthreads();
  if ((int)threadIdx.x == pick_owner) {
    const double S = total;
    float uu = u[(size_t)b * u_stride];
    uu = uu < 0.f ? 0.f : (uu >= 1.f ? 0.99999994f : uu);
    const double target = (double)uu * S;
    double run = pick_base;
    int pick = -1;
    for (int v = v0; v < v1; ++v) {
      const double e = (double)__builtin_amdgcn_exp2f((to_f(z[v]) - M) * 1.4426950408889634f);
      if (e > 0.0) pick = v;
      run += e;
      if (run > target && e > 0.0) break;
    }
    tok[(size_t)b * tok_stride] = pick;
    if (logprob) logprob[(size_t)b * lp_stride] = (to_f(z[pick]) - M) - (float)log(S);
  }
}

hipError_t sample(const void* logits, int dt, int ld, int row_stride, int row0, int V, int B, const float* u,
                  int u_stride, int32_t* tok, int tok_stride, float* logprob, int lp_stride, hipStream_t st) {
  if (B < 1 || V < 1 || V > ld) return hipErrorInvalidValue;
  if (dt == ACT_F16)
    k_sample<f16><<<B, 256, 0, st>>>((const f16*)logits, ld, row_stride, row0, V, u, u_stride, tok, tok_stride,
                                      logprob, lp_stride);
  else if (dt == ACT_BF16)
    k_sample<bf16><<<B, 256, 0, st>>>((const bf16*)logits, ld, row_stride, row0, V, u, u_stride, tok, tok_stride,
                                       logprob, lp_stride);
  else
    k_sample<float><<<B, 256, 0, st>>>((const float*)logits, ld, row_stride, row0, V, u, u_stride, tok,
                                        tok_stride, logprob, lp_stride);
  return hipGetLastError();
}

}  // namespace gk
