// Causal multi-head self-attention, flash style ("Let's reproduce GPT-2
// (124M)" key takeaways, "Efficient Training Infrastructure": attention
// computed without materializing the T x T scores; chapter "flash
// attention").  softmax(q k^T / sqrt(hd)) v with query i attending keys
// j <= i.  q, k, v are read in place from the packed qkv rows [B*T, 3C].
//
// head_dim 64, bf16: matrix-core kernels.  Each wave owns 32 queries (or
// 32 keys in the dK/dV kernel) as the 32-wide MFMA column; K/V (or Q/dO)
// tiles of 64 rows are staged in LDS and shared by the 4 waves of a block.
// Scores are formed transposed (S^T = K Q^T) so that a lane holds 16 scores
// of one query: the online softmax needs one cross-lane exchange and the
// probabilities feed the next MFMA straight from registers.  exp2 with the
// scale folded into log2 units.
//   forward: O and the row log-sum-exp (log2 units) per query.
//   backward: D = rowsum(dO * O); dQ kernel (query-block parallel) and
//   dK/dV kernel (key-block parallel), both recomputing P from the saved
//   log-sum-exp; no atomics, so results are deterministic.
// Other head sizes / fp32: simple one-thread-per-row kernels.
#include "common.h"
#include "kernels.h"

namespace gk {

constexpr float LOG2E_F = 1.4426950408889634f;
constexpr int ALD = 72;  // padded LDS row (bf16 elements)

__device__ __forceinline__ uint4 ldg16(const bf16* p) { return *(const uint4*)p; }

// 8 bf16 for the MFMA operand slots s = 0..7 gathered as keys
// base + {0,1,2,3} and base + 8 + {0,1,2,3} from an LDS row (two 8-byte reads).
__device__ __forceinline__ bf16x8 lds_two_runs(const uint16_t* row, int base) {
  uint2 a = *(const uint2*)(row + base);
  uint2 b = *(const uint2*)(row + base + 8);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// Pack accumulator values e = 8h .. 8h+7 of one 32x32 block to bf16 slots.
__device__ __forceinline__ bf16x8 pack_slots(const f32x16& v, int h) {
  uint4 u = make_uint4(pack_bf2(v[8 * h + 0], v[8 * h + 1]), pack_bf2(v[8 * h + 2], v[8 * h + 3]),
                       pack_bf2(v[8 * h + 4], v[8 * h + 5]), pack_bf2(v[8 * h + 6], v[8 * h + 7]));
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return z;
}

// A 64-row x 64-column bf16 tile held in registers between its global load
// and its LDS store (2 x 16 bytes per thread), so the next tile's loads are
// in flight while the current one is being consumed.  Rows >= T load as 0.
struct Tile64 {
  uint4 v[2];
  __device__ __forceinline__ void load(const bf16* base, int ld, int r0, int T) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int c = threadIdx.x + i * 256;
      int row = c & 63, oct = c >> 6;
      int gr = r0 + row;
      v[i] = gr < T ? ldg16(base + (size_t)gr * ld + oct * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  // [row][col] layout
  __device__ __forceinline__ void store(uint16_t* dn) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int c = threadIdx.x + i * 256;
      int row = c & 63, oct = c >> 6;
      *(uint4*)(dn + row * ALD + oct * 8) = v[i];
    }
  }
  // [col][row] layout
  __device__ __forceinline__ void store_t(uint16_t* dt) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int c = threadIdx.x + i * 256;
      int row = c & 63, oct = c >> 6;
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        dt[(oct * 8 + j) * ALD + row] = (uint16_t)((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu));
    }
  }
};

// ------------------------------------------------------------------ forward, hd = 64
__global__ __launch_bounds__(256) void k_attn_fwd64(const bf16* __restrict__ qkv,
                                                    bf16* __restrict__ out, float* __restrict__ lse,
                                                    int T, int H, float sl2) {
  __shared__ uint16_t Ks[64 * ALD];
  __shared__ uint16_t Vt[64 * ALD];
  const int C = H * 64, ld = 3 * C;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q0 = (gridDim.x - 1 - blockIdx.x) * 128;  // heavy blocks first
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 31, g = lane >> 5;
  const int q = q0 + 32 * w + fr;
  const bf16* base = qkv + (size_t)b * T * ld;
  const bf16* kbase_p = base + C + h * 64;
  const bf16* vbase_p = base + 2 * C + h * 64;

  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = __builtin_bit_cast(
        bf16x8, q < T ? ldg16(base + (size_t)q * ld + h * 64 + ks * 16 + g * 8) : make_uint4(0, 0, 0, 0));

  f32x16 oacc[2] = {zero16(), zero16()};
  float m_i = -INFINITY, l_i = 0.f;
  const int qlast = min(q0 + 127, T - 1);
  const int ntiles = qlast / 64 + 1;
  const int wq_hi = min(q0 + 32 * w + 31, T - 1);

  Tile64 kt_r, vt_r;
  kt_r.load(kbase_p, ld, 0, T);
  vt_r.load(vbase_p, ld, 0, T);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * 64;
    __syncthreads();
    kt_r.store(Ks);
    vt_r.store_t(Vt);
    __syncthreads();
    if (kt + 1 < ntiles) {
      kt_r.load(kbase_p, ld, k0 + 64, T);
      vt_r.load(vbase_p, ld, k0 + 64, T);
    }
    if (k0 > wq_hi) continue;
    f32x16 s[2] = {zero16(), zero16()};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 a = __builtin_bit_cast(bf16x8, *(const uint4*)(Ks + (kb * 32 + fr) * ALD + ks * 16 + g * 8));
        s[kb] = mfma(a, qf[ks], s[kb]);
      }
    const bool diag = k0 + 63 > q0 + 32 * w;  // tile reaches past the wave's first query
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = s[kb][e] * sl2;
        if (diag) {
          int key = k0 + kb * 32 + (e >> 2) * 8 + g * 4 + (e & 3);
          if (key > q || key >= T) v = -INFINITY;
        }
        s[kb][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_i, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_i - m_new);
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float pv = __builtin_amdgcn_exp2f(s[kb][e] - m_new);
        s[kb][e] = pv;
        ps += pv;
      }
    l_i = l_i * alpha + ps;
    m_i = m_new;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 pb = pack_slots(s[j >> 1], j & 1);
      int kbase = (j >> 1) * 32 + (j & 1) * 16 + g * 4;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        bf16x8 a = lds_two_runs(Vt + (db * 32 + fr) * ALD, kbase);
        oacc[db] = mfma(a, pb, oacc[db]);
      }
    }
  }
  const float l_tot = l_i + __shfl_xor(l_i, 32, 64);
  const float inv = 1.0f / l_tot;
  if (q < T) {
    bf16* orow = out + ((size_t)b * T + q) * C + h * 64;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        int d = db * 32 + e4 * 8 + g * 4;
        *(uint2*)(orow + d) = make_uint2(pack_bf2(oacc[db][e4 * 4 + 0] * inv, oacc[db][e4 * 4 + 1] * inv),
                                         pack_bf2(oacc[db][e4 * 4 + 2] * inv, oacc[db][e4 * 4 + 3] * inv));
      }
    if (g == 0) lse[(size_t)bh * T + q] = m_i + __log2f(l_tot);
  }
}

// ------------------------------------------------------------------ backward preprocessing
// D[bh, t] = sum_d dO[t, h, d] * O[t, h, d].  One thread per (row, head),
// 16-byte loads; neighbouring threads read neighbouring heads of one row.
template <typename TA>
__device__ __forceinline__ float dot16(const uint4& a, const uint4& b);
template <>
__device__ __forceinline__ float dot16<bf16>(const uint4& a, const uint4& b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    s += bfbits2f(x[j] & 0xffffu) * bfbits2f(y[j] & 0xffffu) + bfbits2f(x[j] >> 16) * bfbits2f(y[j] >> 16);
  return s;
}
template <>
__device__ __forceinline__ float dot16<float>(const uint4& a, const uint4& b) {
  return __uint_as_float(a.x) * __uint_as_float(b.x) + __uint_as_float(a.y) * __uint_as_float(b.y) +
         __uint_as_float(a.z) * __uint_as_float(b.z) + __uint_as_float(a.w) * __uint_as_float(b.w);
}

template <typename TA>
__global__ __launch_bounds__(256) void k_attn_bwd_pre(const TA* __restrict__ o,
                                                      const TA* __restrict__ dout,
                                                      float* __restrict__ D, int B, int T, int H,
                                                      int hd) {
  constexpr int E = 16 / sizeof(TA);
  int i = blockIdx.x * 256 + threadIdx.x;  // row * H + h
  if (i >= B * T * H) return;
  int h = i % H, row = i / H;
  int b = row / T, t = row % T;
  const TA* po = o + (size_t)row * H * hd + h * hd;
  const TA* pd = dout + (size_t)row * H * hd + h * hd;
  float s = 0.f;
  for (int d = 0; d < hd; d += E) s += dot16<TA>(*(const uint4*)(po + d), *(const uint4*)(pd + d));
  D[((size_t)b * H + h) * T + t] = s;
}

// ------------------------------------------------------------------ dQ, hd = 64
__global__ __launch_bounds__(256) void k_attn_dq64(const bf16* __restrict__ qkv,
                                                   const bf16* __restrict__ dout,
                                                   const float* __restrict__ lse,
                                                   const float* __restrict__ Dv,
                                                   bf16* __restrict__ dqkv, int T, int H, float sl2,
                                                   float scale) {
  __shared__ uint16_t Ks[64 * ALD];
  __shared__ uint16_t Kt[64 * ALD];
  __shared__ uint16_t Vs[64 * ALD];
  const int C = H * 64, ld = 3 * C;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q0 = (gridDim.x - 1 - blockIdx.x) * 128;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 31, g = lane >> 5;
  const int q = q0 + 32 * w + fr;
  const bf16* base = qkv + (size_t)b * T * ld;
  const bf16* dob = dout + (size_t)b * T * C;
  const bf16* kp = base + C + h * 64;
  const bf16* vp = base + 2 * C + h * 64;

  bf16x8 qf[4], dof[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qf[ks] = __builtin_bit_cast(
        bf16x8, q < T ? ldg16(base + (size_t)q * ld + h * 64 + ks * 16 + g * 8) : make_uint4(0, 0, 0, 0));
    dof[ks] = __builtin_bit_cast(
        bf16x8, q < T ? ldg16(dob + (size_t)q * C + h * 64 + ks * 16 + g * 8) : make_uint4(0, 0, 0, 0));
  }
  const float lq = q < T ? lse[(size_t)bh * T + q] : 0.f;
  const float Dq = q < T ? Dv[(size_t)bh * T + q] : 0.f;
  f32x16 dq[2] = {zero16(), zero16()};
  const int qlast = min(q0 + 127, T - 1);
  const int ntiles = qlast / 64 + 1;
  const int wq_hi = min(q0 + 32 * w + 31, T - 1);

  Tile64 kr, vr;
  kr.load(kp, ld, 0, T);
  vr.load(vp, ld, 0, T);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * 64;
    __syncthreads();
    kr.store(Ks);
    kr.store_t(Kt);
    vr.store(Vs);
    __syncthreads();
    if (kt + 1 < ntiles) {
      kr.load(kp, ld, k0 + 64, T);
      vr.load(vp, ld, k0 + 64, T);
    }
    if (k0 > wq_hi) continue;
    const bool diag = k0 + 63 > q0 + 32 * w;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 a = __builtin_bit_cast(bf16x8, *(const uint4*)(Ks + (kb * 32 + fr) * ALD + ks * 16 + g * 8));
        s = mfma(a, qf[ks], s);
        bf16x8 v = __builtin_bit_cast(bf16x8, *(const uint4*)(Vs + (kb * 32 + fr) * ALD + ks * 16 + g * 8));
        dp = mfma(v, dof[ks], dp);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float p = __builtin_amdgcn_exp2f(s[e] * sl2 - lq);
        if (diag) {
          int key = k0 + kb * 32 + (e >> 2) * 8 + g * 4 + (e & 3);
          if (key > q || key >= T) p = 0.f;
        }
        s[e] = p * (dp[e] - Dq);  // dS^T
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 dsb = pack_slots(s, hh);
        int kbase = kb * 32 + hh * 16 + g * 4;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          bf16x8 a = lds_two_runs(Kt + (db * 32 + fr) * ALD, kbase);
          dq[db] = mfma(a, dsb, dq[db]);
        }
      }
    }
  }
  if (q < T) {
    bf16* row = dqkv + ((size_t)b * T + q) * ld + h * 64;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        int d = db * 32 + e4 * 8 + g * 4;
        *(uint2*)(row + d) = make_uint2(pack_bf2(dq[db][e4 * 4 + 0] * scale, dq[db][e4 * 4 + 1] * scale),
                                        pack_bf2(dq[db][e4 * 4 + 2] * scale, dq[db][e4 * 4 + 3] * scale));
      }
  }
}

// ------------------------------------------------------------------ dK, dV, hd = 64
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_dkv64(const bf16* __restrict__ qkv,
                                                    const bf16* __restrict__ dout,
                                                    const float* __restrict__ lse,
                                                    const float* __restrict__ Dv,
                                                    bf16* __restrict__ dqkv, int T, int H, float sl2,
                                                    float scale) {
  __shared__ uint16_t Qs[64 * ALD];
  __shared__ uint16_t Qt[64 * ALD];
  __shared__ uint16_t Os[64 * ALD];   // dO [q][d]
  __shared__ uint16_t Ot[64 * ALD];   // dO^T [d][q]
  __shared__ float Ls[64], Ds[64];
  const int C = H * 64, ld = 3 * C;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int k0 = blockIdx.x * 128;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 31, g = lane >> 5;
  const int key = k0 + 32 * w + fr;
  const bf16* base = qkv + (size_t)b * T * ld;
  const bf16* dob = dout + (size_t)b * T * C;
  const bf16* qp = base + h * 64;
  const bf16* op = dob + h * 64;

  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kf[ks] = __builtin_bit_cast(
        bf16x8, key < T ? ldg16(base + (size_t)key * ld + C + h * 64 + ks * 16 + g * 8) : make_uint4(0, 0, 0, 0));
    vf[ks] = __builtin_bit_cast(
        bf16x8, key < T ? ldg16(base + (size_t)key * ld + 2 * C + h * 64 + ks * 16 + g * 8) : make_uint4(0, 0, 0, 0));
  }
  f32x16 dk[2] = {zero16(), zero16()}, dv[2] = {zero16(), zero16()};
  const int wk_lo = k0 + 32 * w;
  const int nqt = (T + 63) / 64;
  const int qt0 = k0 / 64;
  Tile64 qr, orr;
  float lr = 0.f, dr = 0.f;
  auto load_q = [&](int qt) {
    qr.load(qp, ld, qt * 64, T);
    orr.load(op, C, qt * 64, T);
    if (tid < 64) {
      int qq = qt * 64 + tid;
      lr = qq < T ? lse[(size_t)bh * T + qq] : 0.f;
      dr = qq < T ? Dv[(size_t)bh * T + qq] : 0.f;
    }
  };
  load_q(qt0);
  for (int qt = qt0; qt < nqt; ++qt) {
    const int q0 = qt * 64;
    __syncthreads();
    qr.store(Qs);
    qr.store_t(Qt);
    orr.store(Os);
    orr.store_t(Ot);
    if (tid < 64) {
      Ls[tid] = lr;
      Ds[tid] = dr;
    }
    __syncthreads();
    if (qt + 1 < nqt) load_q(qt + 1);
    if (q0 + 63 < wk_lo || wk_lo >= T) continue;
    const bool diag = q0 < wk_lo + 31;  // some (q, key) pairs of the tile are masked
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // S and dP for 32 queries x this wave's 32 keys:
      // rows q = q0 + qb*32 + 8(e/4) + 4g + e%4, column key
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 a = __builtin_bit_cast(bf16x8, *(const uint4*)(Qs + (qb * 32 + fr) * ALD + ks * 16 + g * 8));
        s = mfma(a, kf[ks], s);
        bf16x8 o = __builtin_bit_cast(bf16x8, *(const uint4*)(Os + (qb * 32 + fr) * ALD + ks * 16 + g * 8));
        dp = mfma(o, vf[ks], dp);
      }
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int ql0 = qb * 32 + e4 * 8 + g * 4;
        const float4 L4 = *(const float4*)(Ls + ql0);
        const float4 D4 = *(const float4*)(Ds + ql0);
        const float Lr[4] = {L4.x, L4.y, L4.z, L4.w}, Dr[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
        for (int e1 = 0; e1 < 4; ++e1) {
          const int e = e4 * 4 + e1;
          float p = __builtin_amdgcn_exp2f(s[e] * sl2 - Lr[e1]);
          if (diag) {
            int qq = q0 + ql0 + e1;
            if (key > qq || qq >= T) p = 0.f;
          }
          s[e] = p;
          dp[e] = p * (dp[e] - Dr[e1]);
        }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 pb = pack_slots(s, hh);
        bf16x8 dsb = pack_slots(dp, hh);
        int qbase = qb * 32 + hh * 16 + g * 4;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          bf16x8 ao = lds_two_runs(Ot + (db * 32 + fr) * ALD, qbase);
          dv[db] = mfma(ao, pb, dv[db]);
          bf16x8 aq = lds_two_runs(Qt + (db * 32 + fr) * ALD, qbase);
          dk[db] = mfma(aq, dsb, dk[db]);
        }
      }
    }
  }
  if (key < T) {
    bf16* rk = dqkv + ((size_t)b * T + key) * ld + C + h * 64;
    bf16* rv = rk + C;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        int d = db * 32 + e4 * 8 + g * 4;
        *(uint2*)(rk + d) = make_uint2(pack_bf2(dk[db][e4 * 4 + 0] * scale, dk[db][e4 * 4 + 1] * scale),
                                       pack_bf2(dk[db][e4 * 4 + 2] * scale, dk[db][e4 * 4 + 3] * scale));
        *(uint2*)(rv + d) = make_uint2(pack_bf2(dv[db][e4 * 4 + 0], dv[db][e4 * 4 + 1]),
                                       pack_bf2(dv[db][e4 * 4 + 2], dv[db][e4 * 4 + 3]));
      }
  }
}

// ------------------------------------------------------------------ generic kernels
// One thread per (b, h, query): two passes over the visible keys.
template <typename TA, int HDM>
__global__ __launch_bounds__(128) void k_attn_fwd_gen(const TA* __restrict__ qkv, TA* __restrict__ out,
                                                      float* __restrict__ lse, int B, int T, int H,
                                                      int hd, float sl2) {
  int i = blockIdx.x * 128 + threadIdx.x;
  if (i >= B * H * T) return;
  int q = i % T, bh = i / T, b = bh / H, h = bh % H;
  const int C = H * hd, ld = 3 * C;
  const TA* base = qkv + (size_t)b * T * ld;
  float qv[HDM], o[HDM];
  for (int d = 0; d < hd; ++d) { qv[d] = to_f(base[(size_t)q * ld + h * hd + d]); o[d] = 0.f; }
  float m = -INFINITY;
  for (int j = 0; j <= q; ++j) {
    const TA* kr = base + (size_t)j * ld + C + h * hd;
    float s = 0.f;
    for (int d = 0; d < hd; ++d) s += qv[d] * to_f(kr[d]);
    m = fmaxf(m, s * sl2);
  }
  float l = 0.f;
  for (int j = 0; j <= q; ++j) {
    const TA* kr = base + (size_t)j * ld + C + h * hd;
    const TA* vr = kr + C;
    float s = 0.f;
    for (int d = 0; d < hd; ++d) s += qv[d] * to_f(kr[d]);
    float p = __builtin_amdgcn_exp2f(s * sl2 - m);
    l += p;
    for (int d = 0; d < hd; ++d) o[d] += p * to_f(vr[d]);
  }
  TA* orow = out + ((size_t)b * T + q) * C + h * hd;
  for (int d = 0; d < hd; ++d) orow[d] = from_f<TA>(o[d] / l);
  lse[(size_t)bh * T + q] = m + __log2f(l);
}

template <typename TA, int HDM>
__global__ __launch_bounds__(128) void k_attn_dq_gen(const TA* __restrict__ qkv, const TA* __restrict__ dout,
                                                     const float* __restrict__ lse,
                                                     const float* __restrict__ Dv, TA* __restrict__ dqkv,
                                                     int B, int T, int H, int hd, float sl2, float scale) {
  int i = blockIdx.x * 128 + threadIdx.x;
  if (i >= B * H * T) return;
  int q = i % T, bh = i / T, b = bh / H, h = bh % H;
  const int C = H * hd, ld = 3 * C;
  const TA* base = qkv + (size_t)b * T * ld;
  float qv[HDM], dov[HDM], dq[HDM];
  for (int d = 0; d < hd; ++d) {
    qv[d] = to_f(base[(size_t)q * ld + h * hd + d]);
    dov[d] = to_f(dout[((size_t)b * T + q) * C + h * hd + d]);
    dq[d] = 0.f;
  }
  float lq = lse[(size_t)bh * T + q], Dq = Dv[(size_t)bh * T + q];
  for (int j = 0; j <= q; ++j) {
    const TA* kr = base + (size_t)j * ld + C + h * hd;
    const TA* vr = kr + C;
    float s = 0.f, dp = 0.f;
    for (int d = 0; d < hd; ++d) { s += qv[d] * to_f(kr[d]); dp += dov[d] * to_f(vr[d]); }
    float p = __builtin_amdgcn_exp2f(s * sl2 - lq);
    float ds = p * (dp - Dq);
    for (int d = 0; d < hd; ++d) dq[d] += ds * to_f(kr[d]);
  }
  TA* row = dqkv + ((size_t)b * T + q) * ld + h * hd;
  for (int d = 0; d < hd; ++d) row[d] = from_f<TA>(dq[d] * scale);
}

template <typename TA, int HDM>
__global__ __launch_bounds__(128) void k_attn_dkv_gen(const TA* __restrict__ qkv, const TA* __restrict__ dout,
                                                      const float* __restrict__ lse,
                                                      const float* __restrict__ Dv, TA* __restrict__ dqkv,
                                                      int B, int T, int H, int hd, float sl2, float scale) {
  int i = blockIdx.x * 128 + threadIdx.x;
  if (i >= B * H * T) return;
  int j = i % T, bh = i / T, b = bh / H, h = bh % H;
  const int C = H * hd, ld = 3 * C;
  const TA* base = qkv + (size_t)b * T * ld;
  float kv[HDM], vv[HDM], dk[HDM], dv[HDM];
  for (int d = 0; d < hd; ++d) {
    kv[d] = to_f(base[(size_t)j * ld + C + h * hd + d]);
    vv[d] = to_f(base[(size_t)j * ld + 2 * C + h * hd + d]);
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  for (int q = j; q < T; ++q) {
    const TA* qr = base + (size_t)q * ld + h * hd;
    const TA* dor = dout + ((size_t)b * T + q) * C + h * hd;
    float s = 0.f, dp = 0.f;
    for (int d = 0; d < hd; ++d) { s += to_f(qr[d]) * kv[d]; dp += to_f(dor[d]) * vv[d]; }
    float p = __builtin_amdgcn_exp2f(s * sl2 - lse[(size_t)bh * T + q]);
    float ds = p * (dp - Dv[(size_t)bh * T + q]);
    for (int d = 0; d < hd; ++d) { dv[d] += p * to_f(dor[d]); dk[d] += ds * to_f(qr[d]); }
  }
  TA* row = dqkv + ((size_t)b * T + j) * ld + C + h * hd;
  for (int d = 0; d < hd; ++d) {
    row[d] = from_f<TA>(dk[d] * scale);
    row[C + d] = from_f<TA>(dv[d]);
  }
}

// ------------------------------------------------------------------ host side
size_t attn_bwd_workspace(int B, int T, int H) { return (size_t)B * H * T; }

hipError_t attn_fwd(const void* qkv, void* o, float* lse, int B, int T, int H, int hd, bool bf,
                    hipStream_t st) {
  if (hd > 128) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf((float)hd);
  const float sl2 = scale * LOG2E_F;
  if (bf && hd == 64) {
    dim3 grid(cdiv(T, 128), B * H);
    k_attn_fwd64<<<grid, 256, 0, st>>>((const bf16*)qkv, (bf16*)o, lse, T, H, sl2);
  } else if (bf) {
    k_attn_fwd_gen<bf16, 128><<<cdiv((long)B * H * T, 128), 128, 0, st>>>(
        (const bf16*)qkv, (bf16*)o, lse, B, T, H, hd, sl2);
  } else {
    k_attn_fwd_gen<float, 128><<<cdiv((long)B * H * T, 128), 128, 0, st>>>(
        (const float*)qkv, (float*)o, lse, B, T, H, hd, sl2);
  }
  return hipGetLastError();
}

hipError_t attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse, void* dqkv,
                    float* ws, int B, int T, int H, int hd, bool bf, hipStream_t st) {
  if (hd > 128 || hd % 8) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf((float)hd);
  const float sl2 = scale * LOG2E_F;
  int n = B * T * H;
  if (bf)
    k_attn_bwd_pre<bf16><<<cdiv(n, 256), 256, 0, st>>>((const bf16*)o, (const bf16*)dout, ws, B, T, H, hd);
  else
    k_attn_bwd_pre<float><<<cdiv(n, 256), 256, 0, st>>>((const float*)o, (const float*)dout, ws, B, T, H, hd);
  if (bf && hd == 64) {
    dim3 grid(cdiv(T, 128), B * H);
    k_attn_dq64<<<grid, 256, 0, st>>>((const bf16*)qkv, (const bf16*)dout, lse, ws, (bf16*)dqkv, T,
                                      H, sl2, scale);
    k_attn_dkv64<<<grid, 256, 0, st>>>((const bf16*)qkv, (const bf16*)dout, lse, ws, (bf16*)dqkv, T,
                                       H, sl2, scale);
  } else if (bf) {
    int g = cdiv((long)B * H * T, 128);
    k_attn_dq_gen<bf16, 128><<<g, 128, 0, st>>>((const bf16*)qkv, (const bf16*)dout, lse, ws,
                                                (bf16*)dqkv, B, T, H, hd, sl2, scale);
    k_attn_dkv_gen<bf16, 128><<<g, 128, 0, st>>>((const bf16*)qkv, (const bf16*)dout, lse, ws,
                                                 (bf16*)dqkv, B, T, H, hd, sl2, scale);
  } else {
    int g = cdiv((long)B * H * T, 128);
    k_attn_dq_gen<float, 128><<<g, 128, 0, st>>>((const float*)qkv, (const float*)dout, lse, ws,
                                                 (float*)dqkv, B, T, H, hd, sl2, scale);
    k_attn_dkv_gen<float, 128><<<g, 128, 0, st>>>((const float*)qkv, (const float*)dout, lse, ws,
                                                  (float*)dqkv, B, T, H, hd, sl2, scale);
  }
  return hipGetLastError();
}

}  // namespace gk
