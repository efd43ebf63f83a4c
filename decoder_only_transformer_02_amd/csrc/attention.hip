// Causal multi-head self-attention, flash style ("Let's reproduce GPT-2
// (124M)" key takeaways, "Efficient Training Infrastructure": attention
// computed without materializing the T x T scores; chapter "flash
// attention").  softmax(q k^T / sqrt(hd)) v with query i attending keys
// j <= i.  q, k, v are read in place from the packed qkv rows [B*T, 3C].
//
// head_dim 64, 16-bit operands (bf16 or fp16): matrix-core kernels.  Each
// wave owns 32 queries (or 32 keys in the dK/dV kernel) as the 32-wide MFMA
// column; K/V (or Q/dO) tiles of 64 rows are staged in LDS, double-buffered
// (one barrier per tile), and shared by the 4 waves of a block.  This file
// is compiled with the MFMA operands and results in VGPRs (build.py): the
// softmax works on them directly instead of copying them out of AGPRs.  Tiles keep the row-major
// [row][d] layout; operands that need the contraction over rows (P V,
// dS K, P^T dO, dS^T Q) are built with the gfx950 LDS transpose read.
// Scores are formed transposed (S^T = K Q^T) so that a lane holds 16 scores
// of one query: the online softmax needs one cross-lane exchange and the
// probabilities feed the next MFMA straight from registers.  exp2 with the
// scale folded into log2 units.
//   forward: O and the row log-sum-exp (log2 units) per query.
//   backward: D = rowsum(dO * O) (computed by the dQ kernel); dQ kernel
//   (query-block parallel) and dK/dV kernel (key-block parallel), both
//   recomputing P from the saved log-sum-exp; no atomics, so results are
//   deterministic.
// Other head sizes / fp32: simple one-thread-per-row kernels.
#include "common.h"
#include "kernels.h"

namespace gk {

constexpr float LOG2E_F = 1.4426950408889634f;
constexpr float RESCALE_LOG2 = 8.f;  // forward: stale-max slack before rescaling (probabilities < 2^8)
constexpr int TILE = 64 * 64;  // one LDS tile, 16-bit elements

// LDS tiles are 64 rows of 64 16-bit values (128-byte rows, no padding);
// the 16-byte chunk p of row r is stored at chunk p ^ rev3((r / 2) % 8).
// With 64 banks of 4 bytes, row r covers the bank groups (4 banks each)
// 8 (r % 2) + chunk, so
//  * 16 consecutive rows reading (or writing) one chunk, 16 bytes each,
//    hit 16 distinct groups: per row parity, rev3 takes 8 distinct values;
//  * a transpose read of rows 4a .. 4a+3 by chunks 4c .. 4c+3 (the two
//    16-lane groups that share a cycle) hits 16 distinct groups: rows 4a and
//    4a+2 (and 4a+1, 4a+3) differ in bit 2 of their swizzle, which sends
//    their chunk quartets to opposite halves of the row.
__device__ __forceinline__ int rev3(int x) { return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1); }
__device__ __forceinline__ int sw_off(int r, int p) { return r * 64 + ((p ^ rev3((r >> 1) & 7)) << 3); }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <typename TE>
__device__ __forceinline__ uint4 ldg16(const TE* p) { return *(const uint4*)p; }

// Row-major MFMA operand: lane l holds the 8 values of chunk p of tile row r.
template <typename TE>
__device__ __forceinline__ typename H16<TE>::v8 lds_row(const uint16_t* tile, int r, int p) {
  return __builtin_bit_cast(typename H16<TE>::v8, *(const uint4*)(tile + sw_off(r, p)));
}

// Transposed MFMA operand: lane l serves column cbase + l % 32 of a tile
// and its slots s = 0..7 hold rows rbase + {0,1,2,3} and rbase + 8 +
// {0,1,2,3} (rbase is the lane's own, a multiple of 4).  Each
// ds_read_b64_tr_b16 has the 16 lanes of a group read a 4-row x 16-column
// block (lane 4j + c: row rbase + j, columns 4c .. 4c+3 of the group's 16)
// and hands lane i the 4 rows of column i.
template <typename TE>
__device__ __forceinline__ typename H16<TE>::v8 lds_tr(const uint16_t* tile, int cbase, int rbase, int lane) {
  const int q = lane & 15;
  const int col = cbase + 16 * ((lane >> 4) & 1) + 4 * (q & 3);
  v4s h[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = rbase + 8 * hh + (q >> 2);
    h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tile + sw_off(r, col >> 3) + (col & 7)));
  }
  return __builtin_bit_cast(typename H16<TE>::v8,
                            make_uint4(__builtin_bit_cast(uint32_t, (short2){h[0][0], h[0][1]}),
                                       __builtin_bit_cast(uint32_t, (short2){h[0][2], h[0][3]}),
                                       __builtin_bit_cast(uint32_t, (short2){h[1][0], h[1][1]}),
                                       __builtin_bit_cast(uint32_t, (short2){h[1][2], h[1][3]})));
}

// Pack accumulator values e = 8h .. 8h+7 of one 32x32 block to 16-bit slots.
template <typename TE>
__device__ __forceinline__ typename H16<TE>::v8 pack_slots(const f32x16& v, int h) {
  uint4 u = make_uint4(H16<TE>::pack2(v[8 * h + 0], v[8 * h + 1]), H16<TE>::pack2(v[8 * h + 2], v[8 * h + 3]),
                       H16<TE>::pack2(v[8 * h + 4], v[8 * h + 5]), H16<TE>::pack2(v[8 * h + 6], v[8 * h + 7]));
  return __builtin_bit_cast(typename H16<TE>::v8, u);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) { return H16<bf16>::mfma(a, b, c); }
__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) { return H16<f16>::mfma(a, b, c); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return z;
}

// A 64-row x 64-column 16-bit tile held in registers between its global load
// and its LDS store (2 x 16 bytes per thread), so the next tile's loads are
// in flight while the current one is being consumed.  Rows >= T load as 0.
struct Tile64 {
  uint4 v[2];
  template <typename TE>
  __device__ __forceinline__ void load(const TE* base, int ld, int r0, int T) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int c = threadIdx.x + i * 256;
      int row = c & 63, oct = c >> 6;
      int gr = r0 + row;
      v[i] = gr < T ? ldg16(base + (size_t)gr * ld + oct * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  // swizzled [row][col] layout
  __device__ __forceinline__ void store(uint16_t* dn) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int c = threadIdx.x + i * 256;
      int row = c & 63, oct = c >> 6;
      *(uint4*)(dn + sw_off(row, oct)) = v[i];
    }
  }
};

// ------------------------------------------------------------------ forward, hd = 64
// One 64-key tile of the forward for one wave (32 queries from qw0, the
// lane's query q): S^T = K Q^T from the row-major key tile, online-softmax
// update of (m, l), O^T += V^T P^T with V^T from the transpose read.
template <typename TE>
__device__ __forceinline__ void attn_fwd_tile(const uint16_t* Ks, const uint16_t* Vs,
                                              const typename H16<TE>::v8 (&qf)[4], f32x16 (&oacc)[2],
                                              float& m_i, float& l_i, int k0, int qw0, int q, int T, float sl2,
                                              int lane) {
  typedef typename H16<TE>::v8 v8;
  const int fr = lane & 31, g = lane >> 5;
  f32x16 s[2] = {zero16(), zero16()};
  // All eight key fragments are read before the first MFMA, and the two
  // 32-key blocks' MFMAs alternate: the reads' latency is paid once per
  // tile instead of before every MFMA.
  v8 kf[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kf[kb][ks] = lds_row<TE>(Ks, kb * 32 + fr, 2 * ks + g);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = mfma(kf[kb][ks], qf[ks], s[kb]);
  // Raw scores (masked ones -inf); the running max m_i is in log2 units.
  // It is raised only when the tile's max exceeds it by more than
  // RESCALE_LOG2: otherwise the tile's probabilities are taken against the
  // stale max (so they stay below 2^RESCALE_LOG2) and the accumulator needs
  // no rescaling, which would otherwise cost a multiply and two register
  // moves per accumulator element every tile.  O = oacc / l and
  // lse = m_i + log2 l are unchanged in exact arithmetic.
  const bool diag = k0 + 63 > qw0;  // tile reaches past the wave's first query
  if (diag) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int key = k0 + kb * 32 + (e >> 2) * 8 + g * 4 + (e & 3);
        if (key > q || key >= T) s[kb][e] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; e += 2) mx = fmaxf(mx, fmaxf(s[kb][e], s[kb][e + 1]));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));  // lanes l and l + 32 hold one query
  const float mxs = mx * sl2;
  if (mxs > m_i + RESCALE_LOG2) {  // always on the first tile (m_i = -inf)
    const float alpha = __builtin_amdgcn_exp2f(m_i - mxs);
    l_i *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    m_i = mxs;
  }
  float ps = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][e], sl2, -m_i));
      s[kb][e] = pv;
      ps += pv;
    }
  l_i += ps;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v8 pb = pack_slots<TE>(s[j >> 1], j & 1);
    int kbase = (j >> 1) * 32 + (j & 1) * 16 + g * 4;
#pragma unroll
    for (int db = 0; db < 2; ++db) oacc[db] = mfma(lds_tr<TE>(Vs, db * 32, kbase, lane), pb, oacc[db]);
  }
}

template <typename TE>
__global__ __launch_bounds__(256) void k_attn_fwd64(const TE* __restrict__ qkv,
                                                    TE* __restrict__ out, float* __restrict__ lse,
                                                    int T, int H, float sl2) {
  typedef typename H16<TE>::v8 v8;
  __shared__ uint16_t Ks[2][TILE];
  __shared__ uint16_t Vs[2][TILE];
  const int C = H * 64, ld = 3 * C;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q0 = (gridDim.x - 1 - blockIdx.x) * 128;  // heavy blocks first
  // the wave index through readfirstlane: the compiler then knows it (and
  // the tile tests built from it) to be uniform across the wave and keeps
  // those tests as scalar branches
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, g = lane >> 5;
  const int q = q0 + 32 * w + fr;
  const TE* base = qkv + (size_t)b * T * ld;
  const TE* kbase_p = base + C + h * 64;
  const TE* vbase_p = base + 2 * C + h * 64;

  v8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = __builtin_bit_cast(
        v8, q < T ? ldg16(base + (size_t)q * ld + h * 64 + ks * 16 + g * 8) : make_uint4(0, 0, 0, 0));

  f32x16 oacc[2] = {zero16(), zero16()};
  float m_i = -INFINITY, l_i = 0.f;
  const int qlast = min(q0 + 127, T - 1);
  const int ntiles = qlast / 64 + 1;
  const int wq_hi = min(q0 + 32 * w + 31, T - 1);

  // tile kt sits in buffer kt % 2; the registers carry tile kt + 1 from its
  // global load (issued after the compute of tile kt - 1) to its LDS store
  // (after the compute of tile kt), and the one barrier per tile orders
  // that store both after every wave's reads of the buffer's previous tile
  // and before the reads of the next iteration.
  Tile64 kt_r, vt_r;
  kt_r.load(kbase_p, ld, 0, T);
  vt_r.load(vbase_p, ld, 0, T);
  kt_r.store(Ks[0]);
  vt_r.store(Vs[0]);
  if (ntiles > 1) {
    kt_r.load(kbase_p, ld, 64, T);
    vt_r.load(vbase_p, ld, 64, T);
  }
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * 64, cur = kt & 1;
    if (k0 <= wq_hi) attn_fwd_tile<TE>(Ks[cur], Vs[cur], qf, oacc, m_i, l_i, k0, q0 + 32 * w, q, T, sl2, lane);
    if (kt + 1 < ntiles) {
      kt_r.store(Ks[cur ^ 1]);
      vt_r.store(Vs[cur ^ 1]);
      if (kt + 2 < ntiles) {
        kt_r.load(kbase_p, ld, k0 + 128, T);
        vt_r.load(vbase_p, ld, k0 + 128, T);
      }
      __syncthreads();
    }
  }
  const float l_tot = l_i + __shfl_xor(l_i, 32, 64);
  const float inv = 1.0f / l_tot;
  if (q < T) {
    TE* orow = out + ((size_t)b * T + q) * C + h * 64;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        int d = db * 32 + e4 * 8 + g * 4;
        *(uint2*)(orow + d) = make_uint2(H16<TE>::pack2(oacc[db][e4 * 4 + 0] * inv, oacc[db][e4 * 4 + 1] * inv),
                                         H16<TE>::pack2(oacc[db][e4 * 4 + 2] * inv, oacc[db][e4 * 4 + 3] * inv));
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
__device__ __forceinline__ float dot16<f16>(const uint4& a, const uint4& b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    s += H16<f16>::lo(x[j]) * H16<f16>::lo(y[j]) + H16<f16>::hi(x[j]) * H16<f16>::hi(y[j]);
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
// One 64-key tile of dQ for one wave: S^T = K Q^T and dP^T = V dO^T from
// row-major tiles, P from the saved log-sum-exp, dS^T = P (dP - D), and
// dQ^T += K^T dS^T with K^T from the transpose read.
template <typename TE>
__device__ __forceinline__ void attn_dq_tile(const uint16_t* Ks, const uint16_t* Vs,
                                             const typename H16<TE>::v8 (&qf)[4],
                                             const typename H16<TE>::v8 (&dof)[4], f32x16 (&dq)[2], float lq,
                                             float Dq, int k0, int qw0, int q, int T, float sl2, int lane) {
  typedef typename H16<TE>::v8 v8;
  const int fr = lane & 31, g = lane >> 5;
  const bool diag = k0 + 63 > qw0;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 s = zero16(), dp = zero16();
    // fragments read two k steps ahead of their MFMAs (all eight up front
    // would cost this kernel its third wave per SIMD)
    v8 kfr[4], vfr[4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kfr[ks] = lds_row<TE>(Ks, kb * 32 + fr, 2 * ks + g);
      vfr[ks] = lds_row<TE>(Vs, kb * 32 + fr, 2 * ks + g);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s = mfma(kfr[ks], qf[ks], s);
      dp = mfma(vfr[ks], dof[ks], dp);
      if (ks + 2 < 4) {
        kfr[ks + 2] = lds_row<TE>(Ks, kb * 32 + fr, 2 * (ks + 2) + g);
        vfr[ks + 2] = lds_row<TE>(Vs, kb * 32 + fr, 2 * (ks + 2) + g);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (diag) {  // masked scores to -inf: their probability comes out as 0
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int key = k0 + kb * 32 + (e >> 2) * 8 + g * 4 + (e & 3);
        if (key > q || key >= T) s[e] = -INFINITY;
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[e], sl2, -lq));
      s[e] = p * (dp[e] - Dq);  // dS^T
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      v8 dsb = pack_slots<TE>(s, hh);
      int kbase = kb * 32 + hh * 16 + g * 4;
#pragma unroll
      for (int db = 0; db < 2; ++db) dq[db] = mfma(lds_tr<TE>(Ks, db * 32, kbase, lane), dsb, dq[db]);
    }
  }
}

// Also computes D = rowsum(dO * O) for its queries (lanes l and l + 32 hold
// the two halves of a query's 64 dimensions) and writes it for the dK/dV
// kernel, which runs after it.
template <typename TE>
__global__ __launch_bounds__(256) void k_attn_dq64(const TE* __restrict__ qkv, const TE* __restrict__ o,
                                                   const TE* __restrict__ dout,
                                                   const float* __restrict__ lse,
                                                   float* __restrict__ Dv,
                                                   TE* __restrict__ dqkv, int T, int H, float sl2,
                                                   float scale) {
  typedef typename H16<TE>::v8 v8;
  __shared__ uint16_t Ks[2][TILE];
  __shared__ uint16_t Vs[2][TILE];
  const int C = H * 64, ld = 3 * C;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q0 = (gridDim.x - 1 - blockIdx.x) * 128;
  // the wave index through readfirstlane: the compiler then knows it (and
  // the tile tests built from it) to be uniform across the wave and keeps
  // those tests as scalar branches
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, g = lane >> 5;
  const int q = q0 + 32 * w + fr;
  const TE* base = qkv + (size_t)b * T * ld;
  const TE* dob = dout + (size_t)b * T * C;
  const TE* kp = base + C + h * 64;
  const TE* vp = base + 2 * C + h * 64;

  v8 qf[4], dof[4];
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qf[ks] = __builtin_bit_cast(
        v8, q < T ? ldg16(base + (size_t)q * ld + h * 64 + ks * 16 + g * 8) : make_uint4(0, 0, 0, 0));
    const uint4 du = q < T ? ldg16(dob + (size_t)q * C + h * 64 + ks * 16 + g * 8) : make_uint4(0, 0, 0, 0);
    const uint4 ou = q < T ? ldg16(o + ((size_t)b * T + q) * C + h * 64 + ks * 16 + g * 8) : make_uint4(0, 0, 0, 0);
    dof[ks] = __builtin_bit_cast(v8, du);
    dpart += dot16<TE>(du, ou);
  }
  const float lq = q < T ? lse[(size_t)bh * T + q] : 0.f;
  const float Dq = dpart + __shfl_xor(dpart, 32, 64);
  if (g == 0 && q < T) Dv[(size_t)bh * T + q] = Dq;
  f32x16 dq[2] = {zero16(), zero16()};
  const int qlast = min(q0 + 127, T - 1);
  const int ntiles = qlast / 64 + 1;
  const int wq_hi = min(q0 + 32 * w + 31, T - 1);

  // double-buffered tiles, one barrier per tile (as in the forward)
  Tile64 kr, vr;
  kr.load(kp, ld, 0, T);
  vr.load(vp, ld, 0, T);
  kr.store(Ks[0]);
  vr.store(Vs[0]);
  if (ntiles > 1) {
    kr.load(kp, ld, 64, T);
    vr.load(vp, ld, 64, T);
  }
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * 64, cur = kt & 1;
    if (k0 <= wq_hi) attn_dq_tile<TE>(Ks[cur], Vs[cur], qf, dof, dq, lq, Dq, k0, q0 + 32 * w, q, T, sl2, lane);
    if (kt + 1 < ntiles) {
      kr.store(Ks[cur ^ 1]);
      vr.store(Vs[cur ^ 1]);
      if (kt + 2 < ntiles) {
        kr.load(kp, ld, k0 + 128, T);
        vr.load(vp, ld, k0 + 128, T);
      }
      __syncthreads();
    }
  }
  if (q < T) {
    TE* row = dqkv + ((size_t)b * T + q) * ld + h * 64;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        int d = db * 32 + e4 * 8 + g * 4;
        *(uint2*)(row + d) = make_uint2(H16<TE>::pack2(dq[db][e4 * 4 + 0] * scale, dq[db][e4 * 4 + 1] * scale),
                                        H16<TE>::pack2(dq[db][e4 * 4 + 2] * scale, dq[db][e4 * 4 + 3] * scale));
      }
  }
}

// ------------------------------------------------------------------ dK, dV, hd = 64
// One 64-query tile of dK/dV for one wave (32 keys from wk_lo, the lane's
// key): S and dP for the tile's queries x the wave's keys from row-major
// tiles, P from the saved log-sum-exp, dS = P (dP - D); dV^T += dO^T P and
// dK^T += Q^T dS with dO^T and Q^T from the transpose read.
template <typename TE>
__device__ __forceinline__ void attn_dkv_tile(const uint16_t* Qs, const uint16_t* Os, const float* Ls,
                                              const float* Ds, const typename H16<TE>::v8 (&kf)[4],
                                              const typename H16<TE>::v8 (&vf)[4], f32x16 (&dk)[2],
                                              f32x16 (&dv)[2], int q0, int wk_lo, int key, int T, float sl2,
                                              int lane) {
  typedef typename H16<TE>::v8 v8;
  const int fr = lane & 31, g = lane >> 5;
  const bool diag = q0 < wk_lo + 31;  // some (q, key) pairs of the tile are masked
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    // S and dP for 32 queries x this wave's 32 keys:
    // rows q = q0 + qb*32 + 8(e/4) + 4g + e%4, column key
    f32x16 s = zero16(), dp = zero16();
    // the eight fragments first, then the MFMAs (as in the forward)
    v8 qfr[4], ofr[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qfr[ks] = lds_row<TE>(Qs, qb * 32 + fr, 2 * ks + g);
      ofr[ks] = lds_row<TE>(Os, qb * 32 + fr, 2 * ks + g);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s = mfma(qfr[ks], kf[ks], s);
      dp = mfma(ofr[ks], vf[ks], dp);
    }
    if (diag) {  // masked scores to -inf: their probability comes out as 0
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int qq = q0 + qb * 32 + (e >> 2) * 8 + g * 4 + (e & 3);
        if (key > qq || qq >= T) s[e] = -INFINITY;
      }
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
        const float p = __builtin_amdgcn_exp2f(fmaf(s[e], sl2, -Lr[e1]));
        s[e] = p;
        dp[e] = p * (dp[e] - Dr[e1]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      v8 pb = pack_slots<TE>(s, hh);
      v8 dsb = pack_slots<TE>(dp, hh);
      int qbase = qb * 32 + hh * 16 + g * 4;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        dv[db] = mfma(lds_tr<TE>(Os, db * 32, qbase, lane), pb, dv[db]);
        dk[db] = mfma(lds_tr<TE>(Qs, db * 32, qbase, lane), dsb, dk[db]);
      }
    }
  }
}

template <typename TE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_dkv64(const TE* __restrict__ qkv,
                                                    const TE* __restrict__ dout,
                                                    const float* __restrict__ lse,
                                                    const float* __restrict__ Dv,
                                                    TE* __restrict__ dqkv, int T, int H, float sl2,
                                                    float scale) {
  typedef typename H16<TE>::v8 v8;
  __shared__ uint16_t Qs[2][TILE];
  __shared__ uint16_t Os[2][TILE];   // dO [q][d]
  __shared__ float Ls[2][64], Ds[2][64];
  const int C = H * 64, ld = 3 * C;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int k0 = blockIdx.x * 128;
  // the wave index through readfirstlane: the compiler then knows it (and
  // the tile tests built from it) to be uniform across the wave and keeps
  // those tests as scalar branches
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, g = lane >> 5;
  const int key = k0 + 32 * w + fr;
  const TE* base = qkv + (size_t)b * T * ld;
  const TE* dob = dout + (size_t)b * T * C;
  const TE* qp = base + h * 64;
  const TE* op = dob + h * 64;

  v8 kf[4], vf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kf[ks] = __builtin_bit_cast(
        v8, key < T ? ldg16(base + (size_t)key * ld + C + h * 64 + ks * 16 + g * 8) : make_uint4(0, 0, 0, 0));
    vf[ks] = __builtin_bit_cast(
        v8, key < T ? ldg16(base + (size_t)key * ld + 2 * C + h * 64 + ks * 16 + g * 8) : make_uint4(0, 0, 0, 0));
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
  // double-buffered tiles, one barrier per tile (as in the forward)
  auto store_q = [&](int buf) {
    qr.store(Qs[buf]);
    orr.store(Os[buf]);
    if (tid < 64) {
      Ls[buf][tid] = lr;
      Ds[buf][tid] = dr;
    }
  };
  load_q(qt0);
  store_q(0);
  if (qt0 + 1 < nqt) load_q(qt0 + 1);
  __syncthreads();
  for (int qt = qt0; qt < nqt; ++qt) {
    const int q0 = qt * 64, cur = (qt - qt0) & 1;
    if (q0 + 63 >= wk_lo && wk_lo < T)
      attn_dkv_tile<TE>(Qs[cur], Os[cur], Ls[cur], Ds[cur], kf, vf, dk, dv, q0, wk_lo, key, T, sl2, lane);
    if (qt + 1 < nqt) {
      store_q(cur ^ 1);
      if (qt + 2 < nqt) load_q(qt + 2);
      __syncthreads();
    }
  }
  if (key < T) {
    TE* rk = dqkv + ((size_t)b * T + key) * ld + C + h * 64;
    TE* rv = rk + C;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        int d = db * 32 + e4 * 8 + g * 4;
        *(uint2*)(rk + d) = make_uint2(H16<TE>::pack2(dk[db][e4 * 4 + 0] * scale, dk[db][e4 * 4 + 1] * scale),
                                       H16<TE>::pack2(dk[db][e4 * 4 + 2] * scale, dk[db][e4 * 4 + 3] * scale));
        *(uint2*)(rv + d) = make_uint2(H16<TE>::pack2(dv[db][e4 * 4 + 0], dv[db][e4 * 4 + 1]),
                                       H16<TE>::pack2(dv[db][e4 * 4 + 2], dv[db][e4 * 4 + 3]));
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

template <typename TE>
static hipError_t attn_fwd_t(const void* qkv, void* o, float* lse, int B, int T, int H, int hd, float sl2,
                             hipStream_t st) {
  if (hd == 64) {
    dim3 grid(cdiv(T, 128), B * H);
    k_attn_fwd64<TE><<<grid, 256, 0, st>>>((const TE*)qkv, (TE*)o, lse, T, H, sl2);
  } else {
    k_attn_fwd_gen<TE, 128><<<cdiv((long)B * H * T, 128), 128, 0, st>>>((const TE*)qkv, (TE*)o, lse, B, T, H,
                                                                        hd, sl2);
  }
  return hipGetLastError();
}

hipError_t attn_fwd(const void* qkv, void* o, float* lse, int B, int T, int H, int hd, int dt,
                    hipStream_t st) {
  if (hd > 128) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf((float)hd);
  const float sl2 = scale * LOG2E_F;
  if (dt == ACT_BF16) return attn_fwd_t<bf16>(qkv, o, lse, B, T, H, hd, sl2, st);
  if (dt == ACT_F16) return attn_fwd_t<f16>(qkv, o, lse, B, T, H, hd, sl2, st);
  k_attn_fwd_gen<float, 128><<<cdiv((long)B * H * T, 128), 128, 0, st>>>(
      (const float*)qkv, (float*)o, lse, B, T, H, hd, sl2);
  return hipGetLastError();
}

template <typename TA>
static hipError_t attn_bwd_t(const void* qkv, const void* o, const void* dout, const float* lse, void* dqkv,
                             float* ws, int B, int T, int H, int hd, float sl2, float scale, hipStream_t st) {
  const int n = B * T * H;
  if constexpr (sizeof(TA) == 2) {
    if (hd == 64) {  // the dQ kernel computes D itself
      dim3 grid(cdiv(T, 128), B * H);
      k_attn_dq64<TA><<<grid, 256, 0, st>>>((const TA*)qkv, (const TA*)o, (const TA*)dout, lse, ws, (TA*)dqkv, T,
                                            H, sl2, scale);
      k_attn_dkv64<TA><<<grid, 256, 0, st>>>((const TA*)qkv, (const TA*)dout, lse, ws, (TA*)dqkv, T, H, sl2,
                                             scale);
      return hipGetLastError();
    }
  }
  k_attn_bwd_pre<TA><<<cdiv(n, 256), 256, 0, st>>>((const TA*)o, (const TA*)dout, ws, B, T, H, hd);
  const int g = cdiv((long)B * H * T, 128);
  k_attn_dq_gen<TA, 128><<<g, 128, 0, st>>>((const TA*)qkv, (const TA*)dout, lse, ws, (TA*)dqkv, B, T, H, hd,
                                            sl2, scale);
  k_attn_dkv_gen<TA, 128><<<g, 128, 0, st>>>((const TA*)qkv, (const TA*)dout, lse, ws, (TA*)dqkv, B, T, H, hd,
                                             sl2, scale);
  return hipGetLastError();
}

hipError_t attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse, void* dqkv,
                    float* ws, int B, int T, int H, int hd, int dt, hipStream_t st) {
  if (hd > 128 || hd % 8) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf((float)hd);
  const float sl2 = scale * LOG2E_F;
  if (dt == ACT_BF16) return attn_bwd_t<bf16>(qkv, o, dout, lse, dqkv, ws, B, T, H, hd, sl2, scale, st);
  if (dt == ACT_F16) return attn_bwd_t<f16>(qkv, o, dout, lse, dqkv, ws, B, T, H, hd, sl2, scale, st);
  return attn_bwd_t<float>(qkv, o, dout, lse, dqkv, ws, B, T, H, hd, sl2, scale, st);
}

}  // namespace gk
