// GEMMs of the training step (all contractions except attention):
//   forward  Y = X W^T   (A, B both K-contiguous)
//   dX       dX = dY W   (B operand transposed in memory)
//   dW       dW = dY^T X (both operands transposed in memory)
// bf16 operands run on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation).  Tiles are staged global -> registers -> LDS with a
// double-buffered LDS ring; operands that are contiguous along M/N instead
// of K are loaded as 8x8 blocks and transposed in registers (v_perm), so the
// LDS always holds [row][k] and every MFMA fragment is one 16-byte LDS read.
// fp32 operands (the all-fp32 configuration) use an LDS-tiled FMA kernel.
// Epilogues fuse bias, tanh-GELU, residual add, the GELU derivative and
// the weight-gradient accumulation (alpha, beta) into the store.
#include "common.h"
#include "kernels.h"

namespace gk {



struct GP {
  int M, N, K;
  const void* A;
  long lda;
  const void* B;
  long ldb;
  void* out;
  long ldo;
  void* out2;
  const void* aux;
  const float* bias;
  float alpha, beta;
  int kchunk;  // split-K: K range per blockIdx.z (multiple of the K tile)
};

// ------------------------------------------------------------------ epilogues
template <int EPI, typename T>
__device__ __forceinline__ void epi_store(const GP& p, int r, int c, float acc) {
  if (r >= p.M || c >= p.N) return;
  size_t o = (size_t)r * p.ldo + c;
  if constexpr (EPI == EPI_STORE) {
    float v = p.alpha * acc + (p.bias ? p.bias[c] : 0.f);
    ((T*)p.out)[o] = from_f<T>(v);
  } else if constexpr (EPI == EPI_LOGITS) {
    ((T*)p.out)[o] = from_f<T>(acc);
  } else if constexpr (EPI == EPI_GELU) {
    float u = acc + p.bias[c];
    ((T*)p.out)[o] = from_f<T>(u);
    ((T*)p.out2)[o] = from_f<T>(gelu_tanh_f(u));
  } else if constexpr (EPI == EPI_RESID) {
    float v = ((const float*)p.aux)[o] + acc + p.bias[c];
    ((float*)p.out)[o] = v;
  } else if constexpr (EPI == EPI_DGELU) {
    float u = to_f(((const T*)p.aux)[o]);
    ((T*)p.out)[o] = from_f<T>(acc * gelu_tanh_grad_f(u));
  } else {  // EPI_WGRAD (fp32 output; with split-K, raw partials)
    float* op = (float*)p.out + (size_t)blockIdx.z * ((size_t)p.M * p.ldo);
    if (gridDim.z > 1) {
      op[o] = acc;
    } else {
      float v = p.alpha * acc;
      if (p.beta != 0.f) v += p.beta * op[o];
      op[o] = v;
    }
  }
}

// ------------------------------------------------------------------ bf16 MFMA kernel
constexpr int BK = 64;       // K tile (bf16 elements)
constexpr int LDS_LD = 72;   // padded LDS row (elements): 144 B, 16-byte aligned

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *(const uint4*)p; }

// Transpose of a KR x 8 block of bf16 (KR = 4 or 8): in[i] holds the 8
// row values of k = i; out[r] (KR/2 dwords) holds the KR k values of row r.
template <int KR>
__device__ __forceinline__ void transpose_block(const uint4 (&in)[KR], uint32_t (&out)[8][KR / 2]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t sel = (r & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int j = 0; j < KR / 2; ++j) {
      const uint4& lo = in[2 * j];
      const uint4& hi = in[2 * j + 1];
      uint32_t a = (r >> 1) == 0 ? lo.x : (r >> 1) == 1 ? lo.y : (r >> 1) == 2 ? lo.z : lo.w;
      uint32_t b = (r >> 1) == 0 ? hi.x : (r >> 1) == 1 ? hi.y : (r >> 1) == 2 ? hi.z : hi.w;
      out[r][j] = __builtin_amdgcn_perm(b, a, sel);
    }
  }
}

// Loader of one operand tile of ROWS x BK into registers, then into LDS.
// K-contiguous: ROWS * BK / 8 chunks of 16 B.  Transposed (memory [K][rows]):
// blocks of KR k-rows x 8 row-values (KR 16-byte loads), transposed in
// registers, written as 8 rows of KR k-values.
template <int ROWS, int NT, bool TRANS>
struct TileLoader {
  static constexpr int KR = ((BK / 8) * (ROWS / 8) >= NT) ? 8 : 4;
  static constexpr int KG = BK / KR;                       // k groups per tile
  static constexpr int NBLK = TRANS ? (KG * (ROWS / 8)) / NT : 0;
  static constexpr int NCH = TRANS ? NBLK * KR : (ROWS * BK / 8) / NT;
  static_assert(NCH >= 1, "tile too small for the thread count");
  static_assert(!TRANS || NBLK * NT == KG * (ROWS / 8), "transposed tile must split evenly");
  uint4 r[NCH];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, long ld, int row0,
                                       int nrows, int k0, int K, int tid) {
    if constexpr (!TRANS) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        int c = tid + i * NT;
        int row = c >> 3, kc = (c & 7) * 8;
        int gr = row0 + row, gk = k0 + kc;
        if (gr < nrows && gk < K)
          r[i] = ld16(base + (size_t)gr * ld + gk);
        else
          r[i] = make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int bi = 0; bi < NBLK; ++bi) {
        int b = tid + bi * NT;
        int ko = b % KG, ro = b / KG;
        int grow = row0 + ro * 8;
#pragma unroll
        for (int i = 0; i < KR; ++i) {
          int gk = k0 + ko * KR + i;
          if (gk < K && grow < nrows)
            r[bi * KR + i] = ld16(base + (size_t)gk * ld + grow);
          else
            r[bi * KR + i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* __restrict__ lds, int tid) {
    if constexpr (!TRANS) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        int c = tid + i * NT;
        int row = c >> 3, kc = (c & 7) * 8;
        *(uint4*)(lds + row * LDS_LD + kc) = r[i];
      }
    } else {
#pragma unroll
      for (int bi = 0; bi < NBLK; ++bi) {
        int b = tid + bi * NT;
        int ko = b % KG, ro = b / KG;
        uint4 in[KR];
        uint32_t out[8][KR / 2];
#pragma unroll
        for (int i = 0; i < KR; ++i) in[i] = r[bi * KR + i];
        transpose_block<KR>(in, out);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          uint16_t* dst = lds + (ro * 8 + rr) * LDS_LD + ko * KR;
          if constexpr (KR == 8)
            *(uint4*)dst = make_uint4(out[rr][0], out[rr][1], out[rr][2], out[rr][3]);
          else
            *(uint2*)dst = make_uint2(out[rr][0], out[rr][1]);
        }
      }
    }
  }
};

// Block-to-tile map: spread consecutive block ids over the 8 XCDs so that
// each XCD's L2 sees a contiguous band of tiles, then group GROUP_M tile
// rows so neighbouring blocks share A and B panels.
__device__ __forceinline__ void tile_coords(int nm, int nn, int& tm, int& tn) {
  int nb = nm * nn;
  int pid = blockIdx.x;
  int per = nb / 8;
  if (pid < per * 8) pid = (pid & 7) * per + (pid >> 3);
  constexpr int GROUP_M = 8;
  int group = GROUP_M * nn;
  int gid = pid / group;
  int first = gid * GROUP_M;
  int gsz = min(nm - first, GROUP_M);
  int in = pid % group;
  tm = first + in % gsz;
  tn = in / gsz;
}

template <int BM, int BN, int WM, int WN, bool AT, bool BT, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void k_gemm_bf16(GP p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 fragments per wave
  __shared__ uint16_t lds[2][(BM + BN) * LDS_LD];

  int tm, tn;
  tile_coords(cdiv(p.M, BM), cdiv(p.N, BN), tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = (wv / WN) * TM, wn = (wv % WN) * TN;
  const int kbeg = blockIdx.z * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);
  const int nk = cdiv(kend - kbeg, BK);

  const uint16_t* A = (const uint16_t*)p.A;
  const uint16_t* B = (const uint16_t*)p.B;
  TileLoader<BM, NT, AT> la;
  TileLoader<BN, NT, BT> lb;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  if (nk > 0) {
    la.load(A, p.lda, m0, p.M, kbeg, kend, tid);
    lb.load(B, p.ldb, n0, p.N, kbeg, kend, tid);
    la.store(&lds[0][0], tid);
    lb.store(&lds[0][BM * LDS_LD], tid);
  }
  __syncthreads();

  const int fr = lane & 31;        // fragment row / column
  const int fk = (lane >> 5) * 8;  // k offset inside a 16-wide k step
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(A, p.lda, m0, p.M, kbeg + (kt + 1) * BK, kend, tid);
      lb.load(B, p.ldb, n0, p.N, kbeg + (kt + 1) * BK, kend, tid);
    }
    const uint16_t* As = &lds[cur][0];
    const uint16_t* Bs = &lds[cur][BM * LDS_LD];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *(const uint4*)(As + (wm + i * 32 + fr) * LDS_LD + ks * 16 + fk));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, *(const uint4*)(Bs + (wn + j * 32 + fr) * LDS_LD + ks * 16 + fk));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      la.store(&lds[cur ^ 1][0], tid);
      lb.store(&lds[cur ^ 1][BM * LDS_LD], tid);
    }
    __syncthreads();
  }

  // accumulator layout of a 32x32 block: lane l holds column l % 32 and
  // rows 8 * (e / 4) + 4 * (l / 32) + e % 4
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int r = m0 + wm + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        int c = n0 + wn + j * 32 + fr;
        epi_store<EPI, bf16>(p, r, c, acc[i][j][e]);
      }
}

// ------------------------------------------------------------------ fp32 FMA kernel
template <bool AT, bool BT, int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(GP p) {
  constexpr int TB = 64, TK = 16;
  __shared__ float As[TK][TB + 4], Bs[TK][TB + 4];
  const int m0 = blockIdx.y * TB, n0 = blockIdx.x * TB;
  const int tid = threadIdx.x;
  const int tr = (tid / 16) * 4, tc = (tid % 16) * 4;
  const float* A = (const float*)p.A;
  const float* B = (const float*)p.B;
  const int kbeg = blockIdx.z * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += TK) {
    for (int e = tid; e < TB * TK; e += 256) {
      int rr, kk;
      if (AT) { kk = e / TB; rr = e % TB; } else { rr = e / TK; kk = e % TK; }
      int gm = m0 + rr, gk = k0 + kk;
      float v = 0.f;
      if (gm < p.M && gk < kend) v = AT ? A[(size_t)gk * p.lda + gm] : A[(size_t)gm * p.lda + gk];
      As[kk][rr] = v;
      if (BT) { kk = e / TB; rr = e % TB; } else { rr = e / TK; kk = e % TK; }
      int gn = n0 + rr;
      gk = k0 + kk;
      v = 0.f;
      if (gn < p.N && gk < kend) v = BT ? B[(size_t)gk * p.ldb + gn] : B[(size_t)gn * p.ldb + gk];
      Bs[kk][rr] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][tr + i]; b[i] = Bs[kk][tc + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) epi_store<EPI, float>(p, m0 + tr + i, n0 + tc + j, acc[i][j]);
}

// ------------------------------------------------------------------ split-K reduction
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ ws, int S,
                                                       size_t n, float* out, float alpha,
                                                       float beta) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float s = 0.f;
    for (int z = 0; z < S; ++z) s += ws[(size_t)z * n + i];
    float v = alpha * s;
    if (beta != 0.f) v += beta * out[i];
    out[i] = v;
  }
}

// ------------------------------------------------------------------ dispatch
static int splitk_for(int M, int N, int K, int bm, int bn) {
  long tiles = (long)cdiv(M, bm) * cdiv(N, bn);
  int s = 1;
  while (tiles * s < 512 && K / (s * 2) >= 1024 && s < 16) s *= 2;
  return s;
}

size_t gemm_splitk_ws_elems(int M, int N, int K) {
  int s = splitk_for(M, N, K, 128, 128);
  return s > 1 ? (size_t)s * M * N : 0;
}

template <bool AT, bool BT, int EPI>
static hipError_t launch_bf16(const GemmArgs& a, GP p, hipStream_t st) {
  constexpr int BM = 128, BN = 128, WM = 2, WN = 2;
  int nm = cdiv(a.M, BM), nn = cdiv(a.N, BN);
  int S = 1;
  if constexpr (EPI == EPI_WGRAD) {
    S = splitk_for(a.M, a.N, a.K, BM, BN);
    if (a.ldo != a.N || !a.splitk_ws || (size_t)S * a.M * a.N > a.splitk_ws_elems) S = 1;
  }
  int kchunk = cdiv(cdiv(a.K, S), BK) * BK;
  S = cdiv(a.K, kchunk);
  p.kchunk = kchunk;
  GP q = p;
  if (S > 1) q.out = a.splitk_ws;
  k_gemm_bf16<BM, BN, WM, WN, AT, BT, EPI><<<dim3(nm * nn, 1, S), WM * WN * 64, 0, st>>>(q);
  if (S > 1) {
    size_t n = (size_t)a.M * a.N;
    k_splitk_reduce<<<2048, 256, 0, st>>>(a.splitk_ws, S, n, (float*)a.out, a.alpha, a.beta);
  }
  return hipGetLastError();
}

template <bool AT, bool BT, int EPI>
static hipError_t launch_f32(const GemmArgs& a, GP p, hipStream_t st) {
  p.kchunk = a.K;
  k_gemm_f32<AT, BT, EPI><<<dim3(cdiv(a.N, 64), cdiv(a.M, 64), 1), 256, 0, st>>>(p);
  return hipGetLastError();
}

template <int EPI>
static hipError_t dispatch_t(const GemmArgs& a, const GP& p, hipStream_t st) {
  if (a.bf16) {
    if (!a.a_t && !a.b_t) return launch_bf16<false, false, EPI>(a, p, st);
    if (!a.a_t && a.b_t) return launch_bf16<false, true, EPI>(a, p, st);
    if (a.a_t && a.b_t) return launch_bf16<true, true, EPI>(a, p, st);
    return launch_bf16<true, false, EPI>(a, p, st);
  }
  if (!a.a_t && !a.b_t) return launch_f32<false, false, EPI>(a, p, st);
  if (!a.a_t && a.b_t) return launch_f32<false, true, EPI>(a, p, st);
  if (a.a_t && a.b_t) return launch_f32<true, true, EPI>(a, p, st);
  return launch_f32<true, false, EPI>(a, p, st);
}

hipError_t gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  GP p;
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.A = a.A; p.lda = a.lda; p.B = a.B; p.ldb = a.ldb;
  p.out = a.out; p.ldo = a.ldo; p.out2 = a.out2; p.aux = a.aux; p.bias = a.bias;
  p.alpha = a.alpha; p.beta = a.beta; p.kchunk = a.K;
  switch (a.kind) {
    case EPI_STORE: return dispatch_t<EPI_STORE>(a, p, st);
    case EPI_LOGITS: return dispatch_t<EPI_LOGITS>(a, p, st);
    case EPI_GELU: return dispatch_t<EPI_GELU>(a, p, st);
    case EPI_RESID: return dispatch_t<EPI_RESID>(a, p, st);
    case EPI_DGELU: return dispatch_t<EPI_DGELU>(a, p, st);
    case EPI_WGRAD: return dispatch_t<EPI_WGRAD>(a, p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gk
