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
  int kchunk;  // split-K: K range per split (multiple of the K tile)
  int splits;  // TN kernel: number of K splits (1: write the output directly)
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

// Four consecutive output columns c..c+3 of row r (bf16 activations).
template <int EPI>
__device__ __forceinline__ void epi_store4(const GP& p, int r, int c, float v0, float v1, float v2,
                                           float v3) {
  if (r >= p.M) return;
  if (c + 3 >= p.N) {
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (c + j < p.N) epi_store<EPI, bf16>(p, r, c + j, v[j]);
    return;
  }
  const size_t o = (size_t)r * p.ldo + c;
  if constexpr (EPI == EPI_STORE) {
    float4 b = p.bias ? *(const float4*)(p.bias + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    *(uint2*)((bf16*)p.out + o) = make_uint2(pack_bf2(p.alpha * v0 + b.x, p.alpha * v1 + b.y),
                                             pack_bf2(p.alpha * v2 + b.z, p.alpha * v3 + b.w));
  } else if constexpr (EPI == EPI_LOGITS) {
    *(uint2*)((bf16*)p.out + o) = make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
  } else if constexpr (EPI == EPI_GELU) {
    float4 b = *(const float4*)(p.bias + c);
    float u0 = v0 + b.x, u1 = v1 + b.y, u2 = v2 + b.z, u3 = v3 + b.w;
    *(uint2*)((bf16*)p.out + o) = make_uint2(pack_bf2(u0, u1), pack_bf2(u2, u3));
    *(uint2*)((bf16*)p.out2 + o) = make_uint2(pack_bf2(gelu_tanh_f(u0), gelu_tanh_f(u1)),
                                              pack_bf2(gelu_tanh_f(u2), gelu_tanh_f(u3)));
  } else if constexpr (EPI == EPI_RESID) {
    float4 b = *(const float4*)(p.bias + c);
    float4 x = *(const float4*)((const float*)p.aux + o);
    *(float4*)((float*)p.out + o) = make_float4(x.x + v0 + b.x, x.y + v1 + b.y, x.z + v2 + b.z,
                                                x.w + v3 + b.w);
  } else if constexpr (EPI == EPI_DGELU) {
    uint2 uu = *(const uint2*)((const bf16*)p.aux + o);
    float u0 = bfbits2f(uu.x & 0xffffu), u1 = bfbits2f(uu.x >> 16);
    float u2 = bfbits2f(uu.y & 0xffffu), u3 = bfbits2f(uu.y >> 16);
    *(uint2*)((bf16*)p.out + o) =
        make_uint2(pack_bf2(v0 * gelu_tanh_grad_f(u0), v1 * gelu_tanh_grad_f(u1)),
                   pack_bf2(v2 * gelu_tanh_grad_f(u2), v3 * gelu_tanh_grad_f(u3)));
  } else {  // EPI_WGRAD
    float* op = (float*)p.out + (size_t)blockIdx.z * ((size_t)p.M * p.ldo);
    if (gridDim.z > 1) {
      *(float4*)(op + o) = make_float4(v0, v1, v2, v3);
    } else {
      float4 w = make_float4(p.alpha * v0, p.alpha * v1, p.alpha * v2, p.alpha * v3);
      if (p.beta != 0.f) {
        float4 old = *(const float4*)(op + o);
        w.x += p.beta * old.x; w.y += p.beta * old.y; w.z += p.beta * old.z; w.w += p.beta * old.w;
      }
      *(float4*)(op + o) = w;
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
  // KR = 8 unless only KR = 4 splits the blocks evenly over the threads;
  // an uneven split leaves the last round to the first threads.
  static constexpr int KR = (((BK / 8) * (ROWS / 8)) % NT == 0) ? 8
                            : (((BK / 4) * (ROWS / 8)) % NT == 0) ? 4 : 8;
  static constexpr int KG = BK / KR;                       // k groups per tile
  static constexpr int TOT = KG * (ROWS / 8);              // transposed blocks per tile
  static constexpr int NBLK = TRANS ? (TOT + NT - 1) / NT : 0;
  static constexpr bool EVEN = TOT % NT == 0;
  static constexpr int NCH = TRANS ? NBLK * KR : (ROWS * BK / 8) / NT;
  static_assert(NCH >= 1, "tile too small for the thread count");
  static_assert(TRANS || (ROWS * BK / 8) % NT == 0, "K-contiguous tile must split evenly");
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
        const bool live = EVEN || b < TOT;
#pragma unroll
        for (int i = 0; i < KR; ++i) {
          int gk = k0 + ko * KR + i;
          if (live && gk < K && grow < nrows)
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
        if (!EVEN && b >= TOT) continue;
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

  const int fr = lane & 31;        // fragment row (m for A, n for B)
  const int fk = (lane >> 5) * 8;  // k offset inside a 16-wide k step
  // D = B_frag x A_frag: the accumulator is the transposed 32x32 block, so a
  // lane holds one output row and 4 runs of 4 consecutive output columns.
  auto substep = [&](const uint16_t* As, const uint16_t* Bs, int ks) {
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
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
  };

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool nxt = kt + 1 < nk;
    if (nxt) {
      la.load(A, p.lda, m0, p.M, kbeg + (kt + 1) * BK, kend, tid);
      lb.load(B, p.ldb, n0, p.N, kbeg + (kt + 1) * BK, kend, tid);
    }
    const uint16_t* As = &lds[cur][0];
    const uint16_t* Bs = &lds[cur][BM * LDS_LD];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) substep(As, Bs, ks);
    // the next tile's loads had the whole k step to arrive
    if (nxt) {
      la.store(&lds[cur ^ 1][0], tid);
      lb.store(&lds[cur ^ 1][BM * LDS_LD], tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        int r = m0 + wm + i * 32 + fr;
        int c = n0 + wn + j * 32 + e4 * 8 + (lane >> 5) * 4;
        epi_store4<EPI>(p, r, c, acc[i][j][e4 * 4 + 0], acc[i][j][e4 * 4 + 1],
                        acc[i][j][e4 * 4 + 2], acc[i][j][e4 * 4 + 3]);
      }
}

// ------------------------------------------------------------------ bf16 NT kernel, direct-to-LDS
// Both operands K-contiguous.  Persistent workgroups walk an XCD-grouped
// tile order; the K loop runs in stages of 32 k held in an NS-deep LDS ring
// that global_load_lds_dwordx4 fills directly (no VGPR staging), NS - 1
// stages ahead, continuing across tile boundaries so the next tile's loads
// are in flight during the epilogue.  LDS rows are 64 bytes (4 chunks of 8
// k); chunk c of row r sits in slot c ^ ((r >> 2) & 3), which keeps both the
// lane-linear direct loads and the 32-row MFMA fragment reads conflict free.
constexpr int NK = 32;  // k per stage
constexpr int NS = 4;   // LDS ring depth

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would also wait for every in-flight LDS DMA load (vmcnt 0) and collapse the
// ring to depth one.  Callers wait for the stage they need (vmcnt) first;
// LDS stores of this wave are drained here.
__device__ __forceinline__ void stage_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);  // compiler-only: keep LDS accesses on their side
  __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from base + voff + soff (range-checked against nbytes,
// zero outside) into LDS at lds + 16 * lane.
__device__ __attribute__((always_inline)) inline void buffer_load_lds16(void* base, uint32_t nbytes,
                                                                       uint16_t* lds, uint32_t voff,
                                                                       uint32_t soff) {
  auto rsrc = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// One operand's stage loads: NI buffer loads of 16 bytes per lane per stage,
// each filling one 16-row block of the LDS tile.  The per-lane byte offsets
// are loop invariant; the tile row and k position move in the scalar offset.
// Rows past the end of the operand read as zero (buffer range check).
template <int ROWS, int NW>
struct BufLoader {
  static constexpr int NI = ROWS * 4 / 64 / NW;  // 16-row blocks per wave per stage
  static_assert(NI * 64 * NW == ROWS * 4, "rows must split over the waves");
  void* base;
  uint32_t nbytes;
  uint32_t voff[NI];
  int blk0;
  __device__ __forceinline__ void init(const void* b, long ld, int nrows, int wv, int lane) {
    uint64_t bytes = (uint64_t)nrows * ld * 2;
    base = const_cast<void*>(b);
    nbytes = (uint32_t)(bytes > 0xffffffffull ? 0xffffffffull : bytes);
    blk0 = wv * NI;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (blk0 + i) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ ((r >> 2) & 3);
      voff[i] = (uint32_t)((long)r * ld * 2 + c * 16);
    }
  }
  // soff: byte offset of (row0, k0)
  __device__ __forceinline__ void issue(uint32_t soff, uint16_t* lds_op) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) buffer_load_lds16(base, nbytes, lds_op + (blk0 + i) * 512, voff[i], soff);
  }
};

// Ragged last stage (k0 + 32 > K): zero-filled register loads, LDS stores.
template <int ROWS, int NW>
__device__ __forceinline__ void issue_tail(const uint16_t* __restrict__ g, long ld, int row0,
                                           int nrows, int k0, int K, uint16_t* lds_op, int wv,
                                           int lane) {
  constexpr int NI = ROWS * 4 / 64 / NW;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int blk = wv * NI + i;
    const int r = blk * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const int gr = row0 + r, gk = k0 + c * 8;
    uint4 v = (gr < nrows && gk < K) ? *(const uint4*)(g + (size_t)gr * ld + gk)
                                      : make_uint4(0, 0, 0, 0);
    *(uint4*)(lds_op + blk * 512 + lane * 8) = v;
  }
}

__device__ __forceinline__ int tile_pid(int round, int G) {
  const int b = blockIdx.x;
  return round * G + (b & 7) * (G >> 3) + (b >> 3);
}

__device__ __forceinline__ void grouped_coords(int pid, int nm, int nn, int& tm, int& tn) {
  constexpr int GROUP_M = 8;
  int group = GROUP_M * nn;
  int gid = pid / group;
  int first = gid * GROUP_M;
  int gsz = min(nm - first, GROUP_M);
  int in = pid % group;
  tm = first + in % gsz;
  tn = in / gsz;
}

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm_nt(GP p) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int STAGE = (BM + BN) * NK;  // bf16 elements per stage
  constexpr int PER = BufLoader<BM, NW>::NI + BufLoader<BN, NW>::NI;  // loads per stage
  __shared__ __attribute__((aligned(1024))) uint16_t lds[NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = (wv / WN) * TM, wn = (wv % WN) * TN;
  const int fr = lane & 31, g = lane >> 5;
  const int swz = (fr >> 2) & 3;
  const int nm = cdiv(p.M, BM), nn = cdiv(p.N, BN);
  const int tiles = nm * nn;
  const int G = gridDim.x;
  const int nk = cdiv(p.K, NK);
  int my_n = 0;
  while (tile_pid(my_n, G) < tiles) ++my_n;
  const int total = my_n * nk;
  const bool ragged = (p.K % NK) != 0;

  BufLoader<BM, NW> la;
  BufLoader<BN, NW> lb;
  la.init(p.A, p.lda, p.M, wv, lane);
  lb.init(p.B, p.ldb, p.N, wv, lane);

  // issue-side cursor: stage t = (round, kt)
  int i_round = 0, i_kt = 0, i_tm = 0, i_tn = 0;
  if (total > 0) grouped_coords(tile_pid(0, G), nm, nn, i_tm, i_tn);
  auto issue_next = [&](int t) {
    uint16_t* st = lds + (t % NS) * STAGE;
    const int k0 = i_kt * NK;
    if (ragged && k0 + NK > p.K) {
      issue_tail<BM, NW>((const uint16_t*)p.A, p.lda, i_tm * BM, p.M, k0, p.K, st, wv, lane);
      issue_tail<BN, NW>((const uint16_t*)p.B, p.ldb, i_tn * BN, p.N, k0, p.K, st + BM * NK, wv, lane);
    } else {
      la.issue((uint32_t)(((long)i_tm * BM * p.lda + k0) * 2), st);
      lb.issue((uint32_t)(((long)i_tn * BN * p.ldb + k0) * 2), st + BM * NK);
    }
    if (++i_kt == nk) {
      i_kt = 0;
      ++i_round;
      if (i_round < my_n) grouped_coords(tile_pid(i_round, G), nm, nn, i_tm, i_tn);
    }
  };
  auto is_async = [&](int t) { return !(ragged && (t % nk) * NK + NK > p.K); };
  // wait until stage t has landed, stages up to `last` issued
  auto wait_stage = [&](int t, int last) {
    int after = 0;
    for (int u = t + 1; u <= last; ++u) after += is_async(u) ? 1 : 0;
    if (after >= 2) wait_vmcnt<2 * PER>();
    else if (after == 1) wait_vmcnt<PER>();
    else wait_vmcnt<0>();
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8 af[2][FM], bfr[2][FN];
  auto load_frags = [&](int t, int ks, int set) {
    const uint16_t* As = lds + (t % NS) * STAGE;
    const uint16_t* Bs = As + BM * NK;
    const int slot = (ks * 2 + g) ^ swz;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[set][i] = __builtin_bit_cast(bf16x8, *(const uint4*)(As + ((wm + i * 32 + fr) * 4 + slot) * 8));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bfr[set][j] = __builtin_bit_cast(bf16x8, *(const uint4*)(Bs + ((wn + j * 32 + fr) * 4 + slot) * 8));
  };
  auto mfma_set = [&](int set) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[set][j], af[set][i], acc[i][j], 0, 0, 0);
  };

  // Stage s + 1 is made visible (wait + barrier) one stage early, so the
  // first fragments of the next stage are read before the barrier and only
  // the barrier itself separates the two MFMA groups of a stage.
  if (total > 0) {
    const int pro = min(NS - 1, total);
    for (int t = 0; t < pro; ++t) issue_next(t);
    wait_stage(min(1, total - 1), pro - 1);
    stage_barrier();
    load_frags(0, 0, 0);
  }
  int s = 0;
  for (int round = 0; round < my_n; ++round) {
    for (int kt = 0; kt < nk; ++kt, ++s) {
      if (s + NS - 1 < total) issue_next(s + NS - 1);
      load_frags(s, 1, 1);
      mfma_set(0);
      if (s + 1 < total) load_frags(s + 1, 0, 0);
      if (s + 2 < total) wait_stage(s + 2, min(s + NS - 1, total - 1));
      stage_barrier();
      mfma_set(1);
    }
    int tm, tn;
    grouped_coords(tile_pid(round, G), nm, nn, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          int r = m0 + wm + i * 32 + fr;
          int c = n0 + wn + j * 32 + e4 * 8 + g * 4;
          epi_store4<EPI>(p, r, c, acc[i][j][e4 * 4 + 0], acc[i][j][e4 * 4 + 1],
                          acc[i][j][e4 * 4 + 2], acc[i][j][e4 * 4 + 3]);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
      }
  }
}

// ------------------------------------------------------------------ bf16 TN kernel (weight gradients)
// D[r][c] = sum_m A[m * lda + r] * B[m * ldb + c]: both operands keep their
// natural [token][feature] layout.  Stages of 32 tokens are loaded straight
// into LDS (buffer loads, tokens past M read as zero, so a ragged token
// count needs no special path) as [m][cols] tiles whose 16-byte chunk p of
// row m sits at p ^ 4 (m % 4); MFMA operands are built with the LDS
// transpose read (ds_read_b64_tr_b16): each 16-lane group reads a 4 x 16
// (token x feature) block and lane i receives the 4 tokens of feature i, so
// two reads give the 8 k values of a 32x32x16 operand.  The swizzle keeps
// the two 16-lane groups that share a cycle on all 64 banks.
constexpr int TK = 32;  // tokens per stage
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <int COLS, int NW>
struct TokLoader {
  static constexpr int CPR = COLS / 8;      // 16-byte chunks per token row
  static constexpr int NI = TK * CPR / 64 / NW;
  static_assert(CPR >= 16 && NI * 64 * NW == TK * CPR, "tile width must be >= 128, split evenly");
  void* base;
  uint32_t nbytes;
  uint32_t voff[NI];
  int blk0;
  __device__ __forceinline__ void init(const void* b, long ld, int M, int wv, int lane) {
    uint64_t bytes = (uint64_t)M * ld * 2;
    base = const_cast<void*>(b);
    nbytes = (uint32_t)(bytes > 0xffffffffull ? 0xffffffffull : bytes);
    blk0 = wv * NI;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int lin = (blk0 + i) * 64 + lane;   // LDS chunk slot
      const int m = lin / CPR, slot = lin % CPR;
      const int pch = slot ^ (4 * (m & 3));     // global chunk stored in this slot
      voff[i] = (uint32_t)((long)m * ld * 2 + pch * 16);
    }
  }
  __device__ __forceinline__ void issue(uint32_t soff, uint16_t* lds_op) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) buffer_load_lds16(base, nbytes, lds_op + (blk0 + i) * 512, voff[i], soff);
  }
};

// 8 k values (tokens ks*16 + 8g .. +7) of feature column `col` of an LDS tile
// [32][COLS], as an MFMA operand; lane l serves column base + l % 32.
template <int COLS>
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, int cbase, int ks, int lane) {
  const int G = lane >> 4, q = lane & 15;
  const int col = cbase + 16 * (G & 1) + 4 * (q & 3);
  v4s h[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int m = ks * 16 + 8 * (G >> 1) + 4 * hh + (q >> 2);
    const int off = m * COLS + (((col >> 3) ^ (4 * (m & 3))) << 3) + (col & 7);
    h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tile + off));
  }
  return __builtin_bit_cast(bf16x8, make_uint4(__builtin_bit_cast(uint32_t, (short2){h[0][0], h[0][1]}),
                                                 __builtin_bit_cast(uint32_t, (short2){h[0][2], h[0][3]}),
                                                 __builtin_bit_cast(uint32_t, (short2){h[1][0], h[1][1]}),
                                                 __builtin_bit_cast(uint32_t, (short2){h[1][2], h[1][3]})));
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm_tn(GP p) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int STAGE = (BM + BN) * TK;
  constexpr int PER = TokLoader<BM, NW>::NI + TokLoader<BN, NW>::NI;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = (wv / WN) * TM, wn = (wv % WN) * TN;
  const int fr = lane & 31, g = lane >> 5;
  const int nm = cdiv(p.M, BM), nn = cdiv(p.N, BN);
  const int tiles = nm * nn;
  const int S = p.splits;
  const int items = tiles * S;
  const int G = gridDim.x;
  int my_n = 0;
  while (tile_pid(my_n, G) < items) ++my_n;

  TokLoader<BM, NW> la;
  TokLoader<BN, NW> lb;
  la.init(p.A, p.lda, p.K, wv, lane);
  lb.init(p.B, p.ldb, p.K, wv, lane);

  auto item_nk = [&](int z) {
    const int kb = z * p.kchunk;
    return cdiv(min(p.K, kb + p.kchunk) - kb, TK);
  };
  // issue cursor
  int i_round = 0, i_kt = 0, i_tm = 0, i_tn = 0, i_z = 0, i_nk = 0;
  auto set_item = [&](int round, int& tm, int& tn, int& z) {
    const int pid = tile_pid(round, G);
    z = pid / tiles;
    grouped_coords(pid % tiles, nm, nn, tm, tn);
  };
  int total = 0;
  for (int r = 0; r < my_n; ++r) {
    int tm, tn, z;
    set_item(r, tm, tn, z);
    total += item_nk(z);
  }
  if (my_n > 0) {
    set_item(0, i_tm, i_tn, i_z);
    i_nk = item_nk(i_z);
  }
  auto issue_next = [&](int t) {
    uint16_t* st = lds + (t % NS) * STAGE;
    const int m0 = i_z * p.kchunk + i_kt * TK;
    la.issue((uint32_t)(((long)m0 * p.lda + i_tm * BM) * 2), st);
    lb.issue((uint32_t)(((long)m0 * p.ldb + i_tn * BN) * 2), st + BM * TK);
    if (++i_kt == i_nk) {
      i_kt = 0;
      if (++i_round < my_n) {
        set_item(i_round, i_tm, i_tn, i_z);
        i_nk = item_nk(i_z);
      }
    }
  };
  auto wait_stage = [&](int t, int last) {
    const int after = last - t;
    if (after >= 2) wait_vmcnt<2 * PER>();
    else if (after == 1) wait_vmcnt<PER>();
    else wait_vmcnt<0>();
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8 af[2][FM], bfr[2][FN];
  auto load_frags = [&](int t, int ks, int set) {
    const uint16_t* As = lds + (t % NS) * STAGE;
    const uint16_t* Bs = As + BM * TK;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[set][i] = tr_frag<BM>(As, wm + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[set][j] = tr_frag<BN>(Bs, wn + j * 32, ks, lane);
  };
  auto mfma_set = [&](int set) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[set][j], af[set][i], acc[i][j], 0, 0, 0);
  };

  if (total > 0) {
    const int pro = min(NS - 1, total);
    for (int t = 0; t < pro; ++t) issue_next(t);
    wait_stage(min(1, total - 1), pro - 1);
    stage_barrier();
    load_frags(0, 0, 0);
  }
  int s = 0;
  for (int round = 0; round < my_n; ++round) {
    int tm, tn, z;
    set_item(round, tm, tn, z);
    const int nk = item_nk(z);
    for (int kt = 0; kt < nk; ++kt, ++s) {
      if (s + NS - 1 < total) issue_next(s + NS - 1);
      load_frags(s, 1, 1);
      mfma_set(0);
      if (s + 1 < total) load_frags(s + 1, 0, 0);
      if (s + 2 < total) wait_stage(s + 2, min(s + NS - 1, total - 1));
      stage_barrier();
      mfma_set(1);
    }
    const int m0 = tm * BM, n0 = tn * BN;
    float* op = (float*)p.out + (S > 1 ? (size_t)z * p.M * p.ldo : 0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int r = m0 + wm + i * 32 + fr;
          const int c = n0 + wn + j * 32 + e4 * 8 + g * 4;
          if (r < p.M && c < p.N) {   // N % 4 == 0
            float4 v = make_float4(acc[i][j][e4 * 4 + 0], acc[i][j][e4 * 4 + 1], acc[i][j][e4 * 4 + 2],
                                   acc[i][j][e4 * 4 + 3]);
            float* dst = op + (size_t)r * p.ldo + c;
            if (S == 1) {
              v.x *= p.alpha; v.y *= p.alpha; v.z *= p.alpha; v.w *= p.alpha;
              if (p.beta != 0.f) {
                float4 o = *(const float4*)dst;
                v.x += p.beta * o.x; v.y += p.beta * o.y; v.z += p.beta * o.z; v.w += p.beta * o.w;
              }
            }
            *(float4*)dst = v;
          }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
      }
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
  const size_t n4 = n / 4;  // n is a multiple of 4 (N % 4 == 0 when split)
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int z = 0; z < S; ++z) {
      float4 v = *(const float4*)(ws + (size_t)z * n + 4 * i);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    float4 r = make_float4(alpha * s.x, alpha * s.y, alpha * s.z, alpha * s.w);
    if (beta != 0.f) {
      float4 o = *(const float4*)(out + 4 * i);
      r.x += beta * o.x; r.y += beta * o.y; r.z += beta * o.z; r.w += beta * o.w;
    }
    *(float4*)(out + 4 * i) = r;
  }
}

// ------------------------------------------------------------------ dispatch
// Tile shapes (block BM x BN, 2 x 2 waves) and a simple cost model: MFMA
// time of the waves of workgroups the grid needs on 256 CUs (relative
// efficiency per shape), plus the HBM time of the split-K partials.
struct TileCfg {
  int bm, bn, per_cu;
  double eff;
};
static const TileCfg kCfgs[4] = {{256, 256, 1, 1.00}, {256, 192, 1, 0.96}, {256, 128, 1, 0.88},
                                 {128, 128, 2, 0.60}};

struct Plan {
  int cfg, splits, kchunk;
};

static Plan plan_gemm(int M, int N, int K, bool wgrad, size_t ws_elems) {
  const double cu_flops = 2.5e15 / 256.0, hbm = 6.0e12;
  Plan best{3, 1, cdiv(K, BK) * BK};
  double best_t = 1e30;
  for (int ci = 0; ci < 4; ++ci) {
    const TileCfg& t = kCfgs[ci];
    long tiles = (long)cdiv(M, t.bm) * cdiv(N, t.bn);
    for (int S = 1; S <= (wgrad ? 32 : 1); ++S) {
      int kchunk = cdiv(cdiv(K, S), BK) * BK;
      if (cdiv(K, kchunk) != S) continue;
      if (S > 1 && (size_t)S * M * N > ws_elems) continue;
      long wg = tiles * S;
      long waves = (wg + 256L * t.per_cu - 1) / (256L * t.per_cu);
      double tm = waves * t.per_cu * (2.0 * t.bm * t.bn * kchunk) / (cu_flops * t.eff);
      double tr = S > 1 ? ((double)S + 2.0) * M * N * 4.0 / hbm + 3e-6 : 0.0;
      if (tm + tr < best_t) {
        best_t = tm + tr;
        best = Plan{ci, S, kchunk};
      }
    }
  }
  return best;
}

// Weight-gradient (TN) tile / split-K choice: 256x256 (8 waves), 256x128,
// 128x128 (two per CU); MFMA time of the workgroup waves at each shape's
// measured relative throughput plus the HBM time of the split partials.
struct TnPlan {
  int cfg, splits, kchunk;
};
static TnPlan plan_tn(int M, int N, int K, size_t ws_elems) {
  const int bm[3] = {256, 256, 128}, bn[3] = {256, 128, 128}, per_cu[3] = {1, 1, 2};
  const double eff[3] = {1.0, 0.65, 0.55};
  const double cu_flops = 2.5e15 / 256.0, hbm = 6.0e12;
  TnPlan best{2, 1, cdiv(K, TK) * TK};
  double bt = 1e30;
  for (int c = 0; c < 3; ++c) {
    long tiles = (long)cdiv(M, bm[c]) * cdiv(N, bn[c]);
    for (int S = 1; S <= 32; ++S) {
      int kchunk = cdiv(cdiv(K, S), TK) * TK;
      if (cdiv(K, kchunk) != S) continue;
      if (S > 1 && (size_t)S * M * N > ws_elems) continue;
      long slots = 256L * per_cu[c];
      long waves = (tiles * S + slots - 1) / slots;
      double t = waves * per_cu[c] * (2.0 * bm[c] * bn[c] * kchunk) / (cu_flops * eff[c]);
      if (S > 1) t += ((double)S + 2.0) * M * N * 4.0 / hbm + 3e-6;
      if (t < bt) {
        bt = t;
        best = TnPlan{c, S, kchunk};
      }
    }
  }
  return best;
}

size_t gemm_splitk_ws_elems(int M, int N, int K) {
  Plan pl = plan_gemm(M, N, K, true, (size_t)-1);
  size_t a = pl.splits > 1 ? (size_t)pl.splits * M * N : 0;
  TnPlan tp = plan_tn(M, N, K, (size_t)-1);
  size_t b = tp.splits > 1 ? (size_t)tp.splits * M * N : 0;
  return a > b ? a : b;
}

template <int BM, int BN, int WM, int WN>
static void launch_tn(GP q, int per_cu, hipStream_t st) {
  long items = (long)cdiv(q.M, BM) * cdiv(q.N, BN) * q.splits;
  long cap = 256L * per_cu;
  int grid = (int)(items < cap ? ((items + 7) / 8) * 8 : cap);
  k_gemm_tn<BM, BN, WM, WN><<<grid, WM * WN * 64, 0, st>>>(q);
}

template <int BM, int BN, bool AT, bool BT, int EPI>
static void launch_cfg(GP q, int S, hipStream_t st) {
  int nb = cdiv(q.M, BM) * cdiv(q.N, BN);
  k_gemm_bf16<BM, BN, 2, 2, AT, BT, EPI><<<dim3(nb, 1, S), 256, 0, st>>>(q);
}

// NT tile choice: 256x256 (8 waves), 256x192 or 256x128 (4 waves), by the
// number of 256-CU waves of tiles weighted with each shape's measured
// relative throughput.
static int plan_nt(int M, int N) {
  const int bn[3] = {256, 192, 128};
  const double eff[3] = {1.00, 0.93, 0.80};
  int best = 0;
  double bt = 1e30;
  for (int c = 0; c < 3; ++c) {
    long tiles = (long)cdiv(M, 256) * cdiv(N, bn[c]);
    double t = (double)((tiles + 255) / 256) * bn[c] / 256.0 / eff[c];
    if (t < bt - 1e-9) {
      bt = t;
      best = c;
    }
  }
  return best;
}

template <int BM, int BN, int WM, int WN, int EPI>
static void launch_nt(GP q, hipStream_t st) {
  int tiles = cdiv(q.M, BM) * cdiv(q.N, BN);
  int grid = tiles < 256 ? ((tiles + 7) / 8) * 8 : 256;
  k_gemm_nt<BM, BN, WM, WN, EPI><<<grid, WM * WN * 64, 0, st>>>(q);
}

template <bool AT, bool BT, int EPI>
static hipError_t launch_bf16(const GemmArgs& a, GP p, hipStream_t st) {
  if constexpr (AT && BT && EPI == EPI_WGRAD) {
    if (a.N % 4 == 0 && a.ldo == a.N && a.lda % 8 == 0 && a.ldb % 8 == 0 && a.splitk_ws) {
      TnPlan tp = plan_tn(a.M, a.N, a.K, a.splitk_ws_elems);
      p.kchunk = tp.kchunk;
      p.splits = tp.splits;
      GP q = p;
      if (tp.splits > 1) q.out = a.splitk_ws;
      switch (tp.cfg) {
        case 0: launch_tn<256, 256, 4, 2>(q, 1, st); break;
        case 1: launch_tn<256, 128, 2, 2>(q, 1, st); break;
        default: launch_tn<128, 128, 2, 2>(q, 2, st); break;
      }
      if (tp.splits > 1) {
        size_t n = (size_t)a.M * a.N;
        k_splitk_reduce<<<2048, 256, 0, st>>>(a.splitk_ws, tp.splits, n, (float*)a.out, a.alpha, a.beta);
      }
      return hipGetLastError();
    }
  }
  if constexpr (!AT && !BT && EPI != EPI_WGRAD) {
    if (a.K % 8 == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0) {
      p.kchunk = a.K;
      switch (plan_nt(a.M, a.N)) {
        case 0: launch_nt<256, 256, 4, 2, EPI>(p, st); break;
        case 1: launch_nt<256, 192, 2, 2, EPI>(p, st); break;
        default: launch_nt<256, 128, 2, 2, EPI>(p, st); break;
      }
      return hipGetLastError();
    }
  }
  const bool wg = EPI == EPI_WGRAD && a.ldo == a.N && a.splitk_ws;
  Plan pl = plan_gemm(a.M, a.N, a.K, wg, wg ? a.splitk_ws_elems : 0);
  p.kchunk = pl.kchunk;
  GP q = p;
  if (pl.splits > 1) q.out = a.splitk_ws;
  switch (pl.cfg) {
    case 0: launch_cfg<256, 256, AT, BT, EPI>(q, pl.splits, st); break;
    case 1: launch_cfg<256, 192, AT, BT, EPI>(q, pl.splits, st); break;
    case 2: launch_cfg<256, 128, AT, BT, EPI>(q, pl.splits, st); break;
    default: launch_cfg<128, 128, AT, BT, EPI>(q, pl.splits, st); break;
  }
  if (pl.splits > 1) {
    size_t n = (size_t)a.M * a.N;
    k_splitk_reduce<<<2048, 256, 0, st>>>(a.splitk_ws, pl.splits, n, (float*)a.out, a.alpha, a.beta);
  }
  return hipGetLastError();
}

template <bool AT, bool BT, int EPI>
static hipError_t launch_f32(const GemmArgs& a, GP p, hipStream_t st) {
  p.kchunk = a.K;
  k_gemm_f32<AT, BT, EPI><<<dim3(cdiv(a.N, 64), cdiv(a.M, 64), 1), 256, 0, st>>>(p);
  return hipGetLastError();
}

// Operand layouts used by the step: forward NT (A, B K-contiguous) with the
// store / classifier / GELU / residual epilogues; dX as NN (B transposed)
// with the store / GELU-derivative epilogues; dW as TN (both transposed).
template <int EPI>
static hipError_t dispatch_t(const GemmArgs& a, const GP& p, hipStream_t st) {
  constexpr bool NT_OK = EPI == EPI_STORE || EPI == EPI_LOGITS || EPI == EPI_GELU || EPI == EPI_RESID ||
                        EPI == EPI_DGELU;
  constexpr bool NN_OK = EPI == EPI_STORE || EPI == EPI_DGELU;
  constexpr bool TN_OK = EPI == EPI_WGRAD;
  if (a.bf16) {
    if constexpr (NT_OK)
      if (!a.a_t && !a.b_t) return launch_bf16<false, false, EPI>(a, p, st);
    if constexpr (NN_OK)
      if (!a.a_t && a.b_t) return launch_bf16<false, true, EPI>(a, p, st);
    if constexpr (TN_OK)
      if (a.a_t && a.b_t) return launch_bf16<true, true, EPI>(a, p, st);
    return hipErrorInvalidValue;
  }
  if constexpr (NT_OK)
    if (!a.a_t && !a.b_t) return launch_f32<false, false, EPI>(a, p, st);
  if constexpr (NN_OK)
    if (!a.a_t && a.b_t) return launch_f32<false, true, EPI>(a, p, st);
  if constexpr (TN_OK)
    if (a.a_t && a.b_t) return launch_f32<true, true, EPI>(a, p, st);
  return hipErrorInvalidValue;
}

hipError_t gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  GP p;
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.A = a.A; p.lda = a.lda; p.B = a.B; p.ldb = a.ldb;
  p.out = a.out; p.ldo = a.ldo; p.out2 = a.out2; p.aux = a.aux; p.bias = a.bias;
  p.alpha = a.alpha; p.beta = a.beta; p.kchunk = a.K; p.splits = 1;
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
