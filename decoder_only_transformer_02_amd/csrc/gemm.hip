// GEMMs of the training step (all contractions except attention):
//   forward  Y = X W^T   (A, B both K-contiguous)
//   dX       dX = dY W   (B operand transposed in memory)
//   dW       dW = dY^T X (both operands transposed in memory)
// 16-bit operands (bf16, or fp16 for the fp16 workload) run on the gfx950
// matrix cores (v_mfma_f32_32x32x16_bf16 / _f16, fp32 accumulation):
//   * forward and dX: persistent k_gemm_nt, operands loaded straight into an
//     LDS ring; the dX weight stays [out][in] and its MFMA operands come from
//     the LDS transpose read;
//   * dW: persistent k_gemm_tn, both operands [token][feature] in LDS, read
//     with the LDS transpose, split over tokens when the tiles are few;
//   * other layouts or alignments: k_gemm_h16, register-staged tiles with
//     8x8 blocks transposed in registers (v_perm).
// fp32 operands (the all-fp32 configuration) use the fp32 matrix cores for
// large problems and an LDS-tiled FMA kernel for small ones.
// Epilogues fuse bias, tanh-GELU, residual add, the GELU derivative and
// the weight-gradient accumulation (alpha, beta) into the store.
#include <type_traits>

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
  float* dbias;     // TN kernel: bias gradient, column sums of A (null: none)
  float* dbias_ws;  // TN kernel with splits: [splits][M] partial column sums
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

// Four consecutive output columns c..c+3 of row r (16-bit activations TE).
template <int EPI, typename TE>
__device__ __forceinline__ void epi_store4(const GP& p, int r, int c, float v0, float v1, float v2,
                                           float v3) {
  if (r >= p.M) return;
  if (c + 3 >= p.N) {
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (c + j < p.N) epi_store<EPI, TE>(p, r, c + j, v[j]);
    return;
  }
  const size_t o = (size_t)r * p.ldo + c;
  if constexpr (EPI == EPI_STORE) {
    float4 b = p.bias ? *(const float4*)(p.bias + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    *(uint2*)((TE*)p.out + o) = make_uint2(H16<TE>::pack2(p.alpha * v0 + b.x, p.alpha * v1 + b.y),
                                             H16<TE>::pack2(p.alpha * v2 + b.z, p.alpha * v3 + b.w));
  } else if constexpr (EPI == EPI_LOGITS) {
    *(uint2*)((TE*)p.out + o) = make_uint2(H16<TE>::pack2(v0, v1), H16<TE>::pack2(v2, v3));
  } else if constexpr (EPI == EPI_GELU) {
    float4 b = *(const float4*)(p.bias + c);
    float u0 = v0 + b.x, u1 = v1 + b.y, u2 = v2 + b.z, u3 = v3 + b.w;
    *(uint2*)((TE*)p.out + o) = make_uint2(H16<TE>::pack2(u0, u1), H16<TE>::pack2(u2, u3));
    *(uint2*)((TE*)p.out2 + o) = make_uint2(H16<TE>::pack2(gelu_tanh_f(u0), gelu_tanh_f(u1)),
                                              H16<TE>::pack2(gelu_tanh_f(u2), gelu_tanh_f(u3)));
  } else if constexpr (EPI == EPI_RESID) {
    float4 b = *(const float4*)(p.bias + c);
    float4 x = *(const float4*)((const float*)p.aux + o);
    *(float4*)((float*)p.out + o) = make_float4(x.x + v0 + b.x, x.y + v1 + b.y, x.z + v2 + b.z,
                                                x.w + v3 + b.w);
  } else if constexpr (EPI == EPI_DGELU) {
    uint2 uu = *(const uint2*)((const TE*)p.aux + o);
    float u0 = H16<TE>::lo(uu.x), u1 = H16<TE>::hi(uu.x);
    float u2 = H16<TE>::lo(uu.y), u3 = H16<TE>::hi(uu.y);
    *(uint2*)((TE*)p.out + o) =
        make_uint2(H16<TE>::pack2(v0 * gelu_tanh_grad_f(u0), v1 * gelu_tanh_grad_f(u1)),
                   H16<TE>::pack2(v2 * gelu_tanh_grad_f(u2), v3 * gelu_tanh_grad_f(u3)));
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

// The 16-bit epilogues of a tile that lies wholly inside the output: no
// bounds tests, and the bias of columns c..c+3 passed in (loaded once for
// all the row fragments that share those columns), so the compiler can keep
// one row address per fragment and fold the column offsets into the stores.
template <int EPI, typename TE>
__device__ __forceinline__ void epi_store4_full(const GP& p, int r, int c, float4 b, float v0, float v1,
                                                float v2, float v3) {
  const size_t o = (size_t)r * p.ldo + c;
  if constexpr (EPI == EPI_STORE) {
    *(uint2*)((TE*)p.out + o) = make_uint2(H16<TE>::pack2(p.alpha * v0 + b.x, p.alpha * v1 + b.y),
                                             H16<TE>::pack2(p.alpha * v2 + b.z, p.alpha * v3 + b.w));
  } else if constexpr (EPI == EPI_LOGITS) {
    *(uint2*)((TE*)p.out + o) = make_uint2(H16<TE>::pack2(v0, v1), H16<TE>::pack2(v2, v3));
  } else if constexpr (EPI == EPI_GELU) {
    float u0 = v0 + b.x, u1 = v1 + b.y, u2 = v2 + b.z, u3 = v3 + b.w;
    *(uint2*)((TE*)p.out + o) = make_uint2(H16<TE>::pack2(u0, u1), H16<TE>::pack2(u2, u3));
    *(uint2*)((TE*)p.out2 + o) = make_uint2(H16<TE>::pack2(gelu_tanh_f(u0), gelu_tanh_f(u1)),
                                              H16<TE>::pack2(gelu_tanh_f(u2), gelu_tanh_f(u3)));
  } else if constexpr (EPI == EPI_RESID) {
    float4 x = *(const float4*)((const float*)p.aux + o);
    *(float4*)((float*)p.out + o) = make_float4(x.x + v0 + b.x, x.y + v1 + b.y, x.z + v2 + b.z,
                                                x.w + v3 + b.w);
  } else if constexpr (EPI == EPI_DGELU) {
    uint2 uu = *(const uint2*)((const TE*)p.aux + o);
    float u0 = H16<TE>::lo(uu.x), u1 = H16<TE>::hi(uu.x);
    float u2 = H16<TE>::lo(uu.y), u3 = H16<TE>::hi(uu.y);
    *(uint2*)((TE*)p.out + o) =
        make_uint2(H16<TE>::pack2(v0 * gelu_tanh_grad_f(u0), v1 * gelu_tanh_grad_f(u1)),
                   H16<TE>::pack2(v2 * gelu_tanh_grad_f(u2), v3 * gelu_tanh_grad_f(u3)));
  }
}

template <int EPI>
__device__ __forceinline__ float4 epi_bias4(const GP& p, int c) {
  if constexpr (EPI == EPI_GELU || EPI == EPI_RESID) return *(const float4*)(p.bias + c);
  if constexpr (EPI == EPI_STORE) return p.bias ? *(const float4*)(p.bias + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  return make_float4(0.f, 0.f, 0.f, 0.f);
}

// ------------------------------------------------------------------ 16-bit MFMA kernel
constexpr int BK = 64;       // K tile (16-bit elements)
constexpr int LDS_LD = 72;   // padded LDS row (elements): 144 B, 16-byte aligned

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *(const uint4*)p; }

// Transpose of a KR x 8 block of 16-bit values (KR = 4 or 8): in[i] holds the 8
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

template <typename TE, int BM, int BN, int WM, int WN, bool AT, bool BT, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void k_gemm_h16(GP p) {
  typedef typename H16<TE>::v8 v8;
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
    v8 af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[i] = __builtin_bit_cast(v8, *(const uint4*)(As + (wm + i * 32 + fr) * LDS_LD + ks * 16 + fk));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bfr[j] = __builtin_bit_cast(v8, *(const uint4*)(Bs + (wn + j * 32 + fr) * LDS_LD + ks * 16 + fk));
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = H16<TE>::mfma(bfr[j], af[i], acc[i][j]);
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
        epi_store4<EPI, TE>(p, r, c, acc[i][j][e4 * 4 + 0], acc[i][j][e4 * 4 + 1],
                            acc[i][j][e4 * 4 + 2], acc[i][j][e4 * 4 + 3]);
      }
}

// ------------------------------------------------------------------ 16-bit NT kernel, direct-to-LDS
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

// Compiler scheduling fence (emits no instruction): nothing is moved across
// it, so the fragment reads and MFMA groups keep their software-pipelined
// order instead of the scheduler's register-saving one.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from base + soff + voff into LDS at lds + 16 * lane.
// The descriptor starts at base + soff and holds the nbytes - soff bytes
// that remain of the operand (soff < nbytes), so the hardware range check
// sees only the per-lane offset: a lane whose bytes lie past the operand's
// end reads zero, whatever the check does with a scalar offset.
__device__ __attribute__((always_inline)) inline void buffer_load_lds16(void* base, uint32_t nbytes,
                                                                       uint16_t* lds, uint32_t voff,
                                                                       uint32_t soff) {
  auto rsrc = __builtin_amdgcn_make_buffer_rsrc((char*)base + soff, (short)0, (int)(nbytes - soff),
                                                0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// One operand's stage loads: NI buffer loads of 16 bytes per lane per stage,
// each filling one 16-row block of the LDS tile.  The per-lane byte offsets
// are loop invariant; the tile row and k position move the descriptor base.
// Rows past the end of the operand read as zero (range check of the per-lane
// offset against the bytes left after the stage's start).
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

// 16 bytes of row `row` from column k (k % 8 == 0, row 16-byte aligned),
// zero past column K: the chunk that straddles K is read element by element.
__device__ __forceinline__ uint4 load_k_chunk(const uint16_t* __restrict__ row, int k, int K) {
  if (k + 8 <= K) return *(const uint4*)(row + k);
  uint16_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = k + i < K ? row[k + i] : (uint16_t)0;
  return make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16, e[4] | (uint32_t)e[5] << 16,
                    e[6] | (uint32_t)e[7] << 16);
}

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
    uint4 v = (gr < nrows && gk < K) ? load_k_chunk(g + (size_t)gr * ld, gk, K) : make_uint4(0, 0, 0, 0);
    *(uint4*)(lds_op + blk * 512 + lane * 8) = v;
  }
}

// ---------------------------------------------- [k][cols] tiles read with the LDS transpose
// An operand contiguous along its output dimension (the weight of dX = dY W,
// both operands of dW = dY^T X) is staged as it lies in memory: 32 k rows of
// COLS columns, row m's 16-byte chunk p in slot p ^ tok_swz(m).  MFMA
// operands come from the LDS transpose read (ds_read_b64_tr_b16): a 16-lane
// group reads a 4 x 16 (k x column) block and lane i receives the 4 k
// values of column i, so two reads give the 8 k values of a 32x32x16
// operand.  The two 16-lane groups that share an LDS cycle read 4 rows x 4
// chunks; the swizzle puts those 16 chunks on distinct 16-byte bank groups:
// rows 512 or 256 bytes apart (COLS % 128 == 0) start on the same bank and
// take XOR offsets of 0, 4, 8, 12 chunks; rows 384 bytes apart (COLS = 192)
// alternate between two bank halves, so rows 2 and 3 of each four take an
// XOR of 4.  XOR by a multiple of 4 below 8 or 16 keeps the slot in the row.
constexpr int TK = 32;  // k rows per stage
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <int COLS>
__device__ __forceinline__ int tok_swz(int m) {
  static_assert(COLS % 64 == 0 && COLS >= 128, "tile width");
  return COLS % 128 == 0 ? 4 * (m & 3) : 4 * ((m >> 1) & 1);
}

// Direct-to-LDS stage loads of a [k][COLS] tile.  The descriptor starts at
// the stage's (k0, c0) and holds the bytes left of the operand's `krows`
// rows, so rows past the last read as zero (range check of the per-lane
// offset).  Columns past the operand's width read the next row's data or
// zero; they feed only output columns that the epilogue drops.
template <int COLS, int NW>
struct TokLoader {
  static constexpr int CPR = COLS / 8;      // 16-byte chunks per k row
  static constexpr int NI = TK * CPR / 64 / NW;
  static_assert(NI * 64 * NW == TK * CPR, "tile must split evenly over the waves");
  void* base;
  uint32_t nbytes;
  uint32_t voff[NI];
  int blk0;
  __device__ __forceinline__ void init(const void* b, long ld, int krows, int wv, int lane) {
    uint64_t bytes = (uint64_t)krows * ld * 2;
    base = const_cast<void*>(b);
    nbytes = (uint32_t)(bytes > 0xffffffffull ? 0xffffffffull : bytes);
    blk0 = wv * NI;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int lin = (blk0 + i) * 64 + lane;   // LDS chunk slot
      const int m = lin / CPR, slot = lin % CPR;
      const int pch = slot ^ tok_swz<COLS>(m);  // global chunk stored in this slot
      voff[i] = (uint32_t)((long)m * ld * 2 + pch * 16);
    }
  }
  __device__ __forceinline__ void issue(uint32_t soff, uint16_t* lds_op) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) buffer_load_lds16(base, nbytes, lds_op + (blk0 + i) * 512, voff[i], soff);
  }
};

// Ragged last stage of a [k][COLS] tile (k0 + 32 > K): zero-filled register
// loads of rows k0.. and columns c0.. (ncols % 8 == 0), LDS stores.
template <int COLS, int NW>
__device__ __forceinline__ void tok_tail(const uint16_t* __restrict__ g, long ld, int k0, int K, int c0,
                                         int ncols, uint16_t* lds_op, int wv, int lane) {
  constexpr int CPR = COLS / 8, NI = TK * CPR / 64 / NW;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int lin = (wv * NI + i) * 64 + lane;
    const int m = lin / CPR, pch = (lin % CPR) ^ tok_swz<COLS>(m);
    const int gk = k0 + m, gc = c0 + pch * 8;
    uint4 v = (gk < K && gc < ncols) ? *(const uint4*)(g + (size_t)gk * ld + gc) : make_uint4(0, 0, 0, 0);
    *(uint4*)(lds_op + lin * 8) = v;
  }
}

// One LDS transpose read.  Taken through a restrict-qualified pointer, the
// read carries alias-scope information, and the compiler then no longer
// drains every in-flight buffer-to-LDS load (vmcnt 0) before it, which would
// cut the load ring to depth one.  The kernels order these reads against
// the ring loads themselves: each wave waits (vmcnt) for its loads of a
// stage, then the block barrier makes the stage visible to all waves.
__device__ __forceinline__ v4s lds_read_tr(const uint16_t* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
}

// Four bias values staged in LDS, read like lds_read_tr (alias-scoped, so
// the compiler does not drain the ring's in-flight loads before it).
__device__ __forceinline__ float4 lds_read_bias4(const float* __restrict__ p) { return *(const float4*)p; }

// 8 k values (rows ks*16 + 8g .. +7) of column `col` of an LDS tile
// [32][COLS], as an MFMA operand; lane l serves column cbase + l % 32.
template <int COLS>
__device__ __forceinline__ uint4 tr_frag(const uint16_t* tile, int cbase, int ks, int lane) {
  const int G = lane >> 4, q = lane & 15;
  const int col = cbase + 16 * (G & 1) + 4 * (q & 3);
  v4s h[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int m = ks * 16 + 8 * (G >> 1) + 4 * hh + (q >> 2);
    const int off = m * COLS + (((col >> 3) ^ tok_swz<COLS>(m)) << 3) + (col & 7);
    h[hh] = lds_read_tr(tile + off);
  }
  return make_uint4(__builtin_bit_cast(uint32_t, (short2){h[0][0], h[0][1]}),
                    __builtin_bit_cast(uint32_t, (short2){h[0][2], h[0][3]}),
                    __builtin_bit_cast(uint32_t, (short2){h[1][0], h[1][1]}),
                    __builtin_bit_cast(uint32_t, (short2){h[1][2], h[1][3]}));
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

// BKN: B is stored [K][N] (the weight of dX = dY W) and staged as a [k][BN]
// tile read with the LDS transpose (TokLoader / tr_frag); otherwise B is
// [N][K] like A.
template <typename TE, int BM, int BN, int WM, int WN, int EPI, bool BKN>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm_nt(GP p) {
  typedef typename H16<TE>::v8 v8;
  typedef typename std::conditional<BKN, TokLoader<BN, WM * WN>, BufLoader<BN, WM * WN>>::type LoaderB;
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  static_assert(NK == TK, "A and B stages cover the same k");
  constexpr int STAGE = (BM + BN) * NK;  // 16-bit elements per stage
  constexpr int PER = BufLoader<BM, NW>::NI + LoaderB::NI;  // loads per stage
  // The bias vector, staged in LDS once per workgroup when it fits: the
  // epilogues then read it without vector-memory loads.  Such a load in
  // the epilogue has to be waited for, and the wait (one counter for loads
  // and stores) also drains every store the epilogue has issued so far.
  // It sits at the end of the ring's array: a second LDS variable would
  // give the accesses alias scopes, and the compiler would then drain the
  // in-flight ring loads before the ring's fragment reads.
  constexpr bool EPI_HAS_BIAS = EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_RESID;
  constexpr int BIAS_MAX = EPI_HAS_BIAS ? 4096 : 0;  // floats
  __shared__ __attribute__((aligned(1024))) uint16_t lds[NS * STAGE + 2 * BIAS_MAX];
  float* const bias_s = (float*)(lds + NS * STAGE);

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
  LoaderB lb;
  la.init(p.A, p.lda, p.M, wv, lane);
  lb.init(p.B, p.ldb, BKN ? p.K : p.N, wv, lane);

  // issue-side cursor: stage t = (round, kt)
  int i_round = 0, i_kt = 0, i_tm = 0, i_tn = 0;
  if (total > 0) grouped_coords(tile_pid(0, G), nm, nn, i_tm, i_tn);
  auto issue_next = [&](int t) {
    uint16_t* st = lds + (t % NS) * STAGE;
    const int k0 = i_kt * NK;
    if (ragged && k0 + NK > p.K) {
      issue_tail<BM, NW>((const uint16_t*)p.A, p.lda, i_tm * BM, p.M, k0, p.K, st, wv, lane);
      if constexpr (BKN)
        tok_tail<BN, NW>((const uint16_t*)p.B, p.ldb, k0, p.K, i_tn * BN, p.N, st + BM * NK, wv, lane);
      else
        issue_tail<BN, NW>((const uint16_t*)p.B, p.ldb, i_tn * BN, p.N, k0, p.K, st + BM * NK, wv, lane);
    } else {
      la.issue((uint32_t)(((long)i_tm * BM * p.lda + k0) * 2), st);
      if constexpr (BKN)
        lb.issue((uint32_t)(((long)k0 * p.ldb + i_tn * BN) * 2), st + BM * NK);
      else
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

  v8 af[2][FM], bfr[2][FN];
  auto load_frags = [&](int t, int ks, int set) {
    const uint16_t* As = lds + (t % NS) * STAGE;
    const uint16_t* Bs = As + BM * NK;
    const int slot = (ks * 2 + g) ^ swz;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[set][i] = __builtin_bit_cast(v8, *(const uint4*)(As + ((wm + i * 32 + fr) * 4 + slot) * 8));
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (BKN)
        bfr[set][j] = __builtin_bit_cast(v8, tr_frag<BN>(Bs, wn + j * 32, ks, lane));
      else
        bfr[set][j] = __builtin_bit_cast(v8, *(const uint4*)(Bs + ((wn + j * 32 + fr) * 4 + slot) * 8));
    }
  };
  auto mfma_set = [&](int set) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = H16<TE>::mfma(bfr[set][j], af[set][i], acc[i][j]);
  };

  // Stage s + 2 is made visible (wait + barrier) one stage early, so the
  // first fragments of the next stage are read during this stage's second
  // MFMA group.  The barrier comes after that group: the LDS drain it
  // needs (this wave's fragment reads of stage s, whose slot the next
  // issue refills) then overlaps the MFMAs instead of stalling them.
  const bool lds_bias = EPI_HAS_BIAS && p.bias != nullptr && p.N <= BIAS_MAX && (p.N & 3) == 0;  // uniform
  if (total > 0) {
    const int pro = min(NS - 1, total);
    for (int t = 0; t < pro; ++t) issue_next(t);
    if constexpr (EPI_HAS_BIAS) {
      // after the ring's first loads, so their latencies overlap.  No
      // branch around the loads or the stores (a branch lets the compiler
      // sink each load next to its store and wait for it alone): a chunk
      // past N loads the vector's first chunk, and its slot is never read.
      if (lds_bias) {
        constexpr int NB = BIAS_MAX / (NW * 64 * 4);
        static_assert(NB >= 1 && NB * NW * 64 * 4 == BIAS_MAX, "one slot per chunk");
        float4 bv[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int c = (tid + i * NW * 64) * 4;
          bv[i] = *(const float4*)(p.bias + (c < p.N ? c : 0));
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) *(float4*)&bias_s[(tid + i * NW * 64) * 4] = bv[i];
      }
    }
    wait_stage(min(1, total - 1), pro - 1);
    stage_barrier();  // also publishes bias_s
    load_frags(0, 0, 0);
  }
  int s = 0;
  for (int round = 0; round < my_n; ++round) {
    int tm, tn;
    grouped_coords(tile_pid(round, G), nm, nn, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool full = m0 + BM <= p.M && n0 + BN <= p.N;  // whole tile inside the output
    if constexpr (EPI == EPI_RESID) {
      // The residual stream enters the accumulators before the tile's MFMAs
      // (they then add the products to it), so the epilogue has no loads to
      // wait for.  With one tile per workgroup (the 768-wide outputs) these
      // loads overlap the ring's first stages.
      if (full) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const size_t o = (size_t)(m0 + wm + i * 32 + fr) * p.ldo + n0 + wn + j * 32 + e4 * 8 + g * 4;
              const float4 x = *(const float4*)((const float*)p.aux + o);
              acc[i][j][e4 * 4 + 0] = x.x;
              acc[i][j][e4 * 4 + 1] = x.y;
              acc[i][j][e4 * 4 + 2] = x.z;
              acc[i][j][e4 * 4 + 3] = x.w;
            }
      }
    }
    for (int kt = 0; kt < nk; ++kt, ++s) {
      if (s + NS - 1 < total) issue_next(s + NS - 1);
      // Software pipeline of the fragment reads, kept in this order by
      // compiler scheduling fences: each MFMA group consumes fragments read
      // one group earlier.  The next stage's reads are unconditional (a
      // read of a ring slot is always in bounds; on the last stage its
      // values are unused): a conditional read would make the wait before
      // the second group count it as possibly absent and drain it too.
      load_frags(s, 1, 1);
      sched_fence();
      mfma_set(0);
      sched_fence();
      load_frags(s + 1, 0, 0);
      sched_fence();
      mfma_set(1);
      if (s + 2 < total) wait_stage(s + 2, min(s + NS - 1, total - 1));
      stage_barrier();
    }
    if (full) {
      if constexpr (EPI == EPI_DGELU) {
        // The u values in groups of (column block, 4-column run), PD groups
        // ahead of the group being stored: each wait then leaves the later
        // loads and the stores already issued in flight.
        constexpr int NG = FN * 4, PD0 = 16 / FM, PD = PD0 < 1 ? 1 : (PD0 > NG ? NG : PD0);
        uint2 ub[NG][FM];
        auto load_u = [&](int gi) {
          const int c = n0 + wn + (gi >> 2) * 32 + (gi & 3) * 8 + g * 4;
#pragma unroll
          for (int i = 0; i < FM; ++i)
            ub[gi][i] = *(const uint2*)((const TE*)p.aux + (size_t)(m0 + wm + i * 32 + fr) * p.ldo + c);
        };
#pragma unroll
        for (int gi = 0; gi < PD; ++gi) load_u(gi);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          if (gi + PD < NG) load_u(gi + PD);
          const int j = gi >> 2, e4 = gi & 3;
          const int c = n0 + wn + j * 32 + e4 * 8 + g * 4;
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const uint2 uu = ub[gi][i];
            const float v0 = acc[i][j][e4 * 4 + 0], v1 = acc[i][j][e4 * 4 + 1];
            const float v2 = acc[i][j][e4 * 4 + 2], v3 = acc[i][j][e4 * 4 + 3];
            *(uint2*)((TE*)p.out + (size_t)(m0 + wm + i * 32 + fr) * p.ldo + c) = make_uint2(
                H16<TE>::pack2(v0 * gelu_tanh_grad_f(H16<TE>::lo(uu.x)), v1 * gelu_tanh_grad_f(H16<TE>::hi(uu.x))),
                H16<TE>::pack2(v2 * gelu_tanh_grad_f(H16<TE>::lo(uu.y)), v3 * gelu_tanh_grad_f(H16<TE>::hi(uu.y))));
          }
        }
      } else {
        // One body per bias source, picked by a uniform branch: a bias that
        // could come from LDS or from global memory (or be a constant) at the
        // same point makes the compiler wait on both counters there, and the
        // vector-memory wait drains the stores.
        auto full_epi = [&](auto bias_at) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const int c = n0 + wn + j * 32 + e4 * 8 + g * 4;
              const float4 b = bias_at(c);
#pragma unroll
              for (int i = 0; i < FM; ++i) {
                const int r = m0 + wm + i * 32 + fr;
                if constexpr (EPI == EPI_RESID) {  // the residual is already in acc
                  *(float4*)((float*)p.out + (size_t)r * p.ldo + c) =
                      make_float4(acc[i][j][e4 * 4 + 0] + b.x, acc[i][j][e4 * 4 + 1] + b.y,
                                  acc[i][j][e4 * 4 + 2] + b.z, acc[i][j][e4 * 4 + 3] + b.w);
                } else {
                  epi_store4_full<EPI, TE>(p, r, c, b, acc[i][j][e4 * 4 + 0], acc[i][j][e4 * 4 + 1],
                                           acc[i][j][e4 * 4 + 2], acc[i][j][e4 * 4 + 3]);
                }
              }
            }
        };
        auto no_bias = [&](int) { return make_float4(0.f, 0.f, 0.f, 0.f); };
        if constexpr (EPI_HAS_BIAS) {
          if (lds_bias)
            full_epi([&](int c) { return lds_read_bias4(bias_s + c); });
          else if (p.bias != nullptr)
            full_epi([&](int c) { return *(const float4*)(p.bias + c); });
          else
            full_epi(no_bias);
        } else {
          full_epi(no_bias);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            int r = m0 + wm + i * 32 + fr;
            int c = n0 + wn + j * 32 + e4 * 8 + g * 4;
            epi_store4<EPI, TE>(p, r, c, acc[i][j][e4 * 4 + 0], acc[i][j][e4 * 4 + 1],
                                acc[i][j][e4 * 4 + 2], acc[i][j][e4 * 4 + 3]);
          }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  }
}

// ------------------------------------------------------------------ 16-bit TN kernel (weight gradients)
// D[r][c] = sum_m A[m * lda + r] * B[m * ldb + c]: both operands keep their
// natural [token][feature] layout and are staged as [k][cols] tiles of 32
// tokens.  A ragged token count needs no special path: tokens past the last
// one fail the range check of the per-lane offset and read as zero.
template <typename TE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm_tn(GP p) {
  typedef typename H16<TE>::v8 v8;
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

  v8 af[2][FM], bfr[2][FN];
  auto load_frags = [&](int t, int ks, int set) {
    const uint16_t* As = lds + (t % NS) * STAGE;
    const uint16_t* Bs = As + BM * TK;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[set][i] = __builtin_bit_cast(v8, tr_frag<BM>(As, wm + i * 32, ks, lane));
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[set][j] = __builtin_bit_cast(v8, tr_frag<BN>(Bs, wn + j * 32, ks, lane));
  };
  auto mfma_set = [&](int set) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = H16<TE>::mfma(bfr[set][j], af[set][i], acc[i][j]);
  };
  // Bias gradient: column sums of A over the tokens.  Lane l's A fragment
  // holds 8 tokens of row wm + i*32 + l % 32, so the waves of the first
  // column tile with wn == 0 (one per row block) add up the fragments they
  // already hold; lanes l and l + 32 hold the two token halves.
  float bsum[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) bsum[i] = 0.f;
  auto add_sums = [&](int set) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint4 u = __builtin_bit_cast(uint4, af[set][i]);
      float v = H16<TE>::add_pair(u.x, bsum[i]);
      v = H16<TE>::add_pair(u.y, v);
      v = H16<TE>::add_pair(u.z, v);
      bsum[i] = H16<TE>::add_pair(u.w, v);
    }
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
    const bool sums = p.dbias != nullptr && tn == 0 && wn == 0;  // uniform per wave
    for (int kt = 0; kt < nk; ++kt, ++s) {
      if (s + NS - 1 < total) issue_next(s + NS - 1);
      load_frags(s, 1, 1);  // the same software pipeline as k_gemm_nt
      sched_fence();
      mfma_set(0);
      if (sums) add_sums(0);
      sched_fence();
      load_frags(s + 1, 0, 0);
      sched_fence();
      mfma_set(1);
      if (sums) add_sums(1);
      // after the second MFMA group, as in k_gemm_nt
      if (s + 2 < total) wait_stage(s + 2, min(s + NS - 1, total - 1));
      stage_barrier();
    }
    const int m0 = tm * BM, n0 = tn * BN;
    if (sums) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const float v = bsum[i] + __shfl_xor(bsum[i], 32, 64);
        bsum[i] = 0.f;
        const int r = m0 + wm + i * 32 + fr;
        if (g == 0 && r < p.M) {
          if (S > 1) {
            p.dbias_ws[(size_t)z * p.M + r] = v;
          } else {
            float o = p.alpha * v;
            if (p.beta != 0.f) o += p.beta * p.dbias[r];
            p.dbias[r] = o;
          }
        }
      }
    }
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

// ------------------------------------------------------------------ fp32 MFMA kernel
// fp32 operands on the matrix cores (v_mfma_f32_32x32x2_f32: 32x32 outputs,
// 2 k per instruction, full fp32 products and sums): 128 x 128 block tiles,
// 4 waves of 64 x 64 (2 x 2 fragments), K in stages of 16 through a
// double-buffered LDS tile stored k-major ([k][row], rows padded to 160
// floats so the two half-waves of a fragment read fall on disjoint banks).
// Lane l supplies A[row l%32][k l/32] and B[k l/32][col l%32]; element e of
// the accumulator is row 8(e/4) + 4(l/32) + e%4, column l%32.  Global loads
// are 16 bytes along whichever of (row, k) is contiguous in memory and go
// through registers, so the next stage's loads overlap the current MFMAs.
// With blockIdx.z > 0 (split-K) each split covers p.kchunk of K.
constexpr int F32M_BM = 128, F32M_BK = 16, F32M_LD = 160;

template <bool TRANS>
struct F32Loader {
  // 128 rows x 16 k = 512 float4 per operand tile, 2 per thread.
  float4 r[2];
  __device__ __forceinline__ void load(const float* __restrict__ base, long ld, int row0, int nrows, int k0,
                                       int kend, int tid) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      int row, k;
      if constexpr (TRANS) {  // memory [k][row]: 4 consecutive rows
        k = c >> 5;
        row = (c & 31) * 4;
      } else {                // memory [row][k]: 4 consecutive k
        row = c >> 2;
        k = (c & 3) * 4;
      }
      const int gr = row0 + row, gk = k0 + k;
      const bool whole = TRANS ? (gr + 3 < nrows && gk < kend) : (gr < nrows && gk + 3 < kend);
      if (whole && (ld & 3) == 0) {  // 16-byte aligned: row0, k0, row, k are multiples of 4
        r[i] = TRANS ? *(const float4*)(base + (size_t)gk * ld + gr) : *(const float4*)(base + (size_t)gr * ld + gk);
        continue;
      }
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = TRANS ? gr + j : gr, kk = TRANS ? gk : gk + j;
        v[j] = (rr < nrows && kk < kend) ? (TRANS ? base[(size_t)kk * ld + rr] : base[(size_t)rr * ld + kk])
                                         : 0.f;
      }
      r[i] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
  // The whole 128 x 16 tile in bounds and 16-byte aligned: plain loads, no
  // tests (a test around each load left a register copy where its paths
  // joined, and that copy waited for the load, so the next stage's loads
  // no longer overlapped the current stage's MFMAs).
  __device__ __forceinline__ void load_whole(const float* __restrict__ base, long ld, int row0, int k0,
                                             int tid) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      const int row = TRANS ? (c & 31) * 4 : c >> 2, k = TRANS ? c >> 5 : (c & 3) * 4;
      r[i] = TRANS ? *(const float4*)(base + (size_t)(k0 + k) * ld + row0 + row)
                   : *(const float4*)(base + (size_t)(row0 + row) * ld + k0 + k);
    }
  }
  __device__ __forceinline__ void store(float* __restrict__ lds, int tid) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      if constexpr (TRANS) {
        const int k = c >> 5, row = (c & 31) * 4;
        *(float4*)(lds + k * F32M_LD + row) = r[i];
      } else {
        const int row = c >> 2, k = (c & 3) * 4;
        lds[(k + 0) * F32M_LD + row] = r[i].x;
        lds[(k + 1) * F32M_LD + row] = r[i].y;
        lds[(k + 2) * F32M_LD + row] = r[i].z;
        lds[(k + 3) * F32M_LD + row] = r[i].w;
      }
    }
  }
};

template <bool AT, bool BT, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_gemm_f32m(GP p) {
  __shared__ float As[2][F32M_BK * F32M_LD], Bs[2][F32M_BK * F32M_LD];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m0 = blockIdx.y * F32M_BM, n0 = blockIdx.x * F32M_BM;
  const int wm = (wv >> 1) * 64, wn = (wv & 1) * 64;
  const int fr = lane & 31, fk = lane >> 5;
  const int kbeg = blockIdx.z * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);
  const int nk = kend > kbeg ? cdiv(kend - kbeg, F32M_BK) : 0;
  const float* A = (const float*)p.A;
  const float* B = (const float*)p.B;
  F32Loader<AT> la;
  F32Loader<BT> lb;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  auto mfma_stage = [&](int cur) {
#pragma unroll
    for (int ks = 0; ks < F32M_BK; ks += 2) {
      const float* ar = As[cur] + (ks + fk) * F32M_LD;
      const float* br = Bs[cur] + (ks + fk) * F32M_LD;
      const float a0 = ar[wm + fr], a1 = ar[wm + 32 + fr];
      const float b0 = br[wn + fr], b1 = br[wn + 32 + fr];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
    }
  };
  // uniform per block: every stage of this tile is whole and aligned
  const bool whole = m0 + F32M_BM <= p.M && n0 + F32M_BM <= p.N && (kend - kbeg) % F32M_BK == 0 &&
                     (p.lda & 3) == 0 && (p.ldb & 3) == 0;
  if (whole) {
    // The next stage's loads, with no branch around them (the last stage
    // reloads itself), are in flight during this stage's MFMAs.
    if (nk > 0) {
      la.load_whole(A, p.lda, m0, kbeg, tid);
      lb.load_whole(B, p.ldb, n0, kbeg, tid);
      la.store(As[0], tid);
      lb.store(Bs[0], tid);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const int kn = kbeg + (kt + 1 < nk ? kt + 1 : kt) * F32M_BK;
      la.load_whole(A, p.lda, m0, kn, tid);
      lb.load_whole(B, p.ldb, n0, kn, tid);
      sched_fence();  // keep the loads ahead of the MFMAs
      mfma_stage(cur);
      la.store(As[cur ^ 1], tid);  // unused after the last stage
      lb.store(Bs[cur ^ 1], tid);
      __syncthreads();
    }
  } else {
    if (nk > 0) {
      la.load(A, p.lda, m0, p.M, kbeg, kend, tid);
      lb.load(B, p.ldb, n0, p.N, kbeg, kend, tid);
      la.store(As[0], tid);
      lb.store(Bs[0], tid);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool nxt = kt + 1 < nk;
      if (nxt) {
        la.load(A, p.lda, m0, p.M, kbeg + (kt + 1) * F32M_BK, kend, tid);
        lb.load(B, p.ldb, n0, p.N, kbeg + (kt + 1) * F32M_BK, kend, tid);
      }
      mfma_stage(cur);
      if (nxt) {
        la.store(As[cur ^ 1], tid);
        lb.store(Bs[cur ^ 1], tid);
      }
      __syncthreads();
    }
  }
  if (m0 + F32M_BM <= p.M && n0 + F32M_BM <= p.N) {
    // A whole tile: the lane's two bias values first, then per fragment its
    // 16 inputs (residual, u, or the accumulated gradient) loaded together
    // before its 16 stores; one element at a time, each load's wait had
    // also drained every store before it.
    float bj[2] = {0.f, 0.f};
    if constexpr (EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_RESID) {
      if (p.bias != nullptr) {
        bj[0] = p.bias[n0 + wn + fr];
        bj[1] = p.bias[n0 + wn + 32 + fr];
      }
    }
    constexpr bool LOADS = EPI == EPI_RESID || EPI == EPI_DGELU || EPI == EPI_WGRAD;
    float* wout = (float*)p.out + (EPI == EPI_WGRAD ? (size_t)blockIdx.z * ((size_t)p.M * p.ldo) : 0);
    const bool wg_acc = EPI == EPI_WGRAD && gridDim.z == 1 && p.beta != 0.f;  // uniform
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = n0 + wn + j * 32 + fr;
        // one 64-bit base per fragment, 32-bit row offsets (rows 8 (e/4) +
        // e%4 below the fragment's first row of this lane)
        const size_t o0 = (size_t)(m0 + wm + i * 32 + 4 * fk) * p.ldo + c;
        const int ld = (int)p.ldo;
        float in[16];
        if constexpr (LOADS) {
          if (EPI != EPI_WGRAD || wg_acc) {
            const float* src = (EPI == EPI_WGRAD ? (const float*)wout : (const float*)p.aux) + o0;
#pragma unroll
            for (int e = 0; e < 16; ++e) in[e] = src[(8 * (e >> 2) + (e & 3)) * ld];
          }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const size_t o = o0 + (size_t)((8 * (e >> 2) + (e & 3)) * ld);
          const float a = acc[i][j][e];
          if constexpr (EPI == EPI_STORE) {
            ((float*)p.out)[o] = p.alpha * a + bj[j];
          } else if constexpr (EPI == EPI_LOGITS) {
            ((float*)p.out)[o] = a;
          } else if constexpr (EPI == EPI_GELU) {
            const float u = a + bj[j];
            ((float*)p.out)[o] = u;
            ((float*)p.out2)[o] = gelu_tanh_f(u);
          } else if constexpr (EPI == EPI_RESID) {
            ((float*)p.out)[o] = in[e] + a + bj[j];
          } else if constexpr (EPI == EPI_DGELU) {
            ((float*)p.out)[o] = a * gelu_tanh_grad_f(in[e]);
          } else {  // EPI_WGRAD: raw partials with split-K
            if (gridDim.z > 1) wout[o] = a;
            else wout[o] = wg_acc ? p.alpha * a + p.beta * in[e] : p.alpha * a;
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          epi_store<EPI, float>(p, m0 + wm + i * 32 + 8 * (e >> 2) + 4 * fk + (e & 3), n0 + wn + j * 32 + fr,
                                acc[i][j][e]);
  }
}

// ------------------------------------------------------------------ split-K reduction
// out = alpha * sum_z ws[z][0..n) + beta * out, and likewise out2 from the
// [S][n2] partials ws2 (the TN kernel's bias-gradient sums; n2 may be 0),
// the splits added in order.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ ws, int S,
                                                       size_t n, float* out,
                                                       const float* __restrict__ ws2, size_t n2,
                                                       float* out2, float alpha, float beta) {
  const size_t n4 = n / 4;  // n is a multiple of 4 (N % 4 == 0 when split)
  for (size_t j = n4 + (size_t)blockIdx.x * 256 + threadIdx.x; j < n4 + n2; j += (size_t)gridDim.x * 256) {
    const size_t i = j - n4;
    float sum = 0.f;
    for (int z = 0; z < S; ++z) sum += ws2[(size_t)z * n2 + i];
    float r = alpha * sum;
    if (beta != 0.f) r += beta * out2[i];
    out2[i] = r;
  }
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    // the partials are added in split order; loads go out 8 at a time so
    // their latencies overlap instead of adding up
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    int z = 0;
    for (; z + 8 <= S; z += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *(const float4*)(ws + (size_t)(z + u) * n + 4 * i);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
      }
    }
    for (; z < S; ++z) {
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
// extra: workspace floats per split beyond the M x N partial (bias sums).
static TnPlan plan_tn(int M, int N, int K, size_t ws_elems, size_t extra) {
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
      if (S > 1 && (size_t)S * ((size_t)M * N + extra) > ws_elems) continue;
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
  TnPlan tp = plan_tn(M, N, K, (size_t)-1, M);
  size_t b = tp.splits > 1 ? (size_t)tp.splits * ((size_t)M * N + M) : 0;
  return a > b ? a : b;
}

template <typename TE, int BM, int BN, int WM, int WN>
static void launch_tn(GP q, int per_cu, hipStream_t st) {
  long items = (long)cdiv(q.M, BM) * cdiv(q.N, BN) * q.splits;
  long cap = 256L * per_cu;
  int grid = (int)(items < cap ? ((items + 7) / 8) * 8 : cap);
  k_gemm_tn<TE, BM, BN, WM, WN><<<grid, WM * WN * 64, 0, st>>>(q);
}

template <typename TE, int BM, int BN, bool AT, bool BT, int EPI>
static void launch_cfg(GP q, int S, hipStream_t st) {
  int nb = cdiv(q.M, BM) * cdiv(q.N, BN);
  k_gemm_h16<TE, BM, BN, 2, 2, AT, BT, EPI><<<dim3(nb, 1, S), 256, 0, st>>>(q);
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

template <typename TE, int BM, int BN, int WM, int WN, int EPI, bool BKN>
static void launch_nt(GP q, hipStream_t st) {
  int tiles = cdiv(q.M, BM) * cdiv(q.N, BN);
  int grid = tiles < 256 ? ((tiles + 7) / 8) * 8 : 256;
  k_gemm_nt<TE, BM, BN, WM, WN, EPI, BKN><<<grid, WM * WN * 64, 0, st>>>(q);
}

// The direct-to-LDS kernels address an operand with 32-bit byte offsets
// from its base: rows x ld 16-bit elements must stay below 4 GiB.
static bool fits32(long rows, long ld) { return rows * ld * 2 < (1L << 32); }

// The weight-gradient shapes the TN kernel takes (it also forms the bias
// gradient, when asked, from the A fragments it holds).
static bool tn_direct(const GemmArgs& a) {
  return (a.dt == ACT_BF16 || a.dt == ACT_F16) && a.kind == EPI_WGRAD && a.a_t && a.b_t && a.N % 4 == 0 &&
         a.ldo == a.N && a.lda % 8 == 0 && a.ldb % 8 == 0 && a.splitk_ws && fits32(a.K, a.lda) &&
         fits32(a.K, a.ldb);
}

template <typename TE, bool AT, bool BT, int EPI>
static hipError_t launch_h16(const GemmArgs& a, GP p, hipStream_t st) {
  if constexpr (AT && BT && EPI == EPI_WGRAD) {
    if (tn_direct(a)) {
      TnPlan tp = plan_tn(a.M, a.N, a.K, a.splitk_ws_elems, a.dbias ? a.M : 0);
      p.kchunk = tp.kchunk;
      p.splits = tp.splits;
      GP q = p;
      q.dbias = a.dbias;
      if (tp.splits > 1) {
        q.out = a.splitk_ws;
        if (a.dbias) q.dbias_ws = a.splitk_ws + (size_t)tp.splits * a.M * a.N;
      }
      switch (tp.cfg) {
        case 0: launch_tn<TE, 256, 256, 4, 2>(q, 1, st); break;
        case 1: launch_tn<TE, 256, 128, 2, 2>(q, 1, st); break;
        default: launch_tn<TE, 128, 128, 2, 2>(q, 2, st); break;
      }
      if (tp.splits > 1) {
        size_t n = (size_t)a.M * a.N;
        k_splitk_reduce<<<2048, 256, 0, st>>>(a.splitk_ws, tp.splits, n, (float*)a.out, q.dbias_ws,
                                              a.dbias ? (size_t)a.M : 0, a.dbias, a.alpha, a.beta);
      }
      return hipGetLastError();
    }
  }
  // Forward (B = [N][K]) and dX (B = [K][N], N % 8 == 0): any K, the last
  // partial stage zero-filled.
  if constexpr (!AT && EPI != EPI_WGRAD) {
    if (a.lda % 8 == 0 && a.ldb % 8 == 0 && (!BT || a.N % 8 == 0) && fits32(a.M, a.lda) &&
        fits32(BT ? a.K : a.N, a.ldb)) {
      p.kchunk = a.K;
      switch (plan_nt(a.M, a.N)) {
        case 0: launch_nt<TE, 256, 256, 4, 2, EPI, BT>(p, st); break;
        case 1: launch_nt<TE, 256, 192, 2, 2, EPI, BT>(p, st); break;
        default: launch_nt<TE, 256, 128, 2, 2, EPI, BT>(p, st); break;
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
    case 0: launch_cfg<TE, 256, 256, AT, BT, EPI>(q, pl.splits, st); break;
    case 1: launch_cfg<TE, 256, 192, AT, BT, EPI>(q, pl.splits, st); break;
    case 2: launch_cfg<TE, 256, 128, AT, BT, EPI>(q, pl.splits, st); break;
    default: launch_cfg<TE, 128, 128, AT, BT, EPI>(q, pl.splits, st); break;
  }
  if (pl.splits > 1) {
    size_t n = (size_t)a.M * a.N;
    k_splitk_reduce<<<2048, 256, 0, st>>>(a.splitk_ws, pl.splits, n, (float*)a.out, nullptr, 0, nullptr,
                                          a.alpha, a.beta);
  }
  return hipGetLastError();
}

// fp32 problems of 2^27 multiply-adds or more go to the matrix cores; the
// small ones (the tiny model) keep the FMA kernel.  Weight gradients split K
// (the tokens) so that the grid covers the 256 CUs, summed by the same
// fixed-order reduction as the 16-bit path.
template <bool AT, bool BT, int EPI>
static hipError_t launch_f32(const GemmArgs& a, GP p, hipStream_t st) {
  if ((double)a.M * a.N * a.K >= 134217728.0) {
    const int tiles = cdiv(a.M, F32M_BM) * cdiv(a.N, F32M_BM);
    int S = 1;
    if (EPI == EPI_WGRAD && a.ldo == a.N && a.splitk_ws && a.N % 4 == 0) {
      S = min(16, max(1, 256 / tiles));
      while (S > 1 && (size_t)S * a.M * a.N > a.splitk_ws_elems) --S;
    }
    p.kchunk = cdiv(cdiv(a.K, S), F32M_BK) * F32M_BK;
    S = cdiv(a.K, p.kchunk);
    GP q = p;
    if (S > 1) q.out = a.splitk_ws;
    k_gemm_f32m<AT, BT, EPI><<<dim3(cdiv(a.N, F32M_BM), cdiv(a.M, F32M_BM), S), 256, 0, st>>>(q);
    if (S > 1)
      k_splitk_reduce<<<2048, 256, 0, st>>>(a.splitk_ws, S, (size_t)a.M * a.N, (float*)a.out, nullptr, 0,
                                            nullptr, a.alpha, a.beta);
    return hipGetLastError();
  }
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
  if (a.dt == ACT_BF16) {
    if constexpr (NT_OK)
      if (!a.a_t && !a.b_t) return launch_h16<bf16, false, false, EPI>(a, p, st);
    if constexpr (NN_OK)
      if (!a.a_t && a.b_t) return launch_h16<bf16, false, true, EPI>(a, p, st);
    if constexpr (TN_OK)
      if (a.a_t && a.b_t) return launch_h16<bf16, true, true, EPI>(a, p, st);
    return hipErrorInvalidValue;
  }
  if (a.dt == ACT_F16) {
    if constexpr (NT_OK)
      if (!a.a_t && !a.b_t) return launch_h16<f16, false, false, EPI>(a, p, st);
    if constexpr (NN_OK)
      if (!a.a_t && a.b_t) return launch_h16<f16, false, true, EPI>(a, p, st);
    if constexpr (TN_OK)
      if (a.a_t && a.b_t) return launch_h16<f16, true, true, EPI>(a, p, st);
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
  if (a.dbias && (a.kind != EPI_WGRAD || !a.a_t || a.alpha != 1.f)) return hipErrorInvalidValue;
  const bool bias_apart = a.dbias && !tn_direct(a);
  if (bias_apart && !a.colsum_ws) return hipErrorInvalidValue;
  GP p;
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.A = a.A; p.lda = a.lda; p.B = a.B; p.ldb = a.ldb;
  p.out = a.out; p.ldo = a.ldo; p.out2 = a.out2; p.aux = a.aux; p.bias = a.bias;
  p.alpha = a.alpha; p.beta = a.beta; p.kchunk = a.K; p.splits = 1;
  p.dbias = nullptr; p.dbias_ws = nullptr;
  hipError_t e = hipErrorInvalidValue;
  switch (a.kind) {
    case EPI_STORE: e = dispatch_t<EPI_STORE>(a, p, st); break;
    case EPI_LOGITS: e = dispatch_t<EPI_LOGITS>(a, p, st); break;
    case EPI_GELU: e = dispatch_t<EPI_GELU>(a, p, st); break;
    case EPI_RESID: e = dispatch_t<EPI_RESID>(a, p, st); break;
    case EPI_DGELU: e = dispatch_t<EPI_DGELU>(a, p, st); break;
    case EPI_WGRAD: e = dispatch_t<EPI_WGRAD>(a, p, st); break;
  }
  // A ([K tokens][M features]) column sums where the GEMM kernel did not form them
  if (e == hipSuccess && bias_apart) e = colsum(a.A, a.dt, a.K, a.M, a.lda, a.dbias, a.beta, a.colsum_ws, st);
  return e;
}

}  // namespace gk
