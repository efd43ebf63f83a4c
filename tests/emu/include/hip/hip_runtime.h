// CPU emulation of the subset of HIP that the library's kernels use.
//
// TEST INFRASTRUCTURE ONLY.  The kernel sources under csrc/ are compiled
// unchanged for the host against this header (after a mechanical rewrite of
// the <<<...>>> launch syntax, see build_emu.py), and every work-item runs
// as a fiber.  Operations that act on a whole wavefront on the hardware
// (matrix instructions, lane shuffles, LDS transpose reads, buffer loads
// into LDS, waits on the vector-memory counter) are rendezvous points of the
// 64 fibers of that wavefront; barriers are rendezvous points of the block.
//
// The lane layouts follow the CDNA3/CDNA4 instruction set reference:
//  * v_mfma_f32_32x32x16_bf16: lane l supplies row l%32 of A (k = 8*(l/32)
//    .. +7) and column l%32 of B (same k); accumulator element e of lane l
//    is D[8*(e/4) + 4*(l/32) + e%4][l%32].
//  * v_mfma_f32_32x32x16_f16: as the bf16 instruction, with fp16 values.
//  * v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][l/32] and
//    B[l/32][l%32]; the same accumulator layout.
//  * ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives
//    element i%4 of the 64-bit words read by lanes 4j + i/4, j = 0..3.
//  * buffer_load ... lds: lane l's 16 bytes land at the LDS base + 16 l;
//    the write becomes visible at the s_waitcnt vmcnt that retires it, or,
//    in the second landing mode (emu_set_land_early), right at issue; a
//    kernel correct under both extremes neither reads a slot before its
//    wait nor overwrites a slot another wave still reads.
// The buffer range check is a run-time choice (emu_set_range_mode): either
// the scalar offset counts towards the check or it does not, in which case
// bytes that lie beyond the buffer but pass the check read as a poison
// pattern, so a kernel that relies on either behaviour fails one mode.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <tuple>
#include <utility>

// ------------------------------------------------------------------ qualifiers
#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __noinline__
#define __launch_bounds__(...)
#define __shared__ static thread_local
#define __restrict__ __restrict

// ------------------------------------------------------------------ vector types
struct dim3 {
  unsigned x, y, z;
  constexpr dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
struct uint2 { uint32_t x, y; };
struct uint4 { uint32_t x, y, z, w; };
struct int2 { int32_t x, y; };
struct int4 { int32_t x, y, z, w; };
struct float2 { float x, y; };
struct float4 { float x, y, z, w; };
struct short2 { int16_t x, y; };
struct short4 { int16_t x, y, z, w; };
inline uint2 make_uint2(uint32_t a, uint32_t b) { return {a, b}; }
inline uint4 make_uint4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) { return {a, b, c, d}; }
inline int2 make_int2(int32_t a, int32_t b) { return {a, b}; }
inline int4 make_int4(int32_t a, int32_t b, int32_t c, int32_t d) { return {a, b, c, d}; }
inline float2 make_float2(float a, float b) { return {a, b}; }
inline float4 make_float4(float a, float b, float c, float d) { return {a, b, c, d}; }

// ------------------------------------------------------------------ runtime API
typedef void* hipStream_t;
typedef struct emu_event* hipEvent_t;
enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorOutOfMemory = 2,
  hipErrorNotInitialized = 3,
  hipErrorInvalidDevice = 101,
  hipErrorLaunchFailure = 719,
};
enum hipMemcpyKind {
  hipMemcpyHostToHost = 0,
  hipMemcpyHostToDevice = 1,
  hipMemcpyDeviceToHost = 2,
  hipMemcpyDeviceToDevice = 3,
  hipMemcpyDefault = 4
};
enum hipFuncAttribute { hipFuncAttributeMaxDynamicSharedMemorySize = 8 };

const char* hipGetErrorString(hipError_t e);
hipError_t hipGetLastError();
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind k, hipStream_t s);
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind k);
hipError_t hipMemsetAsync(void* dst, int v, size_t n, hipStream_t s);
hipError_t hipMemcpy2DAsync(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width,
                            size_t height, hipMemcpyKind k, hipStream_t s);
hipError_t hipStreamSynchronize(hipStream_t s);
hipError_t hipDeviceSynchronize();
hipError_t hipSetDevice(int d);
hipError_t hipGetDevice(int* d);
hipError_t hipEventCreate(hipEvent_t* e);
hipError_t hipEventDestroy(hipEvent_t e);
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s);
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b);
hipError_t hipFuncSetAttribute(const void* f, hipFuncAttribute a, int v);

// ------------------------------------------------------------------ execution context
namespace emu {

struct Fiber;
Fiber* cur();
const dim3& tid3();
const dim3& bid3();
const dim3& bdim3();
const dim3& gdim3();
void* dyn_shared();

void barrier();        // s_barrier (no memory wait)
void syncthreads();    // vmcnt(0), then s_barrier
void waitcnt(int imm);

// raw wave rendezvous: every live lane of the wave deposits `in` (nbytes);
// the last one to arrive calls fn(ctx) once, which reads all deposits
// (lane_in) and writes every lane's result (lane_out); returns this lane's
// result buffer.
typedef void (*CollFn)(void* ctx);
void* wave_collective(int kind, const void* in, size_t nbytes, CollFn fn, void* ctx);
int lane_id();
int wave_lanes_alive_mask_count();
const void* lane_in(int lane);   // NULL for a lane that has exited
void* lane_out(int lane);

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4s_t __attribute__((ext_vector_type(4)));

f32x16_t mfma_32x32x16_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c);
f32x16_t mfma_32x32x2_f32(float a, float b, f32x16_t c);
f32x16_t mfma_32x32x16_f16(f16x8_t a, f16x8_t b, f32x16_t c);
v4s_t ds_read_tr16_b64(const void* lds_addr);

struct Rsrc {
  const char* base;
  uint32_t nbytes;
};
inline Rsrc make_rsrc(const void* base, short /*stride*/, int nbytes, int /*flags*/) {
  return Rsrc{(const char*)base, (uint32_t)nbytes};
}
void buffer_load_lds(Rsrc r, void* lds, int size, uint32_t voff, uint32_t soff, int off, int aux);

uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel);

template <typename T>
struct ShflCtx {
  int mask, width, mode;  // mode 0 xor, 1 index
};
template <typename T>
void shfl_fn(void* vctx) {
  ShflCtx<T>* c = (ShflCtx<T>*)vctx;
  for (int l = 0; l < 64; ++l) {
    int src;
    if (c->mode == 0) src = l ^ c->mask;
    else src = (l & ~(c->width - 1)) + (c->mask & (c->width - 1));
    const void* p = (src >= 0 && src < 64) ? lane_in(src) : nullptr;
    T v{};
    if (p) std::memcpy(&v, p, sizeof(T));
    std::memcpy(lane_out(l), &v, sizeof(T));
  }
}
template <typename T>
T shfl_xor(T v, int mask, int width) {
  ShflCtx<T> c{mask, width, 0};
  void* r = wave_collective(1000 + (int)sizeof(T), &v, sizeof(T), shfl_fn<T>, &c);
  T o;
  std::memcpy(&o, r, sizeof(T));
  return o;
}
template <typename T>
T shfl_idx(T v, int src, int width) {
  ShflCtx<T> c{src, width, 1};
  void* r = wave_collective(1100 + (int)sizeof(T), &v, sizeof(T), shfl_fn<T>, &c);
  T o;
  std::memcpy(&o, r, sizeof(T));
  return o;
}

// v_readfirstlane: the first active lane's value.  The kernels use it only
// to tell the compiler that a value is the same on every lane, so the
// emulator also checks that it is.
inline void rfl_fn(void*) {
  int first = 0;
  bool have = false;
  for (int l = 0; l < 64; ++l) {
    const void* p = lane_in(l);
    if (!p) continue;
    int v;
    std::memcpy(&v, p, sizeof(v));
    if (!have) {
      first = v;
      have = true;
    } else if (v != first) {
      std::fprintf(stderr, "emu: readfirstlane of a value that differs across the wave\n");
      std::abort();
    }
  }
  for (int l = 0; l < 64; ++l) std::memcpy(lane_out(l), &first, sizeof(first));
}
inline int readfirstlane(int v) {
  void* r = wave_collective(1200, &v, sizeof(v), rfl_fn, nullptr);
  int o;
  std::memcpy(&o, r, sizeof(o));
  return o;
}

// generic launch: runs the whole grid before returning (streams are
// synchronous in the emulator)
typedef void (*BlockThunk)(void* args);
void run_grid(dim3 grid, dim3 block, size_t shmem, BlockThunk thunk, void* args);

template <typename K, typename Tup, size_t... I>
inline void call_with(K k, Tup& t, std::index_sequence<I...>) {
  k(std::get<I>(t)...);
}

template <typename... P>
struct Launcher {
  void (*k)(P...);
  dim3 g, b;
  size_t sh;
  template <typename... A>
  void operator()(A&&... a) {
    using Tup = std::tuple<P...>;
    struct Pack {
      void (*k)(P...);
      Tup t;
    } pack{k, Tup(static_cast<P>(a)...)};
    run_grid(g, b, sh, [](void* v) {
      Pack* p = (Pack*)v;
      Tup copy = p->t;  // every work-item gets its own copy of the arguments
      call_with(p->k, copy, std::index_sequence_for<P...>{});
    }, &pack);
  }
};
template <typename... P>
inline Launcher<P...> launch(void (*k)(P...), dim3 g, dim3 b, size_t sh = 0, hipStream_t = nullptr) {
  return Launcher<P...>{k, g, b, sh};
}

}  // namespace emu

#define threadIdx (::emu::tid3())
#define blockIdx (::emu::bid3())
#define blockDim (::emu::bdim3())
#define gridDim (::emu::gdim3())

inline void __syncthreads() { ::emu::syncthreads(); }

// ------------------------------------------------------------------ builtins
#define __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, x, y, z) ::emu::mfma_32x32x16_bf16(a, b, c)
#define __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, x, y, z) ::emu::mfma_32x32x2_f32(a, b, c)
#define __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, x, y, z) ::emu::mfma_32x32x16_f16(a, b, c)
#define __builtin_amdgcn_ds_read_tr16_b64_v4i16(p) ::emu::ds_read_tr16_b64((const void*)(p))
#define __builtin_amdgcn_readfirstlane(v) ::emu::readfirstlane((int)(v))
#define __builtin_amdgcn_make_buffer_rsrc(b, s, n, f) ::emu::make_rsrc(b, s, n, f)
#define __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, sz, vo, so, of, ax) \
  ::emu::buffer_load_lds(r, (void*)(l), sz, vo, so, of, ax)
#define __builtin_amdgcn_s_waitcnt(imm) ::emu::waitcnt(imm)
#define __builtin_amdgcn_s_barrier() ::emu::barrier()
// compiler scheduling fence: no effect on what the code computes
#define __builtin_amdgcn_sched_barrier(mask) ((void)0)
#define __builtin_amdgcn_perm(a, b, s) ::emu::perm(a, b, s)
#define __builtin_amdgcn_exp2f(x) exp2f(x)
#define __builtin_amdgcn_rcpf(x) (1.0f / (x))
// a.lo * b.lo + a.hi * b.hi + c (two-element dot products into fp32)
#define __builtin_amdgcn_fdot2_f32_bf16(a, b, c, clamp) \
  ((float)(a)[0] * (float)(b)[0] + (float)(a)[1] * (float)(b)[1] + (c))
#define __builtin_amdgcn_fdot2(a, b, c, clamp) ((float)(a)[0] * (float)(b)[0] + (float)(a)[1] * (float)(b)[1] + (c))

template <typename T>
inline T __shfl_xor(T v, int mask, int width = 64) { return ::emu::shfl_xor<T>(v, mask, width); }
template <typename T>
inline T __shfl(T v, int src, int width = 64) { return ::emu::shfl_idx<T>(v, src, width); }

inline int atomicOr(int* p, int v) { return __atomic_fetch_or(p, v, __ATOMIC_SEQ_CST); }
inline unsigned atomicOr(unsigned* p, unsigned v) { return __atomic_fetch_or(p, v, __ATOMIC_SEQ_CST); }
inline int atomicAdd(int* p, int v) { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); }
inline unsigned atomicAdd(unsigned* p, unsigned v) { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); }
inline int atomicMin(int* p, int v) {
  int cur = __atomic_load_n(p, __ATOMIC_SEQ_CST);
  while (v < cur && !__atomic_compare_exchange_n(p, &cur, v, false, __ATOMIC_SEQ_CST, __ATOMIC_SEQ_CST)) {
  }
  return cur;
}

// ------------------------------------------------------------------ math
inline float __uint_as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
inline uint32_t __float_as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }
inline float __int_as_float(int32_t u) { return __builtin_bit_cast(float, u); }
inline int32_t __float_as_int(float f) { return __builtin_bit_cast(int32_t, f); }
inline float rsqrtf(float x) { return 1.0f / std::sqrt(x); }
inline float __logf(float x) { return std::log(x); }
inline float __log2f(float x) { return std::log2(x); }
inline float __expf(float x) { return std::exp(x); }
using std::isfinite;
using std::isnan;

inline int min(int a, int b) { return a < b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }
inline unsigned min(unsigned a, unsigned b) { return a < b ? a : b; }
inline unsigned max(unsigned a, unsigned b) { return a > b ? a : b; }
inline long min(long a, long b) { return a < b ? a : b; }
inline long max(long a, long b) { return a > b ? a : b; }
inline unsigned long min(unsigned long a, unsigned long b) { return a < b ? a : b; }
inline unsigned long max(unsigned long a, unsigned long b) { return a > b ? a : b; }
inline long long min(long long a, long long b) { return a < b ? a : b; }
inline long long max(long long a, long long b) { return a > b ? a : b; }
inline float min(float a, float b) { return a < b ? a : b; }
inline float max(float a, float b) { return a > b ? a : b; }
