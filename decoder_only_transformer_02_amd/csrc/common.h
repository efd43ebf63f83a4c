// Shared device helpers for the gfx950 kernels: bf16 conversion, wavefront
// reductions, vector types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define WAVE 64

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even float -> bf16 (the gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f2bf_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float bfbits2f(uint32_t h) { return __uint_as_float(h << 16); }

// Element conversion for the two storage types of activations.
template <typename T> struct Cvt;
template <> struct Cvt<float> {
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};
template <> struct Cvt<bf16> {
  static __device__ __forceinline__ float to_f(bf16 x) {
    return bfbits2f(__builtin_bit_cast(uint16_t, x));
  }
  static __device__ __forceinline__ bf16 from_f(float x) { return (__bf16)x; }
};
template <> struct Cvt<f16> {
  static __device__ __forceinline__ float to_f(f16 x) { return (float)x; }
  static __device__ __forceinline__ f16 from_f(float x) { return (f16)x; }
};
template <typename T> __device__ __forceinline__ float to_f(T x) { return Cvt<T>::to_f(x); }
template <typename T> __device__ __forceinline__ T from_f(float x) { return Cvt<T>::from_f(x); }

// Two floats -> packed pair of bf16 in one dword (low = a).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// The two 16-bit storage types of the matrix-core path, bf16 and fp16 (IEEE
// half): the 8-element MFMA operand vector, the 32x32x16 matrix instruction
// with fp32 accumulation, packing of two floats into one dword (low half =
// first, round to nearest even) and back, and acc + lo + hi of one dword in
// a single instruction (v_dot2 against a pair of ones).
template <typename T> struct H16;
template <> struct H16<bf16> {
  typedef bf16x8 v8;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf2(a, b); }
  static __device__ __forceinline__ float lo(uint32_t u) { return bfbits2f(u & 0xffffu); }
  static __device__ __forceinline__ float hi(uint32_t u) { return bfbits2f(u >> 16); }
  static __device__ __forceinline__ float add_pair(uint32_t u, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                           acc, false);
  }
};
template <> struct H16<f16> {
  typedef f16x8 v8;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    f16x2 v;
    v[0] = (f16)a;
    v[1] = (f16)b;
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float lo(uint32_t u) { return (float)__builtin_bit_cast(f16, (uint16_t)(u & 0xffffu)); }
  static __device__ __forceinline__ float hi(uint32_t u) { return (float)__builtin_bit_cast(f16, (uint16_t)(u >> 16)); }
  static __device__ __forceinline__ float add_pair(uint32_t u, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, u), __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
  }
};

// Wavefront (64 lanes) all-reduce.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// tanh-GELU and its derivative (Hendrycks & Gimpel), fp32, in the logistic
// form: 0.5 (1 + tanh(z / 2)) = 1 / (1 + exp(-z)) with z = 2k (u + a u^3),
// so gelu(u) = u s and gelu'(u) = s (1 + u (1 - s) z'(u)), s = 1 / (1 +
// exp(-z)), z' = 2k (1 + 3a u^2).  One exp2 and one reciprocal each, and
// the cubic folded into fused multiply-adds: these run once per element of
// the MLP's widest GEMM outputs, inside the GEMM epilogue.
__device__ __forceinline__ float gelu_sigmoid_of(float u) {
  const float c0 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2k / ln 2
  const float c1 = c0 * 0.044715f;
  const float x = u * fmaf(c1, u * u, c0);  // -z / ln 2
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
}
__device__ __forceinline__ float gelu_tanh_f(float u) { return u * gelu_sigmoid_of(u); }
__device__ __forceinline__ float gelu_tanh_grad_f(float u) {
  const float d0 = 2.0f * 0.7978845608028654f, d1 = d0 * 3.0f * 0.044715f;  // z' = d0 + d1 u^2
  const float s = gelu_sigmoid_of(u);
  return s * fmaf(u * (1.0f - s), fmaf(d1, u * u, d0), 1.0f);
}

__host__ __device__ __forceinline__ int cdiv(long a, long b) { return (int)((a + b - 1) / b); }
