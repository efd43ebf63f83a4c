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
template <typename T> __device__ __forceinline__ float to_f(T x) { return Cvt<T>::to_f(x); }
template <typename T> __device__ __forceinline__ T from_f(float x) { return Cvt<T>::from_f(x); }

// Two floats -> packed pair of bf16 in one dword (low = a).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

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

// tanh from its exponential form, tanh(x) = 1 - 2 / (exp(2x) + 1), with the
// hardware exp2 and reciprocal; saturates correctly to +-1.
__device__ __forceinline__ float fast_tanh(float x) {
  float e = __builtin_amdgcn_exp2f(x * 2.8853900817779268f);  // 2 / ln 2
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

// tanh-GELU and its derivative (Hendrycks & Gimpel), fp32.
__device__ __forceinline__ float gelu_tanh_f(float u) {
  const float k = 0.7978845608028654f, a = 0.044715f;
  float t = fast_tanh(k * (u + a * u * u * u));
  return 0.5f * u * (1.0f + t);
}
__device__ __forceinline__ float gelu_tanh_grad_f(float u) {
  const float k = 0.7978845608028654f, a = 0.044715f;
  float t = fast_tanh(k * (u + a * u * u * u));
  return 0.5f * (1.0f + t) + 0.5f * u * (1.0f - t * t) * k * (1.0f + 3.0f * a * u * u);
}

__host__ __device__ __forceinline__ int cdiv(long a, long b) { return (int)((a + b - 1) / b); }
