// Shared device-side definitions for the lookahead decoding kernels (gfx950).
//
// Storage types: fp32 or bf16 (kept as raw uint16 bit patterns); all
// arithmetic is fp32 (fp64 in the sampling verifier).  MFMA wrappers and
// their operand layouts for 16x16 output tiles:
//   D[i][j] (fp32x4): lane l holds rows 4*(l/16)+r (r = 0..3), column l%16.
//   16x16x4  f32 : A lane l = A[l%16][l/16],            B lane l = B[l/16][l%16]
//   16x16x16 bf16: A lane l = A[l%16][4*(l/16)+0..3],   B lane l = B[4*(l/16)+0..3][l%16]
//   16x16x32 bf16: A lane l = A[l%16][8*(l/16)+0..7],   B lane l = B[8*(l/16)+0..7][l%16]
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;

#define LA_WAVE 64

// Kernel arguments a prologue needs, loaded as one batch: an empty asm that
// takes them as scalar operands makes the compiler issue their loads back to
// back behind one wait (left alone, it places the loads behind the first
// branches, one memory round trip each).
#define ARGS_READY(...) asm volatile("" ::__VA_ARGS__)

__device__ __forceinline__ float bf2f(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}
// round to nearest, ties to even (NaN kept quiet)
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> struct StoreT;
template <> struct StoreT<float> {
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
  __device__ static __forceinline__ float round(float v) { return v; }
};
template <> struct StoreT<bf16_t> {
  __device__ static __forceinline__ float load(const bf16_t* p) { return bf2f(*p); }
  __device__ static __forceinline__ void store(bf16_t* p, float v) { *p = f2bf(v); }
  __device__ static __forceinline__ float round(float v) { return bf2f(f2bf(v)); }
};
template <typename T> __device__ __forceinline__ float ld(const T* p) { return StoreT<T>::load(p); }
template <typename T> __device__ __forceinline__ void st(T* p, float v) { StoreT<T>::store(p, v); }

__device__ __forceinline__ f32x4 mfma_f32_4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16_16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16_32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// 128-bit vector helpers
struct alignas(16) u32x4 { uint32_t x, y, z, w; };
