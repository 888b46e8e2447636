// Device helpers for kernels that stream through an LDS ring fed by
// global_load_lds (gfx950): static loop unrolling, explicit vmcnt waits, a
// barrier that leaves global loads in flight, and inline-asm LDS reads the
// compiler cannot mistake for reads of an in-flight DMA target.
#pragma once
#include <type_traits>

#include "la_common.h"

#define LDS_BYTES 163840   // LDS of one gfx950 workgroup

typedef __attribute__((address_space(3))) void lds_void_t;

template <int I, int N, typename F> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier that leaves outstanding global loads in flight (the ring
// waits for its own stages with wait_vm): LDS reads of this wave are complete
// before the barrier, and the compiler may not move memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// The same without the LDS wait, where the slot about to be refilled was read
// (and its values used) before the barrier: LDS reads issued just before it
// from another slot stay in flight across it.
__device__ __forceinline__ void slot_barrier() {
  asm volatile("s_barrier" ::: "memory");
}

// LDS reads of the ring are inline asm: the compiler then sees no LDS load
// that could alias an in-flight stage DMA (it would wait for all of them),
// and the ring's own waits order everything.  lds_wait() waits for every
// outstanding LDS read and ties the values to the wait.
template <int B> struct LdsT;
template <> struct LdsT<16> { typedef uint32_t T __attribute__((ext_vector_type(4))); };
template <> struct LdsT<8> { typedef uint32_t T __attribute__((ext_vector_type(2))); };
template <> struct LdsT<4> { typedef uint32_t T; };
template <int B, int OFF> __device__ __forceinline__ typename LdsT<B>::T lds_read(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  typename LdsT<B>::T v;
  if constexpr (B == 16) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  else if constexpr (B == 8) asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  else asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
template <typename T, int N> __device__ __forceinline__ void lds_wait(T (&v)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }   // low half = LDS offset
