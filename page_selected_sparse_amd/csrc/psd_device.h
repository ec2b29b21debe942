// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psd {

constexpr int kPage = 16;
constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short short4v;
typedef __attribute__((ext_vector_type(4))) float float4v;

// bf16 halves of a 32-bit word widened exactly to fp32.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) {
  return (lo16 & 0xffffu) | (hi16 << 16);
}

// Order-preserving map of an fp64 score onto uint64 (larger score -> larger key);
// -0 is first turned into +0 so that the two zeros tie.
__device__ __forceinline__ uint64_t score_key(double x) {
  x = x + 0.0;
  uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
__device__ __forceinline__ int round_up(int a, int b) { return ceil_div(a, b) * b; }

// Pages attended by a unit with n pages and the caller's budget.
__device__ __forceinline__ int effective_budget(int n, int budget) {
  if (n <= 2) return n;
  int b = budget < 2 ? 2 : budget;
  return b < n ? b : n;
}

template <typename T>
__device__ __forceinline__ uint4 load16(const T* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace psd
