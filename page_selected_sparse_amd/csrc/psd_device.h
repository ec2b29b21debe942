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

// ---- wave-wide primitives on DPP row moves and lane reads (no LDS round trips) ----
// DPP control codes: row_shr:n = 0x110 + n, row_ror:n = 0x120 + n, row_bcast:15 = 0x142
// (lane 15 of each row to the next row), row_bcast:31 = 0x143 (lane 31 to rows 2 and 3).
// Lanes without a source, or in rows outside ROW_MASK, read 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_move(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes: shifts within each 16-lane row, then the row
// totals carried into the rows above.
__device__ __forceinline__ int wave_scan_incl(int x) {
  x += dpp_move<0x111>(x);
  x += dpp_move<0x112>(x);
  x += dpp_move<0x114>(x);
  x += dpp_move<0x118>(x);
  x += dpp_move<0x142, 0xa>(x);
  x += dpp_move<0x143, 0xc>(x);
  return x;
}

// AND and OR of a 64-bit value over the 64 lanes (uniform results): rotations within
// each row, then the four row results read out of lanes 0, 16, 32 and 48.
__device__ __forceinline__ void wave_and_or64(uint64_t& a, uint64_t& o) {
  int al = (int)(uint32_t)a, ah = (int)(uint32_t)(a >> 32);
  int ol = (int)(uint32_t)o, oh = (int)(uint32_t)(o >> 32);
#define PSD_ROT_STEP(C)      \
  al &= dpp_move<C>(al);     \
  ah &= dpp_move<C>(ah);     \
  ol |= dpp_move<C>(ol);     \
  oh |= dpp_move<C>(oh);
  PSD_ROT_STEP(0x121)
  PSD_ROT_STEP(0x122)
  PSD_ROT_STEP(0x124)
  PSD_ROT_STEP(0x128)
#undef PSD_ROT_STEP
  uint32_t ra = ~0u, rb = ~0u, rc = 0u, rd = 0u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    ra &= (uint32_t)__builtin_amdgcn_readlane(al, 16 * r);
    rb &= (uint32_t)__builtin_amdgcn_readlane(ah, 16 * r);
    rc |= (uint32_t)__builtin_amdgcn_readlane(ol, 16 * r);
    rd |= (uint32_t)__builtin_amdgcn_readlane(oh, 16 * r);
  }
  a = ((uint64_t)rb << 32) | ra;
  o = ((uint64_t)rd << 32) | rc;
}

// Maximum over the 16 lanes of each row, in every lane of the row (rotations by 1, 2, 4
// and 8 within the row).
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, __int_as_float(dpp_move<0x121>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<0x122>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<0x124>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<0x128>(__float_as_int(v))));
  return v;
}

// Value of x in lane `src` (a wave-uniform lane index).
__device__ __forceinline__ int lane_value(int x, int src) {
  return __builtin_amdgcn_readlane(x, src);
}

template <typename T>
__device__ __forceinline__ uint4 load16(const T* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace psd
