// Page statistics of VEC consecutive dims (16 bytes) of one KV head of one page: the min
// and max over the page's valid tokens, written to the page-major statistics layout
// [num_blocks][H_kv][D / CD][2][CD] (CD = 64 bytes of dims). Shared by the statistics
// kernel and the one-launch decode step.
#pragma once

#include "psd_device.h"

namespace psd {
namespace {

// Token rows are requested TB at a time (all 16 at once by default; TB = 8 halves the
// registers); rows past `valid` are not used. Tokens are folded in ascending order. Min/max
// are exact, so the values written are key values themselves.
template <bool BF16, int TB = kPage>
__device__ __forceinline__ void refresh_stats(const void* k, void* meta, int blk, int valid, int h,
                                              int d, int Hkv, int D, int64_t kbs, int64_t kts,
                                              int64_t khs) {
  static_assert(kPage % TB == 0, "token batches");
  constexpr int VEC = BF16 ? 8 : 4;  // elements per 16 bytes
  const int64_t base = (int64_t)blk * kbs + (int64_t)h * khs + d;
  float mn[VEC], mx[VEC];
#pragma unroll 1
  for (int t0 = 0; t0 < kPage; t0 += TB) {
    if (t0 > 0 && t0 >= valid) break;
    float v[TB][VEC];
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const int t = t0 + i;
      const int tt = t < valid ? t : 0;
      if constexpr (BF16) {
        const uint4 w = load16(static_cast<const uint16_t*>(k) + base + (int64_t)tt * kts);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[i][2 * q] = bf_lo(ws[q]);
          v[i][2 * q + 1] = bf_hi(ws[q]);
        }
      } else {
        const float4 w =
            *reinterpret_cast<const float4*>(static_cast<const float*>(k) + base + (int64_t)tt * kts);
        v[i][0] = w.x; v[i][1] = w.y; v[i][2] = w.z; v[i][3] = w.w;
      }
    }
    if (t0 == 0) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) mn[j] = mx[j] = v[0][j];
    }
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const int t = t0 + i;
      if (t > 0 && t < valid) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          mn[j] = v[i][j] < mn[j] ? v[i][j] : mn[j];
          mx[j] = v[i][j] > mx[j] ? v[i][j] : mx[j];
        }
      }
    }
  }
  constexpr int CD = BF16 ? 32 : 16;
  const int64_t mrow = (((int64_t)blk * Hkv + h) * (D / CD) + d / CD) * 2 * CD + d % CD;
  if constexpr (BF16) {
    uint16_t* m = static_cast<uint16_t*>(meta);
    uint4 lo, hi;
    lo.x = pack2(__float_as_uint(mn[0]) >> 16, __float_as_uint(mn[1]) >> 16);
    lo.y = pack2(__float_as_uint(mn[2]) >> 16, __float_as_uint(mn[3]) >> 16);
    lo.z = pack2(__float_as_uint(mn[4]) >> 16, __float_as_uint(mn[5]) >> 16);
    lo.w = pack2(__float_as_uint(mn[6]) >> 16, __float_as_uint(mn[7]) >> 16);
    hi.x = pack2(__float_as_uint(mx[0]) >> 16, __float_as_uint(mx[1]) >> 16);
    hi.y = pack2(__float_as_uint(mx[2]) >> 16, __float_as_uint(mx[3]) >> 16);
    hi.z = pack2(__float_as_uint(mx[4]) >> 16, __float_as_uint(mx[5]) >> 16);
    hi.w = pack2(__float_as_uint(mx[6]) >> 16, __float_as_uint(mx[7]) >> 16);
    *reinterpret_cast<uint4*>(m + mrow) = lo;
    *reinterpret_cast<uint4*>(m + mrow + CD) = hi;
  } else {
    float* m = static_cast<float*>(meta);
    *reinterpret_cast<float4*>(m + mrow) = make_float4(mn[0], mn[1], mn[2], mn[3]);
    *reinterpret_cast<float4*>(m + mrow + CD) = make_float4(mx[0], mx[1], mx[2], mx[3]);
  }
}

// The statistics of sequence s's tail page for KV head g (the page launch_meta_update
// refreshes when it is given no first_page). Threads tid of nt share the dims; every
// thread of the group calls it. Rows are requested TB at a time (8 keeps registers low).
template <bool BF16, int TB = 8>
__device__ __forceinline__ void refresh_tail_page(const void* k, void* meta, const int32_t* bt,
                                  const int32_t* lens, int max_pages, int s, int g, int Hkv,
                                  int D, int64_t kbs, int64_t kts, int64_t khs, int tid, int nt) {
  const int L = lens[s];
  const int p = ceil_div(L, kPage) - 1;
  if (p < 0) return;
  const int blk = bt[(int64_t)s * max_pages + p];
  const int valid = min(kPage, L - p * kPage);
  constexpr int VEC = BF16 ? 8 : 4;
  for (int d = tid * VEC; d < D; d += nt * VEC)
    refresh_stats<BF16, TB>(k, meta, blk, valid, g, d, Hkv, D, kbs, kts, khs);
}

}  // namespace
}  // namespace psd
