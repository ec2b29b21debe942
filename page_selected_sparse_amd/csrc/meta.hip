// Per-page key min/max refresh (EntmaxKV README, package tree: per-page k_min / k_max
// refresh kept beside the paged cache).
//
// One workgroup refreshes one logical page of one sequence for every KV head: the page's
// K rows for all heads form a [16, H_kv * D] tile whose rows are token-strided, so each
// thread owns 16 contiguous bytes of a row, requests all 16 rows at once and folds the
// page's valid tokens. Loads are coalesced across the workgroup (consecutive threads read
// consecutive 16-byte pieces of a token row) and each statistic is written once. Min/max
// are exact, so the values written are key values themselves. The statistics of one
// (block, head) are one contiguous record of 128-byte lines, each holding the min and the
// max of 64 bytes' worth of dims (the unit the scoring kernel reads back).
#include "psd_device.h"
#include "psd_launch.h"

namespace psd {
namespace {

struct MetaArgs {
  const void* k;
  void* meta;
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* first_page;
  int Hkv, D, max_pages, num_blocks;
  int64_t kbs, kts, khs;
};

template <bool BF16>
__global__ __launch_bounds__(256) void meta_kernel(MetaArgs a) {
  const int s = blockIdx.y;
  const int L = a.lens[s];
  const int n = ceil_div(L, kPage);
  int p;
  if (a.first_page == nullptr) {
    p = n - 1;
  } else {
    int f = a.first_page[s];
    p = (f < 0 ? 0 : f) + (int)blockIdx.x;
  }
  if (p < 0 || p >= n) return;
  const int blk = a.bt[(int64_t)s * a.max_pages + p];
  const int valid = min(kPage, L - p * kPage);
  constexpr int VEC = BF16 ? 8 : 4;  // elements per 16 bytes
  const int cols = a.Hkv * a.D;
  for (int col = threadIdx.x * VEC; col < cols; col += blockDim.x * VEC) {
    const int h = col / a.D, d = col - h * a.D;
    const int64_t base = (int64_t)blk * a.kbs + (int64_t)h * a.khs + d;
    // all 16 token rows are requested at once; rows past the length are not used
    float v[kPage][VEC];
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      const int tt = t < valid ? t : 0;
      if constexpr (BF16) {
        const uint4 w = load16(static_cast<const uint16_t*>(a.k) + base + (int64_t)tt * a.kts);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[t][2 * i] = bf_lo(ws[i]);
          v[t][2 * i + 1] = bf_hi(ws[i]);
        }
      } else {
        const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(a.k) + base +
                                                          (int64_t)tt * a.kts);
        v[t][0] = w.x; v[t][1] = w.y; v[t][2] = w.z; v[t][3] = w.w;
      }
    }
    float mn[VEC], mx[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) mn[i] = mx[i] = v[0][i];
#pragma unroll
    for (int t = 1; t < kPage; ++t) {
      if (t < valid) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          mn[i] = v[t][i] < mn[i] ? v[t][i] : mn[i];
          mx[i] = v[t][i] > mx[i] ? v[t][i] : mx[i];
        }
      }
    }
    // page-major statistics: [num_blocks][H_kv][D / CD][2][CD], CD = 64 bytes of dims
    constexpr int CD = BF16 ? 32 : 16;
    const int64_t mrow = (((int64_t)blk * a.Hkv + h) * (a.D / CD) + d / CD) * 2 * CD + d % CD;
    if constexpr (BF16) {
      uint16_t* m = static_cast<uint16_t*>(a.meta);
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
      float* m = static_cast<float*>(a.meta);
      *reinterpret_cast<float4*>(m + mrow) = make_float4(mn[0], mn[1], mn[2], mn[3]);
      *reinterpret_cast<float4*>(m + mrow + CD) = make_float4(mx[0], mx[1], mx[2], mx[3]);
    }
  }
}

}  // namespace

hipError_t launch_meta_update(const Geo& g, const void* k, void* meta, const int32_t* bt,
                              const int32_t* lens, const int32_t* first_page, hipStream_t st) {
  MetaArgs a{k, meta, bt, lens, first_page, g.Hkv, g.D, g.max_pages, g.num_blocks, g.kbs, g.kts,
             g.khs};
  const dim3 grid(first_page ? g.max_pages : 1, g.B);
  const int vec = g.dtype == 1 ? 8 : 4;
  int threads = (g.Hkv * g.D / vec + 63) / 64 * 64;
  threads = threads > 256 ? 256 : threads;
  if (g.dtype == 1)
    hipLaunchKernelGGL(meta_kernel<true>, grid, dim3(threads), 0, st, a);
  else
    hipLaunchKernelGGL(meta_kernel<false>, grid, dim3(threads), 0, st, a);
  return hipGetLastError();
}

}  // namespace psd
