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
#include "meta_core.h"
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
    refresh_stats<BF16>(a.k, a.meta, blk, valid, h, d, a.Hkv, a.D, a.kbs, a.kts, a.khs);
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
