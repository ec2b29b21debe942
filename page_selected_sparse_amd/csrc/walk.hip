// Diagnostic memory walks of the decode step's reads, with no arithmetic.
//
// They read what the step reads, in the same shapes of request, and fold every 32-bit word
// into one checksum word per unit, so that a run measures what the memory system gives
// these access patterns on the GPU (the practical ceiling of the kernels that make them)
// and a test can check that the walk touched exactly the intended bytes:
//   kind 0: every kept page's K and V rows of every unit, one 1024-thread workgroup per
//           (sequence, KV head) unit, wave w taking list entries w, w + 16, ... (the
//           whole-unit attention's split), whole 256-byte rows per load at D = 128 bf16;
//   kind 1: the statistics record of every candidate page (pages 1 .. n - 2) of every
//           unit, one workgroup per unit, each wave 64 pages per round, one 128-byte line
//           of 8 pages per load (the scoring's staging pattern).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "psd_device.h"
#include "psd_launch.h"

namespace psd {
namespace {

struct WalkArgs {
  const unsigned char* k;
  const unsigned char* v;     // null: V is inside K (latent), not walked again
  const unsigned char* meta;
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* sel;
  const int32_t* cnt;
  uint32_t* checksum;
  int64_t kbs, kts, khs, vbs, vts, vhs;  // bytes
  int Hkv, max_pages, num_blocks, b_max;
};

__device__ __forceinline__ uint32_t fold(const uint4& x) { return x.x ^ x.y ^ x.z ^ x.w; }

// The workgroup's XOR into checksum[unit] (one plain store per unit: a single word
// updated by atomics from every workgroup would serialize them).
__device__ __forceinline__ void publish(uint32_t x, uint32_t* checksum, int unit) {
  __shared__ uint32_t part[16];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) y ^= part[w];
    checksum[unit] = y;
  }
}

// KP / VP: 16-byte pieces per K / V row (V: 0 when it is not walked).
template <int KP, int VP>
__global__ __launch_bounds__(1024) void walk_kv_kernel(WalkArgs a) {
  static_assert((16 * KP) % 64 == 0 && (16 * VP) % 64 == 0, "whole loads per page");
  constexpr int NK = 16 * KP / 64, NV = 16 * VP / 64;  // loads per page and lane
  const int u = blockIdx.x, s = u / a.Hkv, g = u - s * a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = ceil_div(a.lens[s], kPage);
  int count = a.cnt[u];
  count = count < 0 ? 0 : min(count, a.b_max);
  uint32_t x = 0;
  // this wave's entries w, w + 16, ...: block ids looked up 64 at a time, one per lane
  const int mine = wave < count ? (count - wave + 15) / 16 : 0;
  for (int b0 = 0; b0 < mine; b0 += 64) {
    int my_blk = 0;
    if (b0 + lane < mine) {
      const int e = wave + 16 * (b0 + lane);
      const int lp = min(max(a.sel[(int64_t)u * a.b_max + e], 0), max(n - 1, 0));
      my_blk = min(max(a.bt[(int64_t)s * a.max_pages + lp], 0), a.num_blocks - 1);
    }
    const int np = min(64, mine - b0);
    for (int j = 0; j < np; ++j) {
      const int blk = __builtin_amdgcn_readlane(my_blk, j);
      const unsigned char* kb = a.k + blk * a.kbs + g * a.khs;
      uint4 r[NK + NV];
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int p = 64 * i + lane, row = p / KP, c = p - row * KP;
        r[i] = *reinterpret_cast<const uint4*>(kb + row * a.kts + 16 * c);
      }
      if constexpr (VP > 0) {
        const unsigned char* vb = a.v + blk * a.vbs + g * a.vhs;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int p = 64 * i + lane, row = p / VP, c = p - row * VP;
          r[NK + i] = *reinterpret_cast<const uint4*>(vb + row * a.vts + 16 * c);
        }
      }
#pragma unroll
      for (int i = 0; i < NK + NV; ++i) x ^= fold(r[i]);
    }
  }
  publish(x, a.checksum, u);
}

// NL: 128-byte lines per statistics record.
template <int NL>
__global__ __launch_bounds__(1024) void walk_stats_kernel(WalkArgs a) {
  const int u = blockIdx.x, s = u / a.Hkv, g = u - s * a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = ceil_div(a.lens[s], kPage);
  const int inner = n - 2;  // candidate pages 1 .. n - 2
  uint32_t x = 0;
  for (int base = 64 * wave; base < inner; base += 1024) {
    const int pg = 1 + min(base + lane, inner - 1);
    const int blk = min(max(a.bt[(int64_t)s * a.max_pages + pg], 0), a.num_blocks - 1);
    const int64_t rec = ((int64_t)blk * a.Hkv + g) * (NL * 128);
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      uint4 r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = 8 * i + lane / 8;  // the page of this lane's piece in load i
        const int64_t rp = __shfl(rec, p, 64);
        r[i] = *reinterpret_cast<const uint4*>(a.meta + rp + 128 * l + 16 * (lane & 7));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (base + 8 * i + lane / 8 < inner) x ^= fold(r[i]);
    }
  }
  publish(x, a.checksum, u);
}

template <int KP, int VP>
hipError_t launch_kv(const WalkArgs& a, int units, hipStream_t st) {
  hipLaunchKernelGGL((walk_kv_kernel<KP, VP>), dim3(units), dim3(1024), 0, st, a);
  return hipGetLastError();
}

template <int NL>
hipError_t launch_stats(const WalkArgs& a, int units, hipStream_t st) {
  hipLaunchKernelGGL((walk_stats_kernel<NL>), dim3(units), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool walk_supported(const Geo& g, bool latent) {
  const int es = g.dtype == 1 ? 2 : 4;
  const int kp = g.D * es / 16, vp = latent ? 0 : g.Dv * es / 16;
  const bool kv = (kp == 72 && vp == 0) || (kp == vp && (kp == 8 || kp == 16 || kp == 32));
  const int nl = 2 * g.D * es / 128;
  return kv && (nl == 2 || nl == 4 || nl == 8 || nl == 18);
}

hipError_t launch_walk(const Geo& g, int kind, bool latent, const void* k, const void* v,
                       const void* meta, const int32_t* bt, const int32_t* lens,
                       const int32_t* sel, const int32_t* cnt, int b_max, uint32_t* checksum,
                       hipStream_t st) {
  const int es = g.dtype == 1 ? 2 : 4;
  WalkArgs a;
  a.k = static_cast<const unsigned char*>(k);
  a.v = latent ? nullptr : static_cast<const unsigned char*>(v);
  a.meta = static_cast<const unsigned char*>(meta);
  a.bt = bt;
  a.lens = lens;
  a.sel = sel;
  a.cnt = cnt;
  a.checksum = checksum;
  a.kbs = g.kbs * es;
  a.kts = g.kts * es;
  a.khs = g.khs * es;
  a.vbs = g.vbs * es;
  a.vts = g.vts * es;
  a.vhs = g.vhs * es;
  a.Hkv = g.Hkv;
  a.max_pages = g.max_pages;
  a.num_blocks = g.num_blocks;
  a.b_max = b_max;
  const int units = g.B * g.Hkv;
  if (kind == 1) {
    switch (2 * g.D * es / 128) {
      case 2: return launch_stats<2>(a, units, st);
      case 4: return launch_stats<4>(a, units, st);
      case 8: return launch_stats<8>(a, units, st);
      case 18: return launch_stats<18>(a, units, st);
      default: return hipErrorInvalidValue;
    }
  }
  const int kp = g.D * es / 16, vp = latent ? 0 : g.Dv * es / 16;
  if (kp == 72 && vp == 0) return launch_kv<72, 0>(a, units, st);
  if (kp == 8 && vp == 8) return launch_kv<8, 8>(a, units, st);
  if (kp == 16 && vp == 16) return launch_kv<16, 16>(a, units, st);
  if (kp == 32 && vp == 32) return launch_kv<32, 32>(a, units, st);
  return hipErrorInvalidValue;
}

}  // namespace psd
