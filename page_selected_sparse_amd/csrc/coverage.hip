// Adaptive coverage selection: a per-(sequence, KV head) nucleus over exact page masses
// (AMASS README, "Key AmassConfig fields", and LOCKS README, "Configuration": the
// `coverage` knob, 0.95 by default, GQA models only).
//
// Page mass of query head h on page p: the share of h's exact softmax(scale * q_h.k)
// over the sequence's valid tokens that falls on p's tokens. The group mass W(p) is the
// mean over the group's G heads. The kept set is the sink (page 0), the tail (page n-1)
// and the inner pages in (W descending, page ascending) order, added until the kept
// mass reaches `coverage` or the row of b_max entries is full; coverage >= 1 keeps every
// page that fits. The list is written ascending and padded with -1, like the budgeted
// selection's, so that the sparse attention consumes it unchanged.
//
// Two launches:
//  1. page_mass_mfma_kernel (bf16) / page_mass_kernel (fp32): one wave per page, 16
//     pages per 256-thread workgroup. The page's q_h.k for the group's heads come from
//     matrix-core steps (bf16) or from whole-row loads and lane sums (fp32); the wave
//     reduces the page's max m_h(p) and sum s_h(p) = sum_t exp(z_t - m_h(p)), written
//     to the workspace. This reads every valid K row once (the dense K read:
//     exact masses cannot come from the page statistics).
//  2. coverage_cut_kernel: one 1024-thread workgroup per unit. It forms
//     M_h = max_p m_h(p), Z_h = sum_p s_h(p) exp(m_h(p) - M_h) and
//     W(p) = mean_h s_h(p) exp(m_h(p) - M_h) / Z_h in fp64, sorts the inner pages in LDS
//     on 64-bit (fp32 mass, page) keys (bitonic network over at most 4096 entries), finds the cut with a block scan of
//     the sorted masses, and compacts the kept pages in ascending order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "psd_device.h"
#include "psd_launch.h"

namespace psd {
namespace {

constexpr int kCovMaxG = 8;        // query heads per group handled by the mass kernel
constexpr int kCovMaxPages = 4096; // pages per sequence the LDS sort holds
constexpr int kCutThreads = 1024;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

struct CovArgs {
  const void* q;
  const void* k;
  const int32_t* bt;
  const int32_t* lens;
  int32_t* sel;
  int32_t* cnt;
  float* pm;  // [B * Hq, max_pages] page max of each query head
  float* ps;  // [B * Hq, max_pages] page exp-sum of each query head
  float scale, coverage;
  int Hq, Hkv, G, max_pages, num_blocks, b_max;
  int64_t kbs, kts, khs;
};

__device__ __forceinline__ int seq_pages(const CovArgs& a, int s) {
  const int L = a.lens[s];
  return min(max(ceil_div(max(L, 0), kPage), 0), a.max_pages);
}

// Sum over each group of LPR consecutive lanes, in every lane of the group.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPR == 16) {  // a DPP row: rotations by 1, 2, 4 and 8 within the row
    v += __int_as_float(dpp_move<0x121>(__float_as_int(v)));
    v += __int_as_float(dpp_move<0x122>(__float_as_int(v)));
    v += __int_as_float(dpp_move<0x124>(__float_as_int(v)));
    v += __int_as_float(dpp_move<0x128>(__float_as_int(v)));
  } else {
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) v += __shfl_xor(v, o);
  }
  return v;
}

// One wave per page: each load instruction covers whole token rows (LPR lanes x 16 bytes
// per row, 64 / LPR rows per instruction), so a page's K rows arrive as 16 contiguous
// row reads; each lane keeps its 16-byte slice of q for every head of the group in
// registers. A workgroup of 4 waves covers 16 consecutive pages.
template <bool BF16, int D, int GM>
__global__ __launch_bounds__(256) void page_mass_kernel(CovArgs a) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPL = 16 / ES;         // elements per lane and row
  constexpr int LPR = D * ES / 16;     // lanes per row
  constexpr int RPI = kWave / LPR;     // rows per load instruction
  constexpr int RPL = kPage / RPI;     // rows per lane
  static_assert(LPR * RPI == kWave && RPL * RPI == kPage, "row tiling");
  const int s = blockIdx.z, g = blockIdx.y;
  const int L = a.lens[s];
  const int n = seq_pages(a, s);
  if ((int)blockIdx.x * 16 >= n) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = lane % LPR, rs = lane / LPR;
  const int G = a.G;

  float qv[GM][EPL];
  const int64_t q0 = ((int64_t)s * a.Hq + (int64_t)g * G) * D + part * EPL;
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < G) {
      const uint4 w = load16(static_cast<const unsigned char*>(a.q) + (q0 + (int64_t)h * D) * ES);
      if constexpr (BF16) {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qv[h][2 * j] = bf_lo(ws[j]);
          qv[h][2 * j + 1] = bf_hi(ws[j]);
        }
      } else {
        qv[h][0] = __uint_as_float(w.x);
        qv[h][1] = __uint_as_float(w.y);
        qv[h][2] = __uint_as_float(w.z);
        qv[h][3] = __uint_as_float(w.w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) qv[h][j] = 0.f;
    }
  }

  for (int it = 0; it < 4; ++it) {
    const int lp = blockIdx.x * 16 + it * 4 + wave;
    if (lp >= n) break;  // uniform over the wave
    int blk = a.bt[(int64_t)s * a.max_pages + lp];
    blk = min(max(blk, 0), a.num_blocks - 1);
    const unsigned char* kb = static_cast<const unsigned char*>(a.k) +
        ((int64_t)blk * a.kbs + (int64_t)g * a.khs + part * EPL) * ES;
    // Rows past the length are loaded (they lie inside the block) and masked below.
    uint4 raw[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) raw[i] = load16(kb + (int64_t)(rs + RPI * i) * a.kts * ES);
    float z[RPL][GM];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      float kv[EPL];
      if constexpr (BF16) {
        const uint32_t ws[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kv[2 * j] = bf_lo(ws[j]);
          kv[2 * j + 1] = bf_hi(ws[j]);
        }
      } else {
        kv[0] = __uint_as_float(raw[i].x);
        kv[1] = __uint_as_float(raw[i].y);
        kv[2] = __uint_as_float(raw[i].z);
        kv[3] = __uint_as_float(raw[i].w);
      }
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        float acc = 0.f;
        if (h < G) {
#pragma unroll
          for (int j = 0; j < EPL; ++j) acc = fmaf(qv[h][j], kv[j], acc);
          acc = group_sum<LPR>(acc);
        }
        z[i][h] = acc;
      }
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
          const bool valid = lp * kPage + rs + RPI * i < L;
          z[i][h] = valid ? a.scale * z[i][h] : -INFINITY;
          m = fmaxf(m, z[i][h]);
        }
#pragma unroll
        for (int o = LPR; o < kWave; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        float e = 0.f;
#pragma unroll
        for (int i = 0; i < RPL; ++i) e += z[i][h] == -INFINITY ? 0.f : expf(z[i][h] - m);
#pragma unroll
        for (int o = LPR; o < kWave; o <<= 1) e += __shfl_xor(e, o);
        if (lane == 0) {
          const int64_t at = ((int64_t)s * a.Hq + (int64_t)g * G + h) * a.max_pages + lp;
          a.pm[at] = m;
          a.ps[at] = e;
        }
      }
    }
  }
}

// bf16 pages on the matrix cores: one wave per page computes S^T = K_page Q^T (16 tokens x
// up to 16 heads) with D/32 v_mfma_f32_16x16x32_bf16 steps. Lane l loads 16 bytes of token
// row l % 16 at dims 32c + 8 (l / 16) (the A operand) and holds the same dims of head
// l % 16 (the B operand; heads past the group are zero). The result leaves in lane l the
// scores of head l % 16 for tokens 4 (l / 16) .. +3, so the page's max and exp-sum per
// head take two lane exchanges each.
template <int D>
__global__ __launch_bounds__(256) void page_mass_mfma_kernel(CovArgs a) {
  constexpr int NQ = D / 32;
  const int s = blockIdx.z, g = blockIdx.y;
  const int L = a.lens[s];
  const int n = seq_pages(a, s);
  if ((int)blockIdx.x * 16 >= n) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int G = a.G;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  uint4 qf[NQ];
  const int64_t qrow = ((int64_t)s * a.Hq + (int64_t)g * G + (r < G ? r : 0)) * D + 8 * grp;
#pragma unroll
  for (int c = 0; c < NQ; ++c)
    qf[c] = r < G ? load16(q + qrow + 32 * c) : make_uint4(0, 0, 0, 0);
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + (int64_t)g * a.khs +
                          (int64_t)r * a.kts + 8 * grp;

  // The wave's four pages: block ids up front, then each page's rows requested while
  // the previous page is reduced. Rows past the length are loaded (they lie inside the
  // block) and masked below.
  int blks[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int lp = blockIdx.x * 16 + it * 4 + wave;
    blks[it] = lp < n ? min(max(a.bt[(int64_t)s * a.max_pages + lp], 0), a.num_blocks - 1) : 0;
  }
  uint4 kf[NQ], nx[NQ];
  if (blockIdx.x * 16 + wave < n) {
#pragma unroll
    for (int c = 0; c < NQ; ++c) kf[c] = load16(kbase + (int64_t)blks[0] * a.kbs + 32 * c);
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int lp = blockIdx.x * 16 + it * 4 + wave;
    if (lp >= n) break;  // uniform over the wave
    if (it < 3 && lp + 4 < n) {
#pragma unroll
      for (int c = 0; c < NQ; ++c) nx[c] = load16(kbase + (int64_t)blks[it + 1] * a.kbs + 32 * c);
    }
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      const u32x4 kv = {kf[c].x, kf[c].y, kf[c].z, kf[c].w};
      const u32x4 qv = {qf[c].x, qf[c].y, qf[c].z, qf[c].w};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv),
                                                    __builtin_bit_cast(bf16x8, qv), acc, 0, 0, 0);
    }
    const int t0 = lp * kPage + 4 * grp;
    float z[4];
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      z[k] = t0 + k < L ? a.scale * acc[k] : -INFINITY;
      m = fmaxf(m, z[k]);
    }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    float e = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) e += z[k] == -INFINITY ? 0.f : expf(z[k] - m);
    e += __shfl_xor(e, 16);
    e += __shfl_xor(e, 32);
    if (grp == 0 && r < G) {
      const int64_t at = ((int64_t)s * a.Hq + (int64_t)g * G + r) * a.max_pages + lp;
      a.pm[at] = m;
      a.ps[at] = e;
    }
#pragma unroll
    for (int c = 0; c < NQ; ++c) kf[c] = nx[c];
  }
}

// Block-wide inclusive scan of one double per thread (Hillis-Steele in LDS).
__device__ double block_scan_incl(double v, double* buf) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int off = 1; off < kCutThreads; off <<= 1) {
    const double add = t >= off ? buf[t - off] : 0.0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  const double r = buf[t];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kCutThreads) void coverage_cut_kernel(CovArgs a) {
  constexpr int NW = kCutThreads / kWave;
  // Sort keys: the group mass as fp32 bits (non-negative, so the bits order like the
  // values) above the inverted page index, so that a descending sort gives
  // (mass descending, page ascending); 0 pads and sorts last.
  __shared__ uint64_t key[kCovMaxPages];
  __shared__ double buf[kCutThreads];
  __shared__ unsigned char flag[kCovMaxPages];
  __shared__ float redf[NW][kCovMaxG];
  __shared__ double redd[NW][kCovMaxG];
  __shared__ float Mh[kCovMaxG];
  __shared__ double Zh[kCovMaxG];
  __shared__ double ends[2];
  __shared__ int kcut, total;

  const int g = blockIdx.x, s = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int unit = s * a.Hkv + g;
  const int G = a.G;
  int32_t* out = a.sel + (int64_t)unit * a.b_max;
  const int n = seq_pages(a, s);
  if (n <= 2) {
    for (int i = t; i < a.b_max; i += kCutThreads) out[i] = i < n ? i : -1;
    if (t == 0) a.cnt[unit] = n;
    return;
  }
  const int64_t h0 = (int64_t)s * a.Hq + (int64_t)g * G;

  // Each head's max over the pages, then its normaliser: per-thread values, wave
  // shuffles, one pass through LDS.
  float mloc[kCovMaxG];
#pragma unroll
  for (int h = 0; h < kCovMaxG; ++h) mloc[h] = -INFINITY;
  for (int p = t; p < n; p += kCutThreads) {
#pragma unroll
    for (int h = 0; h < kCovMaxG; ++h)
      if (h < G) mloc[h] = fmaxf(mloc[h], a.pm[(h0 + h) * a.max_pages + p]);
  }
#pragma unroll
  for (int h = 0; h < kCovMaxG; ++h) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mloc[h] = fmaxf(mloc[h], __shfl_xor(mloc[h], o));
    if (lane == 0) redf[wave][h] = mloc[h];
  }
  __syncthreads();
  if (t < G) {
    float m = -INFINITY;
    for (int w = 0; w < NW; ++w) m = fmaxf(m, redf[w][t]);
    Mh[t] = m;
  }
  __syncthreads();
  double zloc[kCovMaxG];
#pragma unroll
  for (int h = 0; h < kCovMaxG; ++h) zloc[h] = 0.0;
  for (int p = t; p < n; p += kCutThreads) {
#pragma unroll
    for (int h = 0; h < kCovMaxG; ++h) {
      if (h < G) {
        const int64_t at = (h0 + h) * a.max_pages + p;
        zloc[h] += (double)a.ps[at] * exp((double)a.pm[at] - (double)Mh[h]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kCovMaxG; ++h) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) zloc[h] += __shfl_xor(zloc[h], o);
    if (lane == 0) redd[wave][h] = zloc[h];
  }
  __syncthreads();
  if (t < G) {
    double z = 0.0;
    for (int w = 0; w < NW; ++w) z += redd[w][t];
    Zh[t] = z;
  }
  __syncthreads();

  // Group masses: inner pages 1..n-2 go to sort slot p-1; the ends are kept aside.
  const int mc = n - 2;
  int np2 = 1;
  while (np2 < mc) np2 <<= 1;
  for (int p = t; p < n; p += kCutThreads) {
    double w = 0.0;
    for (int h = 0; h < G; ++h) {
      const int64_t at = (h0 + h) * a.max_pages + p;
      w += (double)a.ps[at] * exp((double)a.pm[at] - (double)Mh[h]) / Zh[h];
    }
    w /= (double)G;
    if (p == 0) {
      ends[0] = w;
    } else if (p == n - 1) {
      ends[1] = w;
    } else {
      key[p - 1] = ((uint64_t)__float_as_uint((float)w) << 32) | (uint32_t)(0xffffffffu - p);
    }
  }
  for (int i = mc + t; i < np2; i += kCutThreads) key[i] = 0;  // padding sorts last
  __syncthreads();

  // Bitonic sort of slots [0, np2) into descending key order.
  for (int k = 2; k <= np2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = t; i < np2; i += kCutThreads) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t ki = key[i], kl = key[l];
          if ((i & k) == 0 ? kl > ki : ki > kl) {
            key[i] = kl;
            key[l] = ki;
          }
        }
      }
      __syncthreads();
    }
  }
  auto slot_mass = [&](int i) { return (double)__uint_as_float((uint32_t)(key[i] >> 32)); };
  auto slot_page = [&](int i) { return (int)(0xffffffffu - (uint32_t)key[i]); };

  // The cut: the fewest leading slots whose mass, with the ends, reaches the coverage.
  const int room = min(mc, a.b_max - 2);
  constexpr int PER = kCovMaxPages / kCutThreads;  // sorted slots per thread
  const double base = ends[0] + ends[1];
  if (t == 0) kcut = mc;
  double local = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = t * PER + j;
    if (i < mc) local += slot_mass(i);
  }
  const double incl = block_scan_incl(local, buf);  // also orders kcut's init before use
  int take;
  if (a.coverage >= 1.f) {
    take = room;
  } else if (base >= (double)a.coverage) {
    take = 0;
  } else {
    double run = base + incl - local;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = t * PER + j;
      if (i < mc) {
        run += slot_mass(i);
        if (run >= (double)a.coverage) {
          atomicMin(&kcut, i + 1);
          break;
        }
      }
    }
    __syncthreads();
    take = min(kcut, room);
  }

  // Flags in page order, then an ascending compaction.
  for (int p = t; p < n; p += kCutThreads) flag[p] = (p == 0 || p == n - 1) ? 1 : 0;
  __syncthreads();
  for (int i = t; i < take; i += kCutThreads) {
    const int p = slot_page(i);
    if ((unsigned)p < (unsigned)n) flag[p] = 1;  // padding decodes past n
  }
  __syncthreads();
  int mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int p = t * PER + j;
    if (p < n) mine += flag[p];
  }
  const int incl_cnt = (int)block_scan_incl((double)mine, buf);
  if (t == kCutThreads - 1) total = incl_cnt;
  int at = incl_cnt - mine;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int p = t * PER + j;
    if (p < n && flag[p]) out[at++] = p;
  }
  __syncthreads();
  const int count = total;  // take + 2 for finite masses
  for (int i = count + t; i < a.b_max; i += kCutThreads) out[i] = -1;
  if (t == 0) a.cnt[unit] = count;
}

template <bool BF16, int D>
hipError_t launch_mass(const CovArgs& a, int B, hipStream_t st) {
  dim3 grid((a.max_pages + 15) / 16, a.Hkv, B);
  if constexpr (BF16)  // the matrix cores take the page's q.k
    hipLaunchKernelGGL((page_mass_mfma_kernel<D>), grid, dim3(256), 0, st, a);
  else if (a.G <= 4)  // head slots held in registers: 4 or 8
    hipLaunchKernelGGL((page_mass_kernel<BF16, D, 4>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((page_mass_kernel<BF16, D, kCovMaxG>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

size_t coverage_workspace_bytes(const Geo& g) {
  return 2 * sizeof(float) * (size_t)g.B * g.Hq * g.max_pages;
}

bool coverage_supported(const Geo& g) {
  return g.G <= kCovMaxG && g.max_pages <= kCovMaxPages && (g.D == 64 || g.D == 128);
}

hipError_t launch_coverage_select(const Geo& g, const void* q, const void* k, const int32_t* bt,
                                  const int32_t* lens, float coverage, float scale, int b_max,
                                  int32_t* sel, int32_t* cnt, void* ws, hipStream_t st) {
  CovArgs a;
  a.q = q;
  a.k = k;
  a.bt = bt;
  a.lens = lens;
  a.sel = sel;
  a.cnt = cnt;
  a.pm = static_cast<float*>(ws);
  a.ps = a.pm + (size_t)g.B * g.Hq * g.max_pages;
  a.scale = scale;
  a.coverage = coverage;
  a.Hq = g.Hq;
  a.Hkv = g.Hkv;
  a.G = g.G;
  a.max_pages = g.max_pages;
  a.num_blocks = g.num_blocks;
  a.b_max = b_max;
  a.kbs = g.kbs;
  a.kts = g.kts;
  a.khs = g.khs;
  hipError_t e;
  if (g.dtype == 1)
    e = g.D == 64 ? launch_mass<true, 64>(a, g.B, st) : launch_mass<true, 128>(a, g.B, st);
  else
    e = g.D == 64 ? launch_mass<false, 64>(a, g.B, st) : launch_mass<false, 128>(a, g.B, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(coverage_cut_kernel, dim3(g.Hkv, g.B), dim3(kCutThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace psd
