// Paged attention over a page list (split-K or whole-unit workgroups): argument block,
// fragment helpers and the workgroup body, shared by the attention launches and by the
// fused selection + attention launch.
#pragma once

#include <math.h>

#include "psd_device.h"
#include "psd_launch.h"

namespace psd {
namespace {

// Tuning (defaults measured on MI355X): software-pipelined page loads (bf16), and the
// one-wave variant's occupancy target in waves per SIMD.
#ifndef PSD_ATTN_KV_TOGETHER
#define PSD_ATTN_KV_TOGETHER 1  // a page's K and V loads in flight together
#endif
#ifndef PSD_ATTN_PIPE
#define PSD_ATTN_PIPE 0
#endif
#ifndef PSD_ATTN_W1
#define PSD_ATTN_W1 4
#endif
#ifndef PSD_ATTN_TARGET
#define PSD_ATTN_TARGET 4096  // sparse
#endif
#ifndef PSD_ATTN_TARGET_DENSE
#define PSD_ATTN_TARGET_DENSE 2048
#endif
#ifndef PSD_ATTN_TARGET_WIDE
#define PSD_ATTN_TARGET_WIDE 256  // workgroups of 2+ waves (groups over 16 heads)
#endif
#ifndef PSD_ATTN_UNIT_WAVES
#define PSD_ATTN_UNIT_WAVES 16  // waves of a whole-unit workgroup
#endif
#ifndef PSD_ATTN_UNIT_MIN
#define PSD_ATTN_UNIT_MIN 128  // units that fill the GPU with one workgroup each
#endif
#ifndef PSD_ATTN_UNIT_DENSE
#define PSD_ATTN_UNIT_DENSE 0  // whole-unit workgroups for the dense walk too
#endif

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* sel;  // nullptr: dense (every page)
  const int32_t* cnt;
  float* pacc;  // [B, Hq, nsplit, Dv]
  float2* pml;  // [B, Hq, nsplit]
  float* out;   // [B, Hq, Dv]: written directly when one workgroup holds a whole unit
  int Hq, Hkv, G, max_pages, b_max, pps, nsplit, num_blocks;
  int64_t kbs, kts, khs, vbs, vts, vhs;
  float sl2;  // scale * log2(e)
  // Value tier (TIER builds): entry e of unit u reads V from hot slice vslot[u][e] when
  // it is >= 0 ([slots][16][Dv] elements), else from v through the block table.
  const int32_t* vslot = nullptr;
  const void* hot = nullptr;
  const void* hot_k = nullptr;  // KV tier: [slices][16][D], K of the resident slices
};

constexpr int kMaxSplits = 16384;
constexpr int kKTileBytes = 16 * 17 * 16;  // a wave's K tile: 16 rows of 256 B, 16 B of pad

// Where the K tiles of a whole-unit workgroup go: inside each wave's own part of the
// closing combine's area when that part is big enough (a wave writes it only once its own
// pages are done, and reads the others' only after a barrier), else past `used` bytes.
struct KTilePlace {
  size_t off, stride, end;  // first tile, distance between tiles, end of the LDS used
};
inline KTilePlace ktile_place(const Geo& g, int waves, size_t used) {
  const size_t part = (size_t)g.G * g.Dv * sizeof(float);
  if (part >= (size_t)kKTileBytes) return KTilePlace{0, part, used};
  const size_t off = (used + 255) / 256 * 256;
  return KTilePlace{off, (size_t)kKTileBytes, off + (size_t)waves * kKTileBytes};
}

// LDS of a whole-unit workgroup's closing combine: acc [waves][G][Dv] and (m, l) [waves][16].
inline size_t unit_combine_lds(const Geo& g) {
  return (size_t)PSD_ATTN_UNIT_WAVES * g.G * g.Dv * sizeof(float) +
         (size_t)PSD_ATTN_UNIT_WAVES * 16 * sizeof(float2);
}

// Argument block of a decode plan; `ws` holds the split partials (unused by whole-unit
// plans).
inline AttnArgs make_attn_args(const Geo& g, const DecodePlan& p, const void* q, const void* k,
                               const void* v, const int32_t* bt, const int32_t* lens,
                               const int32_t* sel, const int32_t* cnt, int b_max, float scale,
                               float* out, void* ws) {
  unsigned char* w = static_cast<unsigned char*>(ws);
  return AttnArgs{q, k, v, bt, lens, sel, cnt,
                  reinterpret_cast<float*>(w), reinterpret_cast<float2*>(w + p.off_ml), out,
                  g.Hq, g.Hkv, g.G, g.max_pages, b_max, p.pps, p.nsplit, g.num_blocks,
                  g.kbs, g.kts, g.khs, g.vbs, g.vts, g.vhs, scale * 1.4426950408889634f};
}

struct MergeArgs {
  const int32_t* lens;
  const int32_t* cnt;  // nullptr: dense
  const float* pacc;
  const float2* pml;
  float* out;
  int Hq, Hkv, G, pps, nsplit, Dv, b_max;
};

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) {
  u32x4 v = {w.x, w.y, w.z, w.w};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ short4v as_short4(uint32_t lo, uint32_t hi) {
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
  u32x2 v = {lo, hi};
  return __builtin_bit_cast(short4v, v);
}

// 8 fp32 values -> bf16 hi part and bf16 lo (residual) part, packed 2 per word.
__device__ __forceinline__ void split8(const float* x, uint4& hi, uint4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = f2bf(x[i]);
    l[i] = f2bf(x[i] - __uint_as_float(h[i] << 16));
  }
  hi = make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
  lo = make_uint4(pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7]));
}

// Reductions over lanes l, l^16, l^32, l^48 with the lane-swap instructions: a 16-lane
// swap pairs each lane with lane l^16, a 32-lane swap with lane l^32 (both operands of a
// swap are x, so each lane receives both halves of its pair).
__device__ __forceinline__ float wave_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Loads the 8-element fragment of row `row` at dim `d` as bf16 (hi, lo for fp32 data).
template <bool BF16>
__device__ __forceinline__ void load_frag8(const void* base, int64_t off, uint4& hi, uint4& lo) {
  if constexpr (BF16) {
    hi = load16(static_cast<const uint16_t*>(base) + off);
  } else {
    const float* p = static_cast<const float*>(base) + off;
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    split8(x, hi, lo);
  }
}

// NWS > 0: one workgroup per unit (groups of up to 16 heads), its NWS waves being the
// splits: wave w takes the unit's list entries w, w + NWS, w + 2 NWS, ..., and the waves'
// partials are combined in LDS at the end, so that no partial leaves the workgroup.
// The body of one workgroup: split `split` of unit (s, g), or, with NWS > 0, the whole
// unit. When `list` is given it replaces the selection row and count in memory (a list
// in LDS written by the same workgroup: ascending pages, list_count entries, negative for
// a flagged unit). A whole-unit workgroup calls `before_combine()` in every thread once
// its wave has attended all of its pages, before the waves are combined.
struct NoHook {
  __device__ void operator()() const {}
};

// KT (bf16, D = 128): each page's K rows are loaded whole (4 rows of 256 bytes per load
// instruction, as V is) and pass through an LDS tile of the wave (kKTileBytes at `ktile` +
// wave * kt_stride) to reach the matrix cores' operand layout (16 rows of 64 bytes per
// fragment). Loads of that layout straight from memory touch 16 rows per instruction; on
// the ragged batch the step took 1.6 us longer with them.
template <bool BF16, int DQK, int DV, int WAVES, int NWS, typename Hook = NoHook,
          bool TIER = false, bool KT = false>
__device__ __forceinline__ void attn_body(const AttnArgs& a, int split_x, int g, int s,
                                          const int32_t* list, int list_count,
                                          const Hook& before_combine = Hook(),
                                          unsigned char* ktile = nullptr,
                                          int kt_stride = kKTileBytes) {
  constexpr bool UNIT = NWS > 0;
  static_assert(!TIER || DQK <= 128, "value tier: D <= 128");
  static_assert(!KT || (BF16 && DQK == 128), "K through LDS: bf16, D = 128");
  static_assert(!UNIT || (WAVES == 1 && DQK <= 128), "unit workgroups: one head tile");
  constexpr bool PIPE = PSD_ATTN_PIPE != 0 && BF16;
  constexpr int NQ = DQK / 32;   // QK MFMAs per page (K = 32 dims each)
  constexpr int NC = DV / 16;    // PV MFMAs per page (16 output columns each)
  static_assert(NC % 4 == 0, "Dv must be a multiple of 64");
  constexpr bool QREG = DQK <= 128;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int split = UNIT ? wave : split_x;
  const int hw = UNIT ? 0 : wave;  // head tile of this wave
  // List entries of this split: first + stride * i.
  const int first = UNIT ? wave : split * a.pps;
  const int stride = UNIT ? NWS : 1;
  const int64_t srow = (int64_t)(s * a.Hkv + g) * a.b_max;
  // The first selection entries are requested together with the length and the count
  // (the row holds b_max entries; lanes past it read its last entry), so that only the
  // block-table lookup stands between them and the first K/V loads.
  int sel_lp = first + stride * lane;
  if (list)
    sel_lp = list[min(sel_lp, max(list_count, 1) - 1)];
  else if (a.sel)
    sel_lp = a.sel[srow + min(sel_lp, a.b_max - 1)];
  const int L = a.lens[s];
  const int n = ceil_div(L, kPage);
  int count = list ? list_count : (a.sel ? min(a.cnt[s * a.Hkv + g], a.b_max) : n);
  if (count < 0) count = 0;  // flagged unit: its output is NaN
  const int total = first >= count ? 0
                    : (UNIT ? ceil_div(count - first, stride) : min(a.pps, count - first));
  if (!UNIT && total == 0) return;

  // Page list of a batch of up to 64 entries: lane i holds entry first + stride * (b0 + i).
  // Entries are clamped to the sequence's pages so that a malformed list can never
  // address outside the table.
  int my_lp = 0, my_blk = 0, my_vs = -1;
  auto set_batch = [&](int np, int e) {  // e: this lane's list entry
    my_lp = my_blk = 0;
    my_vs = -1;
    if (lane < np) {
      my_lp = min(max(sel_lp, 0), n - 1);
      my_blk = a.bt[(int64_t)s * a.max_pages + my_lp];
      my_blk = min(max(my_blk, 0), a.num_blocks - 1);
      if constexpr (TIER) my_vs = a.vslot[srow + min(e, a.b_max - 1)];
    }
  };

  // Q tile as the B operand of S^T = K Q^T: lane holds head r, dims 32c + 8grp .. +8.
  const int head = hw * 16 + r;  // within the group
  const bool hvalid = head < a.G;
  const int64_t qrow = ((int64_t)s * a.Hq + g * a.G + (hvalid ? head : 0)) * DQK;
  uint4 qhi[QREG ? NQ : 1], qlo[QREG ? NQ : 1];
  if constexpr (QREG) {
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      qhi[c] = make_uint4(0, 0, 0, 0);
      qlo[c] = make_uint4(0, 0, 0, 0);
      if (hvalid) load_frag8<BF16>(a.q, qrow + 32 * c + 8 * grp, qhi[c], qlo[c]);
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  float4v acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};

  // Raw fragments of one page: K row r at dims 32c + 8grp (A operand of S^T = K Q^T) and
  // V rows 4grp + j at columns r*NC + w*CW (B operand of O += P V). For D <= 128 all of a
  // page's K and V loads are issued together at the start of the page; for the wide
  // latent rows they are streamed next to the MFMAs that use them (register budget).
  constexpr int CW = (BF16 && NC >= 8) ? 8 : 4;  // V columns per load group
  constexpr int NG = NC / CW;
  constexpr bool EARLY = DQK <= 128;
  auto load_k = [&](int blk, int c, uint4& k0, uint4& k1) {
    const int64_t off = (int64_t)blk * a.kbs + (int64_t)r * a.kts + (int64_t)g * a.khs +
                        32 * c + 8 * grp;
    if constexpr (BF16) {
      k0 = load16(static_cast<const uint16_t*>(a.k) + off);
    } else {
      k0 = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.k) + off);
      k1 = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.k) + off + 4);
    }
  };
  auto load_v = [&](int blk, int w, int j) -> uint4 {
    const int64_t off = (int64_t)blk * a.vbs + (int64_t)g * a.vhs + (int64_t)r * NC +
                        (int64_t)(4 * grp + j) * a.vts + w * CW;
    if constexpr (BF16 && CW == 8) {
      return load16(static_cast<const uint16_t*>(a.v) + off);
    } else if constexpr (BF16) {
      const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.v) + off);
      return make_uint4(x.x, x.y, 0u, 0u);
    } else {
      return *reinterpret_cast<const uint4*>(static_cast<const float*>(a.v) + off);
    }
  };

  // K/V fragments of one page (EARLY: all of them, loaded ahead of use).
  struct PageRegs {
    uint4 kr[EARLY ? NQ : 1][2], vr[EARLY ? NG : 1][4];
  };
  auto issue = [&](int i, PageRegs& R) {
    if constexpr (EARLY) {
      const int blk = __builtin_amdgcn_readlane(my_blk, i);
      const int vs = TIER ? __builtin_amdgcn_readlane(my_vs, i) : -1;
      if (TIER && vs >= 0 && a.hot_k) {
        // KV tier, resident slice: K rows at [16][D] of slice vs, the same fragments
        const int64_t row0 = (int64_t)vs * kPage;
        if constexpr (KT) {
#pragma unroll
          for (int c = 0; c < NQ; ++c)
            R.kr[c][0] = load16(static_cast<const uint16_t*>(a.hot_k) +
                                (row0 + 4 * c + grp) * DQK + 8 * r);
        } else {
#pragma unroll
          for (int c = 0; c < NQ; ++c) {
            const int64_t off = (row0 + r) * DQK + 32 * c + 8 * grp;
            if constexpr (BF16) {
              R.kr[c][0] = load16(static_cast<const uint16_t*>(a.hot_k) + off);
            } else {
              const float* src = static_cast<const float*>(a.hot_k) + off;
              R.kr[c][0] = *reinterpret_cast<const uint4*>(src);
              R.kr[c][1] = *reinterpret_cast<const uint4*>(src + 4);
            }
          }
        }
      } else if constexpr (KT) {  // instruction c: rows 4c + grp, 16 bytes at dims 8r
#pragma unroll
        for (int c = 0; c < NQ; ++c)
          R.kr[c][0] = load16(static_cast<const uint16_t*>(a.k) + (int64_t)blk * a.kbs +
                              (int64_t)(4 * c + grp) * a.kts + (int64_t)g * a.khs + 8 * r);
      } else {
#pragma unroll
        for (int c = 0; c < NQ; ++c) load_k(blk, c, R.kr[c][0], R.kr[c][1]);
      }
      if (TIER && vs >= 0) {  // the page's V slice is resident: [16][Dv] at slice vs
#pragma unroll
        for (int w = 0; w < NG; ++w)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int64_t off = ((int64_t)vs * kPage + 4 * grp + j) * DV + (int64_t)r * NC + w * CW;
            if constexpr (BF16 && CW == 8) {
              R.vr[w][j] = load16(static_cast<const uint16_t*>(a.hot) + off);
            } else if constexpr (BF16) {
              const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.hot) + off);
              R.vr[w][j] = make_uint4(x.x, x.y, 0u, 0u);
            } else {
              R.vr[w][j] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.hot) + off);
            }
          }
      } else {
#pragma unroll
        for (int w = 0; w < NG; ++w)
#pragma unroll
          for (int j = 0; j < 4; ++j) R.vr[w][j] = load_v(blk, w, j);
      }
    }
  };
  auto compute = [&](int i, const PageRegs& R) {
    const int lp = __builtin_amdgcn_readlane(my_lp, i);
    const int blk = __builtin_amdgcn_readlane(my_blk, i);
    const int valid = min(kPage, L - lp * kPage);  // tokens of this page before L

    // ---- S^T = K Q^T -------------------------------------------------------------------
    float4v sacc = {0.f, 0.f, 0.f, 0.f};
    uint4 kt[KT ? NQ : 1];
    if constexpr (KT) {
      // Row t, 16-byte piece k of the page sits at slot 17 t + k of the wave's tile: the
      // padding puts the 16 lanes that write one row, and the 16 lanes that read one piece
      // of 16 rows, on 16 different 4-bank groups; each lane's slots differ by constants.
      // The wave's LDS operations run in order; the fences keep the compiler from moving
      // one lane's accesses across another lane's (the last page's reads, these writes).
      uint4* tile = reinterpret_cast<uint4*>(ktile + (threadIdx.x >> 6) * kt_stride);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      uint4* wr = tile + 17 * grp + r;  // row 4c + grp, piece r
#pragma unroll
      for (int c = 0; c < NQ; ++c) wr[68 * c] = R.kr[c][0];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint4* rd = tile + 17 * r + grp;  // row r, piece 4c + grp
#pragma unroll
      for (int c = 0; c < NQ; ++c) kt[c] = rd[4 * c];
    }
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      uint4 x0, x1, khi, klo, qh, ql;
      if constexpr (KT) {
        x0 = kt[c];
      } else if constexpr (EARLY) {
        x0 = R.kr[c][0];
        x1 = R.kr[c][1];
      } else {
        load_k(blk, c, x0, x1);
      }
      if constexpr (BF16) {
        khi = x0;
      } else {
        const float x[8] = {__uint_as_float(x0.x), __uint_as_float(x0.y), __uint_as_float(x0.z),
                            __uint_as_float(x0.w), __uint_as_float(x1.x), __uint_as_float(x1.y),
                            __uint_as_float(x1.z), __uint_as_float(x1.w)};
        split8(x, khi, klo);
      }
      if constexpr (QREG) {
        qh = qhi[c];
        ql = qlo[c];
      } else {
        qh = ql = make_uint4(0, 0, 0, 0);
        if (hvalid) load_frag8<BF16>(a.q, qrow + 32 * c + 8 * grp, qh, ql);
      }
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(khi), as_bf16x8(qh), sacc, 0, 0, 0);
      if constexpr (!BF16) {
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(klo), as_bf16x8(qh), sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(khi), as_bf16x8(ql), sacc, 0, 0, 0);
      }
    }

    // ---- online softmax: lane holds head r, tokens 4grp .. 4grp+3 ----------------------
    float z[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * grp + j;
      z[j] = t < valid ? sacc[j] * a.sl2 : -INFINITY;
    }
    const float m_loc = wave_max4(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
    const float m_new = fmaxf(m_run, m_loc);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? exp2f(m_run - m_new) : 1.f;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = live ? exp2f(z[j] - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum4(p[0] + p[1] + p[2] + p[3]);
    m_run = m_new;

    // P as the A operand (head r, tokens 4grp + j), bf16 hi + lo.
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ph[j] = f2bf(p[j]);
      pl[j] = f2bf(p[j] - __uint_as_float(ph[j] << 16));
    }
    const short4v Ph = as_short4(pack2(ph[0], ph[1]), pack2(ph[2], ph[3]));
    const bf16x8 PP = as_bf16x8(make_uint4(pack2(ph[0], ph[1]), pack2(ph[2], ph[3]),
                                           pack2(pl[0], pl[1]), pack2(pl[2], pl[3])));

    // Rescale the output rows (heads 4grp + j) by their alpha.
    float al[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) al[j] = __shfl(alpha, 4 * grp + j, 64);
    if (__ballot(alpha != 1.f)) {  // skipped once no head's running max moves
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[c][j] *= al[j];
      }
    }

    // ---- O += P V ------------------------------------------------------------------------
    const bool tail = valid < kPage;
#pragma unroll
    for (int w = 0; w < NG; ++w) {
      uint32_t vh[4][4], vl[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 x;
        if constexpr (EARLY) {
          x = R.vr[w][j];
        } else {
          x = load_v(blk, w, j);
        }
        if (tail && 4 * grp + j >= valid) x = make_uint4(0u, 0u, 0u, 0u);  // unwritten slots
        if constexpr (BF16) {
          vh[j][0] = x.x; vh[j][1] = x.y; vh[j][2] = x.z; vh[j][3] = x.w;
        } else {
          const float xs[8] = {__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                               __uint_as_float(x.w), 0.f, 0.f, 0.f, 0.f};
          uint4 hh, ll;
          split8(xs, hh, ll);
          vh[j][0] = hh.x; vh[j][1] = hh.y; vh[j][2] = 0u; vh[j][3] = 0u;
          vl[j][0] = ll.x; vl[j][1] = ll.y; vl[j][2] = 0u; vl[j][3] = 0u;
        }
      }
#pragma unroll
      for (int cc = 0; cc < CW; ++cc) {
        const int c = w * CW + cc;
        const int wd = cc >> 1;
        const bool hiw = cc & 1;
        uint32_t e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = hiw ? (vh[j][wd] >> 16) : (vh[j][wd] & 0xffffu);
        // one K=32 MFMA: k = 8grp + i pairs token 4grp + (i & 3) with the hi (i < 4) or
        // lo part of P, and V's 4 values repeat, so it adds (P_hi + P_lo) V
        const uint32_t v01 = pack2(e[0], e[1]), v23 = pack2(e[2], e[3]);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(PP, as_bf16x8(make_uint4(v01, v23, v01, v23)),
                                                         acc[c], 0, 0, 0);
        if constexpr (!BF16) {
          uint32_t f[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) f[j] = hiw ? (vl[j][wd] >> 16) : (vl[j][wd] & 0xffffu);
          const short4v Vl = as_short4(pack2(f[0], f[1]), pack2(f[2], f[3]));
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Ph, Vl, acc[c], 0, 0, 0);
        }
      }
    }
  };

  for (int b0 = 0; b0 < total; b0 += 64) {
    const int np = min(64, total - b0);
    const int e = first + stride * (b0 + lane);
    if (b0 > 0)
      sel_lp = list ? list[min(e, count - 1)] : (a.sel ? a.sel[srow + min(e, a.b_max - 1)] : e);
    set_batch(np, e);
    if constexpr (EARLY && PIPE) {
      // Two register sets: page i + 1's loads are in flight while page i is computed.
      PageRegs A, B;
      issue(0, A);
      for (int i = 0; i < np; i += 2) {
        if (i + 1 < np) issue(i + 1, B);
        compute(i, A);
        if (i + 1 >= np) break;
        if (i + 2 < np) issue(i + 2, A);
        compute(i + 1, B);
      }
    } else {
      PageRegs A;
      for (int i = 0; i < np; ++i) {
        issue(i, A);
#if PSD_ATTN_KV_TOGETHER
        // Whole-unit workgroups: keep every load of the page ahead of its first use. Left
        // alone, the scheduler sinks the V loads below the QK products into K's registers,
        // and each page costs two dependent memory round trips instead of one (measured:
        // 0.7 us off the ragged batch step; the split-K form is faster without it).
        if constexpr (EARLY && UNIT) __builtin_amdgcn_sched_barrier(0);
#endif
        compute(i, A);
      }
    }
  }

  if constexpr (UNIT) {
    // Combine the waves: M = max m_w, out = sum acc_w 2^(m_w - M) / sum l_w 2^(m_w - M).
    // A wave without pages has m = -inf, l = 0 and acc = 0 and weighs nothing.
    before_combine();
    extern __shared__ float ush[];  // acc [NWS][G][DV] | (m, l) [NWS][16]
    float2* lml = reinterpret_cast<float2*>(ush + NWS * a.G * DV);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = 4 * grp + j;
      if (hh < a.G) {
        float* dst = ush + (wave * a.G + hh) * DV + r * NC;
#pragma unroll
        for (int c = 0; c < NC; c += 4)
          *reinterpret_cast<float4*>(dst + c) =
              make_float4(acc[c][j], acc[c + 1][j], acc[c + 2][j], acc[c + 3][j]);
      }
    }
    if (grp == 0 && hvalid) lml[wave * 16 + head] = make_float2(m_run, l_run);
    __syncthreads();
    float* out = a.out + ((int64_t)s * a.Hq + g * a.G) * DV;
    for (int t = threadIdx.x; t < a.G * DV; t += 64 * NWS) {
      const int h = t / DV, d = t - h * DV;
      if (count == 0) {
        out[t] = __builtin_nanf("");
        continue;
      }
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWS; ++w) M = fmaxf(M, lml[w * 16 + h].x);
      float l = 0.f, o = 0.f;
#pragma unroll
      for (int w = 0; w < NWS; ++w) {
        const float2 ml = lml[w * 16 + h];
        const float wt = exp2f(ml.x - M);
        l += ml.y * wt;
        o += ush[(w * a.G + h) * DV + d] * wt;
      }
      out[t] = o / l;
    }
    return;
  }

  // ---- partials: acc rows are heads 4grp + j, columns d = r*NC + c ----------------------
  const int64_t ubase = (int64_t)s * a.Hq + g * a.G;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hh = hw * 16 + 4 * grp + j;
    if (hh < a.G) {
      float* dst = a.pacc + ((ubase + hh) * a.nsplit + split) * DV + r * NC;
#pragma unroll
      for (int c = 0; c < NC; c += 4)
        *reinterpret_cast<float4*>(dst + c) =
            make_float4(acc[c][j], acc[c + 1][j], acc[c + 2][j], acc[c + 3][j]);
    }
  }
  if (grp == 0 && hvalid) a.pml[(ubase + head) * a.nsplit + split] = make_float2(m_run, l_run);
}

// KT: wave w's K tile is at byte kt_off + w * kt_stride of the dynamic LDS.
template <bool BF16, int DQK, int DV, int WAVES, int MIN_WAVES_PER_SIMD, int NWS = 0,
          bool TIER = false, bool KT = false>
__global__ __launch_bounds__(64 * (NWS > 0 ? NWS : WAVES))
__attribute__((amdgpu_waves_per_eu(MIN_WAVES_PER_SIMD))) void attn_kernel(AttnArgs a,
                                                                           int kt_off,
                                                                           int kt_stride) {
  extern __shared__ unsigned char kdyn[];
  unsigned char* ktile = KT ? kdyn + kt_off : nullptr;
  if constexpr (NWS > 0)
    attn_body<BF16, DQK, DV, WAVES, NWS, NoHook, TIER, KT>(a, 0, blockIdx.x, blockIdx.y,
                                                           nullptr, 0, NoHook(), ktile,
                                                           kt_stride);
  else
    attn_body<BF16, DQK, DV, WAVES, NWS, NoHook, TIER, KT>(a, blockIdx.x, blockIdx.y,
                                                           blockIdx.z, nullptr, 0, NoHook(),
                                                           ktile, kt_stride);
}

}  // namespace
}  // namespace psd
