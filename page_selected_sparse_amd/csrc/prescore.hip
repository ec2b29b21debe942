// Certified selection for many-head groups (G a multiple of 16, bf16).
//
// The exact page bound (EntmaxKV README, "Two selection strategies": a Quest-style
// upper bound from the page key min/max; LOCKS README, "How it works": many-head (MLA)
// scores max-unioned over the query heads) costs 2 G D fp64 FMAs per page, which for
// G = 128, D = 576 makes the fp64 ALU, not HBM, the bound. Here the bound is first
// computed approximately on bf16 MFMAs, with a proven error bound, and the fp64 bound
// is only evaluated where the approximation cannot decide:
//
//   UB_h(p) = sum_d q+_hd kmax_pd + q-_hd kmin_pd = [Q+ | Q-] . [Kmax ; Kmin]
//
// is a contraction over k = 2D whose operands are bf16 values: every product is exact in
// fp32. Chains of at most C MFMAs (32 products each; the even and the odd k blocks of
// each run of 2C form two chains) accumulate from zero, and each chain's fp32 result is
// added into a running fp32 sum (one sum per (head, page)). With K k blocks there are at
// most 2 ceil(K / 2C) <= K/C + 1 chains, so every product passes a bounded number of
// roundings: at most 33 C inside its chain (any summation order inside an MFMA, faithful
// rounding: unit 2^-23) and K/C + 1 in the sum (2^-24):
//   |UB~ - UB| <= (gamma_33C(2^-23) + gamma_{K/C+1}(2^-24)(1 + ...)) sum_d |q_hd||c_pd|
//              <= 1.6e-5 * ||q_h||_1 * M_p + tiny          (C = 4, K <= 36 k blocks)
// with M_p the largest |statistic| of the page record and gamma_n(u) = n u / (1 - n u).
// The group score error is bounded by the same expression with max_h ||q_h||_1.
//
// certify_kernel then ranks exactly: with L_p = S~_p - e_p and U_p = S~_p + e_p,
//   page p is certainly kept     if L_p > V     (V = the (b-1)-th largest U),
//   page p is certainly dropped  if U_p < T     (T = the (b-2)-th largest L),
// and the pages in between are rescored with the exact sequential fp64 bound (the same
// arithmetic as the scoring kernel and the oracle); the remaining b-2-|kept| slots go to
// the best of them by (exact score desc, page asc). The result is the exact top-(b-2).
#include <type_traits>

#include "meta_core.h"
#include "psd_device.h"
#include "psd_launch.h"

namespace psd {
namespace {

struct PreArgs {
  const uint16_t* q;          // [B, Hq, D] bf16
  const unsigned char* meta;  // page-major statistics records
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* budgets;
  float* approx;  // [unit][max_inner] approximate group score of inner page i (page i + 1)
  float* pmax;    // [unit][max_inner] largest |statistic| of that page's record
  float* second;  // [unit][max_inner] largest approximate head score outside the leading tile
  int32_t* best;  // [unit][max_inner] 16-head tile holding the largest approximate score
  double* qnorm;  // [unit] max over the group's heads of ||q_h||_1
  int32_t* sel;
  int32_t* cnt;
  int Hq, Hkv, G, max_pages, b_max, num_blocks, max_inner, tiles_per_wg;
  // tail refresh in the certify launch (decode step): workgroups z = 1, one per unit
  void* meta_w = nullptr;
  const void* k = nullptr;
  int64_t kbs = 0, kts = 0, khs = 0;
};

struct UnitN {
  int n, b, kp;
  bool trivial;
};

__device__ __forceinline__ UnitN unit_n(const PreArgs& a, int s) {
  UnitN u;
  u.n = ceil_div(a.lens[s], kPage);
  u.b = effective_budget(u.n, a.budgets[s]);
  u.kp = u.b - 2;
  u.trivial = u.n <= u.b || u.kp <= 0 || u.b > a.b_max;
  return u;
}

// Every row entry except the ranked winners (see the scoring kernel of select.hip).
template <int NT>
__device__ void write_header(const PreArgs& a, int unit, const UnitN& u) {
  const int tid = threadIdx.x;
  int32_t* row = a.sel + (int64_t)unit * a.b_max;
  if (u.b > a.b_max) {
    for (int i = tid; i < a.b_max; i += NT) row[i] = -1;
    if (tid == 0) a.cnt[unit] = -1;
    return;
  }
  if (u.n <= u.b) {
    for (int i = tid; i < a.b_max; i += NT) row[i] = i < u.n ? i : -1;
    if (tid == 0) a.cnt[unit] = u.n;
    return;
  }
  for (int i = u.b + tid; i < a.b_max; i += NT) row[i] = -1;
  if (tid == 0) {
    a.cnt[unit] = u.b;
    row[0] = 0;
    row[u.b - 1] = u.n - 1;
  }
}

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4p;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;

__device__ __forceinline__ bf16x8 as_bf8(uint4 w) {
  u32x4p v = {w.x, w.y, w.z, w.w};
  return __builtin_bit_cast(bf16x8, v);
}

// Two 16-byte LDS reads and the wait for them, as one asm block (the compiler would
// otherwise make them wait for loads still streaming into other stages).
__device__ __forceinline__ void lds2(uint32_t a0, uint32_t a1, uint4& x0, uint4& x1) {
  u32x4p r0, r1;
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(a0), "v"(a1)
      : "memory");
  x0 = make_uint4(r0.x, r0.y, r0.z, r0.w);
  x1 = make_uint4(r1.x, r1.y, r1.z, r1.w);
}

// Two 16-byte LDS reads at base + O0 and base + O1 (immediate offsets) and the wait for
// them, as one asm block.
template <int O0, int O1>
__device__ __forceinline__ void lds2i(uint32_t base, uint4& x0, uint4& x1) {
  u32x4p r0, r1;
  asm volatile(
      "ds_read_b128 %0, %2 offset:%3\n\t"
      "ds_read_b128 %1, %2 offset:%4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(base), "n"(O0), "n"(O1)
      : "memory");
  x0 = make_uint4(r0.x, r0.y, r0.z, r0.w);
  x1 = make_uint4(r1.x, r1.y, r1.z, r1.w);
}

// The same two reads without the wait: the registers are defined once a later
// lgkm_wait2 on them has run (LDS reads complete in order).
template <int O0, int O1>
__device__ __forceinline__ void lds2i_issue(uint32_t base, u32x4p& r0, u32x4p& r1) {
  asm volatile(
      "ds_read_b128 %0, %2 offset:%3\n\t"
      "ds_read_b128 %1, %2 offset:%4"
      : "=&v"(r0), "=&v"(r1)
      : "v"(base), "n"(O0), "n"(O1)
      : "memory");
}
// Waits until at most N LDS / scalar-memory operations are outstanding; r0 and r1 are
// tied to the wait so that no use of them can move above it.
template <int N>
__device__ __forceinline__ void lgkm_wait2(u32x4p& r0, u32x4p& r1) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(r0), "+v"(r1) : "n"(N));
}

template <int KB, int KPW, typename F>
__device__ __forceinline__ void for_kb(F&& f) {
  if constexpr (KB < KPW) {
    f(std::integral_constant<int, KB>{});
    for_kb<KB + 2, KPW>(f);
  }
}

// Waits until at most n vector memory operations of this wave are outstanding, n <= 40.
__device__ __forceinline__ void wait_vm_upto40(int n) {
#define PSD_W(N) case N: __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70); break;
  switch (n) {
    PSD_W(0) PSD_W(1) PSD_W(2) PSD_W(3) PSD_W(4) PSD_W(5) PSD_W(6) PSD_W(7) PSD_W(8) PSD_W(9)
    PSD_W(10) PSD_W(11) PSD_W(12) PSD_W(13) PSD_W(14) PSD_W(15) PSD_W(16) PSD_W(17)
    PSD_W(18) PSD_W(19) PSD_W(20) PSD_W(21) PSD_W(22) PSD_W(23) PSD_W(24) PSD_W(25)
    PSD_W(26) PSD_W(27) PSD_W(28) PSD_W(29) PSD_W(30) PSD_W(31) PSD_W(32) PSD_W(33)
    PSD_W(34) PSD_W(35) PSD_W(36) PSD_W(37) PSD_W(38) PSD_W(39)
    default: __builtin_amdgcn_s_waitcnt(0xF70); break;
  }
#undef PSD_W
}

#ifndef PSD_PRE_STAGES
#define PSD_PRE_STAGES 3
#endif
constexpr int kPreStages = PSD_PRE_STAGES;
#ifndef PSD_PRE_CHAIN
#define PSD_PRE_CHAIN 4
#endif
// k blocks accumulated inside one MFMA chain before joining the fp32 sum (even)
constexpr int kPreChain = PSD_PRE_CHAIN;
#ifndef PSD_PRE_KS576
#define PSD_PRE_KS576 1  // contraction halves per head tile at D = 576
#endif

// One workgroup scores tiles of 16 candidate pages of one unit. Wave w owns query heads
// 16 (w % HT) .. +15 and the k blocks of half w / HT (KS halves) of the contraction, and
// keeps those [q+ | q-] MFMA fragments in registers; with KS = 2 the second half's fp32
// partial sums are added to the first's through LDS. A tile's statistics records are
// staged once in LDS (rows padded to an odd number of 16-byte pieces so that fragment
// reads are conflict-free), three tiles deep.
template <int D, int HT, int KS>
__global__ __launch_bounds__(64 * HT * KS) void prescore_kernel(PreArgs a) {
  constexpr int NCH = D / 32;              // 128-byte lines per record
  constexpr int NKB = 2 * NCH;             // 32-wide k blocks: (chunk, min | max)
  constexpr int KPW = NKB / KS;            // k blocks per wave
  constexpr int SLP = NCH * 8 + 1;         // padded 16-byte pieces per staged row
  constexpr int NLD = (16 * SLP + 63) / 64;  // 1 KB loads per tile
  constexpr int STG = NLD * 64;            // uint4 per stage
  constexpr int WAVES = HT * KS;
  constexpr int NT = 64 * WAVES;
  static_assert(NKB % KS == 0 && KPW % 2 == 0, "k split");
  __shared__ uint4 stage[kPreStages * STG];
  __shared__ int32_t blk_of[16 * 64];  // physical block of each page of the workgroup
  __shared__ float wmax[2][HT][16];
  __shared__ uint32_t wabs[2][WAVES][16];
  __shared__ float4 psum[KS > 1 ? HT : 1][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ht = wave % HT, kh = wave / HT;
  const int r = lane & 15, grp = lane >> 4;
  const int g = blockIdx.y, s = blockIdx.z;
  const int unit = s * a.Hkv + g;
  const UnitN u = unit_n(a, s);
  if (blockIdx.x == 0) write_header<NT>(a, unit, u);
  if (u.trivial) return;
  const int inner = u.n - 2;
  const int t0 = blockIdx.x * a.tiles_per_wg;
  const int T = min(a.tiles_per_wg, ceil_div(inner, 16) - t0);
  if (T <= 0) return;
  const int first = 1 + 16 * t0;  // logical page of the first row

  for (int i = tid; i < 16 * T; i += NT)
    blk_of[i] = a.bt[(int64_t)s * a.max_pages + min(first + i, u.n - 2)];

  // [q+ | q-] fragments of head 16 ht + r: k block 2c + h covers dims 32c + 8grp .. +8 of
  // q- (h = 0, paired with the minima) or q+ (h = 1, the maxima).
  const int head = 16 * ht + r;
  const uint16_t* qrow = a.q + ((int64_t)s * a.Hq + g * a.G + head) * D;
  const int kb0 = kh * KPW;
  uint4 qf[KPW];
#pragma unroll
  for (int c2 = 0; c2 < KPW / 2; ++c2) {
    const int c = kb0 / 2 + c2;
    const uint4 w = load16(qrow + 32 * c + 8 * grp);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t neg[4], pos[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // per bf16 half: keep it in q- if its sign bit is set, else in q+
      const uint32_t sgn = ((ws[i] >> 15) & 1u) * 0xffffu | ((ws[i] >> 31) & 1u) * 0xffff0000u;
      neg[i] = ws[i] & sgn;
      pos[i] = ws[i] & ~sgn;
    }
    qf[2 * c2] = make_uint4(neg[0], neg[1], neg[2], neg[3]);
    qf[2 * c2 + 1] = make_uint4(pos[0], pos[1], pos[2], pos[3]);
  }
  if (blockIdx.x == 0) {
    // max_h ||q_h||_1 of the group, from the fragments: every dim sits in exactly one
    // of q+ / q- (the other is zero); fp64 sums of exact terms, combined over the four
    // lanes of a head, the k halves and the head tiles
    __shared__ double qn[KS][HT * 16];
    double part = 0.0;
#pragma unroll
    for (int kb = 0; kb < KPW; ++kb) {
      const uint32_t ws[4] = {qf[kb].x, qf[kb].y, qf[kb].z, qf[kb].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t h = (ws[i >> 1] >> (16 * (i & 1))) & 0x7fffu;
        part += (double)__uint_as_float(h << 16);
      }
    }
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    if (grp == 0) qn[kh][head] = part;
    __syncthreads();
    if (tid == 0) {
      double best = 0.0;
      for (int h = 0; h < HT * 16; ++h) {
        double v = 0.0;
        for (int k = 0; k < KS; ++k) v += qn[k][h];
        best = fmax(best, v);
      }
      a.qnorm[unit] = best;
    }
  }
  __syncthreads();  // blk_of

  const int64_t rec_bytes = NCH * 128;
  const int my_loads = (NLD - wave + WAVES - 1) / WAVES;
  constexpr int MLW0 = (NLD + WAVES - 1) / WAVES;  // most load instructions per wave and tile
  auto issue = [&](int t, int st) {
    // every block id first (one LDS round trip), then the loads
    int blk[MLW0], piece[MLW0];
#pragma unroll
    for (int j = 0; j < MLW0; ++j) {
      const int ins = wave + j * WAVES;
      const int slot = ins * 64 + lane;
      int row = slot / SLP, pc = slot - row * SLP;
      if (row >= 16) {
        row = 15;
        pc = 0;
      }
      if (pc == SLP - 1) pc = 0;
      piece[j] = pc;
      blk[j] = ins < NLD ? blk_of[16 * t + row] : 0;
    }
#pragma unroll
    for (int j = 0; j < MLW0; ++j) {
      const int ins = wave + j * WAVES;
      if (ins < NLD) {
        const unsigned char* src =
            a.meta + ((int64_t)blk[j] * a.Hkv + g) * rec_bytes + (int64_t)piece[j] * 16;
        __builtin_amdgcn_global_load_lds(
            src, (__attribute__((address_space(3))) void*)(stage + st * STG + ins * 64), 16, 0, 0);
      }
    }
  };
  // combines tile t's per-wave head maxima and writes its pages' results
  float* approx = a.approx + (int64_t)unit * a.max_inner;
  float* pmax = a.pmax + (int64_t)unit * a.max_inner;
  float* second = a.second + (int64_t)unit * a.max_inner;
  int32_t* best = a.best + (int64_t)unit * a.max_inner;
  auto finish = [&](int t) {
    if (tid < 16) {  // wave 0 (every wave contributed its share of the record maxima)
      const int i = 16 * (t0 + t) + tid;  // inner page index
      if (i < inner) {
        // the leading 16-head tile and the best of the other tiles
        float m = wmax[t & 1][0][tid], m2 = -__builtin_inff();
        int arg = 0;
#pragma unroll
        for (int w = 1; w < HT; ++w) {
          const float b = wmax[t & 1][w][tid];
          if (b > m) {
            m2 = m;
            m = b;
            arg = w;
          } else {
            m2 = fmaxf(m2, b);
          }
        }
        approx[i] = m;
        second[i] = m2;
        best[i] = arg;
        uint32_t bits = wabs[t & 1][0][tid];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) bits = max(bits, wabs[t & 1][w][tid]);
        pmax[i] = bits > 0x7f80u ? __builtin_inff() : __uint_as_float(bits << 16);
      }
    }
  };

  // tiles in flight ahead of the one computed (bounded so that the vmcnt wait fits)
  constexpr int MLW = (NLD + WAVES - 1) / WAVES;  // most loads one wave issues per tile
  constexpr int AH0 = 39 / MLW < 1 ? 1 : 39 / MLW;
  constexpr int AH = kPreStages - 1 < AH0 ? kPreStages - 1 : AH0;
  constexpr int NST = AH + 1;  // stages used
  const uint32_t sbase = (uint32_t)(uintptr_t)stage;
  for (int j = 0; j < AH && j < T; ++j) issue(j, j);
  for (int t = 0; t < T; ++t) {
    // tile t has landed once only the tiles issued after it are outstanding
    wait_vm_upto40(min(AH - 1, T - 1 - t) * my_loads);
    __syncthreads();  // tile t is in; tile t - 1 is read by every wave; its maxima are in
    if (t + AH < T) issue(t + AH, (t + AH) % NST);
    if (t > 0) finish(t - 1);
    const uint32_t row =
        sbase + (uint32_t)((t % NST) * STG + r * SLP + grp) * 16 + 64 * kb0;
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    float4v chain = {0.f, 0.f, 0.f, 0.f}, chain2 = {0.f, 0.f, 0.f, 0.f};
    // the reads of step kb + 2 are in flight while step kb's MFMAs run
    u32x4p ra[2][2];
    lds2i_issue<0, 64>(row, ra[0][0], ra[0][1]);
    for_kb<0, KPW>([&](auto kbc) {
      constexpr int kb = decltype(kbc)::value;
      constexpr int cur = (kb / 2) & 1;
      if constexpr (kb + 2 < KPW) {
        lds2i_issue<64 * (kb + 2), 64 * (kb + 3)>(row, ra[cur ^ 1][0], ra[cur ^ 1][1]);
        lgkm_wait2<2>(ra[cur][0], ra[cur][1]);
      } else {
        lgkm_wait2<0>(ra[cur][0], ra[cur][1]);
      }
      const uint4 x0 = make_uint4(ra[cur][0].x, ra[cur][0].y, ra[cur][0].z, ra[cur][0].w);
      const uint4 x1 = make_uint4(ra[cur][1].x, ra[cur][1].y, ra[cur][1].z, ra[cur][1].w);
      // two independent chains (even and odd k blocks), each of up to kPreChain MFMAs,
      // so that consecutive MFMAs do not wait on each other; each chain then joins the
      // fp32 sum (the same number of additions as one chain per kPreChain k blocks)
      if constexpr (kb % (2 * kPreChain) == 0) {
        chain = float4v{0.f, 0.f, 0.f, 0.f};
        chain2 = float4v{0.f, 0.f, 0.f, 0.f};
      }
      chain = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(x0), as_bf8(qf[kb]), chain, 0, 0, 0);
      chain2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(x1), as_bf8(qf[kb + 1]), chain2, 0, 0, 0);
      if constexpr ((kb + 2) % (2 * kPreChain) == 0 || kb + 2 >= KPW) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[i] += chain[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[i] += chain2[i];
      }
      // keep each step's reads, MFMAs and adds together (short register live ranges)
      __builtin_amdgcn_sched_barrier(0);
    });
    {
      // The largest |statistic| of each page's record, shared out: wave w takes the k
      // blocks [w per, (w + 1) per) of the staged tile (lane (r, grp) holds 16 bytes of
      // page r's block), after its MFMA stream, whose LDS reads have all completed.
      constexpr int PER = (NKB + WAVES - 1) / WAVES;
      const unsigned char* tb = reinterpret_cast<const unsigned char*>(stage) +
                                ((t % NST) * STG + r * SLP + grp) * 16;
      const int kb0w = __builtin_amdgcn_readfirstlane(wave) * PER;
      u16x2 amax = {0, 0};
      for (int kb = kb0w; kb < NKB && kb < kb0w + PER; ++kb) {
        const uint4 x = *reinterpret_cast<const uint4*>(tb + 64 * kb);
        const uint32_t ws[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          amax = __builtin_elementwise_max(amax, __builtin_bit_cast(u16x2, ws[i] & 0x7fff7fffu));
      }
      uint32_t m = amax.x > amax.y ? amax.x : amax.y;
      m = max(m, (uint32_t)__shfl_xor((int)m, 16, 64));
      m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
      if (grp == 0) wabs[t & 1][wave][r] = m;
    }
    if constexpr (KS > 1) {
      if (kh == 1) psum[ht][lane] = make_float4(sum[0], sum[1], sum[2], sum[3]);
      __syncthreads();
      if (kh == 0) {
        const float4 o = psum[ht][lane];
        sum[0] += o.x;
        sum[1] += o.y;
        sum[2] += o.z;
        sum[3] += o.w;
      }
    }
    // lane (r, grp) holds pages 4grp + i for head r: max over the 16 heads of the wave;
    // a non-finite sum (overflow) is made +inf so that the page can never be dropped
    // on an approximate score.
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sum[i];
        if (!__builtin_isfinite(v)) v = __builtin_inff();
        v = row_max16(v);
        if (r == 0) wmax[t & 1][ht][4 * grp + i] = v;
      }
    }
  }
  __syncthreads();
  finish(T - 1);
}

// ---- certification and exact ranking -------------------------------------------------------

struct SelScr {
  uint32_t hist[256];
  int wave_cnt[16];
  uint64_t wand[16], wor[16];
  int digit, k;
  bool done;
  double red[16];
};

template <int NT>
__device__ __forceinline__ int excl_sum(int x, SelScr& sc, int& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_scan_incl(x);
  if (lane == 63) sc.wave_cnt[w] = incl;
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int c = sc.wave_cnt[i];
    off += i < w ? c : 0;
    total += c;
  }
  __syncthreads();
  return off + incl - x;
}

// The K-th largest key (1 <= K <= N) of keys[0..N), exactly: radix select over 8-bit
// digits, starting at the highest bit where two keys differ (the bits every key shares
// are skipped) and resolving every bit below it. Equal digits met in a row by one thread
// are counted with one atomic.
template <int NT>
__device__ uint64_t kth_key(const uint64_t* keys, int N, int K, SelScr& sc) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint64_t kand = ~0ull, kor = 0;
  for (int i = tid; i < N; i += NT) {
    kand &= keys[i];
    kor |= keys[i];
  }
  wave_and_or64(kand, kor);
  if (lane == 0) {
    sc.wand[w] = kand;
    sc.wor[w] = kor;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    kand &= sc.wand[i];
    kor |= sc.wor[i];
  }
  __syncthreads();  // sc.wand / sc.wor are rewritten by the next call
  const uint64_t diff = kand ^ kor;
  if (diff == 0) return kand;  // every key is equal
  const int hb = 63 - __clzll(diff);
  uint64_t mask = hb == 63 ? 0ull : ~((2ull << hb) - 1ull);
  uint64_t prefix = kand & mask;
  int k = K;
  for (int sh = hb - 7;; sh -= 8) {
    const int lo = sh > 0 ? sh : 0;
    const uint64_t dmask = (1ull << (sh + 8 - lo)) - 1ull;
    for (int i = tid; i < 256; i += NT) sc.hist[i] = 0;
    __syncthreads();
    int run_d = -1, run_c = 0;
    for (int i = tid; i < N; i += NT) {
      const uint64_t key = keys[i];
      if ((key & mask) == prefix) {
        const int dg = (int)((key >> lo) & dmask);
        if (dg == run_d) {
          ++run_c;
        } else {
          if (run_c) atomicAdd(&sc.hist[run_d], (uint32_t)run_c);
          run_d = dg;
          run_c = 1;
        }
      }
    }
    if (run_c) atomicAdd(&sc.hist[run_d], (uint32_t)run_c);
    __syncthreads();
    if (tid < 64) {
      const int base = 255 - 4 * tid;
      const int c0 = sc.hist[base], c1 = sc.hist[base - 1], c2 = sc.hist[base - 2],
                c3 = sc.hist[base - 3];
      const int local = c0 + c1 + c2 + c3;
      const int incl = wave_scan_incl(local);
      const int excl = incl - local;
      if (excl < k && k <= incl) {
        int rr = k - excl, dg;
        if (rr <= c0) {
          dg = base;
        } else if (rr <= c0 + c1) {
          rr -= c0;
          dg = base - 1;
        } else if (rr <= c0 + c1 + c2) {
          rr -= c0 + c1;
          dg = base - 2;
        } else {
          rr -= c0 + c1 + c2;
          dg = base - 3;
        }
        sc.digit = dg;
        sc.k = rr;
      }
    }
    __syncthreads();
    prefix |= (uint64_t)sc.digit << lo;
    mask |= dmask << lo;
    k = sc.k;
    __syncthreads();
    if (lo == 0) break;
  }
  return prefix;
}

// The KA-th largest of keysA and the KB-th largest of keysB (same length N) in one radix
// sweep with two histograms: digits start at the highest bit where any two keys of either
// array differ. After max_passes digits it stops with a lower bound of A's and an upper
// bound of B's (exact when every bit was resolved).
template <int NT>
__device__ void kth_key2(const uint64_t* keysA, int KA, const uint64_t* keysB, int KB, int N,
                         SelScr& sc, uint32_t* histB, uint64_t& outA, uint64_t& outB,
                         int max_passes = 8) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint64_t kand = ~0ull, kor = 0;
  for (int i = tid; i < N; i += NT) {
    kand &= keysA[i] & keysB[i];
    kor |= keysA[i] | keysB[i];
  }
  wave_and_or64(kand, kor);
  if (lane == 0) {
    sc.wand[w] = kand;
    sc.wor[w] = kor;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    kand &= sc.wand[i];
    kor |= sc.wor[i];
  }
  __syncthreads();
  const uint64_t diff = kand ^ kor;
  if (diff == 0) {
    outA = outB = kand;
    return;
  }
  const int hb = 63 - __clzll(diff);
  uint64_t mask = hb == 63 ? 0ull : ~((2ull << hb) - 1ull);
  uint64_t pa = kand & mask, pb = pa;
  int ka = KA, kb = KB;
  __shared__ int res[4];
  for (int sh = hb - 7, pass = 0;; sh -= 8, ++pass) {
    const int lo = sh > 0 ? sh : 0;
    const uint64_t dmask = (1ull << (sh + 8 - lo)) - 1ull;
    for (int i = tid; i < 256; i += NT) {
      sc.hist[i] = 0;
      histB[i] = 0;
    }
    __syncthreads();
    int ra = -1, ca = 0, rb = -1, cb = 0;
    for (int i = tid; i < N; i += NT) {
      const uint64_t x = keysA[i], y = keysB[i];
      if ((x & mask) == pa) {
        const int dg = (int)((x >> lo) & dmask);
        if (dg == ra) {
          ++ca;
        } else {
          if (ca) atomicAdd(&sc.hist[ra], (uint32_t)ca);
          ra = dg;
          ca = 1;
        }
      }
      if ((y & mask) == pb) {
        const int dg = (int)((y >> lo) & dmask);
        if (dg == rb) {
          ++cb;
        } else {
          if (cb) atomicAdd(&histB[rb], (uint32_t)cb);
          rb = dg;
          cb = 1;
        }
      }
    }
    if (ca) atomicAdd(&sc.hist[ra], (uint32_t)ca);
    if (cb) atomicAdd(&histB[rb], (uint32_t)cb);
    __syncthreads();
    if (tid < 128) {  // wave 0 resolves A, wave 1 resolves B
      const uint32_t* h = tid < 64 ? sc.hist : histB;
      const int k = tid < 64 ? ka : kb;
      const int l = tid & 63;
      const int base = 255 - 4 * l;
      const int c0 = h[base], c1 = h[base - 1], c2 = h[base - 2], c3 = h[base - 3];
      const int local = c0 + c1 + c2 + c3;
      const int incl = wave_scan_incl(local);
      const int excl = incl - local;
      if (excl < k && k <= incl) {
        int rr = k - excl, dg;
        if (rr <= c0) {
          dg = base;
        } else if (rr <= c0 + c1) {
          rr -= c0;
          dg = base - 1;
        } else if (rr <= c0 + c1 + c2) {
          rr -= c0 + c1;
          dg = base - 2;
        } else {
          rr -= c0 + c1 + c2;
          dg = base - 3;
        }
        res[(tid >> 6) * 2] = dg;
        res[(tid >> 6) * 2 + 1] = rr;
      }
    }
    __syncthreads();
    pa |= (uint64_t)res[0] << lo;
    pb |= (uint64_t)res[2] << lo;
    mask |= dmask << lo;
    ka = res[1];
    kb = res[3];
    __syncthreads();
    if (lo == 0) break;
    if (pass + 1 == max_passes) {
      // stop early: A is bounded below by its prefix with zero low bits, B above by its
      // prefix with all low bits set
      outA = pa;
      outB = pb | ~mask;
      return;
    }
  }
  outA = pa;
  outB = pb;
}

struct CertArgs {
  PreArgs p;
  int D;
};

// Exact fp64 bound of one logical page for one head: the sum over ascending d of the exact
// product q_d * (q_d >= 0 ? kmax_d : kmin_d) (the sequential definition, bit for bit),
// returned as its order-preserving key. The q row and the page record are
// streamed in chunks of 32 dims, two chunks in flight ahead of the FMA chain.
template <int D>
__device__ uint64_t exact_head_key(const PreArgs& a, int s, int g, int head, int blk) {
  constexpr int NCH = D / 32;
  constexpr int DEPTH = 2;  // chunks in flight; divides NCH
  static_assert(NCH % DEPTH == 0, "chunk ring");
  const uint16_t* qrow = a.q + ((int64_t)s * a.Hq + g * a.G + head) * D;
  const uint16_t* rec =
      reinterpret_cast<const uint16_t*>(a.meta + ((int64_t)blk * a.Hkv + g) * NCH * 128);
  uint4 qb[DEPTH][4], nb[DEPTH][4], xb[DEPTH][4];
  auto load = [&](int c, int slot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qb[slot][j] = load16(qrow + 32 * c + 8 * j);
      nb[slot][j] = load16(rec + 64 * c + 8 * j);
      xb[slot][j] = load16(rec + 64 * c + 32 + 8 * j);
    }
  };
#pragma unroll
  for (int c = 0; c < DEPTH; ++c) load(c, c);
  double acc = 0.0;
  // rolled over rings of DEPTH chunks: each ring computes its chunks in order and refills
  // their slots with the chunks DEPTH ahead
#pragma unroll 1
  for (int c0 = 0; c0 < NCH; c0 += DEPTH) {
#pragma unroll
    for (int slot = 0; slot < DEPTH; ++slot) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t qa[4] = {qb[slot][j].x, qb[slot][j].y, qb[slot][j].z, qb[slot][j].w};
        const uint32_t na[4] = {nb[slot][j].x, nb[slot][j].y, nb[slot][j].z, nb[slot][j].w};
        const uint32_t xa[4] = {xb[slot][j].x, xb[slot][j].y, xb[slot][j].z, xb[slot][j].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t qh = (qa[i >> 1] >> (16 * (i & 1))) & 0xffffu;
          const uint32_t nh = (na[i >> 1] >> (16 * (i & 1))) & 0xffffu;
          const uint32_t xh = (xa[i >> 1] >> (16 * (i & 1))) & 0xffffu;
          // the product q * (q >= 0 ? kmax : kmin), exact, added once per dim
          const double qd = (double)__uint_as_float(qh << 16);
          const uint32_t ch = qd >= 0.0 ? xh : nh;
          acc = __builtin_fma(qd, (double)__uint_as_float(ch << 16), acc);
        }
      }
      if (c0 + slot + DEPTH < NCH) load(c0 + slot + DEPTH, slot);
    }
  }
  return score_key(acc);
}

// One workgroup per ranking unit: certified classification from the approximate scores,
// exact rescoring of the undecided pages, and the exact top-(b-2) written in page order.
template <int D, int NT>
__global__ __launch_bounds__(NT) void certify_kernel(PreArgs a) {
  __shared__ SelScr sc;
  extern __shared__ unsigned char lds[];
  const int tid = threadIdx.x;
  const int g = blockIdx.x, s = blockIdx.y;
  if (blockIdx.z == 1) {  // the unit's tail-page statistics; no ranking reads them
    refresh_tail_page<true>(a.k, a.meta_w, a.bt, a.lens, a.max_pages, s, g, a.Hkv, D, a.kbs,
                            a.kts, a.khs, tid, NT);
    return;
  }
  const int unit = s * a.Hkv + g;
  const UnitN u = unit_n(a, s);
  if (u.trivial) return;
  const int cnt = u.n - 2, kp = u.kp;
  uint64_t* kL = reinterpret_cast<uint64_t*>(lds);        // [cnt] lower-bound keys, then exact
  uint64_t* kU = kL + cnt;                                 // [cnt] upper-bound keys, then R list
  unsigned char* flag = reinterpret_cast<unsigned char*>(kU + cnt);  // [cnt] 1 kept, 2 undecided
  int32_t* rlist = reinterpret_cast<int32_t*>(kU);

  // max_h ||q_h||_1 (written by the scoring stage), rounded up by a relative 2^-40: its
  // fp64 sum of at most 576 exact terms is off by far less
  const double q1 = a.qnorm[unit] * (1.0 + 0x1p-40);
  // relative error factor of the approximate score (see the file comment): a product
  // passes at most 33 faithful fp32 roundings in each MFMA of its chain of kPreChain,
  // then at most (2D/32)/kPreChain + 1 rounded additions into the running sum
  constexpr double u23 = 0x1p-23, u24 = 0x1p-24;
  constexpr double nin = 33.0 * kPreChain;
  constexpr double nout = 2.0 * D / 32.0 / kPreChain + 1.0;
  constexpr double gin = nin * u23 / (1.0 - nin * u23);
  constexpr double gout = nout * u24 / (1.0 - nout * u24);
  const double rel = (gin + gout * (1.0 + gin)) * (1.0 + 0x1p-20);

  const float* approx = a.approx + (int64_t)unit * a.max_inner;
  const float* pmax = a.pmax + (int64_t)unit * a.max_inner;
#pragma unroll 4
  for (int i = tid; i < cnt; i += NT) {
    const double sv = (double)approx[i];
    const double mv = (double)pmax[i];
    double L = -__builtin_inf(), U = __builtin_inf();
    if (__builtin_isfinite(sv) && __builtin_isfinite(mv)) {
      const double e = rel * q1 * mv + fabs(sv) * 0x1p-50 + 0x1p-100;
      L = sv - e;
      U = sv + e;
    }
    kL[i] = score_key(L);
    kU[i] = score_key(U);
  }
  __syncthreads();
  // T: the (b-2)-th largest lower bound or less; V: the (b-1)-th largest upper bound or
  // more (two digits below the first differing bit; looser bounds only leave more pages
  // undecided)
  __shared__ uint32_t histB[256];
  uint64_t T, V;
  kth_key2<NT>(kL, kp, kU, kp + 1, cnt, sc, histB, T, V, 2);
  for (int i = tid; i < cnt; i += NT) flag[i] = kL[i] > V ? 1 : (kU[i] >= T ? 2 : 0);
  __syncthreads();

  // undecided pages in page order (one contiguous segment per thread)
  const int per = ceil_div(cnt, NT);
  const int b0 = min(tid * per, cnt), e0 = min(b0 + per, cnt);
  int nr = 0, ni = 0;
  for (int i = b0; i < e0; ++i) {
    nr += flag[i] == 2;
    ni += flag[i] == 1;
  }
  int total_r, total_i;
  int pos = excl_sum<NT>(nr, sc, total_r);
  excl_sum<NT>(ni, sc, total_i);
  for (int i = b0; i < e0; ++i)
    if (flag[i] == 2) rlist[pos++] = i;
  for (int i = tid; i < total_r; i += NT) kL[i] = 0;
  __syncthreads();

  // Exact keys of the undecided pages (max over heads). A page whose best head outside
  // its leading 16-head tile lies more than 2e below the leading score has its group
  // score inside that tile (every other head's exact bound is below the leader's), so
  // only the tile's 16 heads are rescored; other pages rescore every head, one
  // (page, head) per lane.
  const float* second = a.second + (int64_t)unit * a.max_inner;
  const int32_t* best = a.best + (int64_t)unit * a.max_inner;
  // work lists in LDS: pages rescored at their leading head only, then pages rescored
  // at every head (one list from each end of a total_r-entry array)
  int32_t* lists = reinterpret_cast<int32_t*>(flag + ((cnt + 15) & ~15));  // [total_r]
  __shared__ int nsep, nfull;
  if (tid == 0) nsep = nfull = 0;
  __syncthreads();
  for (int ri = tid; ri < total_r; ri += NT) {
    const int i = rlist[ri];
    const double m1 = (double)approx[i], m2 = (double)second[i];
    const double e = rel * q1 * (double)pmax[i] + fabs(m1) * 0x1p-50 + 0x1p-100;
    if (__builtin_isfinite(m1) && __builtin_isfinite(e) && m2 < m1 - 2.0 * e)
      lists[atomicAdd(&nsep, 1)] = ri;
    else
      lists[total_r - 1 - atomicAdd(&nfull, 1)] = ri;
  }
  __syncthreads();
  const int work = 16 * nsep + nfull * a.G;
  for (int it = tid; it < work; it += NT) {
    int ri, head;
    if (it < 16 * nsep) {
      ri = lists[it >> 4];
      head = 16 * best[rlist[ri]] + (it & 15);
    } else {
      const int f = (it - 16 * nsep) / a.G;
      head = (it - 16 * nsep) - f * a.G;
      ri = lists[total_r - 1 - f];
    }
    const int page = rlist[ri] + 1;
    const int blk = a.bt[(int64_t)s * a.max_pages + page];
    atomicMax(reinterpret_cast<unsigned long long*>(&kL[ri]),
              (unsigned long long)exact_head_key<D>(a, s, g, head, blk));
  }
  __syncthreads();

  // the remaining slots go to the best undecided pages, ties to the lower page
  const int need = kp - total_i;
  if (need > 0 && total_r <= 64) {
    // few undecided pages: one wave ranks them directly by (key desc, page asc)
    if (tid < total_r) {
      const uint64_t key = kL[tid];
      int rank = 0;
      for (int j = 0; j < total_r; ++j) {
        const uint64_t kj = kL[j];
        rank += kj > key || (kj == key && j < tid);
      }
      if (rank < need) flag[rlist[tid]] = 1;
    }
  } else if (need > 0) {
    const uint64_t P = kth_key<NT>(kL, total_r, need, sc);
    // pages strictly above P, then the first `need - above` at P in page order
    int above = 0, at = 0;
    const int rper = ceil_div(total_r, NT);
    const int rb = min(tid * rper, total_r), re = min(rb + rper, total_r);
    for (int i = rb; i < re; ++i) {
      above += kL[i] > P;
      at += kL[i] == P;
    }
    int tot_above, tot_at;
    excl_sum<NT>(above, sc, tot_above);
    const int at_before = excl_sum<NT>(at, sc, tot_at);
    int take = min(max(need - tot_above - at_before, 0), at);
    for (int i = rb; i < re; ++i) {
      bool pick = kL[i] > P;
      if (kL[i] == P && take > 0) {
        pick = true;
        --take;
      }
      if (pick) flag[rlist[i]] = 1;
    }
  }
  __syncthreads();

  // kept pages in page order into row[1 ..]
  int32_t* row = a.sel + (int64_t)unit * a.b_max;
  int nk = 0;
  for (int i = b0; i < e0; ++i) nk += flag[i] == 1;
  int tot_k;
  int wpos = excl_sum<NT>(nk, sc, tot_k);
  for (int i = b0; i < e0; ++i)
    if (flag[i] == 1) {
      if (wpos < kp) row[1 + wpos] = i + 1;  // exactly kp by construction; never past b - 2
      ++wpos;
    }
}

}  // namespace

// ---- host side ---------------------------------------------------------------------------

bool prescore_applies(const Geo& g) {
  return g.dtype == 1 && g.G >= 16 && g.G % 16 == 0 && g.G <= 128 &&
         (g.D == 64 || g.D == 128 || g.D == 576) && g.max_pages - 2 <= kPreMaxInner;
}

size_t prescore_lds(int max_inner) { return (size_t)max_inner * 21 + 64; }

hipError_t launch_prescore(const Geo& g, const SelectPlan& p, const void* q, const void* meta,
                           const int32_t* bt, const int32_t* lens, const int32_t* budgets,
                           int b_max, int32_t* sel, int32_t* cnt, void* ws, hipStream_t st) {
  unsigned char* w = static_cast<unsigned char*>(ws);
  const int max_inner = g.max_pages > 2 ? g.max_pages - 2 : 1;
  PreArgs a{static_cast<const uint16_t*>(q), static_cast<const unsigned char*>(meta), bt, lens,
            budgets, reinterpret_cast<float*>(w), reinterpret_cast<float*>(w + p.off_idx),
            reinterpret_cast<float*>(w + 2 * p.off_idx), reinterpret_cast<int32_t*>(w + 3 * p.off_idx),
            reinterpret_cast<double*>(w + p.off_cnt), sel, cnt, g.Hq, g.Hkv, g.G, g.max_pages,
            b_max, g.num_blocks, max_inner, p.ppt};
  const dim3 grid(p.nchunk, g.Hkv, g.B);
  const int ht = g.G / 16;
  // the 576-wide contraction is split over two waves per head tile (register budget)
#define PSD_LAUNCH(DD, HH, KK) \
  hipLaunchKernelGGL((prescore_kernel<DD, HH, KK>), grid, dim3(64 * HH * KK), 0, st, a)
#define PSD_BY_HT(DD, KK)                       \
  switch (ht) {                                 \
    case 1: PSD_LAUNCH(DD, 1, KK); break;       \
    case 2: PSD_LAUNCH(DD, 2, KK); break;       \
    case 3: PSD_LAUNCH(DD, 3, KK); break;       \
    case 4: PSD_LAUNCH(DD, 4, KK); break;       \
    case 5: PSD_LAUNCH(DD, 5, KK); break;       \
    case 6: PSD_LAUNCH(DD, 6, KK); break;       \
    case 7: PSD_LAUNCH(DD, 7, KK); break;       \
    default: PSD_LAUNCH(DD, 8, KK); break;      \
  }
  if (g.D == 64) {
    PSD_BY_HT(64, 1)
  } else if (g.D == 128) {
    PSD_BY_HT(128, 1)
  } else {
    PSD_BY_HT(576, PSD_PRE_KS576)
  }
#undef PSD_BY_HT
#undef PSD_LAUNCH
  return hipGetLastError();
}

hipError_t launch_certify(const Geo& g, const SelectPlan& p, const void* q, const void* meta,
                          const int32_t* bt, const int32_t* lens, const int32_t* budgets,
                          int b_max, int32_t* sel, void* ws, hipStream_t st, void* meta_tail,
                          const void* k) {
  unsigned char* w = static_cast<unsigned char*>(ws);
  const int max_inner = g.max_pages > 2 ? g.max_pages - 2 : 1;
  PreArgs a{static_cast<const uint16_t*>(q), static_cast<const unsigned char*>(meta), bt, lens,
            budgets, reinterpret_cast<float*>(w), reinterpret_cast<float*>(w + p.off_idx),
            reinterpret_cast<float*>(w + 2 * p.off_idx), reinterpret_cast<int32_t*>(w + 3 * p.off_idx),
            reinterpret_cast<double*>(w + p.off_cnt), sel, nullptr, g.Hq, g.Hkv, g.G,
            g.max_pages, b_max, g.num_blocks, max_inner, p.ppt};
  a.meta_w = meta_tail;
  a.k = k;
  a.kbs = g.kbs;
  a.kts = g.kts;
  a.khs = g.khs;
  const size_t lds = prescore_lds(max_inner);
  const dim3 grid(g.Hkv, g.B, meta_tail ? 2 : 1);
  hipError_t e;
#define PSD_CERT(DD)                                                                        \
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&certify_kernel<DD, 512>),   \
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) !=   \
      hipSuccess)                                                                           \
    return e;                                                                               \
  hipLaunchKernelGGL((certify_kernel<DD, 512>), grid, dim3(512), lds, st, a);
  if (g.D == 64) {
    PSD_CERT(64)
  } else if (g.D == 128) {
    PSD_CERT(128)
  } else {
    PSD_CERT(576)
  }
#undef PSD_CERT
  return hipGetLastError();
}

}  // namespace psd
