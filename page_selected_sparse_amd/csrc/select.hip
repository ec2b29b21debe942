// Page scoring and top-b selection.
//
// Score (EntmaxKV README, "Two selection strategies", top-k: a Quest-style upper bound
// on each page's best score from its key min/max, without reading cached tokens):
//   UB_h(p) = sum_d max(q_hd * kmin_pd, q_hd * kmax_pd), group score = max_h UB_h(p)
// (LOCKS README, "Configuration": GQA combine by max; "How it works": MLA scores are
// max-unioned over the query heads).
//
// The bound is accumulated in fp64 over ascending d, one exact product per step. With
// q+ = max(q, 0) and q- = min(q, 0) the step is two fused multiply-adds,
//   acc = fma(q+, kmax, acc); acc = fma(q-, kmin, acc),
// of which one adds an exact zero: the nonzero one adds exactly the product a plain
// sequential loop adds, so the result is bit-identical to it (up to the sign of an
// all-zero sum, which score_key() folds). Products of two bf16 (or two fp32) values are
// exact in fp64.
//
// Selection (EntmaxKV README, top-k with the budget counting the always-kept tail page;
// LOCKS README, introduction and "Results": sink and most-recent pages kept, counted
// inside b) is two-level so that a unit with tens of thousands of pages still spreads
// over many workgroups:
//   1. score_kernel: a workgroup scores a chunk of candidate pages (1..n-2) of one
//      (sequence, KV head) unit, finds the chunk's top-(b-2) by (score desc, page asc)
//      with an LDS radix select on order-preserving 64-bit keys, and writes them in
//      page order.
//   2. merge_kernel: a workgroup per unit concatenates the chunk candidates (still in
//      page order), radix-selects the global top-(b-2), and writes sink, the winners
//      and the tail in ascending page order.
// The global top-(b-2) is contained in the union of the chunk top-(b-2) lists, since a
// page outranked by fewer than b-2 pages overall is outranked by fewer than b-2 pages of
// its own chunk.
#include "psd_device.h"
#include "psd_launch.h"

namespace psd {
namespace {

constexpr int kThreads = 256;
constexpr int kMergeCap = 8192;  // candidates one merge workgroup holds in LDS
constexpr int kMaxChunks = 1024;  // chunks per unit

// Everything the three selection kernels need; device pointers into the caller's
// buffers and the select workspace.
struct SelArgs {
  const void* q;
  const void* meta;
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* budgets;
  uint64_t* ckey;    // [unit][nchunk][cap] chunk candidates (order-preserving keys)
  int32_t* cidx;     // [unit][nchunk][cap] their logical pages
  int32_t* ccnt;     // [unit][nchunk] candidates written per chunk
  int32_t* sel;
  int32_t* cnt;
  int Hq, Hkv, G, D, max_pages, b_max, chunk, ppt, nchunk, cap, num_blocks;
};

struct SelScratch {
  uint32_t hist[256];
  int wave_cnt[16];
  int digit, k;
  bool done;
};

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Exclusive count of `flag` over the threads before this one (thread order), and the
// total, for an NT-thread workgroup. Contains barriers: every thread must call it.
template <int NT>
__device__ __forceinline__ int block_excl_count(bool flag, SelScratch& sc, int& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  if constexpr (NW == 1) {
    total = __popcll(m);
    return below;
  }
  if (lane == 0) sc.wave_cnt[w] = __popcll(m);
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
  return off + below;
}

// Finds the top K (1 <= K <= N) of keys[0..N) in LDS by radix select over 8-bit digits
// from the most significant. Returns a prefix P over the bits covered by `mask` such that
// every key with (key & mask) > P is in the top K and `need` of the keys with
// (key & mask) == P complete it (the lowest positions among them). It stops as soon as all
// keys of the chosen digit are needed; otherwise it ends with mask = all bits, P = the
// K-th largest key. Equal digits met in a row by one thread are counted once.
template <int NT>
__device__ void block_kth_largest(const uint64_t* keys, int N, int K, SelScratch& sc,
                                  uint64_t& P, uint64_t& M, int& need) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0, mask = 0;
  int k = K;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) sc.hist[i] = 0;
    __syncthreads();
    int run_d = -1, run_c = 0;
    for (int i = tid; i < N; i += NT) {
      const uint64_t key = keys[i];
      if ((key & mask) == prefix) {
        const int dg = (int)((key >> shift) & 255u);
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
      // lane handles digits 255-4l .. 252-4l, i.e. descending digit order
      const int base = 255 - 4 * tid;
      const int c0 = sc.hist[base], c1 = sc.hist[base - 1], c2 = sc.hist[base - 2],
                c3 = sc.hist[base - 3];
      const int local = c0 + c1 + c2 + c3;
      const int incl = wave_inclusive_scan(local);
      const int excl = incl - local;
      if (excl < k && k <= incl) {
        int r = k - excl, dg, cnt;
        if (r <= c0) {
          dg = base;
          cnt = c0;
        } else if (r <= c0 + c1) {
          r -= c0;
          dg = base - 1;
          cnt = c1;
        } else if (r <= c0 + c1 + c2) {
          r -= c0 + c1;
          dg = base - 2;
          cnt = c2;
        } else {
          r -= c0 + c1 + c2;
          dg = base - 3;
          cnt = c3;
        }
        sc.digit = dg;
        sc.k = r;
        sc.done = r == cnt;  // every key of this digit is in the top K
      }
    }
    __syncthreads();
    prefix |= (uint64_t)sc.digit << shift;
    mask |= 255ull << shift;
    k = sc.k;
    const bool done = sc.done;
    __syncthreads();  // sc is rewritten by the next pass
    if (done) break;
  }
  P = prefix;
  M = mask;
  need = k;
}

// Emits, in position order, every key with (key & M) > P and the first `need` keys with
// (key & M) == P; calls out(rank, position) for each. Returns the number emitted. Every
// thread must call it.
template <int NT, typename Out>
__device__ int block_emit_top(const uint64_t* keys, int N, uint64_t P, uint64_t M, int need,
                              SelScratch& sc, Out out) {
  int run_eq = 0, run_out = 0;
  for (int base = 0; base < N; base += NT) {
    const int i = base + threadIdx.x;
    const bool ok = i < N;
    const uint64_t key = ok ? (keys[i] & M) : 0;
    const bool gt = ok && key > P, eq = ok && key == P;
    int tot_eq, tot_sel;
    const int eq_rank = run_eq + block_excl_count<NT>(eq, sc, tot_eq);
    const bool pick = gt || (eq && eq_rank < need);
    const int pos = run_out + block_excl_count<NT>(pick, sc, tot_sel);
    if (pick) out(pos, i);
    run_eq += tot_eq;
    run_out += tot_sel;
  }
  return run_out;
}

template <bool BF16>
__device__ __forceinline__ double q_value(const void* q, int64_t idx) {
  if constexpr (BF16) {
    return (double)__uint_as_float((uint32_t) static_cast<const uint16_t*>(q)[idx] << 16);
  } else {
    return (double)static_cast<const float*>(q)[idx];
  }
}


// Unit status shared by the three kernels: pages n, effective budget b, free slots kp.
struct UnitInfo {
  int n, b, kp;
  bool trivial;  // no ranking needed (all pages, sink + tail only, or over capacity)
};

__device__ __forceinline__ UnitInfo unit_info(const SelArgs& a, int s) {
  UnitInfo u;
  u.n = ceil_div(a.lens[s], kPage);
  u.b = effective_budget(u.n, a.budgets[s]);
  u.kp = u.b - 2;
  u.trivial = u.n <= u.b || u.kp <= 0 || u.b > a.b_max;
  return u;
}

// Writes every selection row entry except the ranked winners: sink, tail, padding and
// count for units that rank; the whole row for units that need no ranking; a -1 row and
// count for units over capacity (never truncated). NT threads of one workgroup.
template <int NT>
__device__ void write_row_header(const SelArgs& a, int unit, const UnitInfo& u) {
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

// Element j of a chunk held as 16-byte vectors, widened exactly to fp64.
template <bool BF16>
__device__ __forceinline__ double chunk_elem(const uint4* v, int j) {
  if constexpr (BF16) {
    const uint4 w = v[j >> 3];
    const int k = (j >> 1) & 3;
    const uint32_t word = k == 0 ? w.x : (k == 1 ? w.y : (k == 2 ? w.z : w.w));
    return (double)((j & 1) ? bf_hi(word) : bf_lo(word));
  } else {
    const uint4 w = v[j >> 2];
    const int k = j & 3;
    return (double)__uint_as_float(k == 0 ? w.x : (k == 1 ? w.y : (k == 2 ? w.z : w.w)));
  }
}

// Statistics are chunk-major: [D / CD][num_blocks][H_kv][2][CD] with CD = 64 bytes of
// dims, so the minima and maxima of CD dims of one (block, head) are one 128-byte line.
template <bool BF16>
struct MetaGeo {
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int CD = 64 / ES;  // dims per chunk
  // byte offset of chunk c of (block, head)
  __device__ static int64_t piece(int c, int nb, int hkv, int blk, int g) {
    return (((int64_t)c * nb + blk) * hkv + g) * 128;
  }
};

// Four fp64 FMAs per head pair of one dim: acc_h += q+_h kmax + q-_h kmin, with q read
// from lane B + 2h (+1) of each 16-lane row of `q` by a DPP row broadcast. The leading
// s_nop covers the VALU-write -> DPP-read hazard on the q register.
template <int B>
__device__ __forceinline__ void fma4_dpp(double& a0, double& a1, double& a2, double& a3, double q,
                                         double kx, double kn) {
  asm("s_nop 1\n\t"
      "v_fmac_f64_dpp %0, %4, %5 row_newbcast:%7 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %0, %4, %6 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %1, %4, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %1, %4, %6 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %2, %4, %5 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %2, %4, %6 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %3, %4, %5 row_newbcast:%13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f64_dpp %3, %4, %6 row_newbcast:%14 row_mask:0xf bank_mask:0xf"
      : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)
      : "v"(q), "v"(kx), "v"(kn), "n"(B), "n"(B + 1), "n"(B + 2), "n"(B + 3), "n"(B + 4),
        "n"(B + 5), "n"(B + 6), "n"(B + 7));
}

// Bound of one page per lane for HB (4 or 8) heads. The group's (q+, q-) values for a
// chunk of CD dims are spread over the lanes of each 16-lane row (value v of the chunk in
// register v / 16 of lane v % 16, loaded from the LDS table once per chunk) and reach the
// fp64 FMAs through DPP row broadcasts, so no per-dim operand traffic is needed.
// Statistics lines (128 bytes per page and chunk) are loaded cooperatively and straight
// into LDS: in each of 8 load instructions, 8 lanes read the 8 pieces of one page's line,
// so every line is one coalesced request. The wave's `stage` (8 KB) holds its 64 lines
// with each page's pieces rotated by the page index, so that each lane reads back its own
// line without bank conflicts. The next chunk's lines land while the current one is
// accumulated; dims ascend.
template <bool BF16, int D, int HB>
__device__ __forceinline__ void bound_dpp(const void* meta, int nb, int hkv, int blk, int g,
                                          const double* qv, uint4* stage, double* acc) {
  using M = MetaGeo<BF16>;
  constexpr int CD = M::CD;
  constexpr int NQ = CD * 2 * HB / 16;  // q registers per chunk
  constexpr int NCH = D / CD;
  const int lane = threadIdx.x & 63, lane16 = lane & 15;
  const int sub = lane & 7;  // which slot of its line this lane fills
  const unsigned char* base = static_cast<const unsigned char*>(meta);
  // In load step i this lane fills slot `sub` of page 8i + lane / 8 with piece
  // (sub + page) & 7 of that page's line.
  int64_t src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int page = 8 * i + (lane >> 3);
    src[i] = M::piece(0, nb, hkv, __shfl(blk, page, 64), g) + 16 * ((sub + page) & 7);
  }
  const int64_t cstride = (int64_t)nb * hkv * 128;  // bytes between chunks of one line
  auto load = [&](int c) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(base + src[i] + c * cstride,
                                       (__attribute__((address_space(3))) void*)(stage + 64 * i),
                                       16, 0, 0);
  };
  auto accumulate = [&](int c, const uint4* mv) {
    double Q[NQ];
#pragma unroll
    for (int m = 0; m < NQ; ++m) Q[m] = qv[c * CD * 2 * HB + 16 * m + lane16];
#pragma unroll
    for (int j = 0; j < CD; ++j) {
      const double kmn = chunk_elem<BF16>(mv, j), kmx = chunk_elem<BF16>(mv + 4, j);
      if constexpr (HB == 4) {
        if (j & 1)
          fma4_dpp<8>(acc[0], acc[1], acc[2], acc[3], Q[j >> 1], kmx, kmn);
        else
          fma4_dpp<0>(acc[0], acc[1], acc[2], acc[3], Q[j >> 1], kmx, kmn);
      } else {
        fma4_dpp<0>(acc[0], acc[1], acc[2], acc[3], Q[j], kmx, kmn);
        fma4_dpp<8>(acc[4], acc[5], acc[6], acc[7], Q[j], kmx, kmn);
      }
    }
  };
  load(0);
  // kept rolled: the q reads and loads of one chunk stay inside their iteration
#pragma unroll 1
  for (int c = 0; c < NCH; ++c) {
    __builtin_amdgcn_s_waitcnt(0);  // this chunk's lines have landed in LDS
    uint4 mv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) mv[k] = stage[lane * 8 + ((k - lane) & 7)];
    __builtin_amdgcn_s_waitcnt(0);  // read back before the next lines overwrite the stage
    if (c + 1 < NCH) load(c + 1);
    accumulate(c, mv);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// Bound contribution of dims [d0, d0 + DC) of one page for HB heads, with the (q+, q-)
// table of those dims staged in LDS and read as broadcasts; dims ascend.
template <bool BF16, int DC, int HB>
__device__ __forceinline__ void bound_lds(const void* meta, int nb, int hkv, int blk, int g,
                                          int d0, const double2* qt, double* acc) {
  using M = MetaGeo<BF16>;
  constexpr int CD = M::CD;
  constexpr int PER = 16 / M::ES;  // dims per 16-byte vector
  const unsigned char* base = static_cast<const unsigned char*>(meta);
#pragma unroll
  for (int dd = 0; dd < DC; dd += PER) {
    const int d = d0 + dd;
    const unsigned char* pc = base + M::piece(d / CD, nb, hkv, blk, g) + (d % CD) * M::ES;
    const uint4 av = *reinterpret_cast<const uint4*>(pc);
    const uint4 bv = *reinterpret_cast<const uint4*>(pc + 64);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const double kmn = chunk_elem<BF16>(&av, j), kmx = chunk_elem<BF16>(&bv, j);
#pragma unroll
      for (int h = 0; h < HB; ++h) {
        const double2 qq = qt[(dd + j) * HB + h];
        acc[h] = __builtin_fma(qq.x, kmx, acc[h]);
        acc[h] = __builtin_fma(qq.y, kmn, acc[h]);
      }
    }
  }
}

// Global top-kp of one unit from its chunk candidate lists, written to row[1 .. kp] in
// ascending page order. The unit's slots are copied as one block (chunk-major, so in page
// order); slots past a chunk's count get key 0, below every score key. When every chunk
// keeps all its pages (cap == chunk) a slot's page is its position + 1.
template <int NT>
__device__ void merge_unit(const SelArgs& a, int unit, int n, int kp, unsigned char* lds,
                           SelScratch& sc) {
  const int tid = threadIdx.x;
  int32_t* row = a.sel + (int64_t)unit * a.b_max;
  const int nch = ceil_div(n - 2, a.chunk);
  const int total = nch * a.cap;
  const bool dense = a.cap == a.chunk;
  uint64_t* keys = reinterpret_cast<uint64_t*>(lds);
  int32_t* idx = reinterpret_cast<int32_t*>(lds + sizeof(uint64_t) * (size_t)a.nchunk * a.cap);
  int* cnts = reinterpret_cast<int*>(idx + (size_t)a.nchunk * a.cap);
  const int64_t src = (int64_t)unit * a.nchunk * a.cap;
  for (int c = tid; c < nch; c += NT) cnts[c] = a.ccnt[(int64_t)unit * a.nchunk + c];
#pragma unroll 4
  for (int j = tid; j < total; j += NT) {
    keys[j] = a.ckey[src + j];
    if (!dense) idx[j] = a.cidx[src + j];
  }
  __syncthreads();
  for (int j = tid; j < total; j += NT) {
    const int c = j / a.cap;
    if (j - c * a.cap >= cnts[c]) keys[j] = 0;
  }
  __syncthreads();
  uint64_t P, M;
  int need;
  block_kth_largest<NT>(keys, total, kp, sc, P, M, need);
  block_emit_top<NT>(keys, total, P, M, need, sc,
                     [&](int pos, int i) { row[1 + pos] = dense ? i + 1 : idx[i]; });
}

// One workgroup scores one chunk of a unit's candidate pages 1..n-2, one page per thread.
// DPP (groups of up to 8 heads, D <= 128): the whole (q+, q-) table in LDS, fed to the
// FMAs by row broadcasts. Otherwise the table is staged 16 heads x DC dims at a time and
// read as LDS broadcasts.
template <bool BF16, int D, int HB, bool DPP, int NT>
__global__ __launch_bounds__(NT) void score_kernel(SelArgs a) {
  constexpr int DC = DPP ? D : ((HB * D * 16 <= 32768) ? D : 32);
  constexpr int NDC = D / DC;
  __shared__ double2 qlds[DC * HB];
  __shared__ SelScratch sc;
  extern __shared__ unsigned char lds[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(lds);  // [chunk]

  const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x;
  const UnitInfo u = unit_info(a, s);
  if (c == 0) write_row_header<NT>(a, s * a.Hkv + g, u);
  if (u.trivial) return;
  const int kp = u.kp, n = u.n;
  const int lo = 1 + c * a.chunk;
  const int hi = min(lo + a.chunk, n - 1);
  if (lo >= hi) return;
  const int cnt = hi - lo;
  const int unit = s * a.Hkv + g;
  const int nhp = ceil_div(a.G, HB);

  auto load_qlds = [&](int hp, int dc) {
    for (int e = tid; e < DC * HB; e += NT) {
      const int d = e / HB, h = e - d * HB, hh = hp * HB + h;
      double qv = 0.0;
      if (hh < a.G) qv = q_value<BF16>(a.q, ((int64_t)s * a.Hq + g * a.G + hh) * D + dc * DC + d);
      qlds[e] = make_double2(qv >= 0.0 ? qv : 0.0, qv >= 0.0 ? 0.0 : qv);
    }
  };
  const bool once = nhp == 1 && NDC == 1;
  if (once) {
    load_qlds(0, 0);
    __syncthreads();
  }
  const int64_t bt0 = (int64_t)s * a.max_pages;
  for (int it = 0; it < a.ppt; ++it) {
    const int o = it * NT + tid;
    const bool have = o < cnt;
    const int blk = a.bt[bt0 + (have ? lo + o : 0)];
    double best = -__builtin_inf();
    if constexpr (DPP) {
      double acc[HB];
#pragma unroll
      for (int h = 0; h < HB; ++h) acc[h] = 0.0;
      uint4* stage = reinterpret_cast<uint4*>(lds + a.chunk * sizeof(uint64_t)) + (tid >> 6) * 512;
      bound_dpp<BF16, D, HB>(a.meta, a.num_blocks, a.Hkv, blk, g,
                             reinterpret_cast<const double*>(qlds), stage, acc);
#pragma unroll
      for (int h = 0; h < HB; ++h)
        if (h < a.G && acc[h] > best) best = acc[h];
    } else {
      for (int hp = 0; hp < nhp; ++hp) {
        double acc[HB];
#pragma unroll
        for (int h = 0; h < HB; ++h) acc[h] = 0.0;
        for (int dc = 0; dc < NDC; ++dc) {
          if (!once) {
            __syncthreads();
            load_qlds(hp, dc);
            __syncthreads();
          }
          bound_lds<BF16, DC, HB>(a.meta, a.num_blocks, a.Hkv, blk, g, dc * DC, qlds, acc);
        }
#pragma unroll
        for (int h = 0; h < HB; ++h)
          if (hp * HB + h < a.G && acc[h] > best) best = acc[h];
      }
    }
    keys[o] = score_key(best);  // every slot written; slots past cnt are never read
  }
  __syncthreads();

  // Chunk candidates: all pages when they fit in kp, else the chunk's top-kp.
  uint64_t* okey = a.ckey + ((int64_t)unit * a.nchunk + c) * a.cap;
  int32_t* oidx = a.cidx + ((int64_t)unit * a.nchunk + c) * a.cap;
  if (cnt <= kp || a.cap == a.chunk) {  // every page of the chunk is a candidate
    for (int o = tid; o < cnt; o += NT) {
      okey[o] = keys[o];
      if (a.cap < a.chunk) oidx[o] = lo + o;
    }
    if (tid == 0) a.ccnt[(int64_t)unit * a.nchunk + c] = cnt;
  } else {
    uint64_t P, M;
    int need;
    block_kth_largest<NT>(keys, cnt, kp, sc, P, M, need);
    const int emitted = block_emit_top<NT>(keys, cnt, P, M, need, sc, [&](int pos, int i) {
      okey[pos] = keys[i];
      oidx[pos] = lo + i;
    });
    if (tid == 0) a.ccnt[(int64_t)unit * a.nchunk + c] = emitted;
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void merge_kernel(SelArgs a) {
  __shared__ SelScratch sc;
  extern __shared__ unsigned char lds[];
  const int g = blockIdx.x, s = blockIdx.y;
  const UnitInfo u = unit_info(a, s);
  if (u.trivial) return;
  merge_unit<NT>(a, s * a.Hkv + g, u.n, u.kp, lds, sc);
}

template <typename K>
hipError_t set_lds(K kernel, size_t lds) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <bool BF16, int D, int HB, bool DPP, int NT>
hipError_t launch_score(const SelArgs& a, const SelectPlan& p, dim3 sgrid, hipStream_t st) {
  hipError_t e = set_lds(&score_kernel<BF16, D, HB, DPP, NT>, p.score_lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_kernel<BF16, D, HB, DPP, NT>), sgrid, dim3(NT), p.score_lds, st, a);
  return hipGetLastError();
}

template <bool BF16, int D, int HB, bool DPP>
hipError_t dispatch_nt(const SelArgs& a, const SelectPlan& p, dim3 grid, hipStream_t st) {
  return p.threads == 64 ? launch_score<BF16, D, HB, DPP, 64>(a, p, grid, st)
                         : launch_score<BF16, D, HB, DPP, kThreads>(a, p, grid, st);
}

template <bool BF16, int D>
hipError_t dispatch_hb(const SelArgs& a, const SelectPlan& p, dim3 grid, hipStream_t st) {
  if constexpr (D > 128) {
    return launch_score<BF16, D, 16, false, kThreads>(a, p, grid, st);
  } else {
    switch (p.head_block) {
      case 4: return dispatch_nt<BF16, D, 4, true>(a, p, grid, st);
      case 8: return dispatch_nt<BF16, D, 8, true>(a, p, grid, st);
      default: return dispatch_nt<BF16, D, 16, false>(a, p, grid, st);
    }
  }
}

}  // namespace

bool plan_select(const Geo& g, int b_max, SelectPlan* p) {
  if (b_max < 2) return false;
  const int kcap = b_max - 2;
  const int inner = g.max_pages > 2 ? g.max_pages - 2 : 1;
  const int64_t units = (int64_t)g.B * g.Hkv;
  // Groups of up to 8 heads with D <= 128 take q through DPP broadcasts (whole table in
  // LDS); other groups read it as LDS broadcasts, 16 heads at a time.
  p->all_q = g.G <= 16 && g.D <= 128;
  p->head_block = !p->all_q ? 16 : (g.G <= 4 ? 4 : (g.G <= 8 ? 8 : 16));
  p->d_chunk = p->all_q ? g.D : ((16 * g.D * 16 <= 32768) ? g.D : 32);
  p->pages_per_lane = 1;
  // one-wave workgroups when 256-thread ones would leave the GPU mostly idle
  p->threads = (p->all_q && units * ((inner + kThreads - 1) / kThreads) < 512) ? 64 : kThreads;
  const bool multi_pass = !p->all_q && (g.G > 16 || 16 * g.D * 16 > 32768);
  bool ok = false;
  for (int ppt = 1; ppt <= 64; ppt *= 2) {
    if (multi_pass && ppt > 1) break;
    const int chunk = p->threads * p->pages_per_lane * ppt;
    if (chunk * sizeof(uint64_t) > 65536) break;
    const int nchunk = (inner + chunk - 1) / chunk;
    if (nchunk > kMaxChunks) continue;
    // Every page of a chunk is a candidate when they all fit in the merge; otherwise a
    // chunk keeps only its own top b-2.
    int cap = chunk;
    if ((int64_t)nchunk * chunk > kMergeCap) cap = kcap < 1 ? 1 : (kcap < chunk ? kcap : chunk);
    if ((int64_t)nchunk * cap <= kMergeCap) {
      p->ppt = ppt;
      p->chunk = chunk;
      p->nchunk = nchunk;
      p->cap = cap;
      ok = true;
      break;
    }
  }
  if (!ok) return false;
  const size_t slots = (size_t)units * p->nchunk * p->cap;
  p->merge_lds = (size_t)p->nchunk * p->cap * (sizeof(uint64_t) + sizeof(int32_t)) +
                 (size_t)p->nchunk * sizeof(int32_t);
  p->merge_threads = (int64_t)p->nchunk * p->cap <= 512 ? 64 : kThreads;
  p->score_lds = p->chunk * sizeof(uint64_t);
  if (p->head_block <= 8 && p->all_q) p->score_lds += (size_t)(p->threads / 64) * 8192;  // staging
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  p->off_idx = al(slots * sizeof(uint64_t));
  p->off_cnt = al(p->off_idx + slots * sizeof(int32_t));
  p->bytes = p->off_cnt + units * p->nchunk * sizeof(int32_t) + 256;
  return true;
}

static SelArgs make_args(const Geo& g, const SelectPlan& p, const void* q, const void* meta,
                         const int32_t* bt, const int32_t* lens, const int32_t* budgets,
                         int b_max, int32_t* sel, int32_t* cnt, void* ws) {
  unsigned char* w = static_cast<unsigned char*>(ws);
  return SelArgs{q, meta, bt, lens, budgets,
                 reinterpret_cast<uint64_t*>(w), reinterpret_cast<int32_t*>(w + p.off_idx),
                 reinterpret_cast<int32_t*>(w + p.off_cnt), sel, cnt,
                 g.Hq, g.Hkv, g.G, g.D, g.max_pages, b_max, p.chunk, p.ppt, p.nchunk, p.cap,
                 g.num_blocks};
}

hipError_t launch_select_score(const Geo& g, const SelectPlan& p, const void* q,
                               const void* meta, const int32_t* bt, const int32_t* lens,
                               const int32_t* budgets, int b_max, int32_t* sel, int32_t* cnt,
                               void* ws, hipStream_t st) {
  const SelArgs a = make_args(g, p, q, meta, bt, lens, budgets, b_max, sel, cnt, ws);
  const dim3 sgrid(p.nchunk, g.Hkv, g.B);
  const bool bf = g.dtype == 1;
  switch (g.D) {
    case 64: return bf ? dispatch_hb<true, 64>(a, p, sgrid, st)
                       : dispatch_hb<false, 64>(a, p, sgrid, st);
    case 128: return bf ? dispatch_hb<true, 128>(a, p, sgrid, st)
                        : dispatch_hb<false, 128>(a, p, sgrid, st);
    default: return bf ? dispatch_hb<true, 576>(a, p, sgrid, st)
                       : dispatch_hb<false, 576>(a, p, sgrid, st);
  }
}

// The merge runs as its own launch: the kernel boundary makes every chunk's candidates
// visible (a device-scope fence inside the scoring kernel writes back and invalidates
// the L2).
hipError_t launch_select_merge(const Geo& g, const SelectPlan& p, const int32_t* lens,
                               const int32_t* budgets, int b_max, int32_t* sel, void* ws,
                               hipStream_t st) {
  const SelArgs a = make_args(g, p, nullptr, nullptr, nullptr, lens, budgets, b_max, sel,
                              nullptr, ws);
  const dim3 ugrid(g.Hkv, g.B);
  hipError_t e;
  if (p.merge_threads == 64) {
    if ((e = set_lds(&merge_kernel<64>, p.merge_lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(merge_kernel<64>, ugrid, dim3(64), p.merge_lds, st, a);
  } else {
    if ((e = set_lds(&merge_kernel<kThreads>, p.merge_lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(merge_kernel<kThreads>, ugrid, dim3(kThreads), p.merge_lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace psd
