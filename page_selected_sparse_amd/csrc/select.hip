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
// inside b) ranks pages by (score desc, page asc) with an LDS radix select on
// order-preserving 64-bit keys. When there are enough (sequence, KV head) units to fill
// the GPU and a unit has at most 2048 candidate pages, one workgroup scores all of a
// unit's pages and writes its row directly. Otherwise selection is two-level, so that a
// unit with tens of thousands of pages still spreads over many workgroups:
//   1. score_kernel: a workgroup scores a chunk of candidate pages (1..n-2) of one unit,
//      finds the chunk's top-(b-2) and writes them in page order to the workspace.
//   2. merge_kernel: a workgroup per unit concatenates the chunk candidates (still in
//      page order), radix-selects the global top-(b-2), and writes them into the row.
// The global top-(b-2) is contained in the union of the chunk top-(b-2) lists, since a
// page outranked by fewer than b-2 pages overall is outranked by fewer than b-2 pages of
// its own chunk. Sink, tail, padding and counts are written by the scoring kernel.
#include "attn_core.h"
#include "meta_core.h"
#include "psd_device.h"
#include "psd_launch.h"

namespace psd {
namespace {

#ifndef PSD_FUSED_XCD_MAP
#define PSD_FUSED_XCD_MAP 1  // the KV heads of a sequence on one XCD
#endif

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
  uint64_t* ckey;    // [unit][ustride] chunk candidates (order-preserving keys), chunk-major
  int32_t* cidx;     // [unit][ustride] their logical pages
  int32_t* ccnt;     // [unit][nchunk] candidates written per chunk
  int32_t* sel;
  int32_t* cnt;
  int Hq, Hkv, G, D, max_pages, b_max, chunk, ppt, nchunk, cap, num_blocks;
  int ustride;  // candidate slots per unit: nchunk * cap rounded up to 1 KB of keys
  // Tail refresh (decode step): with meta_w, one extra workgroup per unit refreshes the
  // tail page's statistics of its KV head from K: x = 0 of the scoring launch (ahead of
  // the unit's chunks, which then take x = 1 .. nchunk), or z = 1 of the merge launch.
  void* meta_w;
  const void* k;
  int64_t kbs, kts, khs;
  int bf16 = 0;
};

struct SelScratch {
  uint32_t hist[3][256];  // rotating: one barrier per radix pass
  int wave_cnt[2][16];    // wave totals of a block scan (two buffers: back-to-back scans)
  uint64_t wand[16], wor[16];
};

// Finds the top K (1 <= K <= N) of keys[0..N) in LDS by radix select over 8-bit digits.
// Key 0 marks an empty slot: it never ranks (score keys of finite scores are nonzero and
// far above it). The bits every nonzero key shares are skipped: the first digit starts at
// the highest bit where two keys differ. Returns a prefix P over the bits covered by
// `mask` such that every key with (key & mask) > P is in the top K and `need` of the keys
// with (key & mask) == P complete it (the lowest positions among them). It stops as soon
// as all keys of the chosen digit are needed; otherwise it ends with mask = all bits,
// P = the K-th largest key. Equal digits met in a row by one thread are counted once.
// One barrier per pass: histograms rotate over three buffers (a buffer is cleared two
// passes before it is counted into) and every wave scans the histogram itself.
// With `published`, the caller has already run kth_publish with the AND and OR of each
// thread's nonzero keys (as it wrote them) and passed a barrier, which saves a pass over
// the keys and a barrier.
template <int NT>
__device__ __forceinline__ void kth_publish(SelScratch& sc, uint64_t kand, uint64_t kor) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 2 * 256; i += NT) sc.hist[i >> 8][i & 255] = 0;
  wave_and_or64(kand, kor);
  if (lane == 0) {
    sc.wand[w] = kand;
    sc.wor[w] = kor;
  }
}

template <int NT>
__device__ void block_kth_largest(const uint64_t* keys, int N, int K, SelScratch& sc,
                                  uint64_t& P, uint64_t& M, int& need, bool published = false) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  if (!published) {
    uint64_t kand = ~0ull, kor = 0;
    for (int i = tid; i < N; i += NT) {
      const uint64_t key = keys[i];
      if (key) {
        kand &= key;
        kor |= key;
      }
    }
    kth_publish<NT>(sc, kand, kor);
    __syncthreads();
  }
  // the workgroup's AND and OR: lane i < NW brings wave i's, then one wave reduction
  uint64_t kand = lane < NW ? sc.wand[lane] : ~0ull, kor = lane < NW ? sc.wor[lane] : 0ull;
  wave_and_or64(kand, kor);
  const uint64_t diff = kand ^ kor;
  if (diff == 0) {  // every nonzero key is equal: the first K of them
    P = kand;
    M = ~0ull;
    need = K;
    return;
  }
  const int hb = 63 - __clzll(diff);
  uint64_t mask = hb == 63 ? 0ull : ~((2ull << hb) - 1ull);  // bits above hb are shared
  uint64_t prefix = kand & mask;
  int k = K;
  for (int pass = 0, sh = hb - 7;; ++pass, sh -= 8) {
    const int lo = sh > 0 ? sh : 0;
    const uint64_t dmask = (1ull << (sh + 8 - lo)) - 1ull;
    uint32_t* hist = sc.hist[pass % 3];
    int run_d = -1, run_c = 0;
    for (int i = tid; i < N; i += NT) {
      const uint64_t key = keys[i];
      if ((key & mask) == prefix) {
        const int dg = (int)((key >> lo) & dmask);
        if (dg == run_d) {
          ++run_c;
        } else {
          if (run_c) atomicAdd(&hist[run_d], (uint32_t)run_c);
          run_d = dg;
          run_c = 1;
        }
      }
    }
    if (run_c) atomicAdd(&hist[run_d], (uint32_t)run_c);
    __syncthreads();
    // every wave: lane l handles digits 255-4l .. 252-4l (descending digit order)
    const int base = 255 - 4 * lane;
    const int c0 = hist[base], c1 = hist[base - 1], c2 = hist[base - 2], c3 = hist[base - 3];
    const int local = c0 + c1 + c2 + c3;
    const int incl = wave_scan_incl(local);
    const int excl = incl - local;
    const bool mine = excl < k && k <= incl;
    int r = k - excl, dg = base, cnt = c0;
    if (r > c0) {
      r -= c0;
      dg = base - 1;
      cnt = c1;
      if (r > c1) {
        r -= c1;
        dg = base - 2;
        cnt = c2;
        if (r > c2) {
          r -= c2;
          dg = base - 3;
          cnt = c3;
        }
      }
    }
    const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
    dg = lane_value(dg, src);
    r = lane_value(r, src);
    cnt = lane_value(cnt, src);
    // the buffer of the next pass but one was last read before this pass's barrier
    for (int i = tid; i < 256; i += NT) sc.hist[(pass + 2) % 3][i] = 0;
    prefix |= (uint64_t)dg << lo;
    mask |= dmask << lo;
    k = r;
    if (r == cnt || lo == 0) break;  // every key of this digit is needed, or all bits done
  }
  __syncthreads();  // sc is reused by the next call
  P = prefix;
  M = mask;
  need = k;
}

// Exclusive prefix sum of x over the threads of an NT-thread workgroup (thread order),
// and the total, using wave-count buffer `buf`. One barrier; a buffer may be reused only
// after another barrier.
template <int NT>
__device__ __forceinline__ int block_excl_sum(int x, SelScratch& sc, int& total, int buf = 0) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_scan_incl(x);
  if constexpr (NW == 1) {
    total = lane_value(incl, 63);
    return incl - x;
  }
  if (lane == 63) sc.wave_cnt[buf][w] = incl;
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int c = sc.wave_cnt[buf][i];
    off += i < w ? c : 0;
    total += c;
  }
  return off + incl - x;
}

// Emits, in position order, every key with (key & M) > P and the first `need` keys with
// (key & M) == P; calls out(rank, position) for each. Each thread owns one contiguous
// segment of positions: it counts its keys above and at the threshold, and one block scan
// of the two counts packed in 16-bit halves (N < 65536) gives its first rank: the keys
// above before it plus the equal keys before it, at most `need` of them. Returns the
// number emitted. Every thread must call it.
template <int NT, typename Out>
__device__ int block_emit_top(const uint64_t* keys, int N, uint64_t P, uint64_t M, int need,
                              SelScratch& sc, Out out) {
  const int per = ceil_div(N, NT);
  const int b0 = min((int)threadIdx.x * per, N), e0 = min(b0 + per, N);
  int gt = 0, eq = 0;
  for (int i = b0; i < e0; ++i) {
    const uint64_t key = keys[i] & M;
    gt += key > P;
    eq += key == P;
  }
  int tot;
  const int before = block_excl_sum<NT>((gt << 16) | eq, sc, tot, 0);
  const int eq_before = before & 0xffff;
  const int eq_take = min(max(need - eq_before, 0), eq);
  const int emitted = (tot >> 16) + min(tot & 0xffff, need);
  int pos = (before >> 16) + min(eq_before, need);
  int eq_seen = 0;
  for (int i = b0; i < e0; ++i) {
    const uint64_t key = keys[i] & M;
    bool pick = key > P;
    if (key == P) pick = eq_seen++ < eq_take;
    if (pick) out(pos++, i);
  }
  return emitted;
}

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8),
// each waiting on one counter only.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Waits until at most 8 * n vector memory operations of this wave are outstanding.
__device__ __forceinline__ void wait_vm8(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<8>(); break;
    case 2: wait_vm<16>(); break;
    case 3: wait_vm<24>(); break;
    default: wait_vm<32>(); break;
  }
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

// The same entries as write_row_header, into a unit's page list in LDS. Returns the
// list's entry count: b for units that rank, n for units that keep every page, -1 for
// units over capacity (no entries). The list may overlap the statistics staging area:
// call it only after a barrier that follows every wave's wait for its loads.
template <int NT>
__device__ int write_list_header(int32_t* list, const UnitInfo& u, int b_max) {
  const int tid = threadIdx.x;
  if (u.b > b_max) return -1;
  if (u.n <= u.b) {
    for (int i = tid; i < u.n; i += NT) list[i] = i;
    return u.n;
  }
  if (tid == 0) {
    list[0] = 0;
    list[u.b - 1] = u.n - 1;
  }
  return u.b;
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

// Statistics are page-major: [num_blocks][H_kv][D / CD][2][CD] with CD = 64 bytes of
// dims, so the minima and maxima of CD dims of one (block, head) form one 128-byte line
// and the NCH = D / CD lines of a (block, head) record are contiguous.
template <bool BF16>
struct MetaGeo {
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int CD = 64 / ES;  // dims per chunk
  // byte offset of chunk c of (block, head)
  __device__ static int64_t piece(int c, int nch, int hkv, int blk, int g) {
    return (((int64_t)blk * hkv + g) * nch + c) * 128;
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

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Reads one 128-byte statistics line of this lane's page back from the stage: piece k
// (16 bytes) sits in slot (first + k) mod SL of the page's SL-slot region `page`. Waits
// for the reads. Written as one asm block: the compiler would otherwise make every LDS
// read wait for all loads still streaming into the stages.
template <int SL>
__device__ __forceinline__ void read_line(const uint4* page, int first, uint4 (&mv)[8]) {
  const uint32_t b = (uint32_t)(uintptr_t)page;
  uint32_t a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = b + 16u * (uint32_t)((first + k) & (SL - 1));
  u32x4 r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
  const u32x4 r[8] = {r0, r1, r2, r3, r4, r5, r6, r7};
#pragma unroll
  for (int k = 0; k < 8; ++k) mv[k] = make_uint4(r[k].x, r[k].y, r[k].z, r[k].w);
}

// Bound of one page per lane for HB (4 or 8) heads. The group's (q+, q-) values for a
// chunk of CD dims are spread over the lanes of each 16-lane row (value v of the chunk in
// register v / 16 of lane v % 16, loaded from the LDS table once per chunk) and reach the
// fp64 FMAs through DPP row broadcasts, so no per-dim operand traffic is needed.
// Statistics are loaded cooperatively and straight into LDS in groups of C chunks: each
// load instruction moves 1 KB, 8 / C pages' C contiguous lines, so that each page's
// record is fetched as one contiguous request. In a page's region of the stage its 8C
// pieces are rotated by the page index, so that the 64 lanes read their own lines back
// without bank conflicts. S groups are in flight while one is accumulated; dims ascend.
template <bool BF16, int D, int HB, int CPL, int S>
struct DppPage {
  using M = MetaGeo<BF16>;
  static constexpr int CD = M::CD;
  static constexpr int NQ = CD * 2 * HB / 16;  // q registers per chunk
  static constexpr int NCH = D / CD;
  static constexpr int C = CPL < NCH ? CPL : NCH;  // chunks per load group
  static constexpr int NG = NCH / C;               // load groups
  static constexpr int SS = S < NG ? S : NG;       // groups in flight
  static constexpr int SL = 8 * C;                 // 16-byte slots per page in a group
  static constexpr int NI = SL;                    // 1 KB load instructions per group
  static constexpr int PPI = 8 / C;                // pages per load instruction
  static constexpr int GB = 64 * SL;               // uint4 per group stage (64 pages)
  static_assert(NCH % C == 0 && (SS == 1 || SS == 2), "load grouping");

  const unsigned char* base;
  uint4* stage;
  uint32_t rec[NI];

  // Load instruction i: this lane fetches piece (slot - page) mod SL of page
  // i * PPI + lane / SL into slot lane % SL of that page's region.
  __device__ __forceinline__ void init(const void* meta, int hkv, int blk, int g, uint4* st) {
    const int lane = threadIdx.x & 63;
    base = static_cast<const unsigned char*>(meta);
    stage = st;
    const uint32_t own = (uint32_t)blk * (uint32_t)hkv + (uint32_t)g;  // record of this page
#pragma unroll
    for (int i = 0; i < NI; ++i) rec[i] = __shfl(own, i * PPI + lane / SL, 64);
  }
  __device__ __forceinline__ void load(int grp, uint4* st) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int page = i * PPI + lane / SL;
      const int piece = ((lane % SL) - page) & (SL - 1);
      const unsigned char* src =
          base + (uint64_t)rec[i] * (NCH * 128) + (grp * C * 128 + piece * 16);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(st + 64 * i),
                                       16, 0, 0);
    }
  }
  // the first SS groups; may run before the q table is ready
  __device__ __forceinline__ void issue_first() {
#pragma unroll
    for (int j = 0; j < SS; ++j) load(j, stage + GB * j);
  }
  // the rest of the pipeline and the accumulation, after issue_first()
  __device__ __forceinline__ void finish(const float* qv, double* acc) {
    const int lane = threadIdx.x & 63, lane16 = lane & 15;
    auto accumulate = [&](int c, const uint4* mv) {
      double Q[NQ];
#pragma unroll
      for (int m = 0; m < NQ; ++m) Q[m] = (double)qv[c * CD * 2 * HB + 16 * m + lane16];
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
    // kept rolled: the q reads and loads of one group stay inside their iteration
#pragma unroll 1
    for (int j = 0; j < NG; ++j) {
      // group j has landed once only the groups issued after it are outstanding
      wait_vm8(min(SS - 1, NG - 1 - j) * C);
      uint4* st = stage + GB * (j & (SS - 1)) + lane * SL;  // this lane's page region
#pragma unroll 1
      for (int cc = 0; cc < C; ++cc) {
        uint4 mv[8];
        read_line<SL>(st, cc * 8 + lane, mv);
        if (cc == C - 1 && j + SS < NG) load(j + SS, stage + GB * (j & (SS - 1)));
        accumulate(j * C + cc, mv);
      }
    }
  }
};

// Bound of one page per lane for HB (4 or 8) heads. The group's (q+, q-) values for a
// chunk of CD dims are spread over the lanes of each 16-lane row (value v of the chunk in
// register v / 16 of lane v % 16, loaded from the LDS table once per chunk) and reach the
// fp64 FMAs through DPP row broadcasts, so no per-dim operand traffic is needed.
// Statistics are loaded cooperatively and straight into LDS in groups of C chunks: each
// load instruction moves 1 KB, 8 / C pages' C contiguous lines, so that each page's
// record is fetched as one contiguous request. In a page's region of the stage its 8C
// pieces are rotated by the page index, so that the 64 lanes read their own lines back
// without bank conflicts. S groups are in flight while one is accumulated; dims ascend.
template <bool BF16, int D, int HB, int CPL, int S>
__device__ __forceinline__ void bound_dpp(const void* meta, int hkv, int blk, int g,
                                          const float* qv, uint4* stage, double* acc) {
  DppPage<BF16, D, HB, CPL, S> pg;
  pg.init(meta, hkv, blk, g, stage);
  pg.issue_first();
  pg.finish(qv, acc);
}

// Bound contribution of dims [d0, d0 + DC) of one page for HB heads, with the (q+, q-)
// table of those dims staged in LDS and read as broadcasts; dims ascend.
template <bool BF16, int DC, int HB>
__device__ __forceinline__ void bound_lds(const void* meta, int nch, int hkv, int blk, int g,
                                          int d0, const double2* qt, double* acc) {
  using M = MetaGeo<BF16>;
  constexpr int CD = M::CD;
  constexpr int PER = 16 / M::ES;  // dims per 16-byte vector
  const unsigned char* base = static_cast<const unsigned char*>(meta);
#pragma unroll
  for (int dd = 0; dd < DC; dd += PER) {
    const int d = d0 + dd;
    const unsigned char* pc = base + M::piece(d / CD, nch, hkv, blk, g) + (d % CD) * M::ES;
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

// Copies `bytes` (a multiple of 16) from global memory to LDS with every load in flight at
// once (loads straight into LDS, 16 bytes per lane), then waits for them.
template <int NT>
__device__ __forceinline__ void copy_to_lds(const void* src, void* dst, int bytes) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned char* g = static_cast<const unsigned char*>(src);
  unsigned char* l = static_cast<unsigned char*>(dst);
  for (int off = w * 1024; off < bytes; off += NT * 16) {
    // a whole wave's 1 KB slice is in bounds: callers pad to 1 KB
    __builtin_amdgcn_global_load_lds(g + off + lane * 16,
                                     (__attribute__((address_space(3))) void*)(l + off), 16, 0, 0);
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
  const int ustride = a.ustride;
  uint64_t* keys = reinterpret_cast<uint64_t*>(lds);
  int32_t* idx = reinterpret_cast<int32_t*>(lds + sizeof(uint64_t) * (size_t)ustride);
  int* cnts = reinterpret_cast<int*>(idx + ustride);
  const int64_t src = (int64_t)unit * ustride;
  copy_to_lds<NT>(a.ckey + src, keys, round_up(total * 8, 1024));
  if (!dense) copy_to_lds<NT>(a.cidx + src, idx, round_up(total * 4, 1024));
  for (int c = tid; c < nch; c += NT) cnts[c] = a.ccnt[(int64_t)unit * a.nchunk + c];
  wait_vm<0>();
  __syncthreads();
  uint64_t kand = ~0ull, kor = 0;
  for (int j = tid; j < total; j += NT) {
    const int c = j / a.cap;
    if (j - c * a.cap >= cnts[c]) {
      keys[j] = 0;
    } else if (const uint64_t key = keys[j]) {
      kand &= key;
      kor |= key;
    }
  }
  kth_publish<NT>(sc, kand, kor);
  __syncthreads();
  uint64_t P, M;
  int need;
  block_kth_largest<NT>(keys, total, kp, sc, P, M, need, true);
  block_emit_top<NT>(keys, total, P, M, need, sc,
                     [&](int pos, int i) { row[1 + pos] = dense ? i + 1 : idx[i]; });
}

// One workgroup scores one chunk of a unit's candidate pages 1..n-2, one page per lane
// and round (ppt rounds of NT pages). DPP (groups of up to 8 heads, D <= 128): the whole
// (q+, q-) table in LDS, fed to the FMAs by row broadcasts, statistics staged S chunks
// deep per wave. Otherwise the table is staged 16 heads x DC dims at a time and read as
// LDS broadcasts. When a unit has a single chunk, its top-kp is final and goes straight
// into the selection row; otherwise the chunk's candidates go to the workspace.
//
// With `list` (whole-unit plans only, chunk 0) the ranked winners also go to list[1..b-2]
// in LDS; write_list_header completes the list once the workgroup has passed a barrier.
template <bool BF16, int D, int HB, bool DPP, int NT, int CPL, int S>
__device__ __forceinline__ void score_body(const SelArgs& a, int c, int g, int s, int32_t* list) {
  constexpr int DC = DPP ? D : ((HB * D * 16 <= 32768) ? D : 32);
  constexpr int NDC = D / DC;
  constexpr int NCH = D / MetaGeo<BF16>::CD;
  constexpr int CC = CPL < NCH ? CPL : NCH;
  constexpr int SS = S < NCH / CC ? S : NCH / CC;
  constexpr int STAGE = 512 * CC * SS;  // uint4 per wave
  // (q+, q-) table: fp32 for the DPP path (exact: q is bf16 or fp32), fp64 pairs otherwise
  __shared__ float qf[DPP ? DC * HB * 2 : 1];
  __shared__ double2 qlds[DPP ? 1 : DC * HB];
  __shared__ SelScratch sc;
  extern __shared__ unsigned char lds[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(lds);  // [chunk]

  const int tid = threadIdx.x;
  const int unit = s * a.Hkv + g;
  const int lo = 1 + c * a.chunk;
  const int64_t bt0 = (int64_t)s * a.max_pages;
  // one key slot per lane and round (a one-wave chunk may be narrower than the wave)
  uint4* stage = reinterpret_cast<uint4*>(lds + NT * a.ppt * sizeof(uint64_t)) + (tid >> 6) * STAGE;
  // DPP path: the first page set's block ids and statistics loads go out before the
  // sequence length is known and before the q table is built. The block-table index is
  // clamped to the row and the block id to the pool, so that these loads stay in bounds
  // whatever the row holds past the sequence; lanes past the chunk's pages load a record
  // they never use. A wave that issued them waits for them before it exits.
  // Only the block id stays live across the barrier; the record offsets are recomputed
  // after it (the empty asm keeps the compiler from reusing the first ones).
  const bool pre = DPP && lo + (tid & ~63) < a.max_pages - 1;
  int blk0 = 0;
  if constexpr (DPP) {
    if (pre) {
      blk0 = a.bt[bt0 + min(lo + tid, a.max_pages - 1)];
      blk0 = min(max(blk0, 0), a.num_blocks - 1);
      DppPage<BF16, D, HB, CPL, S> first;
      first.init(a.meta, a.Hkv, blk0, g, stage);
      first.issue_first();
    }
  }
  const UnitInfo u = unit_info(a, s);
  if (c == 0) write_row_header<NT>(a, unit, u);
  const int kp = u.kp, n = u.n;
  const int hi = min(lo + a.chunk, n - 1);
  if (u.trivial || lo >= hi) {
    if (pre) wait_vm<0>();
    return;
  }
  const int cnt = hi - lo;
  const int nhp = ceil_div(a.G, HB);

  auto load_qlds = [&](int hp, int dc) {
    for (int e = tid; e < DC * HB; e += NT) {
      const int d = e / HB, h = e - d * HB, hh = hp * HB + h;
      double qv = 0.0;
      if (hh < a.G) qv = q_value<BF16>(a.q, ((int64_t)s * a.Hq + g * a.G + hh) * D + dc * DC + d);
      if constexpr (DPP) {
        qf[2 * e] = (float)(qv >= 0.0 ? qv : 0.0);
        qf[2 * e + 1] = (float)(qv >= 0.0 ? 0.0 : qv);
      } else {
        qlds[e] = make_double2(qv >= 0.0 ? qv : 0.0, qv >= 0.0 ? 0.0 : qv);
      }
    }
  };
  const bool once = nhp == 1 && NDC == 1;
  // the table's barrier waits only for LDS writes: it is built while the loads fly
  if (once) {
    load_qlds(0, 0);
    if constexpr (DPP) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's table writes are done
      __builtin_amdgcn_s_barrier();
    } else {
      __syncthreads();
    }
  }
  uint64_t kand = ~0ull, kor = 0;  // of this thread's keys, for the ranking
  for (int it = 0; it < a.ppt; ++it) {
    const int o = it * NT + tid;
    if constexpr (DPP) {
      // a wave with no page left in the chunk skips the round (no barrier inside)
      if (it * NT + (tid & ~63) >= cnt) continue;
    }
    const bool have = o < cnt;
    double best = -__builtin_inf();
    if constexpr (DPP) {
      double acc[HB];
#pragma unroll
      for (int h = 0; h < HB; ++h) acc[h] = 0.0;
      if (it == 0) {
        asm volatile("" : "+v"(blk0));
        DppPage<BF16, D, HB, CPL, S> first;
        first.init(a.meta, a.Hkv, blk0, g, stage);
        first.finish(qf, acc);
      } else {
        const int blk = a.bt[bt0 + (have ? lo + o : lo)];
        bound_dpp<BF16, D, HB, CPL, S>(a.meta, a.Hkv, blk, g, qf, stage, acc);
      }
#pragma unroll
      for (int h = 0; h < HB; ++h)
        if (h < a.G && acc[h] > best) best = acc[h];
    } else {
      const int blk = a.bt[bt0 + (have ? lo + o : lo)];
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
          bound_lds<BF16, DC, HB>(a.meta, NCH, a.Hkv, blk, g, dc * DC, qlds, acc);
        }
#pragma unroll
        for (int h = 0; h < HB; ++h)
          if (hp * HB + h < a.G && acc[h] > best) best = acc[h];
      }
    }
    const uint64_t key = score_key(best);
    keys[o] = key;  // every slot written; slots past cnt are never read
    if (have && key) {
      kand &= key;
      kor |= key;
    }
  }
  if constexpr (DPP) {
    if (pre) wait_vm<0>();  // a wave that skipped every round still has its first loads
  }
  kth_publish<NT>(sc, kand, kor);
  __syncthreads();

  if (a.nchunk == 1) {  // the chunk is the whole unit: its top-kp is the selection
    int32_t* row = a.sel + (int64_t)unit * a.b_max;
    uint64_t P, M;
    int need;
    block_kth_largest<NT>(keys, cnt, kp, sc, P, M, need, true);
    // the list's sink and tail entries (every staged load has landed: the ranking's
    // barriers follow each wave's wait for its loads)
    if (list && tid == 0) {
      list[0] = 0;
      list[kp + 1] = n - 1;
    }
    block_emit_top<NT>(keys, cnt, P, M, need, sc, [&](int pos, int i) {
      row[1 + pos] = 1 + i;
      if (list) list[1 + pos] = 1 + i;
    });
    return;
  }
  // Chunk candidates: all pages when they fit in kp, else the chunk's top-kp.
  uint64_t* okey = a.ckey + (int64_t)unit * a.ustride + c * a.cap;
  int32_t* oidx = a.cidx + (int64_t)unit * a.ustride + c * a.cap;
  if (cnt <= kp || a.cap == a.chunk) {  // every page of the chunk is a candidate
    for (int o = tid; o < cnt; o += NT) {
      okey[o] = keys[o];
      if (a.cap < a.chunk) oidx[o] = lo + o;
    }
    if (tid == 0) a.ccnt[(int64_t)unit * a.nchunk + c] = cnt;
  } else {
    uint64_t P, M;
    int need;
    block_kth_largest<NT>(keys, cnt, kp, sc, P, M, need, true);
    const int emitted = block_emit_top<NT>(keys, cnt, P, M, need, sc, [&](int pos, int i) {
      okey[pos] = keys[i];
      oidx[pos] = lo + i;
    });
    if (tid == 0) a.ccnt[(int64_t)unit * a.nchunk + c] = emitted;
  }
}

// The tail page's statistics of unit (s, g), as the statistics kernel writes them. The
// tail page is never a ranking candidate, so no scoring or merging workgroup of the same
// step reads them.
__device__ void refresh_tail(const SelArgs& a, int g, int s) {
  if (a.bf16)
    refresh_tail_page<true>(a.k, a.meta_w, a.bt, a.lens, a.max_pages, s, g, a.Hkv, a.D, a.kbs,
                            a.kts, a.khs, threadIdx.x, blockDim.x);
  else
    refresh_tail_page<false>(a.k, a.meta_w, a.bt, a.lens, a.max_pages, s, g, a.Hkv, a.D, a.kbs,
                             a.kts, a.khs, threadIdx.x, blockDim.x);
}

template <bool BF16, int D, int HB, bool DPP, int NT, int CPL, int S>
__global__ __launch_bounds__(NT) void score_kernel(SelArgs a) {
  int c = blockIdx.x;
  if (a.meta_w) {
    if (c == 0) {
      refresh_tail(a, blockIdx.y, blockIdx.z);
      return;
    }
    --c;
  }
  score_body<BF16, D, HB, DPP, NT, CPL, S>(a, c, blockIdx.y, blockIdx.z, nullptr);
}

template <int NT>
__global__ __launch_bounds__(NT) void merge_kernel(SelArgs a) {
  __shared__ SelScratch sc;
  extern __shared__ unsigned char lds[];
  const int g = blockIdx.x, s = blockIdx.y;
  if (blockIdx.z == 1) {  // the unit's tail refresh (decode step)
    refresh_tail(a, g, s);
    return;
  }
  const UnitInfo u = unit_info(a, s);
  if (u.trivial) return;
  merge_unit<NT>(a, s * a.Hkv + g, u.n, u.kp, lds, sc);
}

template <typename K>
hipError_t set_lds(K kernel, size_t lds) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// Tuning of the scoring workgroups (defaults measured on MI355X): statistics chunks per
// load group (CPL) and load groups in flight per wave (STAGES).
#ifndef PSD_UNIT_THREADS
#define PSD_UNIT_THREADS 1024  // whole-unit workgroups
#endif
#ifndef PSD_UNIT_CPL
#define PSD_UNIT_CPL 2
#endif
#ifndef PSD_UNIT_STAGES
#define PSD_UNIT_STAGES 1
#endif
#ifndef PSD_CHUNK_CPL
#define PSD_CHUNK_CPL 1  // 256-thread chunk workgroups
#endif
#ifndef PSD_CHUNK_STAGES
#define PSD_CHUNK_STAGES 1
#endif
#ifndef PSD_WAVE_CHUNK
#define PSD_WAVE_CHUNK 64  // pages of a one-wave chunk workgroup
#endif
#ifndef PSD_MERGE_BIG
#define PSD_MERGE_BIG 1024  // candidates above which a unit merge takes 1024 threads
#endif
#ifndef PSD_WAVE_WG_MAX
#define PSD_WAVE_WG_MAX 512  // one-wave chunk workgroups below this many 256-page chunks
#endif
#ifndef PSD_MIN_PPT
#define PSD_MIN_PPT 1
#endif
#ifndef PSD_UNIT_MIN_UNITS
#define PSD_UNIT_MIN_UNITS 128  // units that fill the GPU with one workgroup each
#endif

template <bool BF16, int D, int HB, bool DPP, int NT, int CPL, int S>
hipError_t launch_score(const SelArgs& a, const SelectPlan& p, dim3 sgrid, hipStream_t st) {
  hipError_t e = set_lds(&score_kernel<BF16, D, HB, DPP, NT, CPL, S>, p.score_lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_kernel<BF16, D, HB, DPP, NT, CPL, S>), sgrid, dim3(NT), p.score_lds,
                     st, a);
  return hipGetLastError();
}

// (threads, chunks per load group, groups in flight) triples the planner picks from;
// (CPL, S) = (1, 1) is the fallback when the tuned staging does not fit in LDS.
// 1024-thread workgroups are built for 4-head groups only: at the 128-VGPR budget of 16
// waves per CU the 8-head accumulators spill, so 8-head whole units take 512 threads.
template <bool BF16, int D, int HB>
hipError_t dispatch_dpp(const SelArgs& a, const SelectPlan& p, dim3 grid, hipStream_t st) {
  const bool tuned = p.cpl > 1 || p.stages > 1;
  switch (p.threads) {
    case 64: return launch_score<BF16, D, HB, true, 64, 4, 1>(a, p, grid, st);
    case 256:
      return tuned ? launch_score<BF16, D, HB, true, 256, PSD_CHUNK_CPL, PSD_CHUNK_STAGES>(a, p, grid, st)
                   : launch_score<BF16, D, HB, true, 256, 1, 1>(a, p, grid, st);
    case 512:
      return tuned ? launch_score<BF16, D, HB, true, 512, PSD_UNIT_CPL, PSD_UNIT_STAGES>(a, p, grid, st)
                   : launch_score<BF16, D, HB, true, 512, 1, 1>(a, p, grid, st);
    default:
      if constexpr (HB == 4) return launch_score<BF16, D, HB, true, 1024, 1, 1>(a, p, grid, st);
      return hipErrorInvalidValue;  // not planned: plan_select gives 8-head units 512 threads
  }
}

template <bool BF16, int D>
hipError_t dispatch_hb(const SelArgs& a, const SelectPlan& p, dim3 grid, hipStream_t st) {
  if constexpr (D > 128) {
    return launch_score<BF16, D, 16, false, kThreads, 1, 1>(a, p, grid, st);
  } else {
    switch (p.head_block) {
      case 4: return dispatch_dpp<BF16, D, 4>(a, p, grid, st);
      case 8: return dispatch_dpp<BF16, D, 8>(a, p, grid, st);
      default: return launch_score<BF16, D, 16, false, kThreads, 1, 1>(a, p, grid, st);
    }
  }
}

// One workgroup per (sequence, KV head) unit does the whole sparse decode of the unit:
// it scores and ranks the unit's pages as score_kernel does for a whole-unit plan (and
// writes the selection row and count the same way), keeps the page list in LDS at
// `list_off`, and then attends over it as the whole-unit attention kernel does, its 16
// waves being the splits. The list lies past both the ranking keys and the attention's
// closing combine area, inside the statistics staging area: a ranking unit's entries
// (winners, sink and tail) are written by the emission, which follows the last staged
// load; a unit that needs no ranking writes its entries after the barrier that follows
// the scoring.
//
// With `meta_w` (decode step) the workgroup also refreshes the statistics of its
// sequence's tail page for its KV head, as the statistics kernel does for the tail page.
// The tail page is never a ranking candidate, so the refresh is independent of the
// ranking; the last wave, which has the fewest pages to attend, does it before the waves
// are combined.
template <bool BF16, int D, int HB, bool REFRESH, bool KT>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4)))
void select_attn_kernel(SelArgs a, AttnArgs aa, int list_off, int kt_off, int kt_stride,
                        void* meta_w, int64_t kbs, int64_t kts, int64_t khs) {
  static_assert(PSD_ATTN_UNIT_WAVES == 16, "one attention split per wave of the workgroup");
  // Built only where it fits the 128 VGPRs of 16 waves per CU without spilling: 4-head
  // groups, and fp32 only at D = 64 (8-head groups and fp32 at D = 128 spill).
  static_assert(HB == 4 && (BF16 || D <= 64), "fused step: no spill-free build");
  extern __shared__ unsigned char lds[];
  int32_t* list = reinterpret_cast<int32_t*>(lds + list_off);
#if PSD_FUSED_XCD_MAP
  // workgroup i runs on XCD i % 8: give each XCD a contiguous range of units, so that
  // the KV heads of a sequence share an XCD (and its L2)
  const int U = gridDim.x * gridDim.y, i = blockIdx.x + blockIdx.y * gridDim.x;
  const int u = (U % 8 == 0) ? (i % 8) * (U / 8) + i / 8 : i;
  const int g = u % a.Hkv, s = u / a.Hkv;
#else
  const int g = blockIdx.x, s = blockIdx.y;
#endif
  score_body<BF16, D, HB, true, 1024, 1, 1>(a, 0, g, s, list);
  __syncthreads();  // every staged load has landed; the ranking keys are no longer read
  // A ranking unit's list is complete (its emission wrote the sink and tail too); a unit
  // that needs no ranking writes its list now.
  const UnitInfo ui = unit_info(a, s);
  int count = ui.b;
  if (ui.trivial) {
    count = write_list_header<1024>(list, ui, a.b_max);
    __syncthreads();
  }
  // The tail refresh feeds only later steps (a tail page is always kept, never scored),
  // so of each pair of sequences (s, s ^ 1) the shorter one's workgroup refreshes both
  // tails of head g and the longer one's none: the longest units end without it.
  auto refresh_tail = [&]() {
    if constexpr (REFRESH) {
      if ((threadIdx.x >> 6) == 15) {  // all 16 rows at once: the attention's registers are free
        const int ps = s ^ 1;
        bool own = true, pair = false;
        if (ps < (int)gridDim.y) {
          const int ls = a.lens[s], lp = a.lens[ps];
          own = pair = ls < lp || (ls == lp && (s & 1) == 0);
        }
        if (own)
          refresh_tail_page<BF16, kPage>(aa.k, meta_w, a.bt, a.lens, a.max_pages, s, g, a.Hkv,
                                         D, kbs, kts, khs, threadIdx.x & 63, 64);
        if (pair)
          refresh_tail_page<BF16, kPage>(aa.k, meta_w, a.bt, a.lens, a.max_pages, ps, g, a.Hkv,
                                         D, kbs, kts, khs, threadIdx.x & 63, 64);
      }
    }
  };
  attn_body<BF16, D, D, 1, 16, decltype(refresh_tail), false, KT>(aa, 0, g, s, list, count,
                                                                   refresh_tail, lds + kt_off,
                                                                   kt_stride);
}

struct FusedLayout {
  size_t list_off, lds;        // byte offset of the page list; dynamic LDS
  bool kt;                     // K through the waves' LDS tiles
  size_t kt_off, kt_stride;    // first tile, distance between tiles
};

template <bool BF16, int D, bool REFRESH, bool KT>
hipError_t launch_fused(const SelArgs& a, const AttnArgs& aa, int head_block, dim3 grid,
                        const FusedLayout& L, void* meta_w, const Geo& g, hipStream_t st) {
  if (head_block != 4) return hipErrorInvalidValue;  // fused_applies admits 4-head groups only
  auto kern = &select_attn_kernel<BF16, D, 4, REFRESH, KT>;
  hipError_t e = set_lds(kern, L.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(1024), L.lds, st, a, aa, (int)L.list_off, (int)L.kt_off,
                     (int)L.kt_stride, meta_w, g.kbs, g.kts, g.khs);
  return hipGetLastError();
}

// bf16 at D = 128 is built with the K tiles only (fused_applies admits no other layout).
template <bool BF16, int D>
hipError_t launch_fused_r(const SelArgs& a, const AttnArgs& aa, int head_block, dim3 grid,
                          const FusedLayout& L, void* meta_w, const Geo& g, hipStream_t st) {
  constexpr bool KT = BF16 && D == 128;
  if (L.kt != KT) return hipErrorInvalidValue;
  return meta_w ? launch_fused<BF16, D, true, KT>(a, aa, head_block, grid, L, meta_w, g, st)
                : launch_fused<BF16, D, false, KT>(a, aa, head_block, grid, L, meta_w, g, st);
}

// Static LDS of the fused kernel (the scoring's query copies and scratch).
size_t fused_static_lds(const Geo& g, const SelectPlan& sp) {
  return (size_t)g.D * sp.head_block * 2 * sizeof(float) + sizeof(double2) + sizeof(SelScratch);
}

// Dynamic LDS of the fused launch. The scoring's keys and staging come first; once the
// ranking is done, the closing combine's area reuses the start and the page list follows
// it. At bf16, D = 128 the waves' K tiles sit inside their combine parts, or past the
// list where those are too small; `kt` is false where they would not fit, and
// fused_applies then turns the launch down.
FusedLayout fused_layout(const Geo& g, const SelectPlan& sp, int b_max) {
  FusedLayout L;
  const size_t keys = (size_t)sp.threads * sp.ppt * sizeof(uint64_t);
  const size_t combine = unit_combine_lds(g);
  L.list_off = ((keys > combine ? keys : combine) + 255) / 256 * 256;
  const size_t end = L.list_off + (size_t)b_max * sizeof(int32_t);
  L.lds = end > sp.score_lds ? end : sp.score_lds;
  L.kt = false;
  L.kt_off = L.kt_stride = 0;
  if (g.dtype == 1 && g.D == 128) {
    const KTilePlace kp = ktile_place(g, PSD_ATTN_UNIT_WAVES, end);
    const size_t lds = kp.end > L.lds ? kp.end : L.lds;
    if (fused_static_lds(g, sp) + lds <= 160 * 1024) {
      L.kt = true;
      L.kt_off = kp.off;
      L.kt_stride = kp.stride;
      L.lds = lds;
    }
  }
  return L;
}

}  // namespace

bool plan_select(const Geo& g, int b_max, SelectPlan* p) {
  if (b_max < 2) return false;
  p->prescore = false;
  if (prescore_applies(g)) {
    // certified MFMA pre-score: ~256 workgroups of up to 64 tiles of 16 pages
    const int max_inner = g.max_pages > 2 ? g.max_pages - 2 : 1;
    const int64_t tiles = (max_inner + 15) / 16;
    const int64_t units = (int64_t)g.B * g.Hkv;
    int64_t tpw = (units * tiles + 255) / 256;
    tpw = tpw < 1 ? 1 : (tpw > 64 ? 64 : tpw);
    p->prescore = true;
    p->ppt = (int)tpw;
    p->nchunk = (int)((tiles + tpw - 1) / tpw);
    p->chunk = 16 * p->ppt;
    p->threads = 64 * (g.G / 16);
    p->cap = 0;
    p->ustride = 0;
    p->cpl = p->stages = 1;
    p->head_block = 16;
    p->d_chunk = g.D;
    p->all_q = false;
    p->merge_threads = 1024;
    p->merge_lds = prescore_lds(max_inner);
    p->score_lds = 0;
    const size_t plane = ((size_t)units * max_inner * sizeof(float) + 255) / 256 * 256;
    // planes: approximate group score, page maximum, runner-up, leading head; q norms
    p->off_idx = plane;
    p->off_cnt = 4 * plane;
    p->bytes = 4 * plane + (size_t)units * sizeof(double) + 256;
    return true;
  }
  constexpr size_t kLdsLimit = 160 * 1024;
  const int kcap = b_max - 2;
  const int inner = g.max_pages > 2 ? g.max_pages - 2 : 1;
  const int64_t units = (int64_t)g.B * g.Hkv;
  // Groups of up to 8 heads with D <= 128 take q through DPP broadcasts (whole table in
  // LDS); other groups read it as LDS broadcasts, 16 heads at a time.
  p->all_q = g.G <= 16 && g.D <= 128;
  p->head_block = !p->all_q ? 16 : (g.G <= 4 ? 4 : (g.G <= 8 ? 8 : 16));
  p->d_chunk = p->all_q ? g.D : ((16 * g.D * 16 <= 32768) ? g.D : 32);
  const bool dpp = p->all_q && p->head_block <= 8;
  const size_t static_lds = (size_t)p->d_chunk * p->head_block * (dpp ? 8 : 16) + 1536;
  const int nch = g.D / (g.dtype == 1 ? 32 : 16);  // 64-byte statistics chunks per record
  // LDS staging per wave for (chunks per group, groups in flight), as the kernel clamps them
  auto stage_bytes = [&](int cpl, int st) {
    const int c = cpl < nch ? cpl : nch;
    const int ss = st < nch / c ? st : nch / c;
    return (size_t)8192 * c * ss;
  };
  // the tuned staging of a workgroup size if it fits, else one chunk at a time
  auto pick_staging = [&](int cpl, int st) {
    const size_t keys = (size_t)p->threads * p->ppt * 8;
    if (cpl == 4 && p->threads == 64) st = 1;
    if (static_lds + keys + (size_t)(p->threads / 64) * stage_bytes(cpl, st) <= kLdsLimit) {
      p->cpl = cpl;
      p->stages = st;
    } else {
      p->cpl = 1;
      p->stages = 1;
    }
  };
  bool ok = false;
  if (dpp && inner <= 2048 && (units >= PSD_UNIT_MIN_UNITS || small_units(g))) {
    // one workgroup per unit: scores every page and ranks them, no merge
    p->threads = p->head_block == 4 ? PSD_UNIT_THREADS : 512;
    p->ppt = (inner + p->threads - 1) / p->threads;
    p->chunk = p->threads * p->ppt;
    p->nchunk = 1;
    p->cap = p->chunk;
    if (p->threads == 512)
      pick_staging(PSD_UNIT_CPL, PSD_UNIT_STAGES);
    else if (p->threads == 256)
      pick_staging(PSD_CHUNK_CPL, PSD_CHUNK_STAGES);
    else
      pick_staging(1, 1);
    ok = true;
  } else {
    // one-wave workgroups when 256-thread ones would leave the GPU mostly idle
    p->threads = (dpp && units * ((inner + kThreads - 1) / kThreads) < PSD_WAVE_WG_MAX) ? 64 : kThreads;
    const bool multi_pass = !p->all_q && (g.G > 16 || 16 * g.D * 16 > 32768);
    for (int ppt = PSD_MIN_PPT; ppt <= 64; ppt *= 2) {
      if (multi_pass && ppt > 1) break;
      // a one-wave workgroup may take fewer pages than lanes: more waves share a unit
      const int chunk = p->threads == 64 && ppt == 1 ? PSD_WAVE_CHUNK : p->threads * ppt;
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
    if (ok) {
      if (!dpp) {
        p->cpl = 1;
        p->stages = 1;
      } else if (p->threads == 64) {
        pick_staging(4, 1);
      } else {
        pick_staging(PSD_CHUNK_CPL, PSD_CHUNK_STAGES);
      }
    }
  }
  if (!ok) return false;
  // candidate slots per unit, padded so that a merge copies whole 1 KB slices
  p->ustride = p->nchunk == 1 ? 0 : (p->nchunk * p->cap + 255) / 256 * 256;
  const size_t slots = (size_t)units * p->ustride;
  p->merge_lds = (size_t)p->ustride * (sizeof(uint64_t) + sizeof(int32_t)) +
                 (size_t)p->nchunk * sizeof(int32_t);
  const int64_t cands = (int64_t)p->nchunk * p->cap;
  p->merge_threads = cands <= 512 ? 64 : (cands <= PSD_MERGE_BIG ? kThreads : 1024);
  p->score_lds = (size_t)p->threads * p->ppt * sizeof(uint64_t);
  if (dpp) p->score_lds += (size_t)(p->threads / 64) * stage_bytes(p->cpl, p->stages);
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
                 g.num_blocks, p.ustride, nullptr, nullptr, g.kbs, g.kts, g.khs, g.dtype == 1};
}

hipError_t launch_select_score(const Geo& g, const SelectPlan& p, const void* q,
                               const void* meta, const int32_t* bt, const int32_t* lens,
                               const int32_t* budgets, int b_max, int32_t* sel, int32_t* cnt,
                               void* ws, hipStream_t st, void* meta_tail, const void* k) {
  if (p.prescore)
    return launch_prescore(g, p, q, meta, bt, lens, budgets, b_max, sel, cnt, ws, st);
  SelArgs a = make_args(g, p, q, meta, bt, lens, budgets, b_max, sel, cnt, ws);
  a.meta_w = meta_tail;
  a.k = k;
  const dim3 sgrid(p.nchunk + (meta_tail ? 1 : 0), g.Hkv, g.B);
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

RefreshSite refresh_site(const Geo& g, const SelectPlan& p) {
  if (!p.prescore && (int64_t)p.nchunk * g.Hkv * g.B <= kComputeUnits) return kRefreshInScore;
  if (p.prescore || p.nchunk > 1) return kRefreshInMerge;
  return kRefreshOwnLaunch;
}

// The merge runs as its own launch: the kernel boundary makes every chunk's candidates
// visible (a device-scope fence inside the scoring kernel writes back and invalidates
// the L2).
hipError_t launch_select_merge(const Geo& g, const SelectPlan& p, const void* q,
                               const void* meta, const int32_t* bt, const int32_t* lens,
                               const int32_t* budgets, int b_max, int32_t* sel, void* ws,
                               hipStream_t st, void* meta_tail, const void* k) {
  if (p.prescore)
    return launch_certify(g, p, q, meta, bt, lens, budgets, b_max, sel, ws, st, meta_tail, k);
  if (p.nchunk == 1) return hipSuccess;  // the scoring stage ranked every unit completely
  SelArgs a = make_args(g, p, nullptr, nullptr, bt, lens, budgets, b_max, sel, nullptr, ws);
  a.meta_w = meta_tail;
  a.k = k;
  const dim3 ugrid(g.Hkv, g.B, meta_tail ? 2 : 1);
  hipError_t e;
  if (p.merge_threads == 64) {
    if ((e = set_lds(&merge_kernel<64>, p.merge_lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(merge_kernel<64>, ugrid, dim3(64), p.merge_lds, st, a);
  } else if (p.merge_threads == 1024) {
    if ((e = set_lds(&merge_kernel<1024>, p.merge_lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(merge_kernel<1024>, ugrid, dim3(1024), p.merge_lds, st, a);
  } else {
    if ((e = set_lds(&merge_kernel<kThreads>, p.merge_lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(merge_kernel<kThreads>, ugrid, dim3(kThreads), p.merge_lds, st, a);
  }
  return hipGetLastError();
}

bool fused_applies(const Geo& g, const SelectPlan& sp, const DecodePlan& dp, int b_max) {
  if (sp.prescore || sp.nchunk != 1 || sp.threads != 1024 || !sp.all_q) return false;
  if (sp.head_block != 4 || (g.dtype != 1 && g.D > 64)) return false;  // spill-free builds
  if (sp.cpl != 1 || sp.stages != 1) return false;
  if (dp.unit != 16 || g.D > 128 || g.Dv != g.D) return false;
  const FusedLayout L = fused_layout(g, sp, b_max);
  if (L.kt != (g.dtype == 1 && g.D == 128)) return false;  // the build takes K tiles there
  return fused_static_lds(g, sp) + L.lds <= 160 * 1024;
}

hipError_t launch_select_decode(const Geo& g, const SelectPlan& sp, const DecodePlan& dp,
                                const void* q, const void* meta, const void* k, const void* v,
                                const int32_t* bt, const int32_t* lens, const int32_t* budgets,
                                int b_max, float scale, int32_t* sel, int32_t* cnt, float* out,
                                void* ws, void* meta_tail, hipStream_t st) {
  const SelArgs a = make_args(g, sp, q, meta, bt, lens, budgets, b_max, sel, cnt, ws);
  const AttnArgs aa = make_attn_args(g, dp, q, k, v, bt, lens, sel, cnt, b_max, scale, out, ws);
  const FusedLayout L = fused_layout(g, sp, b_max);
  const dim3 grid(g.Hkv, g.B);
  const bool bf = g.dtype == 1;
  if (g.D == 64)
    return bf ? launch_fused_r<true, 64>(a, aa, sp.head_block, grid, L, meta_tail, g, st)
              : launch_fused_r<false, 64>(a, aa, sp.head_block, grid, L, meta_tail, g, st);
  if (!bf) return hipErrorInvalidValue;  // fp32 at D = 128: no fused build (fused_applies)
  return launch_fused_r<true, 128>(a, aa, sp.head_block, grid, L, meta_tail, g, st);
}

}  // namespace psd
