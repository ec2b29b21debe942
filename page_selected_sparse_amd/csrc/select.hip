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

struct ScoreArgs {
  const void* q;
  const void* meta;
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* budgets;
  uint64_t* ckey;
  int32_t* cidx;
  int32_t* ccnt;
  int Hq, Hkv, G, max_pages, chunk, ppt, nchunk, cap;
};

struct MergeArgs {
  const int32_t* lens;
  const int32_t* budgets;
  const uint64_t* ckey;
  const int32_t* cidx;
  const int32_t* ccnt;
  int32_t* sel;
  int32_t* cnt;
  int Hkv, b_max, chunk, nchunk, cap;
};

struct SelScratch {
  uint32_t hist[256];
  int wave_cnt[4];
  int digit, k;
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
// total, for a 256-thread workgroup. Contains barriers: every thread must call it.
__device__ __forceinline__ int block_excl_count(bool flag, SelScratch& sc, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) sc.wave_cnt[w] = __popcll(m);
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = sc.wave_cnt[i];
    off += i < w ? c : 0;
    total += c;
  }
  __syncthreads();
  return off + below;
}

// K-th largest (1-based) of keys[0..N) in LDS, 1 <= K <= N. Returns the key T and how
// many of the keys equal to T belong to the top K. Radix select over 8-bit digits from
// the most significant; equal digits met in a row by one thread are counted once.
__device__ void block_kth_largest(const uint64_t* keys, int N, int K, SelScratch& sc,
                                  uint64_t& T, int& need) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0, mask = 0;
  int k = K;
  for (int shift = 56; shift >= 0; shift -= 8) {
    sc.hist[tid] = 0;
    __syncthreads();
    int run_d = -1, run_c = 0;
    for (int i = tid; i < N; i += kThreads) {
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
        int r = k - excl, dg;
        if (r <= c0) {
          dg = base;
        } else if (r <= c0 + c1) {
          r -= c0;
          dg = base - 1;
        } else if (r <= c0 + c1 + c2) {
          r -= c0 + c1;
          dg = base - 2;
        } else {
          r -= c0 + c1 + c2;
          dg = base - 3;
        }
        sc.digit = dg;
        sc.k = r;
      }
    }
    __syncthreads();
    prefix |= (uint64_t)sc.digit << shift;
    mask |= 255ull << shift;
    k = sc.k;
  }
  T = prefix;
  need = k;
}

// Emits, in position order, every key > T and the first `need` keys == T; calls
// out(rank, position) for each. Returns the number emitted. Every thread must call it.
template <typename Out>
__device__ int block_emit_top(const uint64_t* keys, int N, uint64_t T, int need, SelScratch& sc,
                              Out out) {
  int run_eq = 0, run_out = 0;
  for (int base = 0; base < N; base += kThreads) {
    const int i = base + threadIdx.x;
    const bool ok = i < N;
    const uint64_t key = ok ? keys[i] : 0;
    const bool gt = ok && key > T, eq = ok && key == T;
    int tot_eq, tot_sel;
    const int eq_rank = run_eq + block_excl_count(eq, sc, tot_eq);
    const bool pick = gt || (eq && eq_rank < need);
    const int pos = run_out + block_excl_count(pick, sc, tot_sel);
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

// Bound contribution of dims [d0, d0 + DC) of one page for HB heads, ascending d.
template <bool BF16, int DC, int HB>
__device__ __forceinline__ void accumulate_bound(const void* meta, int64_t row, int D,
                                                 const double2* qt, double* acc) {
  if constexpr (BF16) {
    const uint16_t* mn = static_cast<const uint16_t*>(meta) + row;
    const uint16_t* mx = mn + D;
#pragma unroll
    for (int d0 = 0; d0 < DC; d0 += 8) {
      const uint4 a = load16(mn + d0), b = load16(mx + d0);
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double kmn = (double)((j & 1) ? bf_hi(aw[j >> 1]) : bf_lo(aw[j >> 1]));
        const double kmx = (double)((j & 1) ? bf_hi(bw[j >> 1]) : bf_lo(bw[j >> 1]));
#pragma unroll
        for (int h = 0; h < HB; ++h) {
          const double2 qq = qt[(d0 + j) * HB + h];
          acc[h] = __builtin_fma(qq.x, kmx, acc[h]);
          acc[h] = __builtin_fma(qq.y, kmn, acc[h]);
        }
      }
    }
  } else {
    const float* mn = static_cast<const float*>(meta) + row;
    const float* mx = mn + D;
#pragma unroll
    for (int d0 = 0; d0 < DC; d0 += 4) {
      const float4 a = *reinterpret_cast<const float4*>(mn + d0);
      const float4 b = *reinterpret_cast<const float4*>(mx + d0);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double kmn = (double)av[j], kmx = (double)bv[j];
#pragma unroll
        for (int h = 0; h < HB; ++h) {
          const double2 qq = qt[(d0 + j) * HB + h];
          acc[h] = __builtin_fma(qq.x, kmx, acc[h]);
          acc[h] = __builtin_fma(qq.y, kmn, acc[h]);
        }
      }
    }
  }
}

template <bool BF16, int D, int HB>
__global__ __launch_bounds__(kThreads) void score_kernel(ScoreArgs a) {
  // q table (q+, q-) for HB heads over DC dims; whole D when it fits in 32 KB.
  constexpr int DC = (HB * D * 16 <= 32768) ? D : 32;
  constexpr int NDC = D / DC;
  __shared__ double2 qtab[DC * HB];
  __shared__ SelScratch sc;
  extern __shared__ uint64_t keys[];  // [chunk]

  const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x;
  const int L = a.lens[s];
  const int n = ceil_div(L, kPage);
  const int b = effective_budget(n, a.budgets[s]);
  if (n <= b) return;  // every page kept; the merge writes them
  const int kp = b - 2;
  if (kp <= 0 || kp > a.cap) return;  // kp > cap: budget beyond b_max, the merge flags it
  const int lo = 1 + c * a.chunk;
  const int hi = min(lo + a.chunk, n - 1);
  if (lo >= hi) return;
  const int cnt = hi - lo;
  const int unit = s * a.Hkv + g;
  const int nhp = ceil_div(a.G, HB);
  const bool once = (nhp == 1 && NDC == 1);

  auto load_qtab = [&](int hp, int dc) {
    for (int e = tid; e < DC * HB; e += kThreads) {
      const int d = e / HB, h = e - d * HB, hh = hp * HB + h;
      double qv = 0.0;
      if (hh < a.G) qv = q_value<BF16>(a.q, ((int64_t)s * a.Hq + g * a.G + hh) * D + dc * DC + d);
      qtab[e] = make_double2(qv >= 0.0 ? qv : 0.0, qv >= 0.0 ? 0.0 : qv);
    }
  };

  if (once) {
    load_qtab(0, 0);
    __syncthreads();
  }
  for (int it = 0; it < a.ppt; ++it) {
    const int o = it * kThreads + tid;
    const bool have = o < cnt;
    const int blk = have ? a.bt[(int64_t)s * a.max_pages + lo + o] : 0;
    const int64_t row = ((int64_t)blk * a.Hkv + g) * 2 * D;
    double best = -__builtin_inf();
    for (int hp = 0; hp < nhp; ++hp) {
      double acc[HB];
#pragma unroll
      for (int h = 0; h < HB; ++h) acc[h] = 0.0;
      for (int dc = 0; dc < NDC; ++dc) {
        if (!once) {
          __syncthreads();
          load_qtab(hp, dc);
          __syncthreads();
        }
        if (have) accumulate_bound<BF16, DC, HB>(a.meta, row + dc * DC, D, qtab, acc);
      }
#pragma unroll
      for (int h = 0; h < HB; ++h)
        if (hp * HB + h < a.G && acc[h] > best) best = acc[h];
    }
    if (have) keys[o] = score_key(best);
  }
  __syncthreads();

  uint64_t* okey = a.ckey + ((int64_t)unit * a.nchunk + c) * a.cap;
  int32_t* oidx = a.cidx + ((int64_t)unit * a.nchunk + c) * a.cap;
  if (cnt <= kp) {
    for (int o = tid; o < cnt; o += kThreads) {
      okey[o] = keys[o];
      oidx[o] = lo + o;
    }
    if (tid == 0) a.ccnt[(int64_t)unit * a.nchunk + c] = cnt;
    return;
  }
  uint64_t T;
  int need;
  block_kth_largest(keys, cnt, kp, sc, T, need);
  const int emitted = block_emit_top(keys, cnt, T, need, sc, [&](int pos, int i) {
    okey[pos] = keys[i];
    oidx[pos] = lo + i;
  });
  if (tid == 0) a.ccnt[(int64_t)unit * a.nchunk + c] = emitted;
}

__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  __shared__ SelScratch sc;
  __shared__ int chunk_off[kMaxChunks + 1];
  extern __shared__ unsigned char lds[];
  const int g = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int unit = s * a.Hkv + g;
  const int L = a.lens[s];
  const int n = ceil_div(L, kPage);
  const int b = effective_budget(n, a.budgets[s]);
  int32_t* row = a.sel + (int64_t)unit * a.b_max;
  if (b > a.b_max) {  // never truncate: flag the unit
    for (int i = tid; i < a.b_max; i += kThreads) row[i] = -1;
    if (tid == 0) a.cnt[unit] = -1;
    return;
  }
  if (n <= b) {
    for (int i = tid; i < a.b_max; i += kThreads) row[i] = i < n ? i : -1;
    if (tid == 0) a.cnt[unit] = n;
    return;
  }
  for (int i = b + tid; i < a.b_max; i += kThreads) row[i] = -1;
  if (tid == 0) {
    a.cnt[unit] = b;
    row[0] = 0;
    row[b - 1] = n - 1;
  }
  const int kp = b - 2;
  if (kp <= 0) return;

  // Concatenate the chunk candidate lists; chunks are in page order and so is each list.
  const int nch = ceil_div(n - 2, a.chunk);
  uint64_t* keys = reinterpret_cast<uint64_t*>(lds);
  int32_t* idx = reinterpret_cast<int32_t*>(lds + sizeof(uint64_t) * (size_t)a.nchunk * a.cap);
  for (int c = tid; c < nch; c += kThreads) chunk_off[c] = a.ccnt[(int64_t)unit * a.nchunk + c];
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < nch; base += kThreads) {  // exclusive scan of the counts
    const int c = base + tid;
    const int v = c < nch ? chunk_off[c] : 0;
    const int lane = tid & 63, w = tid >> 6;
    const int incl = wave_inclusive_scan(v);
    if (lane == 63) sc.wave_cnt[w] = incl;
    __syncthreads();
    int off = carry, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      off += i < w ? sc.wave_cnt[i] : 0;
      tot += sc.wave_cnt[i];
    }
    __syncthreads();
    if (c < nch) chunk_off[c] = off + incl - v;
    carry += tot;
  }
  if (tid == 0) chunk_off[nch] = carry;
  __syncthreads();
  const int total = carry;
  for (int j = tid; j < nch * a.cap; j += kThreads) {
    const int c = j / a.cap, i = j - c * a.cap;
    const int o = chunk_off[c];
    if (i < chunk_off[c + 1] - o) {
      const int64_t src = ((int64_t)unit * a.nchunk + c) * a.cap + i;
      keys[o + i] = a.ckey[src];
      idx[o + i] = a.cidx[src];
    }
  }
  __syncthreads();

  uint64_t T;
  int need;
  block_kth_largest(keys, total, kp, sc, T, need);
  block_emit_top(keys, total, T, need, sc, [&](int pos, int i) { row[1 + pos] = idx[i]; });
}

template <bool BF16, int D, int HB>
hipError_t launch_score(const ScoreArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel<BF16, D, HB>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_kernel<BF16, D, HB>), grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t dispatch_hb(const ScoreArgs& a, int hb, dim3 grid, size_t lds, hipStream_t st) {
  switch (hb) {
    case 4: return launch_score<BF16, D, 4>(a, grid, lds, st);
    case 8: return launch_score<BF16, D, 8>(a, grid, lds, st);
    default: return launch_score<BF16, D, 16>(a, grid, lds, st);
  }
}

}  // namespace

bool plan_select(const Geo& g, int b_max, SelectPlan* p) {
  if (b_max < 2) return false;
  const int kcap = b_max - 2;
  const int inner = g.max_pages > 2 ? g.max_pages - 2 : 1;
  p->head_block = g.G <= 4 ? 4 : (g.G <= 8 ? 8 : 16);
  const int hb = p->head_block;
  const bool multi_pass = (g.G > hb) || (hb * g.D * 16 > 32768);
  p->d_chunk = (hb * g.D * 16 <= 32768) ? g.D : 32;
  bool ok = false;
  for (int ppt = 1; ppt <= 32; ppt *= 2) {
    if (multi_pass && ppt > 1) break;
    const int chunk = kThreads * ppt;
    const int nchunk = (inner + chunk - 1) / chunk;
    const int cap = kcap < 1 ? 1 : (kcap < chunk ? kcap : chunk);
    if ((int64_t)nchunk * cap <= kMergeCap && nchunk <= kMaxChunks) {
      p->ppt = ppt;
      p->chunk = chunk;
      p->nchunk = nchunk;
      p->cap = cap;
      ok = true;
      break;
    }
  }
  if (!ok) return false;
  const size_t slots = (size_t)g.B * g.Hkv * p->nchunk * p->cap;
  p->off_idx = slots * sizeof(uint64_t);
  p->off_cnt = (p->off_idx + slots * sizeof(int32_t) + 255) / 256 * 256;
  p->bytes = p->off_cnt + (size_t)g.B * g.Hkv * p->nchunk * sizeof(int32_t) + 256;
  p->merge_lds = (size_t)p->nchunk * p->cap * (sizeof(uint64_t) + sizeof(int32_t));
  return true;
}

hipError_t launch_select(const Geo& g, const SelectPlan& p, const void* q, const void* meta,
                         const int32_t* bt, const int32_t* lens, const int32_t* budgets,
                         int b_max, int32_t* sel, int32_t* cnt, void* ws, hipStream_t st) {
  unsigned char* w = static_cast<unsigned char*>(ws);
  ScoreArgs sa{q, meta, bt, lens, budgets,
               reinterpret_cast<uint64_t*>(w), reinterpret_cast<int32_t*>(w + p.off_idx),
               reinterpret_cast<int32_t*>(w + p.off_cnt),
               g.Hq, g.Hkv, g.G, g.max_pages, p.chunk, p.ppt, p.nchunk, p.cap};
  const dim3 sgrid(p.nchunk, g.Hkv, g.B);
  const size_t slds = (size_t)p.chunk * sizeof(uint64_t);
  hipError_t e;
  const bool bf = g.dtype == 1;
  switch (g.D) {
    case 64: e = bf ? dispatch_hb<true, 64>(sa, p.head_block, sgrid, slds, st)
                    : dispatch_hb<false, 64>(sa, p.head_block, sgrid, slds, st); break;
    case 128: e = bf ? dispatch_hb<true, 128>(sa, p.head_block, sgrid, slds, st)
                     : dispatch_hb<false, 128>(sa, p.head_block, sgrid, slds, st); break;
    default: e = bf ? dispatch_hb<true, 576>(sa, p.head_block, sgrid, slds, st)
                    : dispatch_hb<false, 576>(sa, p.head_block, sgrid, slds, st); break;
  }
  if (e != hipSuccess) return e;
  MergeArgs ma{lens, budgets, sa.ckey, sa.cidx, sa.ccnt, sel, cnt,
               g.Hkv, b_max, p.chunk, p.nchunk, p.cap};
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&merge_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.merge_lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(g.Hkv, g.B), dim3(kThreads), p.merge_lds, st, ma);
  return hipGetLastError();
}

}  // namespace psd
