// Value tier: V in pinned host memory, with a bounded resident buffer in device memory;
// and the KV tier, the same with K in host memory too (each resident slice holds both).
//
// The value cache can live in host DRAM, mapped for the device, while a bounded hot
// buffer in HBM holds the V slices that decode steps keep calling, and only the slices a
// step selects that are not resident cross the host link (AMASS page, "What is in the
// box", item 2, the DRAM value tier with a resident hot buffer and a staging pool; LOCKS
// README, "How it works", the optional DRAM tier). A slice is one (block, KV head): 16
// token rows of Dv elements, the V a unit attends when it keeps that page.
//
// State kept between steps (device memory, the caller's):
//   slot_of [num_blocks * H_kv]  slot of each (block, head) slice, -1 if not resident
//   owner   [slots]              slice held by each slot (block * H_kv + head), -1 if free
//   stamp   [slots]              the last step that used the slot
// A step (psd_value_tier_stage) runs four launches:
//   1. clear the step's counters;
//   2. every kept (unit, entry) whose slice is resident takes that slot (a hit: the
//      slot's stamp becomes the step), the others are listed as misses;
//   3. one workgroup gives the missed slices slots that this step does not use (the
//      staging pool: free slots, then ones whose slice the step did not call), evicting
//      their old slices, and lists the copies; a slice missed by several entries gets one
//      slot; when the slots run out, the remaining entries read V from host memory;
//   4. the copies: each listed slice's 16 rows go from the host pool to its slot.
// The attention then reads each entry's V from its slot (psd_sparse_decode_tiered); in the
// KV tier the copies also bring the slice's K rows into a K hot buffer with the same slots,
// and the attention reads K from there too (psd_sparse_decode_kv_tiered).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "psd_device.h"
#include "psd_launch.h"

namespace psd {
namespace {

struct TierArgs {
  const void* v;  // host pool (device-mapped), the V layout of the shape
  void* hot;      // [slots][16][Dv]
  const void* k;  // KV tier: host K pool (device-mapped), the K layout of the shape; else null
  void* hot_k;    // KV tier: [slots][16][D]
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* sel;
  const int32_t* cnt;
  int32_t* slot_of;
  int32_t* owner;
  int32_t* stamp;
  int32_t* vslot;     // [B * H_kv * b_max] out: slot of each kept entry, -1: read from host
  int32_t* miss;      // [B * H_kv * b_max] entries that missed (unit * b_max + entry)
  int32_t* jobs;      // [B * H_kv * b_max] slots to fill this step
  int32_t* freelist;  // [slots]
  int32_t* ctl;       // [8]: 0 misses, 1 copies, 2 hits, 3 overflow
  unsigned long long* stats;  // [4] out: hits, misses, copies, entries read from host
  int64_t vbs, vts, vhs, kbs, kts, khs;
  int B, Hkv, max_pages, b_max, num_blocks, D, Dv, es, slots, step;
};

__global__ __launch_bounds__(64) void tier_begin_kernel(TierArgs a) {
  if (threadIdx.x < 8) a.ctl[threadIdx.x] = 0;
}

// The slice of kept entry e of unit u, clamped into the pool.
__device__ __forceinline__ int tier_key(const TierArgs& a, int u, int e, int n) {
  const int s = u / a.Hkv, g = u - s * a.Hkv;
  int p = a.sel[(int64_t)u * a.b_max + e];
  p = min(max(p, 0), n - 1);
  int blk = a.bt[(int64_t)s * a.max_pages + p];
  blk = min(max(blk, 0), a.num_blocks - 1);
  return blk * a.Hkv + g;
}

__device__ __forceinline__ int tier_count(const TierArgs& a, int u) {
  const int c = a.cnt[u];
  return c < 0 ? 0 : min(c, a.b_max);
}

// One workgroup per unit: hits take their slot, misses are listed.
__global__ __launch_bounds__(256) void tier_mark_kernel(TierArgs a) {
  const int u = blockIdx.x, s = u / a.Hkv;
  const int count = tier_count(a, u), n = ceil_div(a.lens[s], kPage);
  int hits = 0;
  for (int e = threadIdx.x; e < count; e += 256) {
    const int key = tier_key(a, u, e, n);
    const int slot = a.slot_of[key];
    const int64_t idx = (int64_t)u * a.b_max + e;
    if (slot >= 0) {
      a.stamp[slot] = a.step;
      a.vslot[idx] = slot;
      ++hits;
    } else {
      a.vslot[idx] = -1;
      a.miss[atomicAdd(&a.ctl[0], 1)] = (int)idx;
    }
  }
  if (hits) atomicAdd(&a.ctl[2], hits);
}

// Block-wide exclusive prefix sum of 0/1 flags (NT threads), and the total.
template <int NT>
__device__ int tier_scan(int x, int* buf, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_scan_incl(x);
  if (lane == 63) buf[w] = incl;
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int c = buf[i];
    off += i < w ? c : 0;
    total += c;
  }
  __syncthreads();
  return off + incl - x;
}

// One workgroup: slots for the missed slices, evictions, the copy list, the entries' slots.
__global__ __launch_bounds__(1024) void tier_alloc_kernel(TierArgs a) {
  constexpr int NT = 1024;
  __shared__ int buf[NT / 64];
  __shared__ int nfree, nalloc, njobs, over;
  const int tid = threadIdx.x;
  if (tid == 0) {
    nfree = 0;
    nalloc = 0;
    njobs = 0;
    over = 0;
  }
  __syncthreads();
  // the staging pool: slots this step does not use, in slot order (free ones have no
  // owner and a stamp from an earlier step)
  for (int base = 0; base < a.slots; base += NT) {
    const int f = base + tid;
    const int is_free = f < a.slots && a.stamp[f] != a.step;
    int total;
    const int pos = tier_scan<NT>(is_free, buf, total);
    if (is_free) a.freelist[nfree + pos] = f;
    __syncthreads();
    if (tid == 0) nfree += total;
    __syncthreads();
  }
  const int nmiss = a.ctl[0];
  // A missed slice gets a slot once: the first entry to claim its map word takes a slot
  // from the pool and evicts the slot's old slice (which this step does not call, or the
  // slot would not be in the pool).
  for (int i = tid; i < nmiss; i += NT) {
    const int idx = a.miss[i];
    const int u = idx / a.b_max, e = idx - u * a.b_max;
    const int n = ceil_div(a.lens[u / a.Hkv], kPage);
    const int key = tier_key(a, u, e, n);
    if (atomicCAS(&a.slot_of[key], -1, -2) != -1) continue;  // another entry has it
    const int j = atomicAdd(&nalloc, 1);
    if (j >= nfree) {
      a.slot_of[key] = -1;  // no slot left: read from host
      continue;
    }
    const int f = a.freelist[j];
    const int old = a.owner[f];
    if (old >= 0) a.slot_of[old] = -1;
    a.owner[f] = key;
    a.stamp[f] = a.step;
    a.slot_of[key] = f;
    a.jobs[atomicAdd(&njobs, 1)] = f;
  }
  __syncthreads();
  for (int i = tid; i < nmiss; i += NT) {
    const int idx = a.miss[i];
    const int u = idx / a.b_max, e = idx - u * a.b_max;
    const int n = ceil_div(a.lens[u / a.Hkv], kPage);
    const int slot = a.slot_of[tier_key(a, u, e, n)];
    a.vslot[idx] = slot;
    if (slot < 0) atomicAdd(&over, 1);
  }
  __syncthreads();
  if (tid == 0) {
    a.ctl[1] = njobs;
    a.ctl[3] = over;
    a.stats[0] = (unsigned long long)a.ctl[2];
    a.stats[1] = (unsigned long long)nmiss;
    a.stats[2] = (unsigned long long)njobs;
    a.stats[3] = (unsigned long long)over;
  }
}

// The 16 rows of one slice, from a pool with strides (bs, ts, hs) to a slot of `cols`
// elements per row: 16 bytes per lane per row piece.
__device__ __forceinline__ void copy_slice(const void* pool, void* hot, int f, int blk, int g,
                                           int64_t bs, int64_t ts, int64_t hs, int cols, int es,
                                           int lane) {
  const int row_bytes = cols * es, chunks = row_bytes / 16;
  const unsigned char* src =
      static_cast<const unsigned char*>(pool) + ((int64_t)blk * bs + (int64_t)g * hs) * es;
  unsigned char* dst = static_cast<unsigned char*>(hot) + (int64_t)f * kPage * row_bytes;
  for (int piece = lane; piece < kPage * chunks; piece += 64) {
    const int t = piece / chunks, c = piece - t * chunks;
    const uint4 x = *reinterpret_cast<const uint4*>(src + (int64_t)t * ts * es + c * 16);
    *reinterpret_cast<uint4*>(dst + (int64_t)t * row_bytes + c * 16) = x;
  }
}

// The copies: one wave per listed slot at a time (V, and K in the KV tier).
__global__ __launch_bounds__(256) void tier_copy_kernel(TierArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), waves = gridDim.x * 4;
  const int njobs = a.ctl[1];
  for (int j = wave; j < njobs; j += waves) {
    const int f = a.jobs[j];
    const int key = a.owner[f];
    const int blk = key / a.Hkv, g = key - blk * a.Hkv;
    copy_slice(a.v, a.hot, f, blk, g, a.vbs, a.vts, a.vhs, a.Dv, a.es, lane);
    if (a.k) copy_slice(a.k, a.hot_k, f, blk, g, a.kbs, a.kts, a.khs, a.D, a.es, lane);
  }
}

// Map and slots back to empty.
__global__ __launch_bounds__(256) void tier_reset_kernel(int32_t* slot_of, int64_t keys,
                                                         int32_t* owner, int32_t* stamp,
                                                         int slots) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < keys) slot_of[i] = -1;
  if (i < slots) {
    owner[i] = -1;
    stamp[i] = INT32_MIN;
  }
}

}  // namespace

TierLayout tier_layout(const Geo& g, int slots, int b_max) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  TierLayout t;
  const size_t keys = (size_t)g.num_blocks * g.Hkv;
  t.off_owner = al(keys * 4);
  t.off_stamp = t.off_owner + al((size_t)slots * 4);
  t.state_bytes = t.off_stamp + al((size_t)slots * 4);
  const size_t entries = (size_t)g.B * g.Hkv * b_max;
  t.off_jobs = al(entries * 4);
  t.off_free = t.off_jobs + al(entries * 4);
  t.off_ctl = t.off_free + al((size_t)slots * 4);
  t.work_bytes = t.off_ctl + 256;
  return t;
}

hipError_t launch_tier_reset(const Geo& g, int slots, void* state, hipStream_t st) {
  const TierLayout t = tier_layout(g, slots, 1);
  unsigned char* p = static_cast<unsigned char*>(state);
  const int64_t keys = (int64_t)g.num_blocks * g.Hkv;
  const int64_t n = keys > slots ? keys : slots;
  hipLaunchKernelGGL(tier_reset_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<int32_t*>(p), keys,
                     reinterpret_cast<int32_t*>(p + t.off_owner),
                     reinterpret_cast<int32_t*>(p + t.off_stamp), slots);
  return hipGetLastError();
}

hipError_t launch_tier_stage(const Geo& g, int slots, int step, const void* k, const void* v,
                             void* hot_k, void* hot, void* state, const int32_t* bt,
                             const int32_t* lens, const int32_t* sel, const int32_t* cnt,
                             int b_max, int32_t* vslot, unsigned long long* stats, void* ws,
                             hipStream_t st) {
  const TierLayout t = tier_layout(g, slots, b_max);
  unsigned char* p = static_cast<unsigned char*>(state);
  unsigned char* w = static_cast<unsigned char*>(ws);
  TierArgs a;
  a.v = v;
  a.hot = hot;
  a.k = k;
  a.hot_k = hot_k;
  a.bt = bt;
  a.lens = lens;
  a.sel = sel;
  a.cnt = cnt;
  a.slot_of = reinterpret_cast<int32_t*>(p);
  a.owner = reinterpret_cast<int32_t*>(p + t.off_owner);
  a.stamp = reinterpret_cast<int32_t*>(p + t.off_stamp);
  a.vslot = vslot;
  a.miss = reinterpret_cast<int32_t*>(w);
  a.jobs = reinterpret_cast<int32_t*>(w + t.off_jobs);
  a.freelist = reinterpret_cast<int32_t*>(w + t.off_free);
  a.ctl = reinterpret_cast<int32_t*>(w + t.off_ctl);
  a.stats = stats;
  a.vbs = g.vbs;
  a.vts = g.vts;
  a.vhs = g.vhs;
  a.kbs = g.kbs;
  a.kts = g.kts;
  a.khs = g.khs;
  a.D = g.D;
  a.B = g.B;
  a.Hkv = g.Hkv;
  a.max_pages = g.max_pages;
  a.b_max = b_max;
  a.num_blocks = g.num_blocks;
  a.Dv = g.Dv;
  a.es = g.dtype == 1 ? 2 : 4;
  a.slots = slots;
  a.step = step;
  hipLaunchKernelGGL(tier_begin_kernel, dim3(1), dim3(64), 0, st, a);
  hipLaunchKernelGGL(tier_mark_kernel, dim3(g.B * g.Hkv), dim3(256), 0, st, a);
  hipLaunchKernelGGL(tier_alloc_kernel, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(tier_copy_kernel, dim3(kComputeUnits), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace psd
