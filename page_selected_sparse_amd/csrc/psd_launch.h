// Host-side launch interface between the C-ABI layer (psd_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace psd {

// Plain geometry copied out of psd_shape after validation.
struct Geo {
  int B, Hq, Hkv, G, D, Dv, num_blocks, max_pages, dtype;  // dtype: 0 f32, 1 bf16
  int64_t kbs, kts, khs, vbs, vts, vhs;
};

// A step over few pages per unit: one workgroup per unit scores and attends them in
// about a launch time, so the whole-unit plans (and with them the one-launch step) pay
// even when there are too few units to fill the GPU.
#ifndef PSD_SMALL_PAGES
#define PSD_SMALL_PAGES 256
#endif
inline bool small_units(const Geo& g) { return g.max_pages <= PSD_SMALL_PAGES; }

// ---- page statistics ------------------------------------------------------------------
hipError_t launch_meta_update(const Geo& g, const void* k, void* meta, const int32_t* bt,
                              const int32_t* lens, const int32_t* first_page, hipStream_t st);

// ---- selection --------------------------------------------------------------------------
// Chunking of the candidate pages 1..n-2 of a unit for the two-level top-b. A plan with
// nchunk == 1 scores and ranks every unit in one workgroup and needs no merge.
struct SelectPlan {
  int chunk;       // candidate pages per scoring workgroup (threads * ppt)
  int threads;     // threads per scoring workgroup
  int ppt;         // pages per thread
  int nchunk;      // chunks covering max_pages - 2 candidates
  int cap;         // candidate slots per chunk = min(chunk, b_max - 2)
  int ustride;     // candidate slots per unit in the workspace
  bool prescore;   // many-head bf16 groups: certified MFMA pre-score + exact ranking
  int cpl;         // statistics chunks per load group (DPP path)
  int stages;      // load groups in flight per wave (DPP path)
  int head_block;  // query heads scored per pass (template width)
  int d_chunk;     // dims of q staged in LDS per pass (LDS q path)
  bool all_q;           // whole (q+, q-) table of the group in LDS
  int merge_threads;  // threads of the per-unit merge workgroup
  size_t off_idx, off_cnt, bytes;  // workspace layout
  size_t merge_lds;  // LDS of a unit merge
  size_t score_lds;  // dynamic LDS of the scoring kernel
};
// Returns false when no plan fits (b_max too large).
bool plan_select(const Geo& g, int b_max, SelectPlan* plan);
// Scoring stage: chunk candidates into the workspace and every row entry except the
// ranked winners. Merge stage: the winners, from the workspace.
// With meta_tail the scoring launch (exact path) or the merge launch also refreshes every
// sequence's tail-page statistics from k, as launch_meta_update with no first_page does:
// one extra workgroup per unit. refresh_site() says which launch takes it: the scoring
// launch when its grid has at most one workgroup per CU (more would give some CUs an
// extra scoring workgroup), else the merge launch (one workgroup per unit), else, when
// whole-unit scoring leaves no merge launch, a launch of its own.
constexpr int kComputeUnits = 256;  // MI355X
enum RefreshSite { kRefreshOwnLaunch, kRefreshInScore, kRefreshInMerge };
RefreshSite refresh_site(const Geo& g, const SelectPlan& plan);
hipError_t launch_select_score(const Geo& g, const SelectPlan& plan, const void* q,
                               const void* meta, const int32_t* bt, const int32_t* lens,
                               const int32_t* budgets, int b_max, int32_t* sel, int32_t* cnt,
                               void* ws, hipStream_t st, void* meta_tail = nullptr,
                               const void* k = nullptr);
hipError_t launch_select_merge(const Geo& g, const SelectPlan& plan, const void* q,
                               const void* meta, const int32_t* bt, const int32_t* lens,
                               const int32_t* budgets, int b_max, int32_t* sel, void* ws,
                               hipStream_t st, void* meta_tail = nullptr,
                               const void* k = nullptr);

// Certified many-head path (prescore.hip): the score stage is prescore_kernel (tiles of
// `ppt` 16-page groups per workgroup, nchunk workgroups per unit), the merge stage is
// certify_kernel. Workspace: approximate scores at 0, page maxima at off_idx.
constexpr int kPreMaxInner = 7168;  // certify holds 21 bytes per candidate in LDS
bool prescore_applies(const Geo& g);
size_t prescore_lds(int max_inner);
hipError_t launch_prescore(const Geo& g, const SelectPlan& plan, const void* q, const void* meta,
                           const int32_t* bt, const int32_t* lens, const int32_t* budgets,
                           int b_max, int32_t* sel, int32_t* cnt, void* ws, hipStream_t st);
hipError_t launch_certify(const Geo& g, const SelectPlan& plan, const void* q, const void* meta,
                          const int32_t* bt, const int32_t* lens, const int32_t* budgets,
                          int b_max, int32_t* sel, void* ws, hipStream_t st,
                          void* meta_tail = nullptr, const void* k = nullptr);

// ---- attention -------------------------------------------------------------------------
struct DecodePlan {
  int pps;     // pages per split (one workgroup, or one wave of a whole-unit workgroup)
  int nsplit;  // splits per unit
  int waves;   // waves per workgroup = ceil(G / 16) head tiles
  int unit;    // > 0: one workgroup of `unit` waves per unit, combined in LDS (no merge)
  int latent_tiles;  // > 0: latent sparse plan, one workgroup per (unit, split, 16-head tile)
  size_t off_ml, bytes;
};
// dense: every page of each sequence is attended (splits sized for long page walks).
bool plan_decode(const Geo& g, int max_pages_attended, bool dense, DecodePlan* plan);
hipError_t launch_decode(const Geo& g, const DecodePlan& plan, const void* q, const void* k,
                         const void* v, const int32_t* bt, const int32_t* lens,
                         const int32_t* sel, const int32_t* cnt, int b_max, float scale,
                         float* out, void* ws, hipStream_t st);
// The same attention with V from the value tier: entry e of unit u reads its V from hot
// slice vslot[u][e] ([slots][16][Dv]) when >= 0, else from v (host pool) by the block
// table. GQA shapes with D == Dv in {64, 128} and groups of up to 16 heads.
// hot_k: the KV tier's K hot buffer (K of a resident entry read from its slot), else null.
hipError_t launch_decode_tiered(const Geo& g, const DecodePlan& plan, const void* q,
                                const void* k, const void* v, const void* hot_k,
                                const void* hot, const int32_t* vslot, const int32_t* bt,
                                const int32_t* lens, const int32_t* sel, const int32_t* cnt,
                                int b_max, float scale, float* out, void* ws, hipStream_t st);

// ---- diagnostic memory walks (walk.hip) --------------------------------------------------
// kind 0: the kept pages' K and V rows; kind 1: the candidate pages' statistics records.
// latent: V is the leading part of each K row and is not walked again.
bool walk_supported(const Geo& g, bool latent);
hipError_t launch_walk(const Geo& g, int kind, bool latent, const void* k, const void* v,
                       const void* meta, const int32_t* bt, const int32_t* lens,
                       const int32_t* sel, const int32_t* cnt, int b_max, uint32_t* checksum,
                       hipStream_t st);

// ---- value tier (V in host memory, resident hot buffer) ----------------------------------
struct TierLayout {
  // state: slot_of [num_blocks * H_kv] at 0, owner [slots], stamp [slots]
  size_t off_owner, off_stamp, state_bytes;
  // workspace: misses [entries] at 0, jobs [entries], free list [slots], counters
  size_t off_jobs, off_free, off_ctl, work_bytes;
};
TierLayout tier_layout(const Geo& g, int slots, int b_max);
hipError_t launch_tier_reset(const Geo& g, int slots, void* state, hipStream_t st);
// k / hot_k: the KV tier's host K pool and K hot buffer, or null for the value tier.
hipError_t launch_tier_stage(const Geo& g, int slots, int step, const void* k, const void* v,
                             void* hot_k, void* hot, void* state, const int32_t* bt,
                             const int32_t* lens, const int32_t* sel, const int32_t* cnt,
                             int b_max, int32_t* vslot, unsigned long long* stats, void* ws,
                             hipStream_t st);

// ---- selection and attention in one launch -------------------------------------------------
// Applies when both plans take one workgroup per unit (DPP scoring of groups of up to 8
// heads, whole-unit attention): each workgroup scores, ranks and attends its unit, the page
// list passing through LDS. Writes the selection rows and counts as the separate calls do.
// With meta_tail (the statistics, writable) each workgroup also refreshes its sequence's
// tail-page statistics for its KV head, as launch_meta_update with no first_page does.
bool fused_applies(const Geo& g, const SelectPlan& sp, const DecodePlan& dp, int b_max);
hipError_t launch_select_decode(const Geo& g, const SelectPlan& sp, const DecodePlan& dp,
                                const void* q, const void* meta, const void* k, const void* v,
                                const int32_t* bt, const int32_t* lens, const int32_t* budgets,
                                int b_max, float scale, int32_t* sel, int32_t* cnt, float* out,
                                void* ws, void* meta_tail, hipStream_t st);

// ---- adaptive coverage selection ---------------------------------------------------------
// Exact page masses from every valid K row, then a per-unit nucleus cut (G <= 8,
// max_pages <= 4096, D in {64, 128}). Writes selection rows and counts like the budgeted
// selection. The workspace holds each query head's page max and page exp-sum.
size_t coverage_workspace_bytes(const Geo& g);
bool coverage_supported(const Geo& g);
hipError_t launch_coverage_select(const Geo& g, const void* q, const void* k, const int32_t* bt,
                                  const int32_t* lens, float coverage, float scale, int b_max,
                                  int32_t* sel, int32_t* cnt, void* ws, hipStream_t st);

}  // namespace psd
