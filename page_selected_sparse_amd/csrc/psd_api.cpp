// C-ABI entry points declared in include/psd.h: host-side argument checks, workspace
// sizing and stream-ordered kernel launches. Nothing here allocates or synchronises.
#include "psd.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "psd_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dims(int D, int Dv) {
  return (D == 64 && Dv == 64) || (D == 128 && Dv == 128) || (D == 576 && Dv == 512);
}

bool supported_group(int G) { return (G >= 1 && G <= 16) || (G % 16 == 0 && G <= 128); }

// Shape checks common to every call; fills the kernel geometry.
psd_status check_shape(const psd_shape* sh, psd::Geo* g) {
  if (!sh) return PSD_ERR_INVALID_ARG;
  if (sh->batch < 1 || sh->num_q_heads < 1 || sh->num_kv_heads < 1 || sh->head_dim < 1 ||
      sh->head_dim_v < 1 || sh->num_blocks < 1 || sh->max_pages_per_seq < 1 ||
      sh->reserved != 0)
    return PSD_ERR_INVALID_ARG;
  if (sh->page_size != 16) return PSD_ERR_INVALID_ARG;
  if (sh->dtype != PSD_F32 && sh->dtype != PSD_BF16) return PSD_ERR_INVALID_ARG;
  if (sh->num_q_heads % sh->num_kv_heads != 0) return PSD_ERR_INVALID_ARG;
  if (sh->head_dim_v > sh->head_dim) return PSD_ERR_INVALID_ARG;
  if (!supported_dims(sh->head_dim, sh->head_dim_v)) return PSD_ERR_UNSUPPORTED;
  const int G = sh->num_q_heads / sh->num_kv_heads;
  if (!supported_group(G)) return PSD_ERR_UNSUPPORTED;
  if ((int64_t)sh->batch * sh->max_pages_per_seq > INT32_MAX) return PSD_ERR_UNSUPPORTED;
  g->B = sh->batch;
  g->Hq = sh->num_q_heads;
  g->Hkv = sh->num_kv_heads;
  g->G = G;
  g->D = sh->head_dim;
  g->Dv = sh->head_dim_v;
  g->num_blocks = sh->num_blocks;
  g->max_pages = sh->max_pages_per_seq;
  g->dtype = sh->dtype;
  g->kbs = sh->k_block_stride;
  g->kts = sh->k_token_stride;
  g->khs = sh->k_head_stride;
  g->vbs = sh->v_block_stride;
  g->vts = sh->v_token_stride;
  g->vhs = sh->v_head_stride;
  return PSD_OK;
}

// Cache strides: positive, 16-byte multiples, and rows that fit inside a block.
psd_status check_strides(const psd::Geo& g, bool need_v) {
  const int64_t es = g.dtype == PSD_BF16 ? 2 : 4;
  auto ok = [&](int64_t bs, int64_t ts, int64_t hs, int dims) {
    if (bs <= 0 || ts <= 0 || hs < 0) return false;
    if ((bs * es) % 16 || (ts * es) % 16 || (hs * es) % 16) return false;
    if (g.Hkv > 1 && hs < dims) return false;
    if (ts < (int64_t)(g.Hkv - 1) * hs + dims) return false;
    if (bs < 15 * ts + (int64_t)(g.Hkv - 1) * hs + dims) return false;
    return true;
  };
  if (!ok(g.kbs, g.kts, g.khs, g.D)) return PSD_ERR_INVALID_ARG;
  if (need_v && !ok(g.vbs, g.vts, g.vhs, g.Dv)) return PSD_ERR_INVALID_ARG;
  return PSD_OK;
}

psd_status launched(hipError_t e) { return e == hipSuccess ? PSD_OK : PSD_ERR_LAUNCH; }

}  // namespace

extern "C" {

psd_status psd_page_meta_update(const psd_shape* shape, const void* k_cache, void* meta,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* first_page, hipStream_t stream) {
  psd::Geo g;
  psd_status st = check_shape(shape, &g);
  if (st != PSD_OK) return st;
  if (!k_cache || !meta || !block_table || !seq_lens) return PSD_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(meta)) return PSD_ERR_INVALID_ARG;
  if ((st = check_strides(g, false)) != PSD_OK) return st;
  return launched(psd::launch_meta_update(g, k_cache, meta, block_table, seq_lens, first_page,
                                          stream));
}

size_t psd_select_workspace_bytes(const psd_shape* shape, int32_t b_max) {
  psd::Geo g;
  if (check_shape(shape, &g) != PSD_OK) return 0;
  psd::SelectPlan p;
  if (!psd::plan_select(g, b_max, &p)) return 0;
  return p.bytes;
}

}  // extern "C"

namespace {

// Checks shared by the selection calls; fills the geometry and the plan.
psd_status select_common(const psd_shape* shape, const int32_t* seq_lens,
                         const int32_t* budgets, int32_t b_max, const int32_t* sel_pages,
                         const void* workspace, size_t workspace_bytes, psd::Geo* g,
                         psd::SelectPlan* p) {
  psd_status st = check_shape(shape, g);
  if (st != PSD_OK) return st;
  if (!seq_lens || !budgets || !sel_pages) return PSD_ERR_INVALID_ARG;
  if (b_max < 2) return PSD_ERR_INVALID_ARG;
  if (!psd::plan_select(*g, b_max, p)) return PSD_ERR_CAPACITY;
  if (!workspace || workspace_bytes < p->bytes || !aligned16(workspace)) return PSD_ERR_WORKSPACE;
  return PSD_OK;
}

}  // namespace

extern "C" {

psd_status psd_select_score(const psd_shape* shape, const void* q, const void* meta,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* budgets, int32_t b_max, int32_t* sel_pages,
                            int32_t* sel_count, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  psd::Geo g;
  psd::SelectPlan p;
  psd_status st = select_common(shape, seq_lens, budgets, b_max, sel_pages, workspace,
                                workspace_bytes, &g, &p);
  if (st != PSD_OK) return st;
  if (!q || !meta || !block_table || !sel_count) return PSD_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(meta)) return PSD_ERR_INVALID_ARG;
  return launched(psd::launch_select_score(g, p, q, meta, block_table, seq_lens, budgets, b_max,
                                           sel_pages, sel_count, workspace, stream));
}

psd_status psd_select_merge(const psd_shape* shape, const void* q, const void* meta,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* budgets, int32_t b_max, int32_t* sel_pages,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  psd::Geo g;
  psd::SelectPlan p;
  psd_status st = select_common(shape, seq_lens, budgets, b_max, sel_pages, workspace,
                                workspace_bytes, &g, &p);
  if (st != PSD_OK) return st;
  if (!q || !meta || !block_table) return PSD_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(meta)) return PSD_ERR_INVALID_ARG;
  return launched(psd::launch_select_merge(g, p, q, meta, block_table, seq_lens, budgets, b_max,
                                           sel_pages, workspace, stream));
}

psd_status psd_select_pages(const psd_shape* shape, const void* q, const void* meta,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* budgets, int32_t b_max, int32_t* sel_pages,
                            int32_t* sel_count, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  psd_status st = psd_select_score(shape, q, meta, block_table, seq_lens, budgets, b_max,
                                   sel_pages, sel_count, workspace, workspace_bytes, stream);
  if (st != PSD_OK) return st;
  return psd_select_merge(shape, q, meta, block_table, seq_lens, budgets, b_max, sel_pages,
                          workspace, workspace_bytes, stream);
}

size_t psd_decode_workspace_bytes(const psd_shape* shape, int32_t max_pages_attended) {
  psd::Geo g;
  if (check_shape(shape, &g) != PSD_OK) return 0;
  // the same query serves the sparse and the dense call: room for either plan
  psd::DecodePlan ps, pd;
  if (!psd::plan_decode(g, max_pages_attended, false, &ps) ||
      !psd::plan_decode(g, max_pages_attended, true, &pd))
    return 0;
  return ps.bytes > pd.bytes ? ps.bytes : pd.bytes;
}

static psd_status decode_common(const psd_shape* shape, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* sel_pages,
                                const int32_t* sel_count, int32_t pages_cap, int32_t b_max,
                                float scale, float* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  psd::Geo g;
  psd_status st = check_shape(shape, &g);
  if (st != PSD_OK) return st;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return PSD_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return PSD_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale == __builtin_inff()) return PSD_ERR_INVALID_ARG;
  if ((st = check_strides(g, true)) != PSD_OK) return st;
  psd::DecodePlan p;
  if (!psd::plan_decode(g, pages_cap, sel_pages == nullptr, &p)) return PSD_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < p.bytes || !aligned16(workspace)) return PSD_ERR_WORKSPACE;
  return launched(psd::launch_decode(g, p, q, k_cache, v_cache, block_table, seq_lens, sel_pages,
                                     sel_count, b_max, scale, out, workspace, stream));
}

psd_status psd_sparse_decode(const psd_shape* shape, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* sel_pages,
                             const int32_t* sel_count, int32_t b_max, float scale, float* out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!sel_pages || !sel_count || b_max < 1) return PSD_ERR_INVALID_ARG;
  return decode_common(shape, q, k_cache, v_cache, block_table, seq_lens, sel_pages, sel_count,
                       b_max, b_max, scale, out, workspace, workspace_bytes, stream);
}

psd_status psd_dense_decode(const psd_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, float scale, float* out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!shape) return PSD_ERR_INVALID_ARG;
  return decode_common(shape, q, k_cache, v_cache, block_table, seq_lens, nullptr, nullptr,
                       shape->max_pages_per_seq, 0, scale, out, workspace, workspace_bytes,
                       stream);
}

// ---- diagnostic memory walks ----------------------------------------------------------------
psd_status psd_diag_walk(const psd_shape* shape, int32_t kind, const void* k_cache,
                         const void* v_cache, const void* meta, const int32_t* block_table,
                         const int32_t* seq_lens, const int32_t* sel_pages,
                         const int32_t* sel_count, int32_t b_max, uint32_t* checksum,
                         hipStream_t stream) {
  psd::Geo g;
  psd_status st = check_shape(shape, &g);
  if (st != PSD_OK) return st;
  if ((kind != 0 && kind != 1) || !block_table || !seq_lens || !checksum)
    return PSD_ERR_INVALID_ARG;
  if (kind == 0 && (!k_cache || !v_cache || !sel_pages || !sel_count || b_max < 1))
    return PSD_ERR_INVALID_ARG;
  if (kind == 1 && !meta) return PSD_ERR_INVALID_ARG;
  if ((k_cache && !aligned16(k_cache)) || (v_cache && !aligned16(v_cache)) ||
      (meta && !aligned16(meta)))
    return PSD_ERR_INVALID_ARG;
  if (kind == 0 && (st = check_strides(g, true)) != PSD_OK) return st;
  const bool latent = k_cache == v_cache && g.kbs == g.vbs && g.kts == g.vts && g.khs == g.vhs &&
                      g.Dv <= g.D;
  if (!psd::walk_supported(g, latent)) return PSD_ERR_UNSUPPORTED;
  return launched(psd::launch_walk(g, kind, latent, k_cache, v_cache, meta, block_table,
                                   seq_lens, sel_pages, sel_count, b_max, checksum, stream));
}

// ---- value tier ----------------------------------------------------------------------------
static bool tier_shape(const psd_shape* shape, psd::Geo* g) {
  if (check_shape(shape, g) != PSD_OK) return false;
  return g->D == g->Dv && (g->D == 64 || g->D == 128) && g->G <= 16 &&
         check_strides(*g, true) == PSD_OK;
}

size_t psd_value_tier_state_bytes(const psd_shape* shape, int32_t slots) {
  psd::Geo g;
  if (slots < 0 || !tier_shape(shape, &g)) return 0;
  return psd::tier_layout(g, slots, 1).state_bytes;
}

size_t psd_value_tier_workspace_bytes(const psd_shape* shape, int32_t b_max, int32_t slots) {
  psd::Geo g;
  if (slots < 0 || b_max < 1 || !tier_shape(shape, &g)) return 0;
  return psd::tier_layout(g, slots, b_max).work_bytes;
}

psd_status psd_value_tier_reset(const psd_shape* shape, int32_t slots, void* state,
                                hipStream_t stream) {
  psd::Geo g;
  if (check_shape(shape, &g) != PSD_OK) return PSD_ERR_INVALID_ARG;
  if (!tier_shape(shape, &g)) return PSD_ERR_UNSUPPORTED;
  if (slots < 0 || !state || !aligned16(state)) return PSD_ERR_INVALID_ARG;
  return launched(psd::launch_tier_reset(g, slots, state, stream));
}

// The value tier (k_host and hot_k null) and the KV tier share the stage and the attention.
static psd_status tier_stage_common(const psd_shape* shape, const void* k_host,
                                    const void* v_host, void* hot_k, void* hot, void* state,
                                    int32_t slots, int32_t step, const int32_t* block_table,
                                    const int32_t* seq_lens, const int32_t* sel_pages,
                                    const int32_t* sel_count, int32_t b_max, int32_t* slot,
                                    uint64_t* stats, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  psd::Geo g;
  if (check_shape(shape, &g) != PSD_OK) return PSD_ERR_INVALID_ARG;
  if (!tier_shape(shape, &g)) return PSD_ERR_UNSUPPORTED;
  if (slots < 0 || b_max < 1 || !v_host || !state || !block_table || !seq_lens || !sel_pages ||
      !sel_count || !slot || !stats || (slots > 0 && !hot))
    return PSD_ERR_INVALID_ARG;
  if (k_host && slots > 0 && !hot_k) return PSD_ERR_INVALID_ARG;
  if (!aligned16(v_host) || (hot && !aligned16(hot)) || !aligned16(state))
    return PSD_ERR_INVALID_ARG;
  if ((k_host && !aligned16(k_host)) || (hot_k && !aligned16(hot_k))) return PSD_ERR_INVALID_ARG;
  const psd::TierLayout t = psd::tier_layout(g, slots, b_max);
  if (!workspace || workspace_bytes < t.work_bytes || !aligned16(workspace))
    return PSD_ERR_WORKSPACE;
  return launched(psd::launch_tier_stage(g, slots, step, k_host, v_host, k_host ? hot_k : nullptr,
                                         hot, state, block_table, seq_lens, sel_pages, sel_count,
                                         b_max, slot, reinterpret_cast<unsigned long long*>(stats),
                                         workspace, stream));
}

psd_status psd_value_tier_stage(const psd_shape* shape, const void* v_host, void* hot,
                                void* state, int32_t slots, int32_t step,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* sel_pages, const int32_t* sel_count,
                                int32_t b_max, int32_t* vslot, uint64_t* stats, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return tier_stage_common(shape, nullptr, v_host, nullptr, hot, state, slots, step, block_table,
                           seq_lens, sel_pages, sel_count, b_max, vslot, stats, workspace,
                           workspace_bytes, stream);
}

psd_status psd_kv_tier_stage(const psd_shape* shape, const void* k_host, const void* v_host,
                             void* hot_k, void* hot_v, void* state, int32_t slots, int32_t step,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* sel_pages, const int32_t* sel_count, int32_t b_max,
                             int32_t* slot, uint64_t* stats, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!k_host) return PSD_ERR_INVALID_ARG;
  return tier_stage_common(shape, k_host, v_host, hot_k, hot_v, state, slots, step, block_table,
                           seq_lens, sel_pages, sel_count, b_max, slot, stats, workspace,
                           workspace_bytes, stream);
}

static psd_status tiered_common(const psd_shape* shape, const void* q, const void* k_cache,
                                const void* v_host, const void* hot_k, const void* hot,
                                const int32_t* slot, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* sel_pages,
                                const int32_t* sel_count, int32_t b_max, float scale, float* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  psd::Geo g;
  if (check_shape(shape, &g) != PSD_OK) return PSD_ERR_INVALID_ARG;
  if (!tier_shape(shape, &g)) return PSD_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_host || !slot || !block_table || !seq_lens || !sel_pages ||
      !sel_count || !out || b_max < 1)
    return PSD_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_host) || (hot && !aligned16(hot)) ||
      (hot_k && !aligned16(hot_k)) || !aligned16(out))
    return PSD_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale == __builtin_inff()) return PSD_ERR_INVALID_ARG;
  psd::DecodePlan p;
  if (!psd::plan_decode(g, b_max, false, &p)) return PSD_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < p.bytes || !aligned16(workspace)) return PSD_ERR_WORKSPACE;
  return launched(psd::launch_decode_tiered(g, p, q, k_cache, v_host, hot_k, hot, slot,
                                            block_table, seq_lens, sel_pages, sel_count, b_max,
                                            scale, out, workspace, stream));
}

psd_status psd_sparse_decode_tiered(const psd_shape* shape, const void* q, const void* k_cache,
                                    const void* v_host, const void* hot, const int32_t* vslot,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* sel_pages, const int32_t* sel_count,
                                    int32_t b_max, float scale, float* out, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  return tiered_common(shape, q, k_cache, v_host, nullptr, hot, vslot, block_table, seq_lens,
                       sel_pages, sel_count, b_max, scale, out, workspace, workspace_bytes,
                       stream);
}

psd_status psd_sparse_decode_kv_tiered(const psd_shape* shape, const void* q, const void* k_host,
                                       const void* v_host, const void* hot_k, const void* hot_v,
                                       const int32_t* slot, const int32_t* block_table,
                                       const int32_t* seq_lens, const int32_t* sel_pages,
                                       const int32_t* sel_count, int32_t b_max, float scale,
                                       float* out, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  if ((hot_k == nullptr) != (hot_v == nullptr)) return PSD_ERR_INVALID_ARG;
  return tiered_common(shape, q, k_host, v_host, hot_k, hot_v, slot, block_table, seq_lens,
                       sel_pages, sel_count, b_max, scale, out, workspace, workspace_bytes,
                       stream);
}

// select_pages then sparse_decode, as one launch when the plans allow; with `refresh`,
// the tail-page statistics refresh of page_meta_update (no first_page) comes first.
static psd_status step_common(const psd_shape* shape, const void* q, const void* meta,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              const int32_t* budgets, int32_t b_max, float scale,
                              int32_t* sel_pages, int32_t* sel_count, float* out, void* workspace,
                              size_t workspace_bytes, bool refresh, hipStream_t stream) {
  psd::Geo g;
  psd::SelectPlan sp;
  psd_status st = select_common(shape, seq_lens, budgets, b_max, sel_pages, workspace,
                                workspace_bytes, &g, &sp);
  if (st != PSD_OK) return st;
  if (!q || !meta || !block_table || !sel_count || !k_cache || !v_cache || !out)
    return PSD_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(meta) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(out))
    return PSD_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale == __builtin_inff()) return PSD_ERR_INVALID_ARG;
  if ((st = check_strides(g, true)) != PSD_OK) return st;
  psd::DecodePlan dp;
  if (!psd::plan_decode(g, b_max, false, &dp)) return PSD_ERR_INVALID_ARG;
  if (workspace_bytes < dp.bytes) return PSD_ERR_WORKSPACE;
  void* meta_w = refresh ? const_cast<void*>(meta) : nullptr;
  if (psd::fused_applies(g, sp, dp, b_max))
    return launched(psd::launch_select_decode(g, sp, dp, q, meta, k_cache, v_cache, block_table,
                                              seq_lens, budgets, b_max, scale, sel_pages,
                                              sel_count, out, workspace, meta_w, stream));
  hipError_t e = hipSuccess;
  // The tail refresh rides on the scoring or the merge launch as one extra workgroup per
  // unit (refresh_site picks the launch), else it is a launch of its own.
  const psd::RefreshSite site = psd::refresh_site(g, sp);
  if (refresh && site == psd::kRefreshOwnLaunch)
    e = psd::launch_meta_update(g, k_cache, meta_w, block_table, seq_lens, nullptr, stream);
  if (e == hipSuccess)
    e = psd::launch_select_score(g, sp, q, meta, block_table, seq_lens, budgets, b_max,
                                 sel_pages, sel_count, workspace, stream,
                                 refresh && site == psd::kRefreshInScore ? meta_w : nullptr,
                                 k_cache);
  if (e == hipSuccess)
    e = psd::launch_select_merge(g, sp, q, meta, block_table, seq_lens, budgets, b_max,
                                 sel_pages, workspace, stream,
                                 refresh && site == psd::kRefreshInMerge ? meta_w : nullptr,
                                 k_cache);
  if (e == hipSuccess)
    e = psd::launch_decode(g, dp, q, k_cache, v_cache, block_table, seq_lens, sel_pages,
                           sel_count, b_max, scale, out, workspace, stream);
  return launched(e);
}

size_t psd_select_sparse_decode_workspace_bytes(const psd_shape* shape, int32_t b_max) {
  const size_t sel = psd_select_workspace_bytes(shape, b_max);
  psd::Geo g;
  psd::DecodePlan p;
  if (sel == 0 || check_shape(shape, &g) != PSD_OK || !psd::plan_decode(g, b_max, false, &p))
    return 0;
  // the selection's workspace is dead once its merge stage has run: the attention reuses it
  return sel > p.bytes ? sel : p.bytes;
}

psd_status psd_select_sparse_decode(const psd_shape* shape, const void* q, const void* meta,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* budgets, int32_t b_max, float scale,
                                    int32_t* sel_pages, int32_t* sel_count, float* out,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  return step_common(shape, q, meta, k_cache, v_cache, block_table, seq_lens, budgets, b_max,
                     scale, sel_pages, sel_count, out, workspace, workspace_bytes, false, stream);
}

psd_status psd_decode_step(const psd_shape* shape, const void* q, void* meta, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* seq_lens, const int32_t* budgets, int32_t b_max,
                           float scale, int32_t* sel_pages, int32_t* sel_count, float* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return step_common(shape, q, meta, k_cache, v_cache, block_table, seq_lens, budgets, b_max,
                     scale, sel_pages, sel_count, out, workspace, workspace_bytes, true, stream);
}

const char* psd_status_string(psd_status s) {
  switch (s) {
    case PSD_OK: return "ok";
    case PSD_ERR_INVALID_ARG: return "invalid argument";
    case PSD_ERR_UNSUPPORTED: return "unsupported shape";
    case PSD_ERR_WORKSPACE: return "workspace missing or too small";
    case PSD_ERR_CAPACITY: return "selection capacity (b_max) exceeded";
    case PSD_ERR_LAUNCH: return "kernel launch failed";
    case PSD_ERR_SCRATCH:
      return "step needs more workspace than the library's static scratch (PSD_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int32_t psd_version(void) { return 100; }

}  // extern "C"

extern "C" {

size_t psd_select_coverage_workspace_bytes(const psd_shape* shape) {
  psd::Geo g;
  if (check_shape(shape, &g) != PSD_OK || !psd::coverage_supported(g)) return 0;
  return psd::coverage_workspace_bytes(g);
}

psd_status psd_select_pages_coverage(const psd_shape* shape, const void* q, const void* k_cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     float coverage, float scale, int32_t b_max,
                                     int32_t* sel_pages, int32_t* sel_count, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  psd::Geo g;
  psd_status st = check_shape(shape, &g);
  if (st != PSD_OK) return st;
  if (!q || !k_cache || !block_table || !seq_lens || !sel_pages || !sel_count)
    return PSD_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(q)) return PSD_ERR_INVALID_ARG;
  if (b_max < 2 || !(coverage > 0.f) || !(scale > 0.f) || coverage != coverage)
    return PSD_ERR_INVALID_ARG;
  if ((st = check_strides(g, false)) != PSD_OK) return st;
  if (!psd::coverage_supported(g)) return PSD_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < psd::coverage_workspace_bytes(g) || !aligned16(workspace))
    return PSD_ERR_WORKSPACE;
  return launched(psd::launch_coverage_select(g, q, k_cache, block_table, seq_lens, coverage,
                                              scale, b_max, sel_pages, sel_count, workspace,
                                              stream));
}

}  // extern "C"


// ---- the decode step without a caller workspace -------------------------------------------
//
// psd_decode_step_noalloc keeps its workspace in `scratch`, a file-scope device array of
// PSD_SCRATCH_BYTES that every GPU the library runs on holds until the process ends. In
// host code `scratch` names a host-side stand-in, not device memory: its device address is
// looked up once per device (hipGetSymbolAddress, with that device current) and only that
// address is passed to kernels. The step's kernels need no zeroed workspace, so nothing is
// cleared between calls.
namespace {

__device__ __align__(256) unsigned char scratch[PSD_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, or nullptr if the runtime cannot say.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

psd_status psd_decode_step_noalloc(const psd_shape* shape, const void* q, void* meta,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* budgets, int32_t b_max, float scale,
                                   int32_t* sel_pages, int32_t* sel_count, float* out,
                                   hipStream_t stream) {
  // the size check comes first, before the device is touched
  const size_t need = psd_select_sparse_decode_workspace_bytes(shape, b_max);
  if (need == 0) {
    psd::Geo g;
    psd_status st = check_shape(shape, &g);
    if (st != PSD_OK) return st;
    return b_max < 2 ? PSD_ERR_INVALID_ARG : PSD_ERR_CAPACITY;
  }
  if (need > PSD_SCRATCH_BYTES) return PSD_ERR_SCRATCH;
  void* ws = scratch_on_current_device();
  if (!ws) return PSD_ERR_LAUNCH;
  return step_common(shape, q, meta, k_cache, v_cache, block_table, seq_lens, budgets, b_max,
                     scale, sel_pages, sel_count, out, ws, PSD_SCRATCH_BYTES, true, stream);
}

}  // extern "C"
