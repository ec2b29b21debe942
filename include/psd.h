/*
 * psd.h - page-selected sparse paged decode attention for AMD Instinct MI355X (gfx950).
 *
 * One decode step over a paged KV cache in the vLLM block layout (EntmaxKV README,
 * introduction: [2, num_blocks, page_size, H_kv, D] plus a block table; pages of 16
 * tokens), in three calls:
 *
 *   1. psd_page_meta_update  - refresh the per-page key min/max of the pages an append
 *                              touched (EntmaxKV README, package tree: per-page k_min /
 *                              k_max refresh).
 *   2. psd_select_pages      - score every page from those statistics with a
 *                              Quest-style upper bound, take the max over each GQA
 *                              group, and keep the top-b pages per (sequence, KV head)
 *                              with the sink and the most recent page always kept
 *                              (EntmaxKV README, "Two selection strategies", top-k;
 *                              LOCKS README, introduction, "Configuration", "How it
 *                              works").
 *   3. psd_sparse_decode     - exact softmax attention over only the kept pages
 *                              (EntmaxKV README, introduction; LOCKS README, "How it
 *                              works", sparse decode).
 *
 * plus psd_dense_decode, the same attention over every page (the dense baseline the
 * pages compare against: AMASS page, "Headline results"; LOCKS README, "Efficiency").
 *
 * Conventions shared by every call
 * --------------------------------
 * - All data pointers are DEVICE pointers owned by the caller. The library allocates
 *   nothing, keeps no state between calls and is reentrant. Workspaces are caller-owned
 *   device buffers of at least the size the matching *_workspace_bytes query returns;
 *   their contents need no initialisation and are scratch after the call. The one
 *   exception is psd_decode_step_noalloc, whose workspace is a static device array the
 *   library holds on each GPU (see that call).
 * - Every call only enqueues work on `stream` (HIP stream, may be 0 / the null stream)
 *   and returns without synchronising. A workspace or output may be reused only in
 *   stream order.
 * - Arguments are checked on the host before anything is launched; a failed check
 *   returns a negative psd_status and launches nothing. Device-side preconditions are
 *   documented per call and are not checked: seq_lens[s] in [1, 16 * max_pages_per_seq],
 *   block ids in [0, num_blocks).
 * - Element types: q, K, V and the page statistics share `dtype` (fp32 or bf16). The
 *   attention output is fp32.
 * - GQA grouping: query head h belongs to KV head h / (num_q_heads / num_kv_heads).
 * - A sequence of length L has n = ceil(L / 16) logical pages; page p holds tokens
 *   [16 p, min(16 p + 16, L)); slots past L in the last page are never read as data.
 */
#ifndef PSD_H
#define PSD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum psd_status {
  PSD_OK = 0,
  PSD_ERR_INVALID_ARG = -1, /* null pointer, inconsistent shape, stride or alignment */
  PSD_ERR_UNSUPPORTED = -2, /* head dims / group size outside what the kernels build */
  PSD_ERR_WORKSPACE = -3,   /* workspace null or smaller than the query returned */
  PSD_ERR_CAPACITY = -4,    /* b_max (pages kept per unit) beyond the selection limit */
  PSD_ERR_LAUNCH = -5,      /* the HIP runtime rejected a kernel launch */
  PSD_ERR_SCRATCH = -6      /* psd_decode_step_noalloc: the step needs more workspace than
                               PSD_SCRATCH_BYTES */
} psd_status;

typedef enum psd_dtype { PSD_F32 = 0, PSD_BF16 = 1 } psd_dtype;

/*
 * Shape of one layer's paged cache and decode batch.
 *
 * Supported: page_size == 16; (head_dim, head_dim_v) in {(64, 64), (128, 128),
 * (576, 512)}; group G = num_q_heads / num_kv_heads either <= 16 or a multiple of 16
 * up to 128. A latent (MLA-style) cache passes the same pointer as K and V with
 * head_dim_v < head_dim: V is the first head_dim_v dims of each cached row.
 *
 * Strides are in elements; the last (dim) axis is contiguous. Every pointer and every
 * stride times the element size must be a multiple of 16 bytes.
 */
typedef struct psd_shape {
  int32_t batch;             /* B: sequences in the decode batch */
  int32_t num_q_heads;       /* H_q: a multiple of num_kv_heads */
  int32_t num_kv_heads;      /* H_kv */
  int32_t head_dim;          /* D of q and K */
  int32_t head_dim_v;        /* D_v of V and of the output, <= head_dim */
  int32_t page_size;         /* tokens per page; must be 16 */
  int32_t num_blocks;        /* physical blocks in the cache (and in the statistics) */
  int32_t max_pages_per_seq; /* row length of the block table */
  int32_t dtype;             /* psd_dtype of q, K, V and the page statistics */
  int32_t reserved;          /* must be 0 */
  int64_t k_block_stride, k_token_stride, k_head_stride;
  int64_t v_block_stride, v_token_stride, v_head_stride;
} psd_shape;

/*
 * Page statistics layout (`meta`), in `dtype`, indexed by PHYSICAL block like the cache:
 *   [num_blocks][num_kv_heads][head_dim / CD][2][CD],  CD = 64 bytes of dims
 *   (32 for bf16, 16 for fp32),
 * i.e. the per-dim minimum (index 0) and maximum (index 1) of a page's valid keys, cut
 * into chunks of CD dims; the minima and maxima of one chunk form one 128-byte line and
 * the lines of one (block, head) are one contiguous record of 2 * head_dim elements.
 * Total size: 2 * num_blocks * num_kv_heads * head_dim elements. Values are exact
 * (copied key values). Statistics held as two planes P[2][num_blocks][num_kv_heads]
 * [head_dim] (P[0] the minima, P[1] the maxima) map to this layout element by element:
 * meta[b][h][c][t][i] = P[t][b][h][c * CD + i], a permutation of the same elements.
 * psd_page_meta_update builds the records from the cache, so a caller need not hold
 * statistics of its own.
 */
/*
 * psd_page_meta_update - recompute page statistics from the cached keys.
 *
 * For every sequence s, refreshes the logical pages [first_page[s], n_s) (all pages from
 * first_page on), or only the page holding token L_s - 1 when first_page is NULL (the
 * decode-time refresh after the new token's K/V has been written into the cache).
 * Passing first_page[s] = 0 rebuilds every page (prefill). first_page values < 0 are
 * treated as 0. Writes the statistics of blocks block_table[s][p] of those pages only.
 *
 *   k_cache     [num_blocks, 16, H_kv, D] through the k_* strides (device, read)
 *   meta        statistics in the layout above (device, written)
 *   block_table [B, max_pages_per_seq] int32 physical block ids (device, read)
 *   seq_lens    [B] int32 tokens per sequence including the newest (device, read)
 *   first_page  [B] int32 or NULL (device, read)
 *
 * Source: EntmaxKV README, package tree (per-page k_min / k_max refresh) and
 * introduction (statistics kept beside the vLLM-layout cache).
 */
psd_status psd_page_meta_update(const psd_shape* shape, const void* k_cache, void* meta,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* first_page, hipStream_t stream);

/* Workspace bytes psd_select_pages needs for this shape and b_max. 0 if unsupported. */
size_t psd_select_workspace_bytes(const psd_shape* shape, int32_t b_max);

/*
 * psd_select_pages - pick the pages each (sequence, KV head) attends this step.
 *
 * For query head h and page p: UB_h(p) = sum_d max(q[h,d] kmin[p,d], q[h,d] kmax[p,d]),
 * accumulated in fp64 over ascending d with exact products (bit-identical to a plain
 * sequential fp64 loop). Group score(p) = max of UB_h(p) over the group's query heads.
 * With n pages and b = min(n, max(budgets[s], 2)) (n when n <= 2): if n <= b all pages
 * are kept; else pages 0 and n-1 plus the b-2 best of pages 1..n-2 by (score
 * descending, page index ascending). No scale is applied before ranking.
 *
 *   q           [B, H_q, D] (device, read)
 *   meta        statistics as above, current for every page scored (device, read)
 *   budgets     [B] int32 pages kept per KV head, sink and tail included (device, read)
 *   b_max       capacity of each selection row, >= 2; device precondition:
 *               min(n_s, max(budgets[s], 2)) <= b_max. A row that would exceed it is
 *               not truncated: its count is written as -1 and its pages as -1, and
 *               psd_sparse_decode then writes NaN for that unit's heads.
 *   sel_pages   [B, H_kv, b_max] int32 kept LOGICAL pages, ascending, -1 padded
 *               (device, written)
 *   sel_count   [B, H_kv] int32 number of kept pages (device, written)
 *   workspace   >= psd_select_workspace_bytes(shape, b_max) bytes (device, scratch)
 *
 * Returns PSD_ERR_CAPACITY when b_max is beyond what the two-level selection holds.
 * Source: EntmaxKV README, "Two selection strategies" (top-k from a Quest-style bound,
 * budget counts pages and includes the tail page); LOCKS README, introduction and
 * "Results" (sink + recent kept, inside b), "Configuration" (GQA combine `max`),
 * "How it works" (static top-b, no second exact pass; MLA max-union over heads).
 */
psd_status psd_select_pages(const psd_shape* shape, const void* q, const void* meta,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* budgets, int32_t b_max, int32_t* sel_pages,
                            int32_t* sel_count, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * The two stages of psd_select_pages, for callers that schedule or time them apart.
 * psd_select_pages(args) is exactly psd_select_score(args) followed, on the same stream,
 * by psd_select_merge with the same shape, q, meta, block_table, seq_lens, budgets, b_max,
 * sel_pages and workspace.
 *
 * psd_select_score scores the pages. It writes sel_count and every sel_pages entry except
 * the ranked winners: the sink, the tail and the -1 padding, and the whole row of a unit
 * that keeps every page or exceeds b_max. When one workgroup scores a whole unit (batches
 * of at least 128 units of at most 2050 pages, or rows of at most 256 pages at any batch
 * size; groups of up to 8 heads) it also writes
 * the winners, and psd_select_merge then launches nothing. Otherwise it leaves
 * candidates in the workspace: either each chunk's top pages by exact score or, for
 * groups of 16 or more bf16 heads, approximate scores with a proven error bound.
 * psd_select_merge reads them back and writes the b-2 winners of every ranking unit into
 * sel_pages[..., 1 .. b-2] in ascending order. For the approximate case it first rescores
 * exactly the pages that the bound cannot decide, which is why it takes q, meta and
 * block_table. The workspace must not be
 * touched between the two calls. Arguments, errors and sources are as for
 * psd_select_pages.
 */
psd_status psd_select_score(const psd_shape* shape, const void* q, const void* meta,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* budgets, int32_t b_max, int32_t* sel_pages,
                            int32_t* sel_count, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);
psd_status psd_select_merge(const psd_shape* shape, const void* q, const void* meta,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* budgets, int32_t b_max, int32_t* sel_pages,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Workspace bytes psd_sparse_decode (max_pages_attended = its b_max) or psd_dense_decode
 * (max_pages_attended = max_pages_per_seq) needs. 0 if unsupported.
 */
size_t psd_decode_workspace_bytes(const psd_shape* shape, int32_t max_pages_attended);

/*
 * psd_sparse_decode - softmax attention over the kept pages only.
 *
 * out[s, h, :] = sum_t softmax_t(scale * q[s,h] . K_t) V_t[:D_v] over the valid tokens t
 * of the pages sel_pages[s, h / G, 0 .. sel_count - 1]. Accumulation is fp32; the page
 * splits of a unit are combined by log-sum-exp, inside the workgroup when one workgroup
 * holds a whole unit (batches of at least 128 units, or rows of at most 256 pages at any
 * batch size; groups of up to 16 heads, D <= 128),
 * else by a second launch over partials in the workspace. Units whose sel_count is
 * negative get NaN.
 *
 *   q, k_cache, v_cache, block_table, seq_lens as above (device, read). v_cache may
 *               also be pinned host memory passed by its device address
 *               (hipHostMalloc, then hipHostGetDevicePointer): the value tier in host
 *               DRAM, of which only the kept pages' V rows cross the host link (AMASS
 *               page and LOCKS README, "Configuration": the mem-v variant keeps K
 *               resident and V in DRAM). The same holds for psd_select_sparse_decode,
 *               psd_decode_step and psd_dense_decode.
 *   sel_pages, sel_count, b_max   as written by psd_select_pages (device, read)
 *   scale       softmax scale (1 / sqrt(head_dim) for standard attention)
 *   out         [B, H_q, D_v] fp32 (device, written)
 *   workspace   >= psd_decode_workspace_bytes(shape, b_max) bytes (device, scratch)
 *
 * Source: EntmaxKV README, introduction (attention exact over the selection) and
 * package tree (decode over selected pages); LOCKS README, "How it works" (a paged
 * attention kernel reads only the selected pages).
 */
psd_status psd_sparse_decode(const psd_shape* shape, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* sel_pages,
                             const int32_t* sel_count, int32_t b_max, float scale, float* out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes psd_select_sparse_decode needs for this shape and b_max. 0 if
 * unsupported. */
size_t psd_select_sparse_decode_workspace_bytes(const psd_shape* shape, int32_t b_max);

/*
 * psd_select_sparse_decode - psd_select_pages followed by psd_sparse_decode, as one call.
 *
 * Writes exactly what psd_select_pages(shape, q, meta, block_table, seq_lens, budgets,
 * b_max, sel_pages, sel_count, ...) and then psd_sparse_decode(shape, q, k_cache, v_cache,
 * block_table, seq_lens, sel_pages, sel_count, b_max, scale, out, ...) write, bit for bit.
 * When one workgroup can both rank and attend a whole unit (batches of at least 128
 * units of at most 2050 pages, or rows of at most 256 pages at any batch size; groups of
 * up to 4 heads, D <= 128 in bf16 or D = 64 in fp32) it is a single launch: each
 * workgroup scores and ranks its unit's pages, keeps the page list on chip and attends
 * over it, so that no unit waits for the slowest ranking of the batch before its
 * attention starts, and a short batch-1 step is one launch. Otherwise the call
 * enqueues the two calls' launches in turn, sharing the workspace. sel_pages and
 * sel_count are still written in full.
 *
 *   arguments   as for psd_select_pages and psd_sparse_decode
 *   workspace   >= psd_select_sparse_decode_workspace_bytes(shape, b_max) bytes (scratch)
 *
 * Errors as for the two calls (PSD_ERR_CAPACITY when b_max is beyond what the selection
 * holds). Source: EntmaxKV README, "Two selection strategies" and package tree (select,
 * then decode over the selection); LOCKS README, "How it works" (scores, static top-b,
 * then a paged attention kernel over the selected pages, within one decode step).
 */
psd_status psd_select_sparse_decode(const psd_shape* shape, const void* q, const void* meta,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* budgets, int32_t b_max, float scale,
                                    int32_t* sel_pages, int32_t* sel_count, float* out,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * psd_decode_step - one decode step: psd_page_meta_update with first_page == NULL (the
 * tail page of every sequence, every KV head), then psd_select_sparse_decode.
 *
 * Writes exactly what those two calls write, bit for bit (statistics, rows, counts,
 * outputs). The tail refresh runs inside another launch where it can: inside the single
 * launch of psd_select_sparse_decode, or as one extra workgroup per unit of the exact
 * scoring launch (when that launch has at most one workgroup per compute unit) or of the
 * selection's merge launch; otherwise it is a launch of its own, ahead of the selection.
 * The tail page is never a ranking candidate, so its statistics are not read by the same
 * step's scoring. Running the refresh concurrently
 * with the scoring needs one more device precondition than the two calls: the block
 * holding a sequence's tail page is not an earlier page of any sequence in the batch
 * (true of a paged cache whose partly filled blocks each belong to one sequence).
 *
 *   meta        statistics [num_blocks, H_kv, D / CD, 2, CD] (device, read and written)
 *   others      as for psd_select_sparse_decode, with the same workspace query
 *
 * Source: EntmaxKV README, package tree (per-page k_min / k_max refresh at append time,
 * then selection and decode over the selected pages); LOCKS README, "How it works".
 */
psd_status psd_decode_step(const psd_shape* shape, const void* q, void* meta, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* seq_lens, const int32_t* budgets, int32_t b_max,
                           float scale, int32_t* sel_pages, int32_t* sel_count, float* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Value tier with a resident hot buffer (AMASS page, "What is in the box", item 2: the
 * DRAM value tier keeps a bounded resident hot buffer plus a staging pool in VRAM; LOCKS
 * README, "How it works", the optional DRAM tier keeps only the pages called each step
 * resident). V lives in pinned host memory (v_host: its device address, the V layout of
 * the shape); a device buffer `hot` of `slots` slices, each the 16 token rows of one
 * (block, KV head) ([slots][16][D_v] elements of dtype), keeps the slices that steps
 * call. Each step:
 *
 *   psd_value_tier_stage     - for every kept page of every unit (sel_pages / sel_count
 *                              of psd_select_pages), the slot of its V slice: a slice
 *                              already resident is a hit; a missed slice gets a slot that
 *                              this step does not use (evicting what it held) and its 16
 *                              rows are copied from v_host over the host link. When the
 *                              slots run out, the remaining entries read V from v_host.
 *                              Writes vslot[s][g][e] (slot of entry e, -1: from host) and
 *                              stats[0..3] = hits, misses (entries), slices copied,
 *                              entries read from host (device, uint64).
 *   psd_sparse_decode_tiered - psd_sparse_decode with each entry's V read from its slot
 *                              (or from v_host), the same arithmetic: the same bits as
 *                              psd_sparse_decode over the same V.
 *
 *   state       device, psd_value_tier_state_bytes: the page map and the slots' owners
 *               and last steps, kept between steps; psd_value_tier_reset empties it
 *               (call it once before the first stage, and after any change of v_host's
 *               contents that the hot buffer holds).
 *   step        any value that differs from the previous stage call's since the reset
 *               (a step counter); the slots this call uses are stamped with it.
 *   workspace   psd_value_tier_workspace_bytes(shape, b_max, slots) (scratch).
 * GQA shapes only: D == D_v in {64, 128}, up to 16 query heads per KV head (otherwise
 * PSD_ERR_UNSUPPORTED). The stage enqueues four launches; stats are final once they
 * have run. Calls that share a state or a hot buffer run in stream order.
 */
size_t psd_value_tier_state_bytes(const psd_shape* shape, int32_t slots);
size_t psd_value_tier_workspace_bytes(const psd_shape* shape, int32_t b_max, int32_t slots);
psd_status psd_value_tier_reset(const psd_shape* shape, int32_t slots, void* state,
                                hipStream_t stream);
psd_status psd_value_tier_stage(const psd_shape* shape, const void* v_host, void* hot,
                                void* state, int32_t slots, int32_t step,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* sel_pages, const int32_t* sel_count,
                                int32_t b_max, int32_t* vslot, uint64_t* stats, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);
/* workspace: psd_decode_workspace_bytes(shape, b_max), as for psd_sparse_decode. */
psd_status psd_sparse_decode_tiered(const psd_shape* shape, const void* q, const void* k_cache,
                                    const void* v_host, const void* hot, const int32_t* vslot,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* sel_pages, const int32_t* sel_count,
                                    int32_t b_max, float scale, float* out, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/*
 * KV tier: the same with K in host memory too (AMASS page, "Two variants, one algorithm":
 * the mem-kv residency, K and V offloaded to DRAM with only the page summaries and the
 * called pages resident; LOCKS README, "How it works", the optional DRAM tier's mem-kv).
 * k_host is the device address of the K cache in pinned host memory (the K layout of the
 * shape); hot_k, [slots][16][D] elements of dtype, holds the K rows of each resident slice
 * in the slot that holds its V in hot_v. The page statistics stay in device memory, so
 * the selection reads no K; psd_page_meta_update refreshes the tail pages from k_host.
 *
 *   psd_kv_tier_stage          - psd_value_tier_stage, with each copied slice's K rows
 *                                brought to hot_k as well; slot[s][g][e] is the slot of
 *                                both (-1: entry e reads K and V from host memory).
 *   psd_sparse_decode_kv_tiered - psd_sparse_decode with each entry's K and V read from
 *                                its slot (or from host memory): the same bits as
 *                                psd_sparse_decode over the same K and V.
 *
 * State, workspace sizes and reset are the value tier's (psd_value_tier_state_bytes,
 * psd_value_tier_workspace_bytes, psd_value_tier_reset); a state serves one tier kind
 * from its reset on. hot_k and hot_v may be null only when slots == 0 (both or neither
 * in the attention). Errors and limits as for the value tier.
 */
psd_status psd_kv_tier_stage(const psd_shape* shape, const void* k_host, const void* v_host,
                             void* hot_k, void* hot_v, void* state, int32_t slots, int32_t step,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* sel_pages, const int32_t* sel_count, int32_t b_max,
                             int32_t* slot, uint64_t* stats, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);
/* workspace: psd_decode_workspace_bytes(shape, b_max), as for psd_sparse_decode. */
psd_status psd_sparse_decode_kv_tiered(const psd_shape* shape, const void* q, const void* k_host,
                                       const void* v_host, const void* hot_k, const void* hot_v,
                                       const int32_t* slot, const int32_t* block_table,
                                       const int32_t* seq_lens, const int32_t* sel_pages,
                                       const int32_t* sel_count, int32_t b_max, float scale,
                                       float* out, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * psd_diag_walk - diagnostic: the decode step's memory reads with no arithmetic, to
 * measure what the memory system gives their access patterns on this GPU (the practical
 * ceiling of the kernels that make them). Not part of the method.
 *
 *   kind 0: every kept page's K and V rows of every (sequence, KV head) unit
 *           (sel_pages / sel_count as psd_sparse_decode takes them), one 1024-thread
 *           workgroup per unit, 16 bytes per lane per load (whole 256-byte rows at
 *           D = 128 bf16); a latent cache (v_cache = k_cache, same strides) walks K only.
 *   kind 1: the statistics record of every candidate page 1 .. n - 2 of every unit (meta
 *           as psd_page_meta_update writes it), 128-byte lines of 8 pages per load.
 * Every 32-bit word a unit reads is folded by XOR into checksum[s * H_kv + g] (device,
 * B * H_kv uint32, all written), so a test can check that exactly those bytes were read.
 * Shapes:
 * 16-byte pieces per K row of 8, 16, 32 (with V rows of the same size) or 72 (latent);
 * others give PSD_ERR_UNSUPPORTED. Pointers not needed by the kind may be null.
 */
psd_status psd_diag_walk(const psd_shape* shape, int32_t kind, const void* k_cache,
                         const void* v_cache, const void* meta, const int32_t* block_table,
                         const int32_t* seq_lens, const int32_t* sel_pages,
                         const int32_t* sel_count, int32_t b_max, uint32_t* checksum,
                         hipStream_t stream);

/*
 * psd_dense_decode - the same attention over every page of each sequence (baseline).
 *
 * workspace >= psd_decode_workspace_bytes(shape, shape->max_pages_per_seq) bytes.
 * Source: EntmaxKV README, package tree (exact paged decode); AMASS page, "Headline
 * results" and LOCKS README, "Efficiency" (dense attention as the comparison line).
 */
psd_status psd_dense_decode(const psd_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, float scale, float* out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * psd_select_pages_coverage - adaptive coverage selection: keep, per (sequence, KV head),
 * the fewest pages whose exact attention mass reaches `coverage` (a variant of
 * psd_select_pages that needs K itself instead of the page statistics).
 *
 * For query head h the page mass w_h(p) is the share of h's exact
 * softmax(scale * q_h . k) over the sequence's valid tokens that falls on page p; the
 * group mass W(p) is the mean of w_h(p) over the group's query heads. The kept set is
 * page 0 (sink), page n-1 (tail) and the pages 1..n-2 in (W descending, page index
 * ascending) order, added until the kept mass reaches `coverage` or b_max pages are
 * kept; coverage >= 1 keeps every page that fits. Sequences of n <= 2 pages keep every
 * page.
 *
 *   q            [B, H_q, D] dtype, 16-byte aligned
 *   k_cache      paged K cache (shape strides), 16-byte aligned; every row of each page's
 *                block is read (the tail block's rows at or past the length too, which
 *                must be readable), and rows at or past the length are ignored
 *   block_table  [B, max_pages_per_seq] int32 physical block ids
 *   seq_lens     [B] int32 token counts
 *   coverage     target kept mass, in (0, 1]; larger values act as 1
 *   scale        softmax scale (> 0), normally 1/sqrt(D)
 *   b_max        entries per selection row (>= 2); caps the kept pages
 *   sel_pages    [B, H_kv, b_max] int32 out: kept logical pages ascending, -1 padded
 *   sel_count    [B, H_kv] int32 out: kept pages per row
 *   workspace    >= psd_select_coverage_workspace_bytes(shape) bytes (each query head's
 *                page max and page exp-sum, fp32)
 *
 * Supported: group size G <= 8, D in {64, 128}, max_pages_per_seq <= 4096; otherwise
 * PSD_ERR_UNSUPPORTED (the pages offer the coverage knob for GQA models only). The
 * outputs feed psd_sparse_decode unchanged. Masses are formed in fp32 per page,
 * normalised in fp64 and ranked as fp32 values, so pages whose masses differ by less than
 * about 1e-6 may order either way.
 * Source: AMASS README, "Key AmassConfig fields" (coverage: adaptive per-head nucleus
 * over exact page masses, default 0.95); LOCKS README, "Configuration".
 */
size_t psd_select_coverage_workspace_bytes(const psd_shape* shape);
psd_status psd_select_pages_coverage(const psd_shape* shape, const void* q, const void* k_cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     float coverage, float scale, int32_t b_max,
                                     int32_t* sel_pages, int32_t* sel_count, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/*
 * psd_decode_step_noalloc - psd_decode_step without a caller workspace, for callers that
 * cannot allocate device memory around the call (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).
 *
 * Writes exactly what psd_decode_step with the same arguments writes. Instead of a
 * workspace argument it uses a static device array of PSD_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; its device address is looked up
 * once per device on the first call with that device current. The call allocates and
 * frees nothing. A step whose workspace (psd_select_sparse_decode_workspace_bytes) would
 * exceed PSD_SCRATCH_BYTES returns PSD_ERR_SCRATCH before anything is launched. Every call
 * on one GPU shares that GPU's array and leaves its contents behind: calls that overlap on
 * one GPU (other streams, other host threads) race, so order them on one stream.
 *
 *   arguments   as for psd_decode_step, without workspace and workspace_bytes
 */
#define PSD_SCRATCH_BYTES ((size_t)64 << 20) /* 64 MiB per GPU */
psd_status psd_decode_step_noalloc(const psd_shape* shape, const void* q, void* meta,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* budgets, int32_t b_max, float scale,
                                   int32_t* sel_pages, int32_t* sel_count, float* out,
                                   hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* psd_status_string(psd_status status);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t psd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PSD_H */
