"""Plain fp64 CPU oracle for page-selected sparse paged decode attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The library
(``page_selected_sparse_amd``) never imports it, and it imports nothing from the
library: it is the independent definition the GPU path is checked against.

What it computes, one decode step, for every sequence s and KV head g:

1. Page statistics (EntmaxKV README, introduction and the ``page_metadata.py`` entry of
   its package tree: per-page key min/max kept beside the paged cache). Page p of a
   sequence of length L holds logical tokens [16p, min(16p + 16, L)); its K min and
   max per dim are taken over those valid tokens only.
2. Page bound (EntmaxKV README, "Two selection strategies", top-k: a Quest-style upper
   bound on a page's best score, computed from the statistics without touching cached
   tokens). For query head h: UB_h(p) = sum_d max(q_d * kmin_d, q_d * kmax_d), the
   largest q.k over the page's per-dim bounding box. It is accumulated in fp64 in
   ascending d, one exact product at a time (bf16*bf16 and fp32*fp32 products are exact
   in fp64), so any implementation that adds the same products in the same order
   reproduces it bit for bit.
3. Group score (LOCKS README, "Configuration": the GQA group combine, ``max`` option;
   "How it works": MLA scores are max-unioned over query heads): score_g(p) is the max
   of UB_h(p) over the query heads h of group g; a zero is taken as +0.
4. Selection (EntmaxKV README, top-k: the budget counts pages and includes the always
   attended tail page; LOCKS README introduction and "Results": the sink and the most
   recent page are always kept, counted inside b). With n pages and budget b: if
   n <= b every page is kept; otherwise pages 0 and n-1 plus the b-2 best of pages
   1..n-2 by (score descending, page index ascending). The list is returned ascending.
5. Attention (EntmaxKV README, introduction: attention is exact over the selection):
   softmax(scale * q.k) over the valid tokens of the kept pages, times V.
6. Dense decode: step 5 over every page.

Adaptive coverage (AMASS README, "Key AmassConfig fields"; LOCKS README,
"Configuration", the ``coverage`` knob: a per-head nucleus over exact page masses,
0.95 by default, GQA only) replaces steps 2-4 with:

2'. Page mass: for query head h, the share of its exact softmax(scale * q_h.k) over the
   sequence's valid tokens that falls on page p. Each head's masses sum to 1.
3'. Group mass: the mean of the masses over the query heads of group g (the LOCKS
   ``nrm`` combine of per-head masses; it keeps a distribution over pages).
4'. Selection: the sink and the tail, then pages 1..n-2 in (mass descending, page
   ascending) order, added one at a time until the kept mass reaches ``coverage`` or
   the row (b_max entries) is full; coverage >= 1 keeps every page that fits. The list
   is returned ascending.

Where the pages leave a step open this module takes these readings: the bound is the
exact max of q.k over the min/max box; the group combine is the max; ties go to the
lower page index; the softmax scale is 1/sqrt(D_qk); a budget below 2 still keeps the
sink and the tail. Every function here is pinned by tests in tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np

PAGE = 16


def pages_of(length: int) -> int:
    """Number of 16-token pages holding ``length`` tokens."""
    return (int(length) + PAGE - 1) // PAGE


def valid_in_page(length: int, p: int) -> int:
    """Number of valid tokens in logical page p of a sequence of ``length`` tokens."""
    return max(0, min(PAGE, int(length) - PAGE * int(p)))


def page_minmax(tokens: np.ndarray):
    """Per-dim min and max of a page's valid keys.

    ``tokens``: [T, ...] float64, T >= 1 valid tokens. Returns (kmin, kmax) of shape [...].
    """
    tokens = np.asarray(tokens, dtype=np.float64)
    return tokens.min(axis=0), tokens.max(axis=0)


def sequence_meta(k_cache, block_table_row, length: int, chunk: int = 1024):
    """K min/max of every page of one sequence, in logical page order.

    ``k_cache``: indexable by an array of physical block ids, giving float64
    [m, 16, H_kv, D]. Returns kmin, kmax: [n, H_kv, D]. Pages are read ``chunk`` at a
    time so that long sequences fit in memory.
    """
    n = pages_of(length)
    blocks = np.asarray(block_table_row[:n], dtype=np.int64)
    kmin = kmax = None
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        k = np.asarray(k_cache[blocks[c0:c1]], dtype=np.float64)  # [m, 16, H_kv, D]
        if kmin is None:
            kmin = np.empty((n,) + k.shape[2:])
            kmax = np.empty_like(kmin)
        for p in range(c0, c1):
            kmin[p], kmax[p] = page_minmax(k[p - c0, : valid_in_page(length, p)])
    return kmin, kmax


def page_bounds(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Quest-style upper bound UB[h, p] = sum_d max(q[h,d] kmin[p,d], q[h,d] kmax[p,d]).

    ``q``: [G, D]; ``kmin``, ``kmax``: [n, D]. The sum runs over d in ascending order in
    fp64; each step adds the product picked by the sign of q[h, d] (q >= 0 takes kmax).
    """
    q = np.asarray(q, dtype=np.float64)
    kmin = np.asarray(kmin, dtype=np.float64)
    kmax = np.asarray(kmax, dtype=np.float64)
    G, D = q.shape
    acc = np.zeros((G, kmin.shape[0]), dtype=np.float64)
    for d in range(D):
        qd = q[:, d: d + 1]
        corner = np.where(qd >= 0, kmax[None, :, d], kmin[None, :, d])
        acc = acc + qd * corner
    return acc


def group_scores(ub: np.ndarray) -> np.ndarray:
    """Max of the bounds over the query heads of one group; -0 becomes +0."""
    return np.max(ub, axis=0) + 0.0


def effective_budget(n: int, budget: int) -> int:
    """Pages kept: the budget, at least the sink and the tail, at most every page."""
    if n <= 2:
        return n
    return min(n, max(int(budget), 2))


def select_pages(scores: np.ndarray, n: int, budget: int) -> np.ndarray:
    """Kept logical pages, ascending: sink, tail and the best b-2 inner pages."""
    b = effective_budget(n, budget)
    if n <= b:
        return np.arange(n, dtype=np.int64)
    inner = np.arange(1, n - 1, dtype=np.int64)
    # lexsort sorts by the last key first: score descending, then index ascending.
    order = np.lexsort((inner, -np.asarray(scores, dtype=np.float64)[inner]))
    chosen = inner[order[: b - 2]]
    return np.sort(np.concatenate([[0], chosen, [n - 1]]).astype(np.int64))


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Exact softmax attention of queries [G, D] over keys [T, D] and values [T, Dv]."""
    q = np.asarray(q, dtype=np.float64)
    z = scale * (q @ np.asarray(keys, dtype=np.float64).T)
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    return (w @ np.asarray(values, dtype=np.float64)) / w.sum(axis=1, keepdims=True)


def gather_tokens(cache, block_table_row, length: int, pages, head: int, dims: int):
    """Valid tokens of the given logical pages for one KV head: [T, dims] float64."""
    pages = np.asarray(pages, dtype=np.int64)
    blocks = np.asarray(block_table_row, dtype=np.int64)[pages]
    rows = np.asarray(cache[blocks, :, head, :dims], dtype=np.float64)  # [m, 16, dims]
    parts = [rows[i, : valid_in_page(length, p)] for i, p in enumerate(pages)]
    return np.concatenate(parts, axis=0)


def select_sequence(q_seq, kmin, kmax, num_kv_heads: int, n: int, budget: int):
    """Kept pages for every KV head of one sequence.

    ``q_seq``: [H_q, D]; ``kmin``/``kmax``: [n, H_kv, D]. Returns (pages per head,
    group scores per head [H_kv, n]). Scores are computed for all n pages even when
    every page is kept.
    """
    Hq = q_seq.shape[0]
    G = Hq // num_kv_heads
    sel, scores = [], []
    for g in range(num_kv_heads):
        ub = page_bounds(q_seq[g * G:(g + 1) * G], kmin[:, g], kmax[:, g])
        sc = group_scores(ub)
        scores.append(sc)
        sel.append(select_pages(sc, n, budget))
    return sel, np.stack(scores)


def decode_sequence(q_seq, k_cache, v_cache, block_table_row, length: int, pages_per_head,
                    scale: float, head_dim_v: int):
    """Attention output [H_q, Dv] of one sequence given the kept pages of each KV head."""
    Hq, D = q_seq.shape
    Hkv = len(pages_per_head)
    G = Hq // Hkv
    out = np.empty((Hq, head_dim_v), dtype=np.float64)
    for g in range(Hkv):
        keys = gather_tokens(k_cache, block_table_row, length, pages_per_head[g], g, D)
        vals = gather_tokens(v_cache, block_table_row, length, pages_per_head[g], g,
                             head_dim_v)
        out[g * G:(g + 1) * G] = attend(q_seq[g * G:(g + 1) * G], keys, vals, scale)
    return out


def sparse_step(q, k_cache, v_cache, block_table, seq_lens, budgets, scale: float,
                head_dim_v: int, num_kv_heads: int, sequences=None):
    """One sparse decode step for the given sequences (default: all).

    ``q``: [B, H_q, D] float64. ``k_cache``/``v_cache``: indexable by block ids giving
    float64 [m, 16, H_kv, D(v)]. Returns dict s -> (out [H_q, Dv], pages per head,
    group scores [H_kv, n], kmin, kmax).
    """
    q = np.asarray(q, dtype=np.float64)
    seqs = range(q.shape[0]) if sequences is None else sequences
    res = {}
    for s in seqs:
        L = int(seq_lens[s])
        n = pages_of(L)
        kmin, kmax = sequence_meta(k_cache, block_table[s], L)
        sel, scores = select_sequence(q[s], kmin, kmax, num_kv_heads, n, int(budgets[s]))
        out = decode_sequence(q[s], k_cache, v_cache, block_table[s], L, sel, scale,
                              head_dim_v)
        res[s] = (out, sel, scores, kmin, kmax)
    return res


def dense_step(q, k_cache, v_cache, block_table, seq_lens, scale: float, head_dim_v: int,
               num_kv_heads: int, sequences=None):
    """Dense decode over every page; dict s -> out [H_q, Dv]."""
    q = np.asarray(q, dtype=np.float64)
    seqs = range(q.shape[0]) if sequences is None else sequences
    res = {}
    for s in seqs:
        L = int(seq_lens[s])
        every = [np.arange(pages_of(L))] * num_kv_heads
        res[s] = decode_sequence(q[s], k_cache, v_cache, block_table[s], L, every, scale,
                                 head_dim_v)
    return res


def page_masses(q_group, keys, length: int, scale: float) -> np.ndarray:
    """Group page masses W [n] of one (sequence, KV head) unit (steps 2' and 3').

    ``q_group``: [G, D] queries of the group; ``keys``: [L, D] the sequence's valid keys
    in token order. For each head, w_h(p) is the softmax weight of head h summed over
    the tokens of page p; W(p) is the mean of w_h(p) over the G heads.
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    n = pages_of(length)
    z = scale * (q_group @ keys.T)                    # [G, L]
    e = np.exp(z - z.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)              # each row sums to 1
    page_of_token = np.arange(length) // PAGE
    per_head = np.zeros((q_group.shape[0], n))
    for h in range(q_group.shape[0]):
        per_head[h] = np.bincount(page_of_token, weights=w[h], minlength=n)
    return per_head.mean(axis=0)


def select_coverage(mass: np.ndarray, n: int, coverage: float, b_max: int) -> np.ndarray:
    """Kept logical pages, ascending, for coverage selection (step 4')."""
    if n <= 2:
        return np.arange(n, dtype=np.int64)
    mass = np.asarray(mass, dtype=np.float64)
    inner = np.arange(1, n - 1, dtype=np.int64)
    order = inner[np.lexsort((inner, -mass[inner]))]
    room = min(n - 2, max(int(b_max), 2) - 2)
    if coverage >= 1.0:
        take = room
    else:
        kept = mass[0] + mass[n - 1]
        take = 0
        while kept < coverage and take < room:
            kept += mass[order[take]]
            take += 1
    return np.sort(np.concatenate([[0], order[:take], [n - 1]]).astype(np.int64))


def coverage_select_sequence(q_seq, k_cache, block_table_row, length: int, num_kv_heads: int,
                             scale: float, coverage: float, b_max: int):
    """Coverage selection for every KV head of one sequence.

    Returns (pages per head, group masses per head [H_kv, n]).
    """
    q_seq = np.asarray(q_seq, dtype=np.float64)
    Hq, D = q_seq.shape
    G = Hq // num_kv_heads
    n = pages_of(length)
    sel, masses = [], []
    for g in range(num_kv_heads):
        if n == 0:
            sel.append(np.zeros(0, dtype=np.int64))
            masses.append(np.zeros(0))
            continue
        keys = gather_tokens(k_cache, block_table_row, length, np.arange(n), g, D)
        W = page_masses(q_seq[g * G:(g + 1) * G], keys, length, scale)
        masses.append(W)
        sel.append(select_coverage(W, n, coverage, b_max))
    return sel, masses

