"""GPU parity of adaptive coverage selection (psd_select_pages_coverage) against the oracle.

The GPU forms each page's per-head max m_h(p) and exp-sum s_h(p) in fp32 (they are left
in the workspace) and the group masses W(p) from them; the oracle forms W(p) in fp64. So
the check has three parts:

1. Masses. W_gpu(p), rebuilt on the host from the workspace, lies within a proven bound
   of the oracle's W(p): |W_gpu / W - 1| <= rel, with
     rel = 2 * (exp(2 delta) - 1 + 24 u),  u = 2^-24,
     delta = scale * 1.1 * D * u * max_t sum_d |q_hd k_td|  (over the unit's tokens, heads),
   i.e. a q.k accumulated in fp32 over D exact products (at most D + D/32 roundings, each
   relative to a partial sum bounded by sum |q k|), the exp and the 16-term page sum in
   fp32, and the normalisation by a sum carrying the same relative error.
2. The cut. The GPU row equals the oracle's own selection rule (select_coverage) applied
   to the GPU's masses rounded to fp32, which is the precision the GPU ranks in, with the
   coverage the GPU receives (fp32). This checks the ranking and the cut exactly.
3. Against the oracle's masses. Every GPU row is a valid nucleus under the oracle's W to
   within the bound of part 1 (no page left out that outweighs a kept one by more than the
   bound; kept mass reaches the coverage unless the row is full; no page more than needed).
   Rows equal to the oracle's own row are counted; a row may differ only where the bound
   leaves the oracle's cut undecided, and at most MAX_DIFFERENT of the rows may.

The sparse attention over the GPU's kept pages is checked against the oracle's attention
over the same pages (2e-3).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import check_guards, make_step
from oracle import psd_oracle as O

pytestmark = pytest.mark.gpu

ATOL = 2e-3  # attention outputs
U = 2.0 ** -24
MAX_DIFFERENT = 0.02  # share of rows allowed to differ from the oracle's (undecided cuts)


def run_coverage(w, coverage, b_max):
    print(f"[gpu] coverage {coverage} b_max {b_max}: {w.spec.name} B={w.spec.batch} "
          f"Hq={w.spec.num_q_heads} Hkv={w.spec.num_kv_heads} D={w.spec.head_dim} "
          f"{w.spec.dtype} lens={list(w.seq_lens[:6])}", flush=True)
    step, bands = make_step(w, b_max=b_max)
    step.select_coverage(coverage)
    ws = step.ws_coverage.cpu().numpy().view(np.float32).copy()
    step.sparse()
    check_guards(bands, f"coverage {w.spec.name}")
    B, Hq, P = w.spec.batch, w.spec.num_q_heads, w.block_table.shape[1]
    res = dict(sel=step.sel_pages.cpu().numpy(), cnt=step.sel_count.cpu().numpy(),
               out=step.out.cpu().numpy().astype(np.float64),
               pm=ws[:B * Hq * P].reshape(B, Hq, P), ps=ws[B * Hq * P:2 * B * Hq * P].reshape(B, Hq, P))
    del step, bands
    torch.cuda.empty_cache()
    return res


def gpu_masses(pm, ps, n):
    """Group masses from the GPU's per-head page max and exp-sum, [G, P] each (fp64)."""
    pm = pm[:, :n].astype(np.float64)
    ps = ps[:, :n].astype(np.float64)
    M = pm.max(axis=1, keepdims=True)
    t = ps * np.exp(pm - M)
    return (t / t.sum(axis=1, keepdims=True)).mean(axis=0)


def mass_bound(q_group, keys, scale):
    """Relative bound on |W_gpu / W - 1| for one unit (see the module docstring)."""
    D = q_group.shape[1]
    absdot = np.abs(keys) @ np.abs(q_group).T  # [L, G]: sum_d |q_hd k_td|
    delta = scale * 1.1 * D * U * float(absdot.max())
    return 2.0 * (np.expm1(2.0 * delta) + 24 * U)


def check_nucleus(row, count, W, n, coverage, b_max, rel):
    """The GPU row is a valid nucleus under the oracle's masses W, to the bound rel."""
    kept = [int(p) for p in row[:count]]
    assert np.all(row[count:b_max] == -1)
    assert kept == sorted(set(kept)), kept
    if n <= 2:
        assert kept == list(range(n))
        return
    assert kept[0] == 0 and kept[-1] == n - 1 and kept[-1] < n
    inner = [p for p in kept if 0 < p < n - 1]
    room = min(n - 2, b_max - 2)
    assert len(inner) <= room
    out = np.setdiff1d(np.arange(1, n - 1), inner)
    if inner and len(out):
        lightest, heaviest_out = W[inner].min(), W[out].max()
        assert heaviest_out <= lightest + rel * (lightest + heaviest_out), "a lighter page was kept"
    mass = W[kept].sum()
    slack = rel * min(mass, 1.0 - mass) + 1e-12  # both sides' masses sum to 1
    if coverage >= 1.0:
        assert len(inner) == room
        return
    if len(inner) < room:
        assert mass >= coverage - slack, f"kept mass {mass} below {coverage}"
    if inner:
        last = W[inner].min()
        assert mass - last < coverage + slack + rel * last, "the cut keeps one page too many"


def cut_is_clear(W, n, coverage, b_max, rel):
    """True when masses within the bound rel of W cannot move the oracle's cut."""
    if n <= 2 or coverage >= 1.0:
        return True
    inner = np.arange(1, n - 1)
    order = inner[np.lexsort((inner, -W[inner]))]
    sorted_w = W[order]
    room = min(n - 2, b_max - 2)
    cum = W[0] + W[n - 1] + np.concatenate([[0.0], np.cumsum(sorted_w)])
    take = len(O.select_coverage(W, n, coverage, b_max)) - 2
    slack = lambda c: rel * min(c, 1.0 - c) + 1e-12
    if take < room and abs(cum[take] - coverage) <= slack(cum[take]):
        return False
    if take > 0 and abs(cum[take - 1] - coverage) <= slack(cum[take - 1]):
        return False
    if 0 < take < len(sorted_w) and sorted_w[take - 1] - sorted_w[take] <= rel * (
            sorted_w[take - 1] + sorted_w[take]):
        return False
    return True


def check(w, res, coverage, b_max):
    cov32 = float(np.float32(coverage))  # what the C-ABI hands the kernels
    inp = synth.oracle_inputs(w)
    Hkv, G, D = w.spec.num_kv_heads, w.spec.group, w.spec.head_dim
    equal = units = 0
    worst_out = worst_ratio = 0.0
    for s in range(w.spec.batch):
        L = int(w.seq_lens[s])
        n = O.pages_of(L)
        sel, masses = O.coverage_select_sequence(inp["q"][s], inp["k_cache"], w.block_table[s],
                                                 L, Hkv, w.scale, cov32, b_max)
        got = []
        for g in range(Hkv):
            cnt = int(res["cnt"][s, g])
            row = res["sel"][s, g]
            kept = [int(p) for p in row[:max(cnt, 0)]]
            units += 1
            if n <= 2:
                assert kept == list(range(n)), (s, g, kept)
                got.append(np.array(kept, dtype=np.int64))
                equal += 1
                continue
            qg = inp["q"][s, g * G:(g + 1) * G]
            keys = O.gather_tokens(inp["k_cache"], w.block_table[s], L, np.arange(n), g, D)
            rel = mass_bound(qg, keys, w.scale)
            W = masses[g]
            Wg = gpu_masses(res["pm"][s, g * G:(g + 1) * G], res["ps"][s, g * G:(g + 1) * G], n)
            ratio = float(np.max(np.abs(Wg - W) / (rel * W + 1e-300)))
            worst_ratio = max(worst_ratio, ratio)
            assert ratio <= 1.0, f"s={s} g={g}: GPU page masses outside the bound ({ratio:.3f})"
            # the cut, exactly, from the GPU's masses in the precision it ranks in: inner
            # pages as fp32 values, sink and tail in fp64
            Wr = Wg.copy()
            Wr[1:n - 1] = Wg[1:n - 1].astype(np.float32)
            own = [int(p) for p in O.select_coverage(Wr, n, cov32, b_max)]
            if kept != own:
                # a summation-order difference may move the cut by one page, and only when
                # the kept mass there equals the coverage to within the order's rounding
                extra = sorted(set(kept) ^ set(own))
                shorter = own if len(own) < len(kept) else kept
                assert len(extra) == 1 and abs(Wr[shorter].sum() + Wr[extra].sum() - cov32) < 1e-12 \
                    or abs(Wr[shorter].sum() - cov32) < 1e-12, f"s={s} g={g}: cut {kept[:12]} vs {own[:12]}"
            check_nucleus(row, cnt, W, n, cov32, b_max, rel)
            if kept == [int(p) for p in sel[g]]:
                equal += 1
            else:
                assert not cut_is_clear(W, n, cov32, b_max, rel), \
                    f"s={s} g={g}: GPU {kept[:12]} oracle {list(sel[g][:12])}"
            got.append(np.array(kept, dtype=np.int64))
        ref = O.decode_sequence(inp["q"][s], inp["k_cache"], inp["v_cache"], w.block_table[s], L,
                                got, w.scale, w.spec.head_dim_v)
        err = float(np.max(np.abs(res["out"][s] - ref)))
        worst_out = max(worst_out, err)
        assert err <= ATOL, f"attention over the kept pages s={s}: max abs err {err}"
    print(f"[ok] {equal}/{units} rows equal to the oracle's; GPU masses at most "
          f"{worst_ratio:.3g} of the bound; worst abs err {worst_out:.2e}", flush=True)
    assert units - equal <= MAX_DIFFERENT * units, f"{units - equal} of {units} rows differ"
    return equal, units


SMALL = dict(batch=6, seq_lens=(1000, 37, 4096, 17, 1, 33), max_len=4096)


@pytest.mark.parametrize("coverage", [0.5, 0.9, 0.95, 1.0])
def test_coverage_bf16_d128(coverage):
    w = synth.make_workload(synth.small_spec("cov_bf16", num_q_heads=8, num_kv_heads=2, **SMALL))
    b_max = 258  # every page of the longest sequence fits
    check(w, run_coverage(w, coverage, b_max), coverage, b_max)


@pytest.mark.parametrize("coverage", [0.8, 1.0])
def test_coverage_f32_d64_group8(coverage):
    spec = synth.small_spec("cov_f32", num_q_heads=16, num_kv_heads=2, head_dim=64,
                            head_dim_v=64, dtype="f32", **SMALL)
    w = synth.make_workload(spec)
    check(w, run_coverage(w, coverage, 258), coverage, 258)


def test_coverage_capped_rows():
    # b_max far below what 0.99 needs: every long row is full, the short ones are not
    w = synth.make_workload(synth.small_spec("cov_cap", num_q_heads=8, num_kv_heads=2, **SMALL))
    res = run_coverage(w, 0.99, 8)
    check(w, res, 0.99, 8)
    assert int(res["cnt"][2].min()) == 8


@pytest.mark.timeout(600)
def test_coverage_full_size():
    # the 32-sequence ragged 16K-32K workload, every sequence checked
    w = synth.make_workload("ragged_b32_32k")
    b_max = int(w.block_table.shape[1])
    res = run_coverage(w, 0.95, b_max)
    check(w, res, 0.95, b_max)


@pytest.mark.parametrize("dtype,d,hq", [("bf16", 64, 4), ("f32", 128, 8), ("bf16", 128, 16)])
def test_coverage_row_widths(dtype, d, hq):
    # rows of 8 lanes (bf16 D=64), 32 lanes (fp32 D=128), and 8-head groups at bf16 D=128
    spec = synth.small_spec(f"cov_{dtype}_{d}", num_q_heads=hq, num_kv_heads=2, head_dim=d,
                            head_dim_v=d, dtype=dtype, **SMALL)
    w = synth.make_workload(spec)
    check(w, run_coverage(w, 0.9, 258), 0.9, 258)
