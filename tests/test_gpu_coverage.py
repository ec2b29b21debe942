"""GPU parity of adaptive coverage selection (psd_select_pages_coverage) against the oracle.

The kept set must be the oracle's wherever the cut is decided by more than the masses'
rounding: the GPU forms page masses in fp32 and the oracle in fp64, so where two pages'
masses or the kept mass and the coverage lie within TOL of each other either side may
differ. Every row is also checked to be a valid nucleus under the oracle's masses, and
the sparse attention over the GPU's set is checked against the oracle's attention over
that same set.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import psd_oracle as O
from page_selected_sparse_amd import DecodeStep

pytestmark = pytest.mark.gpu

TOL = 1e-5   # mass: fp32 exp and q.k rounding on masses that sum to 1
ATOL = 2e-3  # attention outputs


def run_coverage(w, coverage, b_max):
    print(f"[gpu] coverage {coverage} b_max {b_max}: {w.spec.name} B={w.spec.batch} "
          f"Hq={w.spec.num_q_heads} Hkv={w.spec.num_kv_heads} D={w.spec.head_dim} "
          f"{w.spec.dtype} lens={list(w.seq_lens[:6])}", flush=True)
    step = DecodeStep.from_arrays(w.q, w.cache, w.block_table, w.seq_lens, w.budgets,
                                  w.spec.dtype, w.spec.head_dim_v, w.spec.latent, b_max=b_max)
    step.select_coverage(coverage)
    step.sparse()
    torch.cuda.synchronize()
    res = dict(sel=step.sel_pages.cpu().numpy(), cnt=step.sel_count.cpu().numpy(),
               out=step.out.cpu().numpy().astype(np.float64))
    del step
    torch.cuda.empty_cache()
    return res


def check_nucleus(row, count, W, n, coverage, b_max):
    """The GPU row is a valid nucleus under the oracle's masses W (to TOL)."""
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
        assert W[out].max() <= W[inner].min() + TOL, "a lighter page was kept"
    mass = W[kept].sum()
    if coverage >= 1.0:
        assert len(inner) == room
        return
    if len(inner) < room:
        assert mass >= coverage - TOL, f"kept mass {mass} below {coverage}"
    if inner:
        assert mass - W[inner].min() < coverage + TOL, "the cut keeps one page too many"


def cut_is_clear(W, n, coverage, b_max):
    """True when rounding of the masses cannot move the oracle's cut."""
    if n <= 2 or coverage >= 1.0:
        return True
    inner = np.arange(1, n - 1)
    order = inner[np.lexsort((inner, -W[inner]))]
    sorted_w = W[order]
    room = min(n - 2, b_max - 2)
    cum = W[0] + W[n - 1] + np.concatenate([[0.0], np.cumsum(sorted_w)])
    take = len(O.select_coverage(W, n, coverage, b_max)) - 2
    if take < room and abs(cum[take] - coverage) < TOL:
        return False
    if take > 0 and abs(cum[take - 1] - coverage) < TOL:
        return False
    # a page at the cut whose mass ties the next one within TOL could swap places
    if 0 < take < len(sorted_w) and sorted_w[take - 1] - sorted_w[take] < TOL:
        return False
    return True


def check(w, res, coverage, b_max, seqs=None):
    inp = synth.oracle_inputs(w)
    seqs = range(w.spec.batch) if seqs is None else seqs
    Hkv = w.spec.num_kv_heads
    exact = units = 0
    worst = 0.0
    for s in seqs:
        L = int(w.seq_lens[s])
        n = O.pages_of(L)
        sel, masses = O.coverage_select_sequence(inp["q"][s], inp["k_cache"], w.block_table[s],
                                                 L, Hkv, w.scale, coverage, b_max)
        got = []
        for g in range(Hkv):
            cnt = int(res["cnt"][s, g])
            row = res["sel"][s, g]
            check_nucleus(row, cnt, masses[g], n, coverage, b_max)
            kept = [int(p) for p in row[:cnt]]
            units += 1
            if kept == [int(p) for p in sel[g]]:
                exact += 1
            else:
                assert not cut_is_clear(masses[g], n, coverage, b_max), \
                    f"s={s} g={g}: GPU {kept[:12]} oracle {list(sel[g][:12])}"
            got.append(np.array(kept, dtype=np.int64))
        ref = O.decode_sequence(inp["q"][s], inp["k_cache"], inp["v_cache"], w.block_table[s], L,
                                got, w.scale, w.spec.head_dim_v)
        err = float(np.max(np.abs(res["out"][s] - ref)))
        worst = max(worst, err)
        assert err <= ATOL, f"attention over the kept pages s={s}: max abs err {err}"
    print(f"[ok] {exact}/{units} rows equal to the oracle's, worst abs err {worst:.2e}",
          flush=True)
    assert exact >= 0.9 * units
    return exact, units


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


def test_coverage_full_size_sampled():
    # the 32-sequence ragged 16K-32K workload, sampled sequences checked one by one
    w = synth.make_workload("ragged_b32_32k")
    b_max = int(w.block_table.shape[1])
    res = run_coverage(w, 0.95, b_max)
    check(w, res, 0.95, b_max, seqs=[0, 13, 31])
    n = [O.pages_of(int(x)) for x in w.seq_lens]
    cnt = res["cnt"]
    for s in range(w.spec.batch):
        assert np.all((cnt[s] >= 2) & (cnt[s] <= n[s])), s


@pytest.mark.parametrize("dtype,d,hq", [("bf16", 64, 4), ("f32", 128, 8), ("bf16", 128, 16)])
def test_coverage_row_widths(dtype, d, hq):
    # rows of 8 lanes (bf16 D=64), 32 lanes (fp32 D=128), and 8-head groups at bf16 D=128
    spec = synth.small_spec(f"cov_{dtype}_{d}", num_q_heads=hq, num_kv_heads=2, head_dim=d,
                            head_dim_v=d, dtype=dtype, **SMALL)
    w = synth.make_workload(spec)
    check(w, run_coverage(w, 0.9, 258), 0.9, 258)
