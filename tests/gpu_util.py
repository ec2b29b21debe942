"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle, compare.

Every buffer the library writes (statistics, selection rows and counts, outputs and the
workspaces) sits between two guard bands of GUARD_BYTES filled with a sentinel byte;
after the calls the bands are checked on the host, so a write past either end of a
buffer fails the test rather than landing silently in a neighbour.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import synth
from oracle import psd_oracle as O
from page_selected_sparse_amd import DecodeStep

ATOL = 2e-3  # max abs error on outputs for bf16 inputs, fp32 accumulation
GUARD_BYTES = 4096
SENTINEL = 0x5A
GUARDED = ("meta", "sel_pages", "sel_count", "out", "out_dense", "ws_select", "ws_decode",
           "ws_dense", "ws_fused")


def workers() -> int:
    """Oracle threads: the CPU share of one GPU (16) or fewer."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def guard_buffers(step: DecodeStep) -> dict:
    """Moves every output and workspace buffer of ``step`` into the middle of a larger
    sentinel-filled allocation (contents copied). Returns name -> (allocation, bytes)."""
    bands = {}
    for name in GUARDED:
        t = getattr(step, name)
        n = t.numel() * t.element_size()
        buf = torch.full((GUARD_BYTES + n + GUARD_BYTES,), SENTINEL, dtype=torch.uint8,
                         device=t.device)
        view = buf[GUARD_BYTES:GUARD_BYTES + n].view(t.dtype).view(t.shape)
        view.copy_(t)
        setattr(step, name, view)
        bands[name] = (buf, n)
    return bands


def check_guards(bands: dict, what: str = ""):
    torch.cuda.synchronize()
    for name, (buf, n) in bands.items():
        head = buf[:GUARD_BYTES].cpu().numpy()
        tail = buf[GUARD_BYTES + n:].cpu().numpy()
        bad_h = np.flatnonzero(head != SENTINEL)
        bad_t = np.flatnonzero(tail != SENTINEL)
        assert bad_h.size == 0 and bad_t.size == 0, (
            f"{what}: write outside {name}: {bad_h.size} bytes before it (nearest at "
            f"-{GUARD_BYTES - int(bad_h.max()) if bad_h.size else 0}), {bad_t.size} bytes "
            f"past its end (first at +{int(bad_t.min()) if bad_t.size else 0})")


def meta_f64(step: DecodeStep, dtype: str) -> np.ndarray:
    """The statistics as float64 [NB, H_kv, 2, D] (min at 0, max at 1)."""
    meta = step.meta.cpu()  # [NB, H_kv, D / CD, 2, CD]
    if dtype == "bf16":
        meta = synth.to_f64(meta.view(torch.int16).numpy().view(np.uint16), "bf16")
    else:
        meta = meta.numpy().astype(np.float64)
    nb, hkv, nc, _, cd = meta.shape
    return meta.transpose(0, 1, 3, 2, 4).reshape(nb, hkv, 2, nc * cd)


def make_step(w: synth.Workload, b_max=None, cache=None, v_host=False, guard=True,
              kv_host=False):
    step = DecodeStep.from_arrays(w.q, w.cache if cache is None else cache, w.block_table,
                                  w.seq_lens, w.budgets, w.spec.dtype, w.spec.head_dim_v,
                                  w.spec.latent, b_max=b_max, v_host=v_host, kv_host=kv_host)
    bands = guard_buffers(step) if guard else {}
    return step, bands


def run_gpu(w: synth.Workload, b_max=None, dense=True, cache=None, v_host=False):
    """Build the statistics, run one sparse step (and the dense decode) on the GPU, with
    every written buffer guarded. With v_host the V cache sits in pinned host memory."""
    print(f"[gpu] {w.spec.name}: B={w.spec.batch} Hq={w.spec.num_q_heads} "
          f"Hkv={w.spec.num_kv_heads} D={w.spec.head_dim} lens={list(w.seq_lens[:4])}... "
          f"v_host={v_host}", flush=True)
    step, bands = make_step(w, b_max=b_max, cache=cache, v_host=v_host)
    step.build_meta()
    step.step()
    if dense:
        step.dense()
    check_guards(bands, w.spec.name)
    res = dict(meta=meta_f64(step, w.spec.dtype), sel=step.sel_pages.cpu().numpy(),
               cnt=step.sel_count.cpu().numpy(),
               out=step.out.cpu().numpy().astype(np.float64), b_max=step.b_max)
    if dense:
        res["dense"] = step.out_dense.cpu().numpy().astype(np.float64)
    del step, bands
    torch.cuda.empty_cache()
    return res


def check_selection_row(row, count, expected, b_max):
    exp = list(map(int, expected))
    assert count == len(exp), (count, len(exp))
    assert list(map(int, row[:count])) == exp
    assert np.all(row[count:b_max] == -1)


def oracle_sparse(w: synth.Workload, seqs) -> dict:
    """The oracle's sparse step for the given sequences, one sequence per thread (BLAS
    single-threaded inside each)."""
    inp = synth.oracle_inputs(w)
    seqs = list(seqs)

    def one(s):
        return O.sparse_step(**inp, sequences=[s])[s]

    with threadpool_limits(limits=1):
        if len(seqs) == 1:
            return {seqs[0]: one(seqs[0])}
        with ThreadPoolExecutor(min(workers(), len(seqs))) as ex:
            return dict(zip(seqs, ex.map(one, seqs)))


def check_workload(w: synth.Workload, res: dict, seqs=None, dense_seqs=None, atol=ATOL):
    """Meta bit-exact, selection bit-exact, outputs within atol, against the oracle, for
    every sequence unless ``seqs`` / ``dense_seqs`` name fewer."""
    inp = synth.oracle_inputs(w)
    seqs = list(range(w.spec.batch)) if seqs is None else list(seqs)
    ref = oracle_sparse(w, seqs)
    Hkv = w.spec.num_kv_heads
    worst = 0.0
    for s in seqs:
        out, sel, scores, kmin, kmax = ref[s]
        n = O.pages_of(int(w.seq_lens[s]))
        blocks = w.block_table[s, :n]
        np.testing.assert_array_equal(res["meta"][blocks, :, 0, :], kmin, err_msg=f"kmin s={s}")
        np.testing.assert_array_equal(res["meta"][blocks, :, 1, :], kmax, err_msg=f"kmax s={s}")
        for g in range(Hkv):
            try:
                check_selection_row(res["sel"][s, g], int(res["cnt"][s, g]), sel[g], res["b_max"])
            except AssertionError:
                got = res["sel"][s, g, : max(0, int(res["cnt"][s, g]))]
                diff = sorted(set(got.tolist()) ^ set(sel[g].tolist()))
                raise AssertionError(
                    f"selection mismatch s={s} g={g}: differing pages {diff[:10]} with oracle "
                    f"scores {[float(scores[g][p]) for p in diff[:10] if p < n]}")
        err = float(np.max(np.abs(res["out"][s] - out)))
        worst = max(worst, err)
        assert err <= atol, f"sparse output s={s}: max abs err {err}"
    dense_seqs = seqs if dense_seqs is None else list(dense_seqs)
    for s in dense_seqs:
        den = O.dense_step(inp["q"], inp["k_cache"], inp["v_cache"], w.block_table, w.seq_lens,
                           w.scale, w.spec.head_dim_v, Hkv, sequences=[s])[s]
        err = float(np.max(np.abs(res["dense"][s] - den)))
        worst = max(worst, err)
        assert err <= atol, f"dense output s={s}: max abs err {err}"
    print(f"[ok] {w.spec.name}: {len(seqs)} sequences sparse, {len(dense_seqs)} dense, "
          f"worst abs err {worst:.2e}", flush=True)
    return worst
