"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle, compare."""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import psd_oracle as O
from page_selected_sparse_amd import DecodeStep

ATOL = 2e-3  # max abs error on outputs for bf16 inputs, fp32 accumulation


def run_gpu(w: synth.Workload, b_max=None, dense=True, cache=None, v_host=False):
    """Build the statistics, run one sparse step (and the dense decode) on the GPU. With
    v_host the V cache sits in pinned host memory."""
    print(f"[gpu] {w.spec.name}: B={w.spec.batch} Hq={w.spec.num_q_heads} "
          f"Hkv={w.spec.num_kv_heads} D={w.spec.head_dim} lens={list(w.seq_lens[:4])}... "
          f"v_host={v_host}", flush=True)
    step = DecodeStep.from_arrays(w.q, w.cache if cache is None else cache, w.block_table,
                                  w.seq_lens, w.budgets, w.spec.dtype, w.spec.head_dim_v,
                                  w.spec.latent, b_max=b_max, v_host=v_host)
    step.build_meta()
    step.step()
    if dense:
        step.dense()
    torch.cuda.synchronize()
    meta = step.meta.cpu()  # [NB, H_kv, D / CD, 2, CD]
    if w.spec.dtype == "bf16":
        meta = synth.to_f64(meta.view(torch.int16).numpy().view(np.uint16), "bf16")
    else:
        meta = meta.numpy().astype(np.float64)
    nb, hkv, nc, _, cd = meta.shape
    meta = meta.transpose(0, 1, 3, 2, 4).reshape(nb, hkv, 2, nc * cd)  # [NB, H_kv, 2, D]
    res = dict(meta=meta, sel=step.sel_pages.cpu().numpy(), cnt=step.sel_count.cpu().numpy(),
               out=step.out.cpu().numpy().astype(np.float64), b_max=step.b_max)
    if dense:
        res["dense"] = step.out_dense.cpu().numpy().astype(np.float64)
    del step
    torch.cuda.empty_cache()
    return res


def check_selection_row(row, count, expected, b_max):
    exp = list(map(int, expected))
    assert count == len(exp), (count, len(exp))
    assert list(map(int, row[:count])) == exp
    assert np.all(row[count:b_max] == -1)


def check_workload(w: synth.Workload, res: dict, seqs=None, dense_seqs=None, atol=ATOL):
    """Meta bit-exact, selection bit-exact, outputs within atol, against the oracle."""
    inp = synth.oracle_inputs(w)
    seqs = list(range(w.spec.batch)) if seqs is None else list(seqs)
    ref = O.sparse_step(**inp, sequences=seqs)
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
    for s in (dense_seqs if dense_seqs is not None else seqs):
        den = O.dense_step(inp["q"], inp["k_cache"], inp["v_cache"], w.block_table, w.seq_lens,
                           w.scale, w.spec.head_dim_v, Hkv, sequences=[s])[s]
        err = float(np.max(np.abs(res["dense"][s] - den)))
        worst = max(worst, err)
        assert err <= atol, f"dense output s={s}: max abs err {err}"
    print(f"[ok] {w.spec.name}: {len(seqs)} sequences, worst abs err {worst:.2e}", flush=True)
    return worst
