"""Pins for the oracle's attention over kept pages and its dense decode.

The independent routine is torch's scaled_dot_product_attention in float64 on the CPU
(GQA via enable_gqa, default 1/sqrt(D) scale), fed with sequences rebuilt token by
token from the block table here, not through the oracle's own gather.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import psd_oracle as O


def _logical(cache_f64, bt_row, L, dims):
    # token t lives in block bt_row[t // 16], slot t % 16
    return np.stack([cache_f64[bt_row[t // 16], t % 16, :, :dims] for t in range(L)])


def _sdpa(q, k, v, mask=None):
    # q [Hq, D], k [L, Hkv, D], v [L, Hkv, Dv]
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(mask)[None, :, None, :]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, enable_gqa=True)
    return o[0, :, 0].numpy()


@pytest.mark.parametrize("latent", [False, True])
def test_dense_and_sparse_match_sdpa(latent):
    if latent:
        spec = synth.small_spec(batch=2, num_q_heads=8, num_kv_heads=1, head_dim=72,
                                head_dim_v=64, latent=True, seq_lens=(300, 77), max_len=320,
                                needles=2)
    else:
        spec = synth.small_spec(batch=3, seq_lens=(300, 77, 16), head_dim=32, head_dim_v=32,
                                max_len=320)
    w = synth.make_workload(spec)
    inp = synth.oracle_inputs(w)
    k = synth.to_f64(w.k_raw, "bf16")
    v = synth.to_f64(w.v_raw, "bf16")
    dense = O.dense_step(inp["q"], inp["k_cache"], inp["v_cache"], w.block_table, w.seq_lens,
                         w.scale, spec.head_dim_v, spec.num_kv_heads)
    sparse = O.sparse_step(**inp)
    G = spec.group
    for s in range(spec.batch):
        L = int(w.seq_lens[s])
        kl = _logical(k, w.block_table[s], L, spec.head_dim)
        vl = _logical(v, w.block_table[s], L, spec.head_dim_v)
        ref = _sdpa(inp["q"][s], kl, vl)
        np.testing.assert_allclose(dense[s], ref, rtol=0, atol=1e-12)
        sel = sparse[s][1]
        mask = np.zeros((spec.num_q_heads, L), dtype=bool)
        for h in range(spec.num_q_heads):
            for p in sel[h // G]:
                mask[h, 16 * p: min(L, 16 * p + 16)] = True
        np.testing.assert_allclose(sparse[s][0], _sdpa(inp["q"][s], kl, vl, mask),
                                   rtol=0, atol=1e-12)


def test_full_budget_sparse_equals_dense():
    spec = synth.small_spec(batch=2, seq_lens=(200, 33), budget_percent=100, head_dim=16,
                            head_dim_v=16, max_len=208)
    w = synth.make_workload(spec)
    inp = synth.oracle_inputs(w)
    sp = O.sparse_step(**inp)
    de = O.dense_step(inp["q"], inp["k_cache"], inp["v_cache"], w.block_table, w.seq_lens,
                      w.scale, 16, spec.num_kv_heads)
    for s in range(2):
        np.testing.assert_allclose(sp[s][0], de[s], rtol=0, atol=1e-14)


def test_closed_forms():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((5, 3))
    # one token: the output is that token's value
    np.testing.assert_allclose(O.attend(rng.standard_normal((2, 4)), rng.standard_normal((1, 4)),
                                        v[:1], 0.5), np.repeat(v[:1], 2, 0), atol=1e-15)
    # identical keys: the mean of the values
    keys = np.repeat(rng.standard_normal((1, 4)), 5, 0)
    np.testing.assert_allclose(O.attend(rng.standard_normal((2, 4)), keys, v, 0.5),
                               np.repeat(v.mean(0, keepdims=True), 2, 0), atol=1e-14)
    # zero query: the uniform mean
    np.testing.assert_allclose(O.attend(np.zeros((1, 4)), rng.standard_normal((5, 4)), v, 0.5),
                               v.mean(0, keepdims=True), atol=1e-14)
