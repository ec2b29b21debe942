"""Pins for the oracle's page statistics (per-page key min/max over valid tokens)."""
import numpy as np

import synth
from oracle import psd_oracle as O


def _brute_meta(k, bt_row, length, page, head, dim):
    vals = []
    for t in range(16):
        pos = 16 * page + t
        if pos < length:
            vals.append(float(k[bt_row[page], t, head, dim]))
    return min(vals), max(vals)


def test_meta_matches_brute_force_ragged():
    spec = synth.small_spec(seq_lens=(37, 16, 1, 50), batch=4, head_dim=8, head_dim_v=8,
                            num_q_heads=4, num_kv_heads=2, max_len=64, needles=0)
    w = synth.make_workload(spec)
    k = synth.to_f64(w.k_raw, "bf16")
    for s in range(spec.batch):
        L = int(w.seq_lens[s])
        kmin, kmax = O.sequence_meta(k, w.block_table[s], L)
        assert kmin.shape == (O.pages_of(L), 2, 8)
        assert np.all(np.isfinite(kmin)) and np.all(np.isfinite(kmax))
        for p in range(O.pages_of(L)):
            for h in range(2):
                for d in range(8):
                    lo, hi = _brute_meta(k, w.block_table[s], L, p, h, d)
                    assert kmin[p, h, d] == lo and kmax[p, h, d] == hi


def test_meta_tail_slots_are_ignored():
    # The generator writes NaN past the length; a page range one slot too long shows up.
    spec = synth.small_spec(seq_lens=(33,), batch=1, head_dim=4, head_dim_v=4,
                            num_q_heads=2, num_kv_heads=1, max_len=48, needles=0)
    w = synth.make_workload(spec)
    k = synth.to_f64(w.k_raw, "bf16")
    assert np.isnan(k[w.block_table[0, 2], 1:]).all()
    kmin, kmax = O.sequence_meta(k, w.block_table[0], 33)
    assert kmin.shape[0] == 3
    np.testing.assert_array_equal(kmin[2], k[w.block_table[0, 2], 0])
    np.testing.assert_array_equal(kmax[2], k[w.block_table[0, 2], 0])


def test_page_geometry():
    assert [O.pages_of(x) for x in (1, 15, 16, 17, 32, 33)] == [1, 1, 1, 2, 2, 3]
    assert [O.valid_in_page(33, p) for p in range(4)] == [16, 16, 1, 0]
