"""The seeded generator: determinism, layout and the stated recipe."""
import numpy as np

import synth


def test_deterministic_and_seeded():
    a = synth.make_workload(synth.small_spec())
    b = synth.make_workload(synth.small_spec())
    c = synth.make_workload(synth.small_spec(), seed=1)
    for x, y in ((a.q, b.q), (a.cache, b.cache), (a.block_table, b.block_table)):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a.q, c.q)


def test_layout_budget_and_tail_sentinels():
    spec = synth.SPECS["ragged_b32_32k"]
    w = synth.make_workload(synth.small_spec(seq_lens=(1000, 37, 4096), budget_percent=5))
    n = [synth.num_pages(x) for x in w.seq_lens]
    assert w.cache.shape == (2, sum(n), 16, 2, 128)
    used = np.concatenate([w.block_table[s, : n[s]] for s in range(3)])
    np.testing.assert_array_equal(np.sort(used), np.arange(sum(n)))  # a permutation
    assert list(w.budgets) == [max(2, x * 5 // 100) for x in n]
    # slots past the length hold NaN in K and V, nothing else does
    k = synth.to_f64(w.k_raw, "bf16")
    tail = w.block_table[0, n[0] - 1]
    assert np.isnan(k[tail, 1000 % 16:]).all() and np.isfinite(k[tail, : 1000 % 16]).all()
    assert spec.len_range == (16384, 32768)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, np.nan], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back[:4], [1.0, 1.0, 1.0 + 2 ** -6, -2.5])
    assert np.isnan(back[4])


def test_needles_are_inner_distinct_pages():
    w = synth.make_workload(synth.small_spec())
    for s in range(3):
        n = synth.num_pages(w.seq_lens[s])
        for g in range(2):
            pg = w.needle_pages[s, g]
            pg = pg[pg >= 0]
            assert len(set(pg.tolist())) == len(pg)
            assert np.all((pg >= 1) & (pg <= n - 2))
