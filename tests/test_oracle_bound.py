"""Pins for the oracle's page bound and group score.

* The closed form equals the brute-force maximum of q.k over all 2^D corners of the
  min/max box (exact rational arithmetic, D <= 10).
* It is an upper bound on every real key of the page (exact rationals on tiny inputs,
  fp64 with a relative slack on a measured workload).
* Hand-worked examples, including one where the ascending-d fp64 order decides.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import psd_oracle as O


def _dyadic(rng, shape):
    # Small dyadic rationals: every product and partial sum is exact in fp64.
    return rng.integers(-64, 65, size=shape).astype(np.float64) / 16.0


@pytest.mark.parametrize("D", [1, 2, 5, 10])
def test_bound_is_max_over_box_corners(D):
    rng = np.random.default_rng(D)
    for _ in range(5):
        q = _dyadic(rng, (3, D))
        a, b = _dyadic(rng, (4, D)), _dyadic(rng, (4, D))
        kmin, kmax = np.minimum(a, b), np.maximum(a, b)
        ub = O.page_bounds(q, kmin, kmax)
        for h in range(3):
            for p in range(4):
                best = max(sum(Fraction(q[h, d]) * Fraction(c[d]) for d in range(D))
                           for c in itertools.product(*[(kmin[p, d], kmax[p, d])
                                                        for d in range(D)]))
                assert Fraction(ub[h, p]) == best


def test_bound_dominates_every_key_exactly():
    rng = np.random.default_rng(7)
    for _ in range(20):
        D, T = 6, int(rng.integers(1, 17))
        keys = _dyadic(rng, (T, D))
        q = _dyadic(rng, (2, D))
        kmin, kmax = O.page_minmax(keys)
        ub = O.page_bounds(q, kmin[None], kmax[None])
        for h in range(2):
            true_max = max(sum(Fraction(q[h, d]) * Fraction(keys[t, d]) for d in range(D))
                           for t in range(T))
            assert Fraction(ub[h, 0]) >= true_max
            if T == 1:
                assert Fraction(ub[h, 0]) == true_max  # a one-key box is that key


def test_group_score_is_max_and_positive_zero():
    ub = np.array([[1.0, -0.0, -3.0], [2.0, -0.0, -4.0]])
    g = O.group_scores(ub)
    np.testing.assert_array_equal(g, [2.0, 0.0, -3.0])
    assert not np.signbit(g[1])


def test_hand_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "bound_hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"])
        ub = O.page_bounds(q, np.array(c["kmin"]), np.array(c["kmax"]))
        np.testing.assert_array_equal(ub, np.array(c["ub"]), err_msg=c["name"])
        np.testing.assert_array_equal(O.group_scores(ub), np.array(c["group"]),
                                      err_msg=c["name"])


def test_bound_dominates_true_max_on_measured_workload():
    w = synth.make_workload("gqa8b_32k")
    inp = synth.oracle_inputs(w)
    q = inp["q"][0]
    L = int(w.seq_lens[0])
    kmin, kmax = O.sequence_meta(inp["k_cache"], w.block_table[0], L)
    n = O.pages_of(L)
    G = 4
    pages = np.arange(0, n, 37)
    keys = inp["k_cache"][w.block_table[0, pages]]  # [m, 16, 8, 128]
    for g in range(8):
        ub = O.page_bounds(q[g * G:(g + 1) * G], kmin[pages, g], kmax[pages, g])
        true = np.einsum("hd,mtd->hmt", q[g * G:(g + 1) * G], keys[:, :, g]).max(axis=2)
        slack = 1e-12 * (np.abs(q[g * G:(g + 1) * G]).sum(1)[:, None]
                         * np.abs(keys[:, :, g]).max(axis=(1, 2))[None, :])
        assert np.all(ub >= true - slack)
