"""Pins of the oracle's coverage selection (page masses and the nucleus cut).

The variant is the adaptive ``coverage`` knob of the AMASS and LOCKS READMEs
("Key AmassConfig fields"; LOCKS "Configuration": a per-head nucleus over exact page
masses). Each pin checks the oracle against something other than itself: brute force
over every admissible page subset, masses in closed form, and invariants of a
softmax distribution.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import psd_oracle as O


def brute_force(mass, n, coverage, b_max):
    """Best admissible set: contains the sink and the tail, fits the row, reaches the
    coverage with the fewest pages (the most mass among those); if nothing fitting
    reaches it, the most mass among the largest fitting sets."""
    inner = list(range(1, n - 1))
    room = min(n - 2, b_max - 2)
    best = None
    for k in range(0, room + 1):
        cands = []
        for extra in itertools.combinations(inner, k):
            s = (0, n - 1) + extra
            cands.append((sum(mass[p] for p in s), sorted(s)))
        top = max(cands, key=lambda c: c[0])
        best = top
        if top[0] >= coverage:
            return top
    return best


@pytest.mark.parametrize("seed", range(40))
def test_cut_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(3, 10))
    mass = rng.dirichlet(np.full(n, 0.5))
    coverage = float(rng.choice([0.3, 0.5, 0.8, 0.9, 0.95]))
    b_max = int(rng.integers(2, n + 2))
    got = O.select_coverage(mass, n, coverage, b_max)
    want_mass, want = brute_force(mass, n, coverage, b_max)
    assert len(got) == len(want)
    assert math.isclose(float(mass[got].sum()), want_mass, rel_tol=0, abs_tol=1e-12)
    assert list(got) == sorted(got)
    assert got[0] == 0 and got[-1] == n - 1


def test_ties_go_to_the_lower_page():
    n = 6
    mass = np.array([0.1, 0.2, 0.2, 0.2, 0.2, 0.1])
    # sink + tail = 0.2; one more page reaches 0.4
    assert list(O.select_coverage(mass, n, 0.4, 16)) == [0, 1, 5]
    assert list(O.select_coverage(mass, n, 0.41, 16)) == [0, 1, 2, 5]


def test_full_coverage_keeps_every_page_that_fits():
    mass = np.full(10, 0.1)
    assert list(O.select_coverage(mass, 10, 1.0, 64)) == list(range(10))
    assert list(O.select_coverage(mass, 10, 1.0, 4)) == [0, 1, 2, 9]


def test_sink_and_tail_alone_can_cover():
    mass = np.array([0.6, 0.01, 0.02, 0.37])
    assert list(O.select_coverage(mass, 4, 0.95, 16)) == [0, 3]


@pytest.mark.parametrize("n", [0, 1, 2])
def test_short_sequences_keep_everything(n):
    assert list(O.select_coverage(np.full(n, 1.0 / max(n, 1)), n, 0.5, 2)) == list(range(n))


def test_zero_query_masses_are_token_shares():
    # q = 0 gives every token the same weight: page mass = valid tokens / L.
    L, D = 53, 8
    keys = np.random.default_rng(1).standard_normal((L, D))
    W = O.page_masses(np.zeros((2, D)), keys, L, 0.3)
    want = np.array([O.valid_in_page(L, p) for p in range(O.pages_of(L))]) / L
    np.testing.assert_allclose(W, want, rtol=0, atol=1e-15)


def test_one_spiked_token_closed_form():
    # L = 17: page 0 holds 16 tokens with z = 0, page 1 one token with z = c.
    D, c, scale = 4, 1.7, 0.5
    q = np.array([[1.0, 0.0, 0.0, 0.0]])
    keys = np.zeros((17, D))
    keys[16, 0] = c / scale
    W = O.page_masses(q, keys, 17, scale)
    e = math.exp(c)
    np.testing.assert_allclose(W, [16 / (16 + e), e / (16 + e)], rtol=1e-14)


def test_group_mass_is_the_mean_over_heads():
    # head 0 spikes on token 20 (page 1), head 1 on token 40 (page 2); 48 tokens.
    L, D, c, scale = 48, 4, 3.0, 1.0
    keys = np.zeros((L, D))
    keys[20, 0] = c
    keys[40, 1] = c
    q = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]])
    W = O.page_masses(q, keys, L, scale)
    e = math.exp(c)
    Z = L - 1 + e
    # each head: 16/Z on a plain page, (15 + e)/Z on its spiked page; the mean halves
    want = np.array([16 + 16, (15 + e) + 16, 16 + (15 + e)]) / Z / 2
    np.testing.assert_allclose(W, want, rtol=1e-14)


@pytest.mark.parametrize("seed", range(5))
def test_masses_form_a_distribution(seed):
    rng = np.random.default_rng(seed)
    L, D, G = int(rng.integers(1, 300)), 16, 4
    W = O.page_masses(rng.standard_normal((G, D)), rng.standard_normal((L, D)), L, 0.25)
    assert W.shape == (O.pages_of(L),)
    assert np.all(W >= 0)
    assert math.isclose(float(W.sum()), 1.0, abs_tol=1e-12)


def test_sequence_selection_ignores_block_placement():
    # The same logical keys behind two different block tables select the same pages.
    rng = np.random.default_rng(7)
    L, Hkv, G, D, nb = 150, 2, 2, 8, 12
    n = O.pages_of(L)
    logical = rng.standard_normal((n, 16, Hkv, D))
    q = rng.standard_normal((Hkv * G, D))
    res = []
    for perm in (np.arange(n), rng.permutation(nb)[:n]):
        cache = np.zeros((nb, 16, Hkv, D))
        cache[perm] = logical
        res.append(O.coverage_select_sequence(q, cache, perm, L, Hkv, 0.35, 0.8, 64))
    for g in range(Hkv):
        assert list(res[0][0][g]) == list(res[1][0][g])
        np.testing.assert_array_equal(res[0][1][g], res[1][1][g])
