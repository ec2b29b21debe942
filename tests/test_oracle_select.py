"""Pins for the oracle's page selection.

A kept set is checked against what defines it rather than against a retyped sort:
sink and tail present, size min(n, max(b, 2)), ascending without repeats, and every
kept inner page ranks above every dropped inner page under (score desc, index asc).
"""
import json
import os

import numpy as np
import pytest

from oracle import psd_oracle as O


def _check_selection(sel, scores, n, budget):
    sel = list(map(int, sel))
    b = n if n <= 2 else min(n, max(budget, 2))
    assert len(sel) == b
    assert sel == sorted(set(sel))
    assert sel[0] == 0 and sel[-1] == n - 1
    kept = set(sel[1:-1])
    dropped = [p for p in range(1, n - 1) if p not in kept]
    for x in kept:
        for y in dropped:
            assert scores[x] > scores[y] or (scores[x] == scores[y] and x < y)


@pytest.mark.parametrize("seed", range(25))
def test_selection_characterisation_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    scores = rng.integers(-3, 4, size=n).astype(np.float64)  # many ties
    budget = int(rng.integers(0, 45))
    sel = O.select_pages(scores, n, budget)
    _check_selection(sel, scores, n, budget)


def test_hand_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "select_hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        sc = np.array(c["scores"], dtype=np.float64)
        got = O.select_pages(sc, len(sc), c["budget"])
        assert list(got) == c["expected"], c["derivation"]


def test_signed_zero_scores_tie():
    scores = np.array([0.0, -0.0, 0.0, -0.0, 0.0, 1.0])
    got = O.select_pages(O.group_scores(scores[None]), 6, 4)
    assert list(got) == [0, 1, 2, 5]


def test_full_budget_keeps_all():
    sc = np.random.default_rng(0).standard_normal(50)
    assert list(O.select_pages(sc, 50, 50)) == list(range(50))
    assert list(O.select_pages(sc, 50, 1000)) == list(range(50))
