"""Pins for the oracle's top-tau selection (blog page section 4)."""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_cases():
    with open(os.path.join(GOLD, "select_cases.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        got = O.select_row(np.array(c["row"], float), c["i"], c["tau"])
        assert got.tolist() == c["expect"], c["why"]


def _dominates(row, a, c):
    va, vc = row[a] + 0.0, row[c] + 0.0
    return va > vc or (va == vc and a < c)


@pytest.mark.parametrize("seed", range(20))
def test_selection_is_the_dominant_set(seed):
    """Every kept earlier block beats every dropped one under (value desc,
    index asc); sizes are min(i, tau) + 1; lists ascending and end with i."""
    rng = np.random.default_rng(seed)
    b = int(rng.integers(1, 40))
    R = np.round(rng.normal(size=(b, b)), 1)          # many ties
    R[rng.random((b, b)) < 0.1] = -0.0
    rho = int(rng.integers(0, 101))
    tau = O.n_select(rho, b)
    lists = O.select(R, rho)
    for i, lst in enumerate(lists):
        assert lst[-1] == i and np.all(np.diff(lst) > 0)
        assert len(lst) == min(i, tau) + 1
        kept = set(lst[:-1].tolist())
        dropped = set(range(i)) - kept
        for a in kept:
            for c in dropped:
                assert _dominates(R[i], a, c)


def test_tau_rules():
    assert O.n_select(20, 16) == 3          # the tiny configuration: tau = 3 + diagonal
    assert O.n_select(20, 1024) == 204
    assert O.n_select(20, 512) == 102
    assert O.n_select(100, 7) == 7
    R = np.random.default_rng(0).normal(size=(9, 9))
    for i, lst in enumerate(O.select(R, 100)):
        assert lst.tolist() == list(range(i + 1))
    for i, lst in enumerate(O.select(R, 20, dense=True)):
        assert lst.tolist() == list(range(i + 1))
