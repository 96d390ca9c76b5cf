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


def test_per_row_budget_hand_case():
    """Per-row budget variant: tau_i = floor(rho (i + 1) / 100).  Rows and the
    expected lists are worked out by hand (b = 6, rho = 50: tau = 0,1,1,2,2,3)."""
    R = np.zeros((6, 6))
    R[0, :1] = [1.0]
    R[1, :2] = [0.5, 1.0]
    R[2, :3] = [0.2, 0.9, 1.0]
    R[3, :4] = [0.7, -0.3, 0.7, 1.0]
    R[4, :5] = [0.1, 0.4, 0.4, 0.4, 1.0]
    R[5, :6] = [0.0, -0.0, 0.3, -1.0, 0.3, 1.0]
    assert [O.n_select_row(50, i) for i in range(6)] == [0, 1, 1, 2, 2, 3]
    got = [x.tolist() for x in O.select_rows_tau(R, 50)]
    assert got == [[0], [0, 1], [1, 2], [0, 2, 3], [1, 2, 4], [0, 2, 4, 5]]
    # the per-sequence budget (tau = 3 for every row) differs on rows 3 and 4
    assert [x.tolist() for x in O.select(R, 50)][3:5] == [[0, 1, 2, 3], [1, 2, 3, 4]]
    assert [x.tolist() for x in O.select_rows_tau(R, 50, dense=True)] == \
        [list(range(i + 1)) for i in range(6)]


def test_per_row_budget_last_row_matches_sequence_budget():
    rng = np.random.default_rng(3)
    for _ in range(50):
        b = int(rng.integers(1, 40))
        rho = int(rng.integers(0, 101))
        assert O.n_select_row(rho, b - 1) == O.n_select(rho, b)
        assert all(O.n_select_row(rho, i) <= i + 1 for i in range(b))


def test_group_scores_hand_case_and_reductions():
    """Group-shared selection scores the row by the fp32 sum of the group's
    walk states.  Hand case: two heads whose own choices differ (block 0 for
    the first, block 1 for the second) agree on block 2 once added."""
    Ra = np.zeros((4, 4), np.float32)
    Rb = np.zeros((4, 4), np.float32)
    Ra[3] = [0.9, 0.1, 0.5, 1.0]
    Rb[3] = [-0.8, 0.6, 0.4, 1.0]
    S = O.group_scores([Ra, Rb])
    assert S.dtype == np.float32
    assert O.select_row(Ra[3], 3, 1).tolist() == [0, 3]
    assert O.select_row(Rb[3], 3, 1).tolist() == [1, 3]
    assert O.select_row(S[3], 3, 1).tolist() == [2, 3]
    # one head: the score is the head's own state; identical heads: exactly 2 R
    rng = np.random.default_rng(4)
    R = np.tril(rng.standard_normal((9, 9))).astype(np.float32)
    assert np.array_equal(O.group_scores([R]), R)
    assert np.array_equal(O.group_scores([R, R]), 2 * R)
    assert [x.tolist() for x in O.select(O.group_scores([R, R]), 30)] == \
        [x.tolist() for x in O.select(R, 30)]
    # fp32 sums in ascending head order
    R3 = [np.tril(rng.standard_normal((9, 9))).astype(np.float32) for _ in range(3)]
    want = (R3[0] + R3[1]).astype(np.float32) + R3[2]
    assert np.array_equal(O.group_scores(R3), want.astype(np.float32))
