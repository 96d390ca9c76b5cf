"""Pins for the oracle's walk state (blog page section 4)."""
import itertools
import math
import json
import os

import numpy as np
import pytest

import gen
import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _lower(rng, b, diag_boost=0.0):
    return np.tril(rng.normal(size=(b, b))) + diag_boost * np.eye(b)


def test_walk_hand_cases():
    with open(os.path.join(GOLD, "walk_small.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        Rp = None if c["R_prev"] is None else np.array(c["R_prev"], float)
        got = O.walk_update(Rp, np.array(c["M"], float), c["s"])
        np.testing.assert_allclose(got, c["R"], atol=1e-15)


@pytest.mark.parametrize("b,s", [(3, 1), (4, 2), (5, 3), (6, 2)])
def test_walk_is_sum_over_causal_paths(b, s):
    """(M^s)[i, m] = sum over block paths i = j0 >= j1 >= ... >= js = m of the
    product of scores, enumerated by brute force."""
    rng = np.random.default_rng(b * 10 + s)
    M = _lower(rng, b)
    P = np.zeros((b, b))
    for path in itertools.product(range(b), repeat=s + 1):
        if all(path[t + 1] <= path[t] for t in range(s)):
            w = 1.0
            for t in range(s):
                w *= M[path[t], path[t + 1]]
            P[path[0], path[-1]] += w
    np.testing.assert_allclose(O.walk_update(None, M, s), O.rownorm(P), rtol=1e-12, atol=1e-12)


def test_eight_hops_equal_repeated_squaring():
    rng = np.random.default_rng(2)
    M = _lower(rng, 12, 1.5)
    M2 = M @ M
    M8 = (M2 @ M2) @ (M2 @ M2)
    np.testing.assert_allclose(O.walk_update(None, M, 8), O.rownorm(M8), rtol=1e-10, atol=1e-12)


def test_one_hop_one_layer_is_rownormed_scores():
    rng = np.random.default_rng(4)
    M = _lower(rng, 9)
    np.testing.assert_allclose(O.walk_update(None, M, 1), O.rownorm(M), atol=1e-15)
    assert np.allclose(np.abs(O.walk_update(None, M, 1)).max(axis=1), 1.0)


def test_layerwise_normalisation_commutes():
    """Normalising rows after every layer gives the same state as one
    normalisation of the raw product R^(-1) M_0^s M_1^s M_2^s."""
    rng = np.random.default_rng(6)
    Ms = [_lower(rng, 10, 1.0) for _ in range(3)]
    R = None
    raw = np.eye(10)
    for M in Ms:
        R = O.walk_update(R, M, 3)
        raw = raw @ np.linalg.matrix_power(M, 3)
    np.testing.assert_allclose(R, O.rownorm(raw), rtol=1e-10, atol=1e-12)


def test_diagonal_scores_keep_state_diagonal_and_lower_triangular():
    rng = np.random.default_rng(8)
    D = np.diag(rng.normal(size=7))
    R = O.walk_update(None, D, 5)
    assert np.count_nonzero(R - np.diag(np.diag(R))) == 0
    R2 = O.walk_update(R, _lower(rng, 7), 4)
    assert np.count_nonzero(np.triu(R2, 1)) == 0


def test_walk_row_equals_matrix_row():
    rng = np.random.default_rng(9)
    M = _lower(rng, 11, 0.5)
    R = O.walk_update(None, M, 8)
    for i in range(11):
        np.testing.assert_allclose(O.walk_row(None, M, i, 8), R[i], rtol=1e-12, atol=1e-13)
    M2 = _lower(rng, 11, 0.5)
    R2 = O.walk_update(R, M2, 8)
    for i in (0, 5, 10):
        np.testing.assert_allclose(O.walk_row(R[i], M2, i, 8), R2[i], rtol=1e-12, atol=1e-13)


def test_positive_scaling_of_queries_keeps_selection():
    cfg = gen.CONFIGS["C1"]
    q, k, v, _ = gen.layer_inputs(cfg, 0)
    Q = q[:, 0].double().numpy()
    K = k[:, 0].double().numpy()
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    lists = []
    for c in (1.0, 3.7):
        M = O.sketched_scores(O.sketch(c * Q, cfg.B, signs, cols), O.sketch(K, cfg.B, signs, cols))
        lists.append(O.select(O.walk_update(None, M, cfg.s), cfg.rho))
    for a, b in zip(*lists):
        np.testing.assert_array_equal(a, b)


def test_planted_two_hop_chain_reached_by_walk():
    """Generator sanity: for a chain i -> j -> m the walk row of block i puts
    m above the median of its candidates although the direct score
    M[i, m] carries no planted term."""
    cfg = gen.CONFIGS["C2"].with_(seqlens=(4096,), hq=8, hkv=2)
    q, k, _, _ = gen.layer_inputs(cfg, 0)
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    Q = q[:, 0].double().numpy()
    K = k[:, 0].double().numpy()
    M = O.sketched_scores(O.sketch(Q, cfg.B, signs, cols), O.sketch(K, cfg.B, signs, cols))
    R = O.walk_update(None, M, 2)
    # first persistent chain of group 0, as the generator drew it
    b = O.n_blocks(4096, cfg.B)
    z = gen.synth._band(cfg.cfg_id, 0, 0, b, cfg.d)
    m_hat = z.mean(axis=0) / np.linalg.norm(z.mean(axis=0))
    trip = gen.synth.chain_draws(cfg, 0, 0, 0, b, m_hat)[0][0]
    i, j, m = (int(x) for x in trip[0])
    assert i > j > m
    assert R[i, j] > np.median(R[i, :i])
    assert R[i, m] > np.median(R[i, :i])


def test_variant_transitions_hand_case():
    """Walk variants: the transition matrices of a 3-block example worked out
    by hand."""
    M = np.array([[2.0, 9.0, 9.0],
                  [1.0, -1.0, 9.0],
                  [0.5, 0.0, -2.0]])
    Tp = O.transition(M, "power", 3)
    assert np.allclose(Tp, [[8.0, 0, 0], [1.0, -1.0, 0], [0.125, 0.0, -8.0]], rtol=0, atol=0)
    Ts = O.transition(M, "softmax", 8)
    e = math.e
    assert np.allclose(Ts[0], [1.0, 0, 0])
    assert np.allclose(Ts[1], [e / (e + 1 / e), (1 / e) / (e + 1 / e), 0])
    den = math.exp(0.5) + 1.0 + math.exp(-2.0)
    assert np.allclose(Ts[2], [math.exp(0.5) / den, 1.0 / den, math.exp(-2.0) / den])


def test_variant_walks_reduce_to_closed_forms():
    rng = np.random.default_rng(11)
    b = 7
    M = np.tril(rng.standard_normal((b, b)))
    # power with s = 1 is the one-hop walk of the default reading
    assert np.allclose(O.walk_update_variant(None, M, 1, "power"), O.walk_update(None, M, 1))
    # power: one product with the elementwise power, from any previous state
    Rp = np.tril(rng.standard_normal((b, b)))
    want = O.rownorm(Rp @ np.tril(M ** 4))
    assert np.allclose(O.walk_update_variant(Rp, M, 4, "power"), want)
    # softmax: rows of T are probability vectors on the causal prefix
    T = O.transition(M, "softmax", 1)
    assert np.allclose(T.sum(axis=1), 1.0) and np.all(np.triu(T, 1) == 0) and np.all(T >= 0)
    # softmax, s hops from the identity: the rows of T^s, row-normalised
    R = O.walk_update_variant(None, M, 3, "softmax")
    assert np.allclose(R, O.rownorm(T @ T @ T))
    # s hops as single-step products: entries are sums over causal paths
    i, m = 5, 1
    paths = sum(T[i, j1] * T[j1, j2] * T[j2, m] for j1 in range(b) for j2 in range(b))
    assert np.isclose((T @ T @ T)[i, m], paths)
    # the row form equals the matrix row
    for mode, s in (("power", 8), ("softmax", 8)):
        full = O.walk_update_variant(Rp, M, s, mode)
        assert np.allclose(O.walk_row_variant(Rp[4], M, 4, s, mode), full[4])
        full0 = O.walk_update_variant(None, M, s, mode)
        assert np.allclose(O.walk_row_variant(None, M, 6, s, mode), full0[6])


def test_floor_hand_case():
    """Dynamic range of the walk state, worked by hand: the row (1, 1) walked
    s = 8 hops with M = diag(1, 2^-10) becomes (1, 2^-10 h) after hop h, so
    the second entry drops below 2^-64 of the row maximum at hop 7 and is zero
    from then on; without the floor it is 2^-80."""
    M = np.diag([1.0, 2.0 ** -10])
    x = np.array([[1.0, 1.0]])
    assert O.walk_update(x, M, 8).tolist() == [[1.0, 0.0]]
    assert O.walk_update(x, M, 8, floor=0.0).tolist() == [[1.0, 2.0 ** -80]]
    assert O.walk_update(x, M, 6).tolist() == [[1.0, 2.0 ** -60]]        # still inside
    assert O.walk_row(x[0], M, 1, 8).tolist() == [1.0, 0.0]
    # the comparison is strict: exactly 2^-64 of the maximum stays
    assert O.floor_rows(np.array([[4.0, 2.0 ** -62, -2.0 ** -62 / 2]])).tolist() == \
        [[4.0, 2.0 ** -62, 0.0]]
    # an all-zero row stays zero; rows are cut independently
    assert O.floor_rows(np.array([[0.0, 0.0], [1.0, 2.0 ** -70]])).tolist() == \
        [[0.0, 0.0], [1.0, 0.0]]


@pytest.mark.parametrize("seed", range(4))
def test_floor_leaves_well_scaled_walks_unchanged(seed):
    """With entries inside 64 binary orders of magnitude of their row maximum
    the floor changes nothing: the floored walk equals the plain one."""
    rng = np.random.default_rng(50 + seed)
    M = _lower(rng, 10, 2.0)
    Rp = O.rownorm(np.tril(rng.uniform(0.5, 1.0, size=(10, 10))))
    a = O.walk_update(Rp, M, 4)
    b = O.walk_update(Rp, M, 4, floor=0.0)
    assert np.abs(np.abs(Rp @ np.linalg.matrix_power(M, 4)) /
                  np.abs(Rp @ np.linalg.matrix_power(M, 4)).max(1, keepdims=True))[
        np.tril(np.ones((10, 10), bool))].min() > 2.0 ** -64
    np.testing.assert_array_equal(a, b)
