"""Pins for the oracle's block means, exact block score and Hadamard sketch
(blog page sections 2, 3.1, 3.2, 6.2)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_block_means_and_a_true_hand_example():
    g = _gold("block_scores.json")
    Q = np.array(g["Q"], float)
    K = np.array(g["K"], float)
    assert O.n_blocks(5, g["B"]) == 3
    np.testing.assert_allclose(O.block_means(Q, g["B"]), g["q_means"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.block_means(K, g["B"]), g["k_means"], rtol=0, atol=1e-15)
    want = np.array(g["a_true_times_sqrt_d"], float) / math.sqrt(2)
    np.testing.assert_allclose(O.a_true_bruteforce(Q, K, g["B"]), want, atol=1e-14)
    np.testing.assert_allclose(O.a_true(O.block_means(Q, 2), O.block_means(K, 2)), want, atol=1e-14)


@pytest.mark.parametrize("n,B,d", [(7, 3, 4), (8, 4, 8), (13, 4, 2)])
def test_a_true_factorised_equals_pairwise_sum(n, B, d):
    rng = np.random.default_rng(n * 100 + B)
    Q = rng.normal(size=(n, d))
    K = rng.normal(size=(n, d))
    brute = O.a_true_bruteforce(Q, K, B)
    fact = O.a_true(O.block_means(Q, B), O.block_means(K, B))
    np.testing.assert_allclose(fact, brute, rtol=1e-12, atol=1e-12)


def test_block_sums_partial_block():
    X = np.arange(10, dtype=float).reshape(5, 2)
    np.testing.assert_array_equal(O.block_sums(X, 2), [[2, 4], [10, 12], [8, 9]])


@pytest.mark.parametrize("d", [1, 2, 4, 16, 64, 128])
def test_sylvester_and_fwht_match_scipy(d):
    H = scipy.linalg.hadamard(d).astype(float)
    np.testing.assert_array_equal(O.sylvester(d), H)
    rng = np.random.default_rng(d)
    x = rng.normal(size=(3, d))
    np.testing.assert_allclose(O.fwht(x), x @ H, rtol=1e-13, atol=1e-12)
    # involution up to d
    np.testing.assert_allclose(O.fwht(O.fwht(x)), d * x, rtol=1e-12, atol=1e-11)


def test_hadamard_hand_example():
    g = _gold("hadamard_d4.json")
    np.testing.assert_array_equal(O.sylvester(4), g["sylvester_4"])
    got = O.sketch_from_means(np.array([g["x"]], float), np.array(g["signs"]), np.array(g["cols"]))
    np.testing.assert_allclose(got[0], np.array(g["sketch_times_sqrt_k"]) / math.sqrt(2), atol=1e-14)


def test_projection_equals_sign_flip_fwht_subsample():
    rng = np.random.default_rng(3)
    d, k = 128, 32
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    cols = np.sort(rng.choice(d, k, replace=False))
    x = rng.normal(size=(5, d))
    via_fwht = O.fwht(x * signs)[:, cols] / math.sqrt(k)
    Hs = scipy.linalg.hadamard(d).astype(float)
    via_scipy = (x * signs) @ Hs[:, cols] / math.sqrt(k)
    got = O.sketch_from_means(x, signs, cols)
    np.testing.assert_allclose(got, via_fwht, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got, via_scipy, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d,B,n", [(64, 64, 1000), (128, 16, 200), (16, 4, 37)])
def test_full_dimension_sketch_is_exact(d, B, n):
    """k = d: H_d is orthonormal, so the sketched score equals A_true."""
    rng = np.random.default_rng(d + n)
    Q = rng.normal(size=(n, d))
    K = rng.normal(size=(n, d))
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    cols = np.arange(d)
    H = O.hadamard_projection(signs, cols, d)
    np.testing.assert_allclose(H @ H.T, np.eye(d), atol=1e-13)
    qs = O.sketch(Q, B, signs, cols)
    ks = O.sketch(K, B, signs, cols)
    A_sws = (qs @ ks.T) / math.sqrt(d)
    A = O.a_true(O.block_means(Q, B), O.block_means(K, B))
    np.testing.assert_allclose(A_sws, A, rtol=1e-10, atol=1e-12)
    M = O.sketched_scores(qs, ks)
    np.testing.assert_allclose(M, np.tril(A), rtol=1e-10, atol=1e-12)


def test_srht_inner_product_unbiased_and_bounded():
    """Section 6.2: the Hadamard sketch preserves inner products; averaged over
    random signs and column subsets it is unbiased, and at k = 32 most draws
    land within eps*|u||v| for eps = 3/sqrt(k)."""
    d, k, trials = 128, 32, 3000
    rng = np.random.default_rng(11)
    u = rng.normal(size=d)
    v = 0.6 * u + 0.8 * rng.normal(size=d)
    H = scipy.linalg.hadamard(d).astype(float)
    est = np.empty(trials)
    for t in range(trials):
        signs = np.where(rng.random(d) < 0.5, -1, 1)
        cols = np.sort(rng.choice(d, k, replace=False))
        Hd = O.hadamard_projection(signs, cols, d)
        est[t] = (u @ Hd) @ (v @ Hd)
    exact = u @ v
    sem = est.std() / math.sqrt(trials)
    assert abs(est.mean() - exact) < 4 * sem
    eps = 3.0 / math.sqrt(k)
    frac_out = np.mean(np.abs(est - exact) > eps * np.linalg.norm(u) * np.linalg.norm(v))
    assert frac_out < 0.01
    # a dropped sign flip or a missing 1/sqrt(k) would be biased
    del H


def test_sketch_scale_and_sign_errors_are_caught():
    """Plausible slips (no 1/sqrt(k), signs ignored) break the k = d identity."""
    rng = np.random.default_rng(5)
    d, B, n = 16, 4, 32
    Q = rng.normal(size=(n, d))
    K = rng.normal(size=(n, d))
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    cols = np.arange(d)
    A = O.a_true(O.block_means(Q, B), O.block_means(K, B))
    bad = (O.block_means(Q, B) @ scipy.linalg.hadamard(d)) @ (O.block_means(K, B) @ scipy.linalg.hadamard(d)).T
    assert not np.allclose(bad / math.sqrt(d), A)
    good = (O.sketch(Q, B, signs, cols) @ O.sketch(K, B, signs, cols).T) / math.sqrt(d)
    np.testing.assert_allclose(good, A, atol=1e-12)
