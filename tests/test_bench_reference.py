"""The exact-score references behind bench.py's selection diagnostics (block
means, the walk on exact block scores, and the attention mass a block
selection captures), checked against the oracle on small inputs, on the CPU."""
import itertools
import math

import numpy as np
import pytest
import torch

import bench
import oracle as O


def _inputs(n, d, seed):
    rng = np.random.default_rng(seed)
    # a shared direction plus noise, so block scores spread over a useful range
    u = rng.standard_normal(d)
    q = rng.standard_normal((n, d)) + 0.7 * u
    k = rng.standard_normal((n, d)) + 0.5 * u
    v = rng.standard_normal((n, d))
    return q, k, v


def test_block_means_match_oracle():
    q, _, _ = _inputs(203, 8, 1)
    got = bench.ref_block_means(torch, torch.from_numpy(q), 16).numpy()
    np.testing.assert_allclose(got, O.block_means(q, 16), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("s,rho", [(1, 20), (3, 30), (8, 20)])
def test_walk_sets_match_oracle(s, rho):
    q, k, _ = _inputs(400, 16, 2 + s)
    B = 16
    qm, km = O.block_means(q, B), O.block_means(k, B)
    want = O.select(O.walk_update(None, O.sketched_scores(qm, km), s), rho)
    got = bench.ref_walk_sets(torch, torch.from_numpy(qm), torch.from_numpy(km), s, rho)
    assert [sorted(x) for x in got] == [w.tolist() for w in want]


def test_captured_mass_matches_oracle_lse_and_brute_force_best():
    """The captured mass of a selection equals exp(lse_sparse - lse_dense) of
    the oracle's attention, row by row; the best selection of a density is the
    tau-subset of earlier blocks (plus the diagonal) with the largest total,
    found here by trying every subset."""
    n, d, B, rho, s = 150, 8, 16, 30, 2
    q, k, v = _inputs(n, d, 7)
    b = O.n_blocks(n, B)
    qm, km = O.block_means(q, B), O.block_means(k, B)
    lists = O.select(O.walk_update(None, O.sketched_scores(qm, km), s), rho)
    dense = O.select(np.zeros((b, b)), rho, dense=True)
    _, lse_s = O.sparse_attention(q, k, v, lists, B)
    _, lse_d = O.sparse_attention(q, k, v, dense, B)
    got = bench.ref_captured_mass(torch, torch.from_numpy(q), torch.from_numpy(k), B,
                                  {"walk": lists}, rhos=(rho,), chunk=3)
    np.testing.assert_allclose(got["walk"], np.exp(lse_s - lse_d), rtol=2e-5)

    tau = O.n_select(rho, b)
    scale = 1.0 / math.sqrt(d)
    best = []
    for i in range(b):
        a, e = i * B, min(n, (i + 1) * B)
        cands = ([list(range(i + 1))] if i <= tau else
                 [list(c) + [i] for c in itertools.combinations(range(i), tau)])
        top, top_rows = -1.0, None
        for c in cands:
            _, lse_c = O.sparse_attention_rows(q, k, v, {i: c}, B, scale, [i])[i]
            rows = np.exp(lse_c - lse_d[a:e])
            if rows.sum() > top:
                top, top_rows = rows.sum(), rows
        best.append(top_rows)
    np.testing.assert_allclose(got[f"best rho={rho}"], np.concatenate(best), rtol=2e-5)
    # no selection of the density captures more than the best one
    assert np.all(got["walk"].reshape(-1).sum() <= got[f"best rho={rho}"].sum() * (1 + 1e-6))
