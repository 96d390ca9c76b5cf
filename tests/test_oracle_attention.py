"""Pins for the oracle's block-sparse attention (blog page sections 4-5)
against torch's scaled_dot_product_attention on the CPU in fp64."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_example():
    with open(os.path.join(GOLD, "attention_small.json")) as f:
        g = json.load(f)
    Q, K, V = (np.array(g[x], float) for x in "QKV")
    for key in ("dense", "sparse"):
        lists = [np.array(x) for x in g[key]["lists"]]
        o, lse = O.sparse_attention(Q, K, V, lists, g["B"], scale=1.0)
        np.testing.assert_allclose(o, g[key]["O"], atol=1e-14)
        np.testing.assert_allclose(lse, g[key]["lse"], atol=1e-14)


def _sdpa_masked(Q, K, V, mask, scale):
    q = torch.from_numpy(Q)[None, None]
    k = torch.from_numpy(K)[None, None]
    v = torch.from_numpy(V)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=torch.from_numpy(mask)[None, None], scale=scale)
    z = (torch.from_numpy(Q) @ torch.from_numpy(K).T) * scale
    z = z.masked_fill(~torch.from_numpy(mask), float("-inf"))
    return o[0, 0].numpy(), torch.logsumexp(z, dim=1).numpy()


@pytest.mark.parametrize("n,B,d", [(64, 8, 16), (70, 16, 8), (33, 32, 4)])
def test_dense_lists_equal_causal_sdpa(n, B, d):
    rng = np.random.default_rng(n + d)
    Q, K, V = (rng.normal(size=(n, d)) for _ in range(3))
    b = O.n_blocks(n, B)
    lists = O.select(np.zeros((b, b)), 100)
    o, lse = O.sparse_attention(Q, K, V, lists, B)
    q = torch.from_numpy(Q)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None], is_causal=True)
    np.testing.assert_allclose(o, ref[0, 0].numpy(), rtol=1e-12, atol=1e-12)
    mask = np.tril(np.ones((n, n), bool))
    _, lse_ref = _sdpa_masked(Q, K, V, mask, 1 / math.sqrt(d))
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_sparse_lists_equal_masked_sdpa(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.choice([4, 8]))
    n = int(rng.integers(B, 12 * B))
    d = 8
    Q, K, V = (rng.normal(size=(n, d)) for _ in range(3))
    b = O.n_blocks(n, B)
    R = O.rownorm(np.tril(rng.normal(size=(b, b))))
    lists = O.select(R, int(rng.integers(0, 60)))
    mask = np.zeros((n, n), bool)
    for i, lst in enumerate(lists):
        for j in lst:
            mask[i * B:(i + 1) * B, j * B:(j + 1) * B] = True
    mask &= np.tril(np.ones((n, n), bool))
    o, lse = O.sparse_attention(Q, K, V, lists, B)
    o_ref, lse_ref = _sdpa_masked(Q, K, V, mask, 1 / math.sqrt(d))
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_single_block_list_is_plain_attention_over_that_block():
    rng = np.random.default_rng(1)
    B, d = 8, 4
    Q, K, V = (rng.normal(size=(40, d)) for _ in range(3))
    lists = [np.array([i]) for i in range(5)]
    o, _ = O.sparse_attention(Q, K, V, lists, B)
    for i in range(5):
        sl = slice(i * B, (i + 1) * B)
        z = Q[sl] @ K[sl].T / 2.0
        z = np.where(np.tril(np.ones((B, B), bool)), z, -np.inf)
        p = np.exp(z - z.max(1, keepdims=True))
        np.testing.assert_allclose(o[sl], (p / p.sum(1, keepdims=True)) @ V[sl], atol=1e-13)


@pytest.mark.parametrize("seed", range(6))
def test_query_attention_equals_masked_sdpa_row(seed):
    """One decode query at position p over the listed blocks (keys u <= p)
    equals torch's masked SDPA on that row, output and log-sum-exp."""
    rng = np.random.default_rng(300 + seed)
    B = int(rng.choice([4, 8]))
    n = int(rng.integers(2, 12 * B))
    d = 8
    Q, K, V = (rng.normal(size=(n, d)) for _ in range(3))
    p = int(rng.integers(0, n))
    c = p // B
    earlier = rng.permutation(c)[:int(rng.integers(0, c + 1))]
    lst = np.sort(np.concatenate([earlier, [c]])).astype(np.int64)
    mask = np.zeros((1, n), bool)
    for j in lst:
        mask[0, j * B:(j + 1) * B] = True
    mask[0, p + 1:] = False
    o, lse = O.query_attention(Q[p], K, V, lst, B, p, 1 / math.sqrt(d))
    o_ref, lse_ref = _sdpa_masked(Q[p:p + 1], K, V, mask, 1 / math.sqrt(d))
    np.testing.assert_allclose(o, o_ref[0], rtol=1e-12, atol=1e-12)
    assert abs(lse - lse_ref[0]) <= 1e-12
    # and it is row p of the block-row form
    rows = O.sparse_attention_rows(Q[:p + 1], K[:p + 1], V[:p + 1], {c: lst}, B,
                                   1 / math.sqrt(d), [c])
    np.testing.assert_allclose(o, rows[c][0][-1], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (6, 3), (8, 1)])
def test_gqa_head_map_equals_sdpa_enable_gqa(hq, hkv):
    """The oracle's grouped-query map (query head h reads KV head h // (hq /
    hkv), reading R14) against torch's grouped-query attention, which fixes
    the same convention independently: one dense layer (every block kept),
    all heads, fp64."""
    n, d, B = 45, 8, 8
    rng = np.random.default_rng(hq * 10 + hkv)
    Q = rng.normal(size=(n, hq, d))
    K = rng.normal(size=(n, hkv, d))
    V = rng.normal(size=(n, hkv, d))
    signs = np.ones(d, np.int8)
    cols = np.arange(4, dtype=np.int32)
    st = O.SeqPrefill(hq)
    recs = O.prefill_layer(Q, K, V, st, signs, cols, B, 1, 20, dense=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q).permute(1, 0, 2)[None], torch.from_numpy(K).permute(1, 0, 2)[None],
        torch.from_numpy(V).permute(1, 0, 2)[None], is_causal=True, enable_gqa=True)[0]
    for h in range(hq):
        got = np.concatenate([recs[h]["attn"][i][0] for i in sorted(recs[h]["attn"])])
        np.testing.assert_allclose(got, ref[h].numpy(), rtol=1e-12, atol=1e-12)
