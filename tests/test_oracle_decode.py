"""Pin for the oracle's decode step: it must equal the row of the prefill on
the prefix (blog page section 5: the same selection rule for each decode step)."""
import numpy as np
import pytest

import gen
import oracle as O


def _prefix_layers(cfg, p_len, layers):
    out = []
    for l in range(layers):
        q, k, v, _ = gen.layer_inputs(cfg, l, seqlens=(p_len,))
        out.append((q.double().numpy(), k.double().numpy(), v.double().numpy()))
    return out


@pytest.mark.parametrize("p_len", [1, 17, 64, 65, 130, 256])
def test_decode_equals_prefix_prefill_row(p_len):
    cfg = gen.CONFIGS["C2"].with_(hq=4, hkv=2, d=16, B=16, k=8, seqlens=(p_len,))
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    layers = _prefix_layers(cfg, p_len, 3)
    dec = O.decode_step(layers, signs, cols, cfg.B, cfg.s, 40, n_dense=1)
    b = O.n_blocks(p_len, cfg.B)
    c = (p_len - 1) // cfg.B
    pre = O.prefill(layers, signs, cols, cfg.B, cfg.s, 40, n_dense=1, attn_rows=[c])
    for l in range(3):
        for h in range(cfg.hq):
            dh, ph = dec[l][h], pre[l][h]
            np.testing.assert_allclose(dh["r"], ph["R"][c], rtol=1e-10, atol=1e-12)
            assert dh["lst"].tolist() == ph["lists"][c].tolist()
            o_blk, lse_blk = ph["attn"][c]
            t = p_len - 1 - c * cfg.B
            np.testing.assert_allclose(dh["o"], o_blk[t], rtol=1e-11, atol=1e-12)
            assert abs(dh["lse"] - lse_blk[t]) < 1e-11
    assert b == c + 1


def test_fp8_e4m3_value_spec_points():
    """Codes whose values the OCP E4M3 definition fixes: one, the largest
    finite value, the smallest normal and subnormal, signed zero, NaN."""
    v = O.fp8_e4m3_value([0x38, 0xB8, 0x7E, 0xFE, 0x08, 0x01, 0x07, 0x00, 0x80, 0x7F, 0xFF,
                          0x40, 0x3C, 0x30])
    want = [1.0, -1.0, 448.0, -448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, 0.0, -0.0,
            np.nan, np.nan, 2.0, 1.5, 0.5]
    np.testing.assert_array_equal(v, want)
    assert np.signbit(v[8]) and not np.signbit(v[7])


def test_fp8_e4m3_value_matches_torch_on_every_code():
    """All 256 codes against torch's float8_e4m3fn, an independent decoder of
    the same format (NaN codes compare as NaN)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = O.fp8_e4m3_value(codes)
    np.testing.assert_array_equal(got, want)
    # monotone over the positive finite codes
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_gather_pages_by_hand():
    """Two pages of B = 2 tokens in swapped order: token t sits in row t % 2
    of page table[t // 2]."""
    pages = np.arange(3 * 2 * 1).reshape(3, 2, 1)   # page p row r holds 2 p + r
    got = O.gather_pages(pages, [2, 0, 1], 5, 2)[:, 0].tolist()
    assert got == [4, 5, 0, 1, 2]


@pytest.mark.parametrize("c", [0, 2, 5])
def test_decode_at_block_end_equals_full_prefill_row_with_row_budget(c):
    """When the new token p is the last of block c, decode(p) equals row p of
    the prefill of a longer sequence, provided the prefill uses the per-row
    budget floor(rho (i + 1) / 100): the walk row c only involves blocks <= c
    (the block graph is causal), and those are complete in both."""
    n = 7 * 16 + 5
    cfg = gen.CONFIGS["C2"].with_(hq=4, hkv=2, d=16, B=16, k=8, seqlens=(n,))
    B, rho = cfg.B, 40
    p_len = (c + 1) * B
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    full = _prefix_layers(cfg, n, 3)
    pre_layers = [(q[:p_len], k[:p_len], v[:p_len]) for q, k, v in full]
    dec = O.decode_step(pre_layers, signs, cols, B, cfg.s, rho, n_dense=1)
    pre = O.prefill(full, signs, cols, B, cfg.s, rho, n_dense=1, with_attention=False)
    grp = cfg.hq // cfg.hkv
    for l in range(3):
        Q, K, V = full[l]
        for h in range(cfg.hq):
            row = pre[l][h]["R"][c]
            np.testing.assert_allclose(dec[l][h]["r"], row[:c + 1], rtol=1e-10, atol=1e-12)
            assert np.all(row[c + 1:] == 0)
            lst = (np.arange(c + 1) if l < 1
                   else O.select_row(row, c, O.n_select_row(rho, c)))
            assert dec[l][h]["lst"].tolist() == lst.tolist()
            g = h // grp
            o_blk, lse_blk = O.sparse_attention_rows(Q[:, h], K[:, g], V[:, g], {c: lst}, B,
                                                     1.0 / np.sqrt(cfg.d), [c])[c]
            np.testing.assert_allclose(dec[l][h]["o"], o_blk[B - 1], rtol=1e-11, atol=1e-12)
            assert abs(dec[l][h]["lse"] - lse_blk[B - 1]) < 1e-11


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_split_kv_combine_equals_unsplit(seed):
    """The split-KV rule the decode kernels use: each chunk of keys keeps its
    (max, sum of exp, exp-weighted V sum); merging them with
    weights exp(m_r - max m) reproduces the unsplit softmax average and its
    log-sum-exp (closed form of the softmax, any chunking, empty chunks
    included)."""
    rng = np.random.default_rng(seed)
    n, d = 300, 8
    z = rng.normal(size=n) * 3
    V = rng.normal(size=(n, d))
    zm = z.max()
    w = np.exp(z - zm)
    o_ref = w @ V / w.sum()
    lse_ref = zm + np.log(w.sum())
    cuts = np.sort(rng.choice(np.arange(1, n), size=6, replace=False))
    bounds = [0, *cuts.tolist(), cuts[-1], n]          # includes an empty chunk
    recs = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b <= a:
            recs.append((-np.inf, 0.0, np.zeros(d)))
            continue
        m = z[a:b].max()
        e = np.exp(z[a:b] - m)
        recs.append((m, e.sum(), e @ V[a:b]))
    M = max(r[0] for r in recs)
    f = [0.0 if r[0] == -np.inf else np.exp(r[0] - M) for r in recs]
    L = sum(fi * r[1] for fi, r in zip(f, recs))
    acc = sum(fi * r[2] for fi, r in zip(f, recs))
    np.testing.assert_allclose(acc / L, o_ref, rtol=1e-12, atol=1e-13)
    assert abs(M + np.log(L) - lse_ref) < 1e-12
