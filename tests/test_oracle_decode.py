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
