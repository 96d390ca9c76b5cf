"""Checks on the synthetic generator (not on the method)."""
import math

import numpy as np
import torch

import gen
import oracle as O


def test_deterministic_and_shaped():
    cfg = gen.CONFIGS["C2"].with_(seqlens=(300, 129))
    a = gen.layer_inputs(cfg, 3)
    b = gen.layer_inputs(cfg, 3)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    q, k, v, cu = a
    assert q.shape == (429, 32, 128) and k.shape == (429, 8, 128) and v.dtype == torch.bfloat16
    assert cu.tolist() == [0, 300, 429]


def test_block_coherence_bound():
    """Section 6.1's concentration: with token = block latent + N(0, I) noise
    the block mean lies within sigma*sqrt(d*log(1/delta))/sqrt(B) of the latent
    for all but about delta of the blocks."""
    cfg = gen.CONFIGS["C1"]
    q, _, _, _ = gen.layer_inputs(cfg, 0, seqlens=(4096,))
    mu, _ = gen.synth.block_latents(cfg, 0, 0, 0, 4096)
    qbar = O.block_means(q[:, 0].double().numpy(), cfg.B)
    delta = 0.05
    bound = math.sqrt(cfg.d * math.log(1 / delta)) / math.sqrt(cfg.B)
    frac = np.mean(np.linalg.norm(qbar - mu, axis=1) > bound)
    assert frac <= delta


def test_tables():
    s, c = gen.hadamard_tables(128, 32)
    assert set(np.unique(s).tolist()) <= {-1, 1} and len(s) == 128
    assert len(set(c.tolist())) == 32 and np.all(np.diff(c) > 0) and c.max() < 128
