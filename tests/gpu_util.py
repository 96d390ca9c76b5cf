"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding and compare every stage with the oracle fed the GPU's own upstream
outputs (so a mismatch is attributed to the stage that produced it)."""
from __future__ import annotations

import math

import numpy as np
import torch

import dynamic_block_sparse_sws_amd as sws
import gen
import oracle as O

TOL_SKETCH = 1e-4      # max |err| per row relative to the row's max magnitude
TOL_WALK = 1e-4
TOL_ATTN_BF16 = 2e-2   # absolute
TOL_ATTN_F32 = 1e-5


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def rowwise_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    got = np.atleast_2d(got)
    want = np.atleast_2d(want)
    den = np.abs(want).max(axis=1)
    den = np.where(den > 0, den, 1.0)
    return float((np.abs(got - want).max(axis=1) / den).max())


def tables(cfg, device):
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    return (signs, cols, torch.from_numpy(signs).to(device), torch.from_numpy(cols).to(device))


class PrefillRun:
    """Runs the layers of one config through the HIP path, keeping host copies
    of every stage for the oracle comparisons."""

    def __init__(self, cfg, seqlens, n_layers, rho, n_dense, device="cuda", dense_idx_null=False):
        self.cfg = cfg
        self.seqlens = list(seqlens)
        self.rho = rho
        self.n_dense = n_dense
        self.geo = sws.Geometry(self.seqlens, cfg.B, device)
        self.signs, self.cols, self.signs_d, self.cols_d = tables(cfg, device)
        self.layers = []
        R = None
        for l in range(n_layers):
            q, k, v, _ = gen.layer_inputs(cfg, l, device=device, seqlens=self.seqlens)
            dense = l < n_dense
            q_sk = sws.sketch(q, self.geo, cfg.k, self.signs_d, self.cols_d)
            k_sk = sws.sketch(k, self.geo, cfg.k, self.signs_d, self.cols_d)
            R_prev_host = None if R is None else R.clone()
            R = sws.walk_update(q_sk, k_sk, self.geo, cfg.s, R, R_out=R)
            if dense and dense_idx_null:
                idx = cnt = None
            else:
                idx, cnt = sws.select_topk(R, cfg.hq, self.geo, rho, dense=dense)
            lse = torch.empty((cfg.hq, self.geo.total_tokens), dtype=torch.float32, device=device)
            out = sws.sparse_attn_prefill(q, k, v, self.geo, idx, cnt, lse=lse)
            torch.cuda.synchronize()
            self.layers.append({
                "q": f64(q), "k": f64(k), "v": f64(v), "q_sk": f64(q_sk), "k_sk": f64(k_sk),
                "R_prev": None if R_prev_host is None else f64(R_prev_host), "R": f64(R),
                "idx": None if idx is None else idx.cpu().numpy(),
                "cnt": None if cnt is None else cnt.cpu().numpy(),
                "out": f64(out), "lse": f64(lse), "dense": dense,
            })

    # -- per-sequence views -------------------------------------------------
    def tok(self, s):
        a = int(self.geo.cu_seqlens_host[s])
        return slice(a, a + self.seqlens[s])

    def blk(self, s):
        a = int(self.geo.cu_blocks_host[s])
        return slice(a, a + self.geo.blocks[s])

    def R_of(self, L, s, h, key="R"):
        arr = L[key]
        if arr is None:
            return None
        b = self.geo.blocks[s]
        off = self.geo.walk_offset(s, self.cfg.hq) + h * b * b
        return arr[off:off + b * b].reshape(b, b)

    def lists_of(self, L, s, h):
        b = self.geo.blocks[s]
        sl = self.blk(s)
        if L["idx"] is None:
            return [np.arange(i + 1) for i in range(b)]
        idx = L["idx"][h, sl]
        cnt = L["cnt"][h, sl]
        return [idx[i, :cnt[i]].astype(np.int64) for i in range(b)]


def check_prefill_run(run: PrefillRun, attn_rows_per_head=None, attn_heads=None):
    """Stage-wise parity of every layer; returns a dict of the worst errors."""
    cfg = run.cfg
    tol_attn = TOL_ATTN_F32 if cfg.dtype == "f32" else TOL_ATTN_BF16
    worst = {"sketch": 0.0, "walk": 0.0, "attn": 0.0, "lse": 0.0}
    grp = cfg.hq // cfg.hkv
    scale = 1.0 / math.sqrt(cfg.d)
    rng = np.random.default_rng(0)
    for li, L in enumerate(run.layers):
        for s in range(len(run.seqlens)):
            ts, bs = run.tok(s), run.blk(s)
            b = run.geo.blocks[s]
            # sketches
            for h in range(cfg.hq):
                want = O.sketch(L["q"][ts, h], cfg.B, run.signs, run.cols)
                e = rowwise_rel_err(L["q_sk"][h, bs], want)
                worst["sketch"] = max(worst["sketch"], e)
                assert e <= TOL_SKETCH, (li, s, h, "q sketch", e)
            for g in range(cfg.hkv):
                want = O.sketch(L["k"][ts, g], cfg.B, run.signs, run.cols)
                e = rowwise_rel_err(L["k_sk"][g, bs], want)
                worst["sketch"] = max(worst["sketch"], e)
                assert e <= TOL_SKETCH, (li, s, g, "k sketch", e)
            heads = range(cfg.hq) if attn_heads is None else attn_heads
            for h in range(cfg.hq):
                g = h // grp
                M = O.sketched_scores(L["q_sk"][h, bs], L["k_sk"][g, bs])
                Rp = run.R_of(L, s, h, "R_prev")
                Rw = O.walk_update(None if Rp is None else np.tril(Rp), M, cfg.s)
                Rg = run.R_of(L, s, h)
                e = rowwise_rel_err(Rg, Rw)
                worst["walk"] = max(worst["walk"], e)
                assert e <= TOL_WALK, (li, s, h, "walk", e)
                assert np.count_nonzero(np.triu(Rg, 1)) == 0
                # selection: bit-exact on the GPU's own fp32 walk scores
                got = run.lists_of(L, s, h)
                want = O.select(Rg, run.rho, L["dense"])
                for i in range(b):
                    assert got[i].tolist() == want[i].tolist(), (li, s, h, i, got[i], want[i])
                if h not in heads:
                    continue
                if attn_rows_per_head is None:
                    rows = list(range(b))
                else:
                    rows = sorted(set([0, b - 1] + rng.choice(b, size=min(b, attn_rows_per_head),
                                                              replace=False).tolist()))
                res = O.sparse_attention_rows(L["q"][ts, h], L["k"][ts, g], L["v"][ts, g], got,
                                              cfg.B, scale, rows)
                for i in rows:
                    o_want, lse_want = res[i]
                    a = ts.start + i * cfg.B
                    o_got = L["out"][a:a + o_want.shape[0], h]
                    lse_got = L["lse"][h, a:a + o_want.shape[0]]
                    e = float(np.abs(o_got - o_want).max())
                    e2 = float(np.abs(lse_got - lse_want).max())
                    worst["attn"] = max(worst["attn"], e)
                    worst["lse"] = max(worst["lse"], e2)
                    assert e <= tol_attn, (li, s, h, i, "attn", e)
                    assert e2 <= max(tol_attn, 1e-4), (li, s, h, i, "lse", e2)
    return worst
