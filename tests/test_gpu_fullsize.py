"""GPU parity at the full workload sizes, in the launch configuration the bench
times (same entry points, same buffers, walk state carried across layers),
checked on outputs the oracle computes one by one:

* 32K prefill (32 query / 8 KV heads, d=128, B=64, k=32): three layers (two
  dense, one sparse), every sketch row, every walk row, every selection, and
  sampled query blocks of attention;
* 128K prefill (B=128, b=1024): two sparse layers, walk state carried from the
  first into the second; every sketch row and selection, full walks of
  sampled heads plus sampled rows of every other head, sampled attention;
* ragged batch (8 sequences of 4096..65536 tokens, 40 query / 8 KV heads);
* decode (16 sequences, 64K-token prefix, 32 query / 8 KV heads): four layers
  over 66 steps, crossing a block boundary.

Each stage is compared with the oracle fed the GPU's own upstream outputs, so a
failure names the stage; bars as in the small tests (sketch and walk 1e-4 of
the row's largest magnitude, selections bit-exact, bf16 attention 2e-2)."""
import math

import numpy as np
import pytest
import torch

import dynamic_block_sparse_sws_amd as sws
import gen
import oracle as O
from gpu_util import rowwise_rel_err, TOL_ATTN_BF16, TOL_SKETCH, TOL_WALK

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def h64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def run_layer(cfg, geo, q, k, v, signs_d, cols_d, R, first, rho, dense):
    """One layer exactly as the bench runs it (R updated in place)."""
    q_sk = sws.sketch(q, geo, cfg.k, signs_d, cols_d)
    k_sk = sws.sketch(k, geo, cfg.k, signs_d, cols_d)
    R_prev = None if first else R.clone()
    sws.walk_update(q_sk, k_sk, geo, cfg.s, None if first else R, R_out=R)
    idx, cnt = sws.select_topk(R, cfg.hq, geo, rho, dense=dense)
    lse = torch.empty((cfg.hq, geo.total_tokens), dtype=torch.float32, device="cuda")
    ws = torch.empty(sws.prefill_workspace_size(sws.BF16, geo.total_blocks, cfg.hkv, cfg.d,
                                                cfg.B), dtype=torch.uint8, device="cuda")
    out = sws.sparse_attn_prefill(q, k, v, geo, idx, cnt, lse=lse, ws=ws)
    torch.cuda.synchronize()
    return {"q_sk": q_sk, "k_sk": k_sk, "R_prev": R_prev, "R": R.clone(), "idx": idx,
            "cnt": cnt, "out": out, "lse": lse}


def check_layer(cfg, geo, lens, q, k, v, st, rho, dense, signs, cols, *, full_walk_heads,
                walk_rows, sel_heads, attn_heads, attn_blocks, seed, label):
    rng = np.random.default_rng(seed)
    grp = cfg.hq // cfg.hkv
    scale = 1.0 / math.sqrt(cfg.d)
    q_sk, k_sk = h64(st["q_sk"]), h64(st["k_sk"])
    R = st["R"].cpu().numpy()
    Rp = None if st["R_prev"] is None else st["R_prev"].cpu().numpy()
    idx, cnt = st["idx"].cpu().numpy(), st["cnt"].cpu().numpy()
    worst = {"sketch": 0.0, "walk": 0.0, "attn": 0.0, "lse": 0.0, "sel_rows": 0}
    for s, n in enumerate(lens):
        t0 = int(geo.cu_seqlens_host[s])
        b0 = int(geo.cu_blocks_host[s])
        b = geo.blocks[s]
        ts, bs = slice(t0, t0 + n), slice(b0, b0 + b)
        woff = geo.walk_offset(s, cfg.hq)
        Kh = [h64(k[ts, g]) for g in range(cfg.hkv)]
        for g in range(cfg.hkv):
            e = rowwise_rel_err(k_sk[g, bs], O.sketch(Kh[g], cfg.B, signs, cols))
            worst["sketch"] = max(worst["sketch"], e)
            assert e <= TOL_SKETCH, (label, s, g, "k sketch", e)
        for h in range(cfg.hq):
            g = h // grp
            Qh = h64(q[ts, h])
            e = rowwise_rel_err(q_sk[h, bs], O.sketch(Qh, cfg.B, signs, cols))
            worst["sketch"] = max(worst["sketch"], e)
            assert e <= TOL_SKETCH, (label, s, h, "q sketch", e)
            # walk: stage-wise on the GPU's sketches and previous state
            M = O.sketched_scores(q_sk[h, bs], k_sk[g, bs])
            Rg = R[woff + h * b * b: woff + (h + 1) * b * b].reshape(b, b).astype(np.float64)
            Rph = (None if Rp is None
                   else np.tril(Rp[woff + h * b * b: woff + (h + 1) * b * b].reshape(b, b)))
            if h in full_walk_heads:
                rows = np.arange(b)
            else:
                rows = np.unique(np.concatenate([[0, b - 1],
                                                 rng.choice(b, size=min(b, walk_rows),
                                                            replace=False)]))
            start = np.eye(b)[rows] if Rph is None else Rph[rows].astype(np.float64)
            want = O.walk_update(start, M, cfg.s)
            e = rowwise_rel_err(Rg[rows], want)
            worst["walk"] = max(worst["walk"], e)
            assert e <= TOL_WALK, (label, s, h, "walk", e)
            upper = np.arange(b)[None, :] > rows[:, None]
            assert np.all(Rg[rows][upper] == 0), (label, s, h, "walk above diagonal")
            # selection, bit-exact on the GPU's fp32 scores
            lists = [idx[h, b0 + i, :cnt[h, b0 + i]].astype(np.int64) for i in range(b)]
            if h in sel_heads:
                tau = O.n_select(rho, b)
                for i in range(b):
                    want_l = np.arange(i + 1) if dense else O.select_row(Rg[i], i, tau)
                    assert lists[i].tolist() == want_l.tolist(), (label, s, h, i)
                worst["sel_rows"] += b
            if h not in attn_heads:
                continue
            blocks = sorted(set([0, b - 1] + rng.choice(b, size=min(b, attn_blocks),
                                                         replace=False).tolist()))
            res = O.sparse_attention_rows(Qh, Kh[g], h64(v[ts, g]), lists, cfg.B, scale, blocks)
            for i in blocks:
                o_want, lse_want = res[i]
                a = t0 + i * cfg.B
                o_got = h64(st["out"][a:a + o_want.shape[0], h])
                lse_got = h64(st["lse"][h, a:a + o_want.shape[0]])
                e = float(np.abs(o_got - o_want).max())
                e2 = float(np.abs(lse_got - lse_want).max())
                worst["attn"] = max(worst["attn"], e)
                worst["lse"] = max(worst["lse"], e2)
                assert e <= TOL_ATTN_BF16, (label, s, h, i, "attn", e)
                assert e2 <= TOL_ATTN_BF16, (label, s, h, i, "lse", e2)
    return worst


def _tables(cfg):
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    return signs, cols, torch.from_numpy(signs).cuda(), torch.from_numpy(cols).cuda()


def test_prefill_32k_full_size():
    cfg = gen.CONFIGS["C2"]
    lens = list(cfg.seqlens)
    geo = sws.Geometry(lens, cfg.B)
    signs, cols, signs_d, cols_d = _tables(cfg)
    R = torch.empty(geo.walk_numel(cfg.hq), dtype=torch.float32, device="cuda")
    for l in range(3):
        dense = l < cfg.n_dense
        _print("32k layer", l, "dense" if dense else "sparse")
        q, k, v, _ = gen.layer_inputs(cfg, l, device="cuda")
        st = run_layer(cfg, geo, q, k, v, signs_d, cols_d, R, l == 0, cfg.rho, dense)
        w = check_layer(cfg, geo, lens, q, k, v, st, cfg.rho, dense, signs, cols,
                        full_walk_heads=set(range(cfg.hq)), walk_rows=0,
                        sel_heads=set(range(cfg.hq)), attn_heads=set(range(0, cfg.hq, 3)),
                        attn_blocks=2, seed=l, label=f"32k/{l}")
        _print("worst", w)


def test_prefill_128k_full_size():
    """The bench's layer: 128K tokens, B=128, rho=20, sparse, walk carried."""
    cfg = gen.CONFIGS["C3"]
    lens = list(cfg.seqlens)
    geo = sws.Geometry(lens, cfg.B)
    signs, cols, signs_d, cols_d = _tables(cfg)
    R = torch.empty(geo.walk_numel(cfg.hq), dtype=torch.float32, device="cuda")
    for j, l in enumerate((2, 3)):
        _print("128k layer", l)
        q, k, v, _ = gen.layer_inputs(cfg, l, device="cuda")
        st = run_layer(cfg, geo, q, k, v, signs_d, cols_d, R, j == 0, 20, False)
        assert int(st["cnt"].long().sum()) == cfg.hq * sum(min(i + 1, 204 + 1) for i in range(1024))
        w = check_layer(cfg, geo, lens, q, k, v, st, 20, False, signs, cols,
                        full_walk_heads={0, 13, 31}, walk_rows=24,
                        sel_heads=set(range(cfg.hq)), attn_heads=set(range(0, cfg.hq, 4)),
                        attn_blocks=1, seed=10 + l, label=f"128k/{l}")
        _print("worst", w)
        del q, k, v, st
        torch.cuda.empty_cache()


def test_prefill_ragged_full_size():
    """Eight sequences of 4096..65536 tokens (lengths not multiples of B), 40
    query / 8 KV heads, per-sequence tau: one dense and one sparse layer."""
    cfg = gen.CONFIGS["C5"]
    lens = list(cfg.seqlens)
    geo = sws.Geometry(lens, cfg.B)
    signs, cols, signs_d, cols_d = _tables(cfg)
    R = torch.empty(geo.walk_numel(cfg.hq), dtype=torch.float32, device="cuda")
    for l, dense in ((0, True), (2, False)):
        _print("ragged layer", l, lens)
        q, k, v, _ = gen.layer_inputs(cfg, l, device="cuda")
        st = run_layer(cfg, geo, q, k, v, signs_d, cols_d, R, l == 0, cfg.rho, dense)
        w = check_layer(cfg, geo, lens, q, k, v, st, cfg.rho, dense, signs, cols,
                        full_walk_heads={7}, walk_rows=8, sel_heads={0, 7, 21, 39},
                        attn_heads={0, 11, 39}, attn_blocks=1, seed=20 + l,
                        label=f"ragged/{l}")
        _print("worst", w)
        del q, k, v, st
        torch.cuda.empty_cache()


def test_decode_full_size():
    """16 sequences with a 65536-token prefix, 32 query / 8 KV heads, B=64: four
    layers (two dense) over 66 steps; steps 0 (opens block 1024), 63 (fills it),
    64 and 65 (open and extend block 1025) are checked for three sequences."""
    cfg = gen.CONFIGS["C4"]
    ns, P, steps, n_layers = cfg.decode_batch, cfg.decode_prefix, 66, 4
    hq, hkv, d, B, kd = cfg.hq, cfg.hkv, cfg.d, cfg.B, cfg.k
    grp = hq // hkv
    max_ctx = P + steps
    b_max = -(-max_ctx // B)
    check_steps = {0, 63, 64, 65}
    check_seqs = (0, 7, 15)
    sketch_heads = (0, 17, 31)
    signs, cols, signs_d, cols_d = _tables(cfg)
    geo_p = sws.Geometry([P], B)
    layers = []
    for l in range(n_layers):
        qpre, qst, kc, vc = gen.decode_layer_inputs(cfg, l, device="cuda", n_seqs=ns, prefix=P,
                                                    steps=steps)
        qsk = torch.zeros((ns, hq, b_max, kd), dtype=torch.float32, device="cuda")
        ksk = torch.zeros((ns, hkv, b_max, kd), dtype=torch.float32, device="cuda")
        rq = torch.zeros((ns, hq, d), dtype=torch.float32, device="cuda")
        rk = torch.zeros((ns, hkv, d), dtype=torch.float32, device="cuda")
        for s in range(ns):
            sws.sketch(qpre[s], geo_p, kd, signs_d, cols_d, out=qsk[s], ld_head=b_max * kd)
            sws.sketch(kc[s, :P], geo_p, kd, signs_d, cols_d, out=ksk[s], ld_head=b_max * kd)
        # host copies for the checked sequences: the sketched heads' queries
        # over the whole context, every head's new-token queries, all K and V
        host = {s: {"q": torch.cat([qpre[s], qst[:, s]], 0)[:, list(sketch_heads)].float().cpu(),
                    "q_new": qst[:, s].float().cpu(),
                    "k": kc[s].float().cpu(), "v": vc[s].float().cpu()} for s in check_seqs}
        del qpre
        knew = kc[:, P:].permute(1, 0, 2, 3).contiguous()
        layers.append({"qst": qst, "knew": knew, "kc": kc, "vc": vc, "qsk": qsk, "ksk": ksk,
                       "rq": rq, "rk": rk, "host": host,
                       "r": torch.zeros((ns, hq, b_max), dtype=torch.float32, device="cuda")})
    torch.cuda.synchronize()
    _print("decode set-up done")
    uw = sws.union_width(cfg.rho, b_max, grp)
    worst = {"sketch": 0.0, "walk": 0.0, "attn": 0.0}
    for t in range(steps):
        pos = torch.full((ns,), P + t, dtype=torch.int32, device="cuda")
        cur = pos // B
        ctx = pos + 1
        recs = []
        for l, L in enumerate(layers):
            dense = l < cfg.n_dense
            sws.sketch_append(L["qst"][t], pos, B, kd, signs_d, cols_d, L["rq"], L["qsk"])
            sws.sketch_append(L["knew"][t], pos, B, kd, signs_d, cols_d, L["rk"], L["ksk"])
            r_prev = None if l == 0 else layers[l - 1]["r"]
            sws.walk_update_row(L["qsk"], L["ksk"], cur, cfg.s, r_prev, L["r"])
            uidx, ucnt, umask, idx, cnt = sws.select_topk_row(L["r"], hq, hkv, cur, b_max,
                                                              cfg.rho, dense=dense,
                                                              per_head=True)
            lse = torch.empty((ns, hq), dtype=torch.float32, device="cuda")
            out = sws.sparse_attn_decode(L["qst"][t], L["kc"], L["vc"], ctx, B, uidx, ucnt,
                                         umask, lse=lse)
            if t in check_steps:
                torch.cuda.synchronize()
                recs.append({"qsk": h64(L["qsk"]), "ksk": h64(L["ksk"]), "r": h64(L["r"]),
                             "uidx": uidx.cpu().numpy(), "ucnt": ucnt.cpu().numpy(),
                             "umask": umask.cpu().numpy().astype(np.uint32),
                             "idx": idx.cpu().numpy(), "cnt": cnt.cpu().numpy(),
                             "out": h64(out), "lse": h64(lse)})
        if t not in check_steps:
            continue
        _print("decode step", t)
        p = P + t
        c = p // B
        for l, (L, rec) in enumerate(zip(layers, recs)):
            dense = l < cfg.n_dense
            assert rec["uidx"].shape[2] <= uw or dense
            for s in check_seqs:
                H = L["host"][s]
                for hi, h in enumerate(sketch_heads):
                    want = O.sketch(H["q"][:p + 1, hi].double().numpy(), B, signs, cols)
                    e = rowwise_rel_err(rec["qsk"][s, h, :c + 1], want)
                    worst["sketch"] = max(worst["sketch"], e)
                    assert e <= TOL_SKETCH, (t, l, s, h, "q sketch", e)
                    g = h // grp
                    want = O.sketch(H["k"][:p + 1, g].double().numpy(), B, signs, cols)
                    e = rowwise_rel_err(rec["ksk"][s, g, :c + 1], want)
                    assert e <= TOL_SKETCH, (t, l, s, g, "k sketch", e)
                for h in range(hq):
                    g = h // grp
                    M = O.sketched_scores(rec["qsk"][s, h, :c + 1], rec["ksk"][s, g, :c + 1])
                    rp = None if l == 0 else recs[l - 1]["r"][s, h, :c + 1]
                    rw = O.walk_row(rp, M, c, cfg.s)
                    rg = rec["r"][s, h]
                    e = rowwise_rel_err(rg[:c + 1], rw)
                    worst["walk"] = max(worst["walk"], e)
                    assert e <= TOL_WALK, (t, l, s, h, "walk", e)
                    assert np.all(rg[c + 1:] == 0)
                    lst = (np.arange(c + 1) if dense
                           else O.select_row(rg, c, O.n_select(cfg.rho, c + 1)))
                    got = rec["idx"][s, h, :rec["cnt"][s, h]]
                    assert got.tolist() == lst.tolist(), (t, l, s, h)
                    keys = np.concatenate([np.arange(j * B, min((j + 1) * B, p + 1)) for j in lst])
                    kk = H["k"][keys, g].double().numpy()
                    z = (kk @ H["q_new"][t, h].double().numpy()) / math.sqrt(d)
                    zm = z.max()
                    wgt = np.exp(z - zm)
                    o_want = (wgt @ H["v"][keys, g].double().numpy()) / wgt.sum()
                    e = float(np.abs(rec["out"][s, h] - o_want).max())
                    worst["attn"] = max(worst["attn"], e)
                    assert e <= TOL_ATTN_BF16, (t, l, s, h, "attn", e)
                    assert abs(rec["lse"][s, h] - (zm + math.log(wgt.sum()))) <= TOL_ATTN_BF16
                for g in range(hkv):
                    want = {}
                    for h in range(g * grp, (g + 1) * grp):
                        for m in rec["idx"][s, h, :rec["cnt"][s, h]]:
                            want[int(m)] = want.get(int(m), 0) | (1 << (h - g * grp))
                    n_u = rec["ucnt"][s, g]
                    assert rec["uidx"][s, g, :n_u].tolist() == sorted(want), (t, l, s, g)
                    assert rec["umask"][s, g, :n_u].tolist() == [want[m] for m in sorted(want)]
        _print("worst", worst)
