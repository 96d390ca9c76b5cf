"""GPU parity through every layer of the full-size workloads, run the way the
bench runs them (same entry points and buffers, the walk state carried from
layer to layer on the GPU), against the oracle:

* 32K prefill: 32 query / 8 KV heads, d=128, B=64, k=32, 32 layers;
* 128K prefill: B=128 (1024 blocks), 32 layers, one sequence;
* ragged prefill: 8 sequences of 4096..65536 tokens, 40 query / 8 KV heads,
  40 layers;
* decode: 16 sequences with a 65536-token prefix, 32 layers, 256 steps,
  checked at steps 0, 1, 62, 63, 64, 127, 128 and 255 (blocks opening,
  filling and completing).

Every layer is checked stage by stage, the oracle fed the GPU's own upstream
outputs, so a mismatch names the stage (sketch and walk rows within 1e-4 of
the row's largest magnitude, selections bit-exact, bf16 attention within
2e-2):
* sketches of sampled query and key heads (rotating over the layers);
* walk rows of sampled heads (all rows of some, sampled rows of others);
* selections of every head on at least three layers, the last included
  (every layer for decode);
* attention of at least 64 query blocks (decode: every sequence) per
  (layer, head) for one head of each KV group on two sparse layers.

End to end (section 4 of the blog page: R^l = R^(l-1) (A^l)^s carried over
all s * L hops): for tracked rows of three or more heads, the oracle carries
its own fp64 walk from its own sketches of the raw Q and K through every
layer, never fed by the GPU; the GPU's walk rows must stay within 1e-4 of
that (the drift per layer is recorded), and its selections on those rows
must match, except where the fp64 scores of the tau-th and (tau+1)-th
candidates are closer than 1e-4 of the row's largest magnitude (a near-tie,
where fp32 may order them either way).  Both walks cut every hop's rows to
the walk state's dynamic range (entries below 2^-64 of the row maximum are
zero); the distance of the GPU's rows to the oracle's walk without that
floor is recorded too: it grows to order one over the deep layers, because
the unfloored walk depends on entries far below any fp32 range."""
import math

import numpy as np
import pytest
import torch

import dynamic_block_sparse_sws_amd as sws
import gen
import oracle as O
import parity_log as PL
from gpu_util import rowwise_rel_err, TOL_ATTN_BF16, TOL_SKETCH, TOL_WALK

pytestmark = pytest.mark.gpu

NEAR_TIE = 1e-4


def _print(*a):
    print(*a, flush=True)


def h64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def _tables(cfg):
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    return signs, cols, torch.from_numpy(signs).cuda(), torch.from_numpy(cols).cuda()


def near_tie(row: np.ndarray, i: int, tau: int) -> bool:
    """True when the tau-th and (tau+1)-th best earlier blocks of row i are
    closer than NEAR_TIE of the row's largest magnitude."""
    if i <= tau:
        return False
    v = np.sort(np.asarray(row[:i], np.float64))[::-1]
    top = np.abs(row).max()
    return bool(v[tau - 1] - v[tau] < NEAR_TIE * (top if top > 0 else 1.0)) if tau > 0 else False


def check_selection_e2e(label, lists_gpu, X, rows, tau, dense):
    """Selections from the oracle's own end-to-end walk rows against the
    GPU's lists; a difference must sit at a near-tie."""
    if dense:
        return 0, 0
    diff = ties = 0
    for r, i in enumerate(rows):
        want = O.select_row(X[r], int(i), tau)
        if lists_gpu[int(i)].tolist() != want.tolist():
            diff += 1
            assert near_tie(X[r], int(i), tau), (label, int(i), "selection differs, not a near-tie")
            ties += 1
    return diff, ties


def prefill_depth(cfg, label, *, sel_layers, attn_layers, track_heads, track_rows,
                  walk_heads_per_layer, walk_full_heads, walk_rows, sketch_q, sketch_k,
                  attn_blocks, seed):
    """Runs every layer of a prefill workload and checks it (see the module
    docstring).  Returns the per-layer end-to-end drift."""
    lens = list(cfg.seqlens)
    geo = sws.Geometry(lens, cfg.B)
    signs, cols, signs_d, cols_d = _tables(cfg)
    hq, hkv, grp = cfg.hq, cfg.hkv, cfg.hq // cfg.hkv
    scale = 1.0 / math.sqrt(cfg.d)
    n_layers = cfg.layers
    rng = np.random.default_rng(seed)
    R = torch.empty(geo.walk_numel(hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(sws.prefill_workspace_size(sws.BF16, geo.total_blocks, hkv, cfg.d, cfg.B),
                     dtype=torch.uint8, device="cuda")
    lse = torch.empty((hq, geo.total_tokens), dtype=torch.float32, device="cuda")
    seqs = range(len(lens))
    tok = [slice(int(geo.cu_seqlens_host[s]), int(geo.cu_seqlens_host[s]) + lens[s]) for s in seqs]
    blk = [slice(int(geo.cu_blocks_host[s]), int(geo.cu_blocks_host[s]) + geo.blocks[s])
           for s in seqs]
    woff = [geo.walk_offset(s, hq) for s in seqs]
    # tracked rows of each sequence (first, last and sampled) for the
    # end-to-end walk; the oracle's own rows per (sequence, tracked head)
    trows = [np.unique(np.concatenate([[0, geo.blocks[s] - 1],
                                        rng.choice(geo.blocks[s], size=min(geo.blocks[s],
                                                                           track_rows),
                                                   replace=False)])) for s in seqs]
    X = {}
    X0 = {}          # the same chain without the walk floor (reported only)
    R_prev = None
    drift = []
    sel_diff = sel_ties = sel_rows_total = 0
    for l in range(n_layers):
        dense = l < cfg.n_dense
        q, k, v, _ = gen.layer_inputs(cfg, l, device="cuda")
        q_sk = sws.sketch(q, geo, cfg.k, signs_d, cols_d)
        k_sk = sws.sketch(k, geo, cfg.k, signs_d, cols_d)
        sws.walk_update(q_sk, k_sk, geo, cfg.s, None if l == 0 else R, R_out=R)
        idx, cnt = sws.select_topk(R, hq, geo, cfg.rho, dense=dense)
        out = sws.sparse_attn_prefill(q, k, v, geo, idx, cnt, lse=lse, ws=ws)
        torch.cuda.synchronize()
        qs_g, ks_g = h64(q_sk), h64(k_sk)
        Rh = R.cpu().numpy()
        idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
        qheads = sorted(set((l * 7 + j * 11) % hq for j in range(sketch_q)) | set(track_heads))
        kheads = sorted(set((l * 3 + j * 5) % hkv for j in range(sketch_k))
                        | {h // grp for h in track_heads})
        Qh = {h: h64(q[:, h]) for h in qheads}
        Kh = {g: h64(k[:, g]) for g in kheads}

        def R_of(arr, s, h):
            b = geo.blocks[s]
            o = woff[s] + h * b * b
            return arr[o:o + b * b].reshape(b, b)

        def lists_of(s, h):
            b0 = blk[s].start
            return [idx_h[h, b0 + i, :cnt_h[h, b0 + i]].astype(np.int64)
                    for i in range(geo.blocks[s])]

        worst = {"sketch": 0.0, "walk": 0.0, "attn": 0.0, "lse": 0.0}
        o_sk = {}
        for s in seqs:
            # sketches of the sampled heads, and the oracle's own sketches
            for h in qheads:
                want = O.sketch(Qh[h][tok[s]], cfg.B, signs, cols)
                o_sk[("q", s, h)] = want
                e = rowwise_rel_err(qs_g[h, blk[s]], want)
                worst["sketch"] = max(worst["sketch"], e)
                assert e <= TOL_SKETCH, (label, l, s, h, "q sketch", e)
            for g in kheads:
                want = O.sketch(Kh[g][tok[s]], cfg.B, signs, cols)
                o_sk[("k", s, g)] = want
                e = rowwise_rel_err(ks_g[g, blk[s]], want)
                worst["sketch"] = max(worst["sketch"], e)
                assert e <= TOL_SKETCH, (label, l, s, g, "k sketch", e)
        # walk, stage-wise: the GPU's sketches and previous state
        whs = sorted(set((l * walk_heads_per_layer + j) % hq for j in range(walk_heads_per_layer)))
        full = set(whs[(l * 3 + j) % len(whs)] for j in range(walk_full_heads))
        for h in whs:
            g = h // grp
            for s in seqs:
                b = geo.blocks[s]
                M = O.sketched_scores(qs_g[h, blk[s]], ks_g[g, blk[s]])
                rows = (np.arange(b) if h in full else
                        np.unique(np.concatenate([[0, b - 1],
                                                  rng.choice(b, size=min(b, walk_rows),
                                                             replace=False)])))
                start = (np.eye(b)[rows] if R_prev is None
                         else np.tril(R_of(R_prev, s, h))[rows].astype(np.float64))
                want = O.walk_update(start, M, cfg.s)
                Rg = R_of(Rh, s, h)[rows].astype(np.float64)
                e = rowwise_rel_err(Rg, want)
                worst["walk"] = max(worst["walk"], e)
                assert e <= TOL_WALK, (label, l, s, h, "walk", e)
                upper = np.arange(b)[None, :] > rows[:, None]
                assert np.all(Rg[upper] == 0), (label, l, s, h, "walk above the diagonal")
        # selection, bit-exact on the GPU's fp32 walk state
        sel_heads = range(hq) if l in sel_layers else [(l * 9) % hq, (l * 9 + 17) % hq]
        nsel = 0
        for h in sel_heads:
            for s in seqs:
                b = geo.blocks[s]
                tau = O.n_select(cfg.rho, b)
                Rs = R_of(Rh, s, h)
                got = lists_of(s, h)
                for i in range(b):
                    want = np.arange(i + 1) if dense else O.select_row(Rs[i], i, tau)
                    assert got[i].tolist() == want.tolist(), (label, l, s, h, i)
                nsel += b
        PL.note_count(label, "selection_rows_bit_exact", nsel)
        # attention on sampled query blocks, one head per KV group
        if l in attn_layers:
            for g in range(hkv):
                h = g * grp + (l + g) % grp
                Qa = h64(q[:, h])
                Ka, Va = h64(k[:, g]), h64(v[:, g])
                per_seq = max(1, -(-attn_blocks // len(lens)))
                for s in seqs:
                    b = geo.blocks[s]
                    blocks = sorted(set([0, b - 1] + rng.choice(b, size=min(b, per_seq),
                                                                replace=False).tolist()))
                    res = O.sparse_attention_rows(Qa[tok[s]], Ka[tok[s]], Va[tok[s]],
                                                  lists_of(s, h), cfg.B, scale, blocks)
                    for i in blocks:
                        o_want, lse_want = res[i]
                        a = tok[s].start + i * cfg.B
                        o_got = h64(out[a:a + o_want.shape[0], h])
                        lse_got = h64(lse[h, a:a + o_want.shape[0]])
                        e = float(np.abs(o_got - o_want).max())
                        e2 = float(np.abs(lse_got - lse_want).max())
                        worst["attn"] = max(worst["attn"], e)
                        worst["lse"] = max(worst["lse"], e2)
                        assert e <= TOL_ATTN_BF16, (label, l, s, h, i, "attn", e)
                        assert e2 <= TOL_ATTN_BF16, (label, l, s, h, i, "lse", e2)
                    PL.note_count(label, "attention_blocks_checked", len(blocks))
        # end to end: the oracle's own fp64 walk from its own sketches
        e_l = e_l0 = 0.0
        for h in track_heads:
            g = h // grp
            for s in seqs:
                b = geo.blocks[s]
                rows = trows[s]
                M = O.sketched_scores(o_sk[("q", s, h)], o_sk[("k", s, g)])
                start = np.eye(b)[rows] if l == 0 else X[(s, h)]
                X[(s, h)] = O.walk_update(start, M, cfg.s)
                X0[(s, h)] = O.walk_update(np.eye(b)[rows] if l == 0 else X0[(s, h)], M, cfg.s,
                                           floor=0.0)
                Rg = R_of(Rh, s, h)[rows].astype(np.float64)
                e_l = max(e_l, rowwise_rel_err(Rg, X[(s, h)]))
                e_l0 = max(e_l0, rowwise_rel_err(Rg, X0[(s, h)]))
                d_, t_ = check_selection_e2e((label, l, s, h), lists_of(s, h), X[(s, h)], rows,
                                             O.n_select(cfg.rho, b), dense)
                sel_diff += d_
                sel_ties += t_
                sel_rows_total += 0 if dense else len(rows)
        drift.append(e_l)
        PL.note_series(label, "walk_drift_end_to_end_by_layer", l, e_l)
        PL.note_series(label, "walk_distance_to_unfloored_fp64_by_layer", l, e_l0)
        for key, bar in (("sketch", TOL_SKETCH), ("walk", TOL_WALK), ("attn", TOL_ATTN_BF16),
                         ("lse", TOL_ATTN_BF16)):
            PL.note(label, key, worst[key], bar)
        _print(f"{label} layer {l}{' dense' if dense else ''}: worst {worst}, "
               f"end-to-end drift {e_l:.3g} (to the unfloored walk {e_l0:.3g})")
        assert e_l <= TOL_WALK, (label, l, "end-to-end walk drift", e_l)
        R_prev = Rh
        del q, k, v, q_sk, k_sk, idx, cnt, out
    PL.note(label, "walk_drift_end_to_end", max(drift), TOL_WALK)
    PL.note_count(label, "e2e_selection_rows", sel_rows_total)
    PL.note_count(label, "e2e_selection_rows_differing_at_near_ties", sel_ties)
    _print(f"{label}: end-to-end selections on {sel_rows_total} tracked rows, "
           f"{sel_diff} differ (all at near-ties)")
    torch.cuda.empty_cache()
    return drift


def test_prefill_32k_all_layers():
    cfg = gen.CONFIGS["C2"]
    prefill_depth(cfg, "C2 32K prefill", sel_layers={0, 2, 16, 31}, attn_layers={2, 31},
                  track_heads=(0, 13, 31), track_rows=64, walk_heads_per_layer=32,
                  walk_full_heads=2, walk_rows=16, sketch_q=4, sketch_k=2, attn_blocks=64,
                  seed=2)


def test_prefill_128k_all_layers():
    cfg = gen.CONFIGS["C3"]
    prefill_depth(cfg, "C3 128K prefill", sel_layers={2, 16, 31}, attn_layers={2, 31},
                  track_heads=(0, 13, 31), track_rows=48, walk_heads_per_layer=16,
                  walk_full_heads=1, walk_rows=8, sketch_q=3, sketch_k=2, attn_blocks=64,
                  seed=3)


def test_prefill_ragged_all_layers():
    cfg = gen.CONFIGS["C5"]
    prefill_depth(cfg, "C5 ragged prefill", sel_layers={0, 2, 20, 39}, attn_layers={2, 39},
                  track_heads=(0, 21, 39), track_rows=16, walk_heads_per_layer=10,
                  walk_full_heads=1, walk_rows=8, sketch_q=3, sketch_k=2, attn_blocks=64,
                  seed=5)


def test_decode_all_layers_and_steps():
    """16 sequences, 65536-token prefix, 32 layers (two dense), 256 steps run
    in order with the bench's buffers (head-major caches, the fused q/k
    append, the walk row carried through the layers in one buffer)."""
    cfg = gen.CONFIGS["C4"]
    label = "C4 decode"
    ns, P, steps, n_layers = cfg.decode_batch, cfg.decode_prefix, cfg.decode_steps, cfg.layers
    hq, hkv, d, B, kd = cfg.hq, cfg.hkv, cfg.d, cfg.B, cfg.k
    grp = hq // hkv
    max_ctx = P + steps
    b_max = -(-max_ctx // B)
    check_steps = (0, 1, 62, 63, 64, 127, 128, 255)
    # (sequence, query head) pairs: sketches, stage-wise walk and the
    # end-to-end walk at every layer
    track = ((0, 0), (5, 13), (10, 22), (15, 31))
    attn_layers = (2, n_layers - 1)
    scale = 1.0 / math.sqrt(d)
    signs, cols, signs_d, cols_d = _tables(cfg)
    geo_p = sws.Geometry([P], B)
    layers = []
    o_pre = {}       # oracle sketches of the prefix: (layer, "q"/"k", seq, head) -> [P/B, k]
    for l in range(n_layers):
        qpre, qst, kc, vc = gen.decode_layer_inputs(cfg, l, device="cuda", n_seqs=ns, prefix=P,
                                                    steps=steps)
        qsk = torch.zeros((ns, hq, b_max, kd), dtype=torch.float32, device="cuda")
        ksk = torch.zeros((ns, hkv, b_max, kd), dtype=torch.float32, device="cuda")
        rq = torch.zeros((ns, hq, d), dtype=torch.float32, device="cuda")
        rk = torch.zeros((ns, hkv, d), dtype=torch.float32, device="cuda")
        sq = torch.empty((hq, geo_p.total_blocks, d), dtype=torch.float32, device="cuda")
        sk = torch.empty((hkv, geo_p.total_blocks, d), dtype=torch.float32, device="cuda")
        for s in range(ns):
            sws.sketch(qpre[s], geo_p, kd, signs_d, cols_d, out=qsk[s], ld_head=b_max * kd,
                       sum_out=sq)
            sws.sketch(kc[s, :P], geo_p, kd, signs_d, cols_d, out=ksk[s], ld_head=b_max * kd,
                       sum_out=sk)
            rq[s] = sq[:, -1]
            rk[s] = sk[:, -1]
        torch.cuda.synchronize()
        for s, h in track:
            g = h // grp
            o_pre[(l, "q", s, h)] = O.sketch(h64(qpre[s, :, h]), B, signs, cols)
            o_pre[(l, "k", s, g)] = O.sketch(h64(kc[s, :P, g]), B, signs, cols)
            for key, got in ((("q", s, h), qsk[s, h, :P // B]), (("k", s, g), ksk[s, g, :P // B])):
                e = rowwise_rel_err(h64(got), o_pre[(l,) + key])
                PL.note(label, "sketch_prefix", e, TOL_SKETCH)
                assert e <= TOL_SKETCH, (l, key, "prefix sketch", e)
        del qpre, sq, sk
        host = {"qst": qst.float().cpu(), "knew": kc[:, P:].float().cpu()}
        if l in attn_layers:
            host["k"] = kc.float().cpu().numpy()
            host["v"] = vc.float().cpu().numpy()
        knew = kc[:, P:].permute(1, 0, 2, 3).contiguous()       # [steps, ns, hkv, d]
        kc_hm = kc.permute(0, 2, 1, 3).contiguous()              # [ns, hkv, ctx, d]
        vc_hm = vc.permute(0, 2, 1, 3).contiguous()
        del kc, vc
        layers.append({"qst": qst, "knew": knew, "kc": kc_hm, "vc": vc_hm, "qsk": qsk,
                       "ksk": ksk, "rq": rq, "rk": rk, "host": host,
                       "out": torch.empty((ns, hq, d), dtype=qst.dtype, device="cuda")})
    torch.cuda.synchronize()
    _print("decode set-up done")
    pos_all = torch.arange(P, P + steps, dtype=torch.int32, device="cuda")[:, None].expand(
        steps, ns).contiguous()
    cur_all = (pos_all // B).contiguous()
    ctx_all = (pos_all + 1).contiguous()
    ws = torch.empty(sws.decode_workspace_size(ns, hq, hkv, d, B, b_max), dtype=torch.uint8,
                     device="cuda")
    r = torch.empty((ns, hq, b_max), dtype=torch.float32, device="cuda")
    lse = torch.empty((ns, hq), dtype=torch.float32, device="cuda")
    sel_rows = ties_total = diff_total = e2e_rows = 0
    for t in range(steps):
        checked = t in check_steps
        recs = []
        for l, L in enumerate(layers):
            dense = l < cfg.n_dense
            sws.sketch_append_qk(L["qst"][t], L["knew"][t], pos_all[t], B, kd, signs_d, cols_d,
                                 L["rq"], L["rk"], L["qsk"], L["ksk"])
            sws.walk_update_row(L["qsk"], L["ksk"], cur_all[t], cfg.s, None if l == 0 else r, r)
            uidx, ucnt, umask, idx, cnt = sws.select_topk_row(r, hq, hkv, cur_all[t], b_max,
                                                              cfg.rho, dense=dense,
                                                              per_head=checked)
            sws.sparse_attn_decode(L["qst"][t], L["kc"], L["vc"], ctx_all[t], B, uidx, ucnt,
                                   umask, out=L["out"], lse=lse if checked else None, ws=ws,
                                   head_major=True)
            if checked:
                torch.cuda.synchronize()
                recs.append({
                    "r": r.cpu().numpy(), "idx": idx.cpu().numpy(), "cnt": cnt.cpu().numpy(),
                    "uidx": uidx.cpu().numpy(), "ucnt": ucnt.cpu().numpy(),
                    "umask": umask.cpu().numpy().astype(np.uint32),
                    "out": h64(L["out"]), "lse": h64(lse),
                    "qsk": {(s, h): h64(L["qsk"][s, h]) for s, h in track},
                    "ksk": {(s, h // grp): h64(L["ksk"][s, h // grp]) for s, h in track}})
        if not checked:
            continue
        p = P + t
        c = p // B
        tau = O.n_select(cfg.rho, c + 1)
        worst = {"sketch": 0.0, "walk": 0.0, "attn": 0.0, "lse": 0.0, "drift": 0.0,
                 "unfloored": 0.0}
        x_e2e = {}
        x_e2e0 = {}
        for l, (L, rec) in enumerate(zip(layers, recs)):
            dense = l < cfg.n_dense
            H = L["host"]
            # sketches of the tracked pairs: the prefix rows stay, the rows
            # of the blocks opened by the steps follow the new tokens
            for s, h in track:
                g = h // grp
                o_q = np.concatenate([o_pre[(l, "q", s, h)],
                                      O.sketch(H["qst"][:t + 1, s, h].double().numpy(), B,
                                               signs, cols)])
                o_k = np.concatenate([o_pre[(l, "k", s, g)],
                                      O.sketch(H["knew"][s, :t + 1, g].double().numpy(), B,
                                               signs, cols)])
                g_q, g_k = rec["qsk"][(s, h)][:c + 1], rec["ksk"][(s, g)][:c + 1]
                e = max(rowwise_rel_err(g_q, o_q), rowwise_rel_err(g_k, o_k))
                worst["sketch"] = max(worst["sketch"], e)
                assert e <= TOL_SKETCH, (t, l, s, h, "sketch", e)
                # walk row, stage-wise (GPU sketches and previous row)
                M = O.sketched_scores(g_q, g_k)
                rp = None if l == 0 else recs[l - 1]["r"][s, h, :c + 1]
                want = O.walk_row(rp, M, c, cfg.s)
                rg = rec["r"][s, h]
                e = rowwise_rel_err(rg[:c + 1], want)
                worst["walk"] = max(worst["walk"], e)
                assert e <= TOL_WALK, (t, l, s, h, "walk", e)
                assert np.all(rg[c + 1:] == 0), (t, l, s, h, "walk past the open block")
                # end to end: the oracle's own walk row from its own sketches
                Mo = O.sketched_scores(o_q, o_k)
                x = O.walk_row(None if l == 0 else x_e2e[(s, h)], Mo, c, cfg.s)
                x_e2e[(s, h)] = x
                e = rowwise_rel_err(rg[:c + 1], x)
                worst["drift"] = max(worst["drift"], e)
                x_e2e0[(s, h)] = O.walk_row(None if l == 0 else x_e2e0[(s, h)], Mo, c, cfg.s,
                                            floor=0.0)
                worst["unfloored"] = max(worst["unfloored"],
                                         rowwise_rel_err(rg[:c + 1], x_e2e0[(s, h)]))
                if not dense:
                    e2e_rows += 1
                    got = rec["idx"][s, h, :rec["cnt"][s, h]]
                    if got.tolist() != O.select_row(x, c, tau).tolist():
                        diff_total += 1
                        assert near_tie(x, c, tau), (t, l, s, h, "e2e selection, not a near-tie")
                        ties_total += 1
            PL.note_series(label, "walk_drift_end_to_end_by_step_layer", [t, l], worst["drift"])
            PL.note_series(label, "walk_distance_to_unfloored_fp64_by_step_layer", [t, l],
                           worst["unfloored"])
            # selection of every head of every sequence, bit-exact on the
            # GPU's fp32 walk row, and the group unions and head masks
            for s in range(ns):
                for h in range(hq):
                    want = (np.arange(c + 1) if dense
                            else O.select_row(rec["r"][s, h], c, tau))
                    got = rec["idx"][s, h, :rec["cnt"][s, h]]
                    assert got.tolist() == want.tolist(), (t, l, s, h, "selection")
                    sel_rows += 1
                for g in range(hkv):
                    heads = range(g * grp, (g + 1) * grp)
                    lists = [rec["idx"][s, h, :rec["cnt"][s, h]] for h in heads]
                    union = np.unique(np.concatenate(lists))
                    n_u = rec["ucnt"][s, g]
                    assert rec["uidx"][s, g, :n_u].tolist() == union.tolist(), (t, l, s, g)
                    mask = np.zeros(len(union), np.uint32)
                    for j, lst in enumerate(lists):
                        mask |= np.isin(union, lst).astype(np.uint32) << np.uint32(j)
                    assert rec["umask"][s, g, :n_u].tolist() == mask.tolist(), (t, l, s, g)
            # attention of one head per KV group for every sequence
            if l in attn_layers:
                for s in range(ns):
                    for g in range(hkv):
                        h = g * grp + (s + t + g) % grp
                        lst = rec["idx"][s, h, :rec["cnt"][s, h]]
                        o_w, lse_w = O.query_attention(H["qst"][t, s, h].double().numpy(),
                                                       H["k"][s, :, g], H["v"][s, :, g], lst,
                                                       B, p, scale)
                        e = float(np.abs(rec["out"][s, h] - o_w).max())
                        e2 = abs(float(rec["lse"][s, h]) - lse_w)
                        worst["attn"] = max(worst["attn"], e)
                        worst["lse"] = max(worst["lse"], e2)
                        assert e <= TOL_ATTN_BF16, (t, l, s, h, "attn", e)
                        assert e2 <= TOL_ATTN_BF16, (t, l, s, h, "lse", e2)
                PL.note_count(label, "attention_queries_checked", ns * hkv)
        for key, bar in (("sketch", TOL_SKETCH), ("walk", TOL_WALK), ("attn", TOL_ATTN_BF16),
                         ("lse", TOL_ATTN_BF16)):
            PL.note(label, key, worst[key], bar)
        PL.note(label, "walk_drift_end_to_end", worst["drift"], TOL_WALK)
        _print(f"{label} step {t}: worst {worst}")
        assert worst["drift"] <= TOL_WALK, (t, "end-to-end walk drift", worst["drift"])
    PL.note_count(label, "selection_rows_bit_exact", sel_rows)
    PL.note_count(label, "e2e_selection_rows", e2e_rows)
    PL.note_count(label, "e2e_selection_rows_differing_at_near_ties", ties_total)
    _print(f"{label}: {sel_rows} selections bit-exact; end-to-end selections on {e2e_rows} "
           f"tracked rows, {diff_total} differ (all at near-ties)")
