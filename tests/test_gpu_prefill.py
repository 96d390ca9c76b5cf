"""GPU parity of the prefill path (sketch -> walk -> select -> attention)
against the oracle, stage by stage, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import dynamic_block_sparse_sws_amd as sws
import gen
import oracle as O
from gpu_util import PrefillRun, check_prefill_run, f64, TOL_ATTN_BF16

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def test_tiny_stack_fp32_all_layers():
    """The tiny configuration: 1 head, 4 layers, n=1024, d=64, B=64, k=16,
    20% density, fp32; every stage of every layer, every query block."""
    cfg = gen.CONFIGS["C1"]
    for n_dense in (0, 2):
        _print("tiny fp32 n_dense", n_dense)
        run = PrefillRun(cfg, cfg.seqlens, cfg.layers, cfg.rho, n_dense)
        w = check_prefill_run(run)
        _print("worst", w)


@pytest.mark.parametrize("d,B,seqlens,hq,hkv,rho", [
    (128, 64, (1000,), 8, 2, 20),
    (128, 128, (700, 129, 1), 4, 1, 30),
    (64, 64, (257, 64, 1500), 6, 3, 20),
    (64, 128, (1024,), 2, 2, 10),
    (128, 64, (900, 64, 3), 4, 4, 20),       # B = 64, one query head per KV head
    (128, 64, (1000, 300), 6, 2, 20),       # B = 64, groups of three: a lone head per group
])
def test_bf16_gqa_ragged(d, B, seqlens, hq, hkv, rho):
    cfg = gen.CONFIGS["C2"].with_(d=d, B=B, hq=hq, hkv=hkv, k=min(32, d))
    _print("bf16", d, B, seqlens, hq, hkv, rho)
    run = PrefillRun(cfg, seqlens, 3, rho, n_dense=1)
    w = check_prefill_run(run)
    _print("worst", w)


@pytest.mark.parametrize("d,B", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_fp32_path_ragged(d, B):
    cfg = gen.CONFIGS["C2"].with_(d=d, B=B, hq=4, hkv=2, k=16, dtype="f32")
    seqlens = (3 * B + 5, B - 3)
    _print("fp32", d, B, seqlens)
    run = PrefillRun(cfg, seqlens, 2, 25, n_dense=0)
    w = check_prefill_run(run)
    _print("worst", w)


@pytest.mark.parametrize("nseq,lo,hi", [(12, 65, 200), (70, 1, 140)])
def test_walk_ragged_tile_orders(nseq, lo, hi):
    """Ragged batches whose rows span several 64-row walk tiles: the
    longest-first tile order over 2 to 64 sequences (12 sequences here) and
    the plain order past 64 sequences (70) must compute every tile exactly
    once; every stage of two layers against the oracle."""
    rng = np.random.default_rng(100 + nseq)
    blocks = rng.integers(lo, hi + 1, size=nseq)
    seqlens = tuple(max(1, int(b) * 64 - int(rng.integers(0, 64))) for b in blocks)
    cfg = gen.CONFIGS["C2"].with_(hq=2, hkv=1, B=64, k=32)
    _print("ragged walk tiles", nseq, max(seqlens), min(seqlens))
    run = PrefillRun(cfg, seqlens, 2, 20, n_dense=0)
    w = check_prefill_run(run, attn_rows_per_head=3)
    _print("worst", w)


def test_dense_null_lists_equal_full_lists():
    """idx == NULL (dense causal) gives the same output as explicit full
    lists, and both match the oracle's dense attention."""
    cfg = gen.CONFIGS["C2"].with_(hq=4, hkv=2, B=64)
    run = PrefillRun(cfg, (777,), 1, 20, n_dense=1, dense_idx_null=True)
    check_prefill_run(run)
    run2 = PrefillRun(cfg, (777,), 1, 20, n_dense=1, dense_idx_null=False)
    assert np.array_equal(run.layers[0]["out"], run2.layers[0]["out"])


def test_bf16_dense_against_sdpa_fp32():
    """Full density equals causal softmax attention computed by torch in fp32
    on the CPU (a library routine, independent of the oracle)."""
    cfg = gen.CONFIGS["C2"].with_(hq=4, hkv=1, B=128)
    n = 640
    geo = sws.Geometry([n], cfg.B)
    q, k, v, _ = gen.layer_inputs(cfg, 0, device="cuda", seqlens=[n])
    out = sws.sparse_attn_prefill(q, k, v, geo, None, None)
    torch.cuda.synchronize()
    qf = q.float().cpu().permute(1, 0, 2)
    kf = k.float().cpu().permute(1, 0, 2).expand(cfg.hq, n, cfg.d).contiguous()
    vf = v.float().cpu().permute(1, 0, 2).expand(cfg.hq, n, cfg.d).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, is_causal=True)
    err = (out.float().cpu().permute(1, 0, 2) - ref).abs().max().item()
    _print("dense vs sdpa", err)
    assert err <= TOL_ATTN_BF16


def test_repeat_runs_bit_identical():
    cfg = gen.CONFIGS["C2"].with_(hq=8, hkv=2, B=64)
    a = PrefillRun(cfg, (900,), 2, 20, 0)
    b = PrefillRun(cfg, (900,), 2, 20, 0)
    for la, lb in zip(a.layers, b.layers):
        for key in ("q_sk", "k_sk", "R", "cnt", "out", "lse"):
            assert np.array_equal(la[key], lb[key]), key
        for h in range(cfg.hq):
            for x, y in zip(a.lists_of(la, 0, h), b.lists_of(lb, 0, h)):
                assert np.array_equal(x, y)


def test_error_codes_from_the_library():
    cfg = gen.CONFIGS["C2"].with_(hq=4, hkv=2)
    geo = sws.Geometry([256], 64)
    q, k, v, _ = gen.layer_inputs(cfg, 0, device="cuda", seqlens=[256])
    with pytest.raises(sws.SwsError) as ei:
        sws.sparse_attn_prefill(q.float()[:, :, :96].contiguous(), k.float()[:, :, :96].contiguous(),
                                v.float()[:, :, :96].contiguous(), geo, None, None)
    assert ei.value.code == 3
    with pytest.raises(sws.SwsError) as ei:
        sws.select_topk(torch.zeros(4 * 16, device="cuda"), 4, geo, 100, width=2)
    assert ei.value.code == 2


@pytest.mark.parametrize("s,kdim,B", [(1, 32, 64), (2, 32, 128), (4, 16, 64), (16, 32, 128),
                                      (8, 64, 64)])
def test_walk_degree_and_sketch_dim(s, kdim, B):
    """The parameter range the sweeps use (walk degree s, sketch dimension k,
    block size B): every stage of a two-layer ragged bf16 stack against the
    oracle, so the walk carried across layers is checked at each s."""
    cfg = gen.CONFIGS["C2"].with_(d=128, B=B, hq=4, hkv=2, k=kdim, s=s)
    _print("walk sweep", s, kdim, B)
    run = PrefillRun(cfg, (5 * B + 17, 3 * B), 2, 20, n_dense=0)
    w = check_prefill_run(run)
    _print("worst", w)


@pytest.mark.parametrize("row_tau,group", [(True, False), (False, True), (True, True)])
def test_selection_variants(row_tau, group):
    """The selection variants behind flags (per-row budget, one shared list per
    KV group) are bit-exact against the oracle on the GPU's own walk states,
    and the attention over the shared lists matches the oracle."""
    cfg = gen.CONFIGS["C2"].with_(d=128, B=64, hq=8, hkv=2, k=32)
    seqlens = (1500, 700)
    geo = sws.Geometry(list(seqlens), cfg.B)
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    sd, cd = torch.from_numpy(signs).cuda(), torch.from_numpy(cols).cuda()
    grp = cfg.hq // cfg.hkv
    rho = 25
    R = None
    for l in range(2):
        q, k, v, _ = gen.layer_inputs(cfg, l, device="cuda", seqlens=list(seqlens))
        q_sk = sws.sketch(q, geo, cfg.k, sd, cd)
        k_sk = sws.sketch(k, geo, cfg.k, sd, cd)
        R = sws.walk_update(q_sk, k_sk, geo, cfg.s, R, R_out=R)
        idx, cnt = sws.select_topk(R, cfg.hq, geo, rho, row_tau=row_tau,
                                   group_hkv=cfg.hkv if group else None)
        out = sws.sparse_attn_prefill(q, k, v, geo, idx, cnt)
        torch.cuda.synchronize()
        Rh, idx_h, cnt_h = R.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
        _print("variant", row_tau, group, "layer", l)
        for s in range(len(seqlens)):
            b = geo.blocks[s]
            b0 = int(geo.cu_blocks_host[s])
            off = geo.walk_offset(s, cfg.hq)
            Rs = [Rh[off + h * b * b: off + (h + 1) * b * b].reshape(b, b) for h in range(cfg.hq)]
            for h in range(cfg.hq):
                g = h // grp
                score = O.group_scores(Rs[g * grp:(g + 1) * grp]) if group else Rs[h]
                want = O.select_rows_tau(score, rho) if row_tau else O.select(score, rho)
                for i in range(b):
                    got = idx_h[h, b0 + i, :cnt_h[h, b0 + i]].tolist()
                    assert got == want[i].tolist(), (row_tau, group, l, s, h, i)
            # attention of sampled blocks over the variant's lists
            t0 = int(geo.cu_seqlens_host[s])
            ts = slice(t0, t0 + seqlens[s])
            for h in (0, cfg.hq - 1):
                g = h // grp
                lists = [idx_h[h, b0 + i, :cnt_h[h, b0 + i]].astype(np.int64) for i in range(b)]
                rows = [0, b // 2, b - 1]
                res = O.sparse_attention_rows(f64(q[ts, h]), f64(k[ts, g]), f64(v[ts, g]), lists,
                                              cfg.B, 1.0 / math.sqrt(cfg.d), rows)
                o = f64(out[ts, h])
                for i in rows:
                    ow, _ = res[i]
                    err = np.abs(o[i * cfg.B:i * cfg.B + ow.shape[0]] - ow).max()
                    assert err <= TOL_ATTN_BF16, (row_tau, group, l, s, h, i, err)


@pytest.mark.parametrize("mode,s,layers", [(sws.WALK_POWER, 8, 2), (sws.WALK_POWER, 3, 1),
                                           (sws.WALK_SOFTMAX, 8, 2), (sws.WALK_SOFTMAX, 1, 1)])
def test_walk_variants(mode, s, layers):
    """The walk variants (elementwise power, softmax transition probabilities)
    against the oracle on the GPU's own sketches and previous walk state,
    ragged batch with a partial and a one-token sequence, then selection on the
    variant's state is bit-exact."""
    cfg = gen.CONFIGS["C2"].with_(d=128, B=64, hq=4, hkv=2, k=32)
    seqlens = (700, 129, 1)
    geo = sws.Geometry(list(seqlens), cfg.B)
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    sd, cd = torch.from_numpy(signs).cuda(), torch.from_numpy(cols).cuda()
    grp = cfg.hq // cfg.hkv
    name = {sws.WALK_POWER: "power", sws.WALK_SOFTMAX: "softmax"}[mode]
    R = None
    for l in range(layers):
        q, k, v, _ = gen.layer_inputs(cfg, l, device="cuda", seqlens=list(seqlens))
        q_sk = sws.sketch(q, geo, cfg.k, sd, cd)
        k_sk = sws.sketch(k, geo, cfg.k, sd, cd)
        R_prev = None if R is None else R.clone()
        R = sws.walk_update_variant(q_sk, k_sk, geo, s, mode, R_prev)
        idx, cnt = sws.select_topk(R, cfg.hq, geo, 30)
        torch.cuda.synchronize()
        qs, ks, Rh = f64(q_sk), f64(k_sk), R.cpu().numpy()
        Rp = None if R_prev is None else R_prev.cpu().numpy()
        idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
        worst = 0.0
        for si in range(len(seqlens)):
            b = geo.blocks[si]
            bs = slice(int(geo.cu_blocks_host[si]), int(geo.cu_blocks_host[si]) + b)
            off = geo.walk_offset(si, cfg.hq)
            for h in range(cfg.hq):
                M = O.sketched_scores(qs[h, bs], ks[h // grp, bs])
                prev = None if Rp is None else np.tril(Rp[off + h * b * b: off + (h + 1) * b * b].reshape(b, b))
                want = O.walk_update_variant(prev, M, s, name)
                got = Rh[off + h * b * b: off + (h + 1) * b * b].reshape(b, b).astype(np.float64)
                e = float((np.abs(got - want).max(axis=1) / np.maximum(np.abs(want).max(axis=1), 1e-300)).max())
                worst = max(worst, e)
                assert e <= 1e-4, (name, s, l, si, h, e)
                lists = O.select(got, 30)
                for i in range(b):
                    assert idx_h[h, bs.start + i, :cnt_h[h, bs.start + i]].tolist() == lists[i].tolist()
        _print("walk variant", name, s, "layer", l, "worst", worst)
