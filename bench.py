#!/usr/bin/env python3
"""Throughput of the Sketch&Walk hot path on one MI355X.

Step = one sparse layer of the 128K-token prefill (32 query / 8 KV heads,
d=128, B=128, k=32, s=8, 20% density): sketch Q, sketch K, walk update, top-tau
selection, block-sparse attention, on inputs already resident in HBM.  The
JSON line reports dense-equivalent TFLOP/s (4 d Hq n(n+1)/2 per layer divided
by the layer time), ms per layer, the per-stage split, the roofline of the
attention kernel against its target, the density sweep (10/30/100%) with the
speed-up over our own 100% run, the 16 x 64K decode step (32 layers, first
two dense, all 256 steps) with the decode attention's HBM roofline, the 32K
and ragged prefill workloads, the tiny stack's latency, and the CPU oracle
timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "128K prefill ms/layer + dense-equiv TFLOP/s at 20% density; decode µs/step"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
# the two roofline targets: prefill attention at >= 50% of the bf16 matrix
# peak on executed FLOPs, sparse decode attention at >= 70% of HBM bandwidth
TARGET_PREFILL_MFMA_FRAC = 0.50
TARGET_DECODE_HBM_FRAC = 0.70


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--rho", type=int, default=20)
    ap.add_argument("--distinct-layers", type=int, default=4)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--decode-layers", type=int, default=32)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--microbatches", type=int, default=2,
                    help="decode graph: the batch as this many micro-batches on as many streams")
    ap.add_argument("--kv-layout", choices=("head", "token"), default="head",
                    help="decode KV cache layout: [seq][kv head][ctx][d] (head) or "
                         "[seq][ctx][kv head][d] (token)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense-ref", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the decode steps replayed as HIP graphs")
    ap.add_argument("--no-serving", action="store_true",
                    help="skip the paged / fp8 KV decode-attention timings")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 128K density sweep (rho = 10, 30, 100)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the 32K, ragged and tiny prefill workloads")
    ap.add_argument("--diag", action="store_true",
                    help="parameter sweep (s, k, B, rho) and selection-quality diagnostics")
    ap.add_argument("--seqlen", type=int, default=None, help="override n (testing only)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def src_hash(name):
    """sha256 prefix of a kernel source's code: comments and whitespace are
    removed first, so a comment edit does not invalidate counters taken on
    the same code."""
    with open(os.path.join(ROOT, "dynamic_block_sparse_sws_amd", "csrc", name)) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_for(kernel_src, launch_bytes_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    ent = t.get(launch_bytes_key)
    if not ent or ent.get("src_sha256_16") != src_hash(kernel_src):
        return None
    return ent.get("hbm_bytes_per_launch")


class Timer:
    """HIP events on the current stream (the one the library launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.acc = {}
        self.n = {}

    def ev(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def add(self, name, e0, e1):
        self.acc.setdefault(name, []).append((e0, e1))

    def ms(self, name):
        pairs = self.acc.get(name, [])
        return sum(a.elapsed_time(b) for a, b in pairs) / max(1, len(pairs))


def bench_prefill(args, torch, sws, gen, timer_cls):
    cfg = gen.CONFIGS["C3"]
    n = args.seqlen or cfg.seqlens[0]
    geo = sws.Geometry([n], cfg.B)
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    signs_d = torch.from_numpy(signs).cuda()
    cols_d = torch.from_numpy(cols).cuda()
    L = max(1, args.distinct_layers)
    layers = []
    for l in range(L):
        q, k, v, _ = gen.layer_inputs(cfg, 2 + l, device="cuda", seqlens=[n])
        layers.append((q, k, v))
    hq, hkv, d, B = cfg.hq, cfg.hkv, cfg.d, cfg.B
    width = sws.select_width(args.rho, geo.max_blocks)
    bufs = {
        "q_sk": torch.empty((hq, geo.total_blocks, cfg.k), dtype=torch.float32, device="cuda"),
        "k_sk": torch.empty((hkv, geo.total_blocks, cfg.k), dtype=torch.float32, device="cuda"),
        "idx": torch.empty((hq, geo.total_blocks, width), dtype=torch.int32, device="cuda"),
        "cnt": torch.empty((hq, geo.total_blocks), dtype=torch.int32, device="cuda"),
        "out": torch.empty_like(layers[0][0]),
        "ws": torch.empty(sws.prefill_workspace_size(sws.BF16, geo.total_blocks, hkv, d, B),
                          dtype=torch.uint8, device="cuda"),
    }
    R = torch.empty(geo.walk_numel(hq), dtype=torch.float32, device="cuda")

    def step(l, first, T=None):
        q, k, v = layers[l % L]
        ev = [T.ev()] if T else None
        sws.sketch(q, geo, cfg.k, signs_d, cols_d, out=bufs["q_sk"])
        sws.sketch(k, geo, cfg.k, signs_d, cols_d, out=bufs["k_sk"])
        if T: ev.append(T.ev())
        sws.walk_update(bufs["q_sk"], bufs["k_sk"], geo, cfg.s, None if first else R, R_out=R)
        if T: ev.append(T.ev())
        sws.select_topk(R, hq, geo, args.rho, idx=bufs["idx"], cnt=bufs["cnt"])
        if T: ev.append(T.ev())
        sws.sparse_attn_prefill(q, k, v, geo, bufs["idx"], bufs["cnt"], out=bufs["out"], ws=bufs["ws"])
        if T:
            ev.append(T.ev())
            for name, a, b in zip(("sketch", "walk", "select", "attention"), ev[:-1], ev[1:]):
                T.add(name, a, b)
            T.add("layer", ev[0], ev[-1])

    for w in range(args.warmup):
        step(w, w == 0)
    torch.cuda.synchronize()
    T = timer_cls(torch)
    t0 = time.perf_counter()
    e_start = T.ev()
    for s in range(args.steps):
        step(s, False, T)
    e_end = T.ev()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e_start.elapsed_time(e_end)
    ms_layer = total_ms / args.steps
    cnt = bufs["cnt"].long()
    pairs = int(cnt.sum().item())
    flops_exec = 4.0 * B * B * d * pairs
    dense_flops = 4.0 * d * hq * n * (n + 1) / 2.0
    attn_ms = T.ms("attention")
    causal_pairs = hq * geo.max_blocks * (geo.max_blocks + 1) // 2
    res = {
        "n": n, "ms_per_layer": ms_layer, "wall_s": wall,
        "stage_us": {k_: T.ms(k_) * 1e3 for k_ in ("sketch", "walk", "select", "attention")},
        "dense_equiv_tflops": dense_flops / (ms_layer * 1e-3) / 1e12,
        "attn_exec_tflops": flops_exec / (attn_ms * 1e-3) / 1e12,
        "executed_block_pairs": pairs, "executed_causal_density": pairs / causal_pairs,
        "attn_flops_per_launch": flops_exec, "attn_ms": attn_ms,
        "sketch_hbm_gbs": (2.0 * (hq + hkv) * d * n) / (T.ms("sketch") * 1e-3) / 1e9,
    }
    # our own dense attention at full density (the speed-up denominator)
    if not args.no_dense_ref:
        Td = timer_cls(torch)
        q, k, v = layers[0]
        sws.sparse_attn_prefill(q, k, v, geo, None, None, out=bufs["out"], ws=bufs["ws"])
        for _ in range(2):
            a = Td.ev()
            sws.sparse_attn_prefill(q, k, v, geo, None, None, out=bufs["out"], ws=bufs["ws"])
            Td.add("dense", a, Td.ev())
        torch.cuda.synchronize()
        dms = Td.ms("dense")
        res["dense_attn_ms"] = dms
        res["dense_attn_tflops"] = dense_flops / (dms * 1e-3) / 1e12
        res["speedup_attn_vs_dense"] = dms / attn_ms
        res["speedup_layer_vs_dense_attn"] = dms / ms_layer
    if not args.no_sweep:
        sweep = {}
        for rho in (10, 30, 100):
            w2 = sws.select_width(rho, geo.max_blocks)
            idx2 = torch.empty((hq, geo.total_blocks, w2), dtype=torch.int32, device="cuda")
            cnt2 = torch.empty((hq, geo.total_blocks), dtype=torch.int32, device="cuda")
            Ts = timer_cls(torch)
            q, k, v = layers[0]
            for it in range(3):
                a = Ts.ev()
                sws.sketch(q, geo, cfg.k, signs_d, cols_d, out=bufs["q_sk"])
                sws.sketch(k, geo, cfg.k, signs_d, cols_d, out=bufs["k_sk"])
                sws.walk_update(bufs["q_sk"], bufs["k_sk"], geo, cfg.s, R, R_out=R)
                sws.select_topk(R, hq, geo, rho, idx=idx2, cnt=cnt2)
                b_ = Ts.ev()
                sws.sparse_attn_prefill(q, k, v, geo, idx2, cnt2, out=bufs["out"], ws=bufs["ws"])
                c_ = Ts.ev()
                if it > 0:
                    Ts.add("layer", a, c_)
                    Ts.add("attention", b_, c_)
            torch.cuda.synchronize()
            p2 = int(cnt2.long().sum().item())
            sweep[str(rho)] = {"ms_per_layer": Ts.ms("layer"), "attn_ms": Ts.ms("attention"),
                               "attn_exec_tflops": 4.0 * B * B * d * p2 / (Ts.ms("attention") * 1e-3) / 1e12,
                               "dense_equiv_tflops": dense_flops / (Ts.ms("layer") * 1e-3) / 1e12,
                               "executed_causal_density": p2 / causal_pairs}
        sweep["20"] = {"ms_per_layer": ms_layer, "attn_ms": attn_ms,
                       "attn_exec_tflops": res["attn_exec_tflops"],
                       "dense_equiv_tflops": res["dense_equiv_tflops"],
                       "executed_causal_density": pairs / causal_pairs}
        full = sweep["100"]
        for rho_, ent in sweep.items():
            ent["speedup_layer_vs_rho100"] = full["ms_per_layer"] / ent["ms_per_layer"]
            ent["speedup_attn_vs_rho100"] = full["attn_ms"] / ent["attn_ms"]
        res["rho_sweep"] = {k_: sweep[k_] for k_ in ("10", "20", "30", "100")}
    ctx = {"cfg": cfg, "geo": geo, "layers": layers, "bufs": bufs, "signs": signs, "cols": cols}
    return res, ctx


def bench_prefill_workload(torch, sws, gen, timer_cls, name, steps=8, warmup=2, distinct=4):
    """ms per sparse layer (sketch Q and K, walk, select, attention) of the
    32K ("C2") or ragged 8-sequence ("C5") prefill workload, cycling over
    `distinct` generated layers with inputs resident in HBM, the walk state
    carried from step to step, timed with HIP events after `warmup` steps."""
    cfg = gen.CONFIGS[name]
    geo = sws.Geometry(list(cfg.seqlens), cfg.B)
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    signs_d, cols_d = torch.from_numpy(signs).cuda(), torch.from_numpy(cols).cuda()
    layers = [gen.layer_inputs(cfg, cfg.n_dense + l, device="cuda")[:3] for l in range(distinct)]
    hq, hkv, d, B = cfg.hq, cfg.hkv, cfg.d, cfg.B
    width = sws.select_width(cfg.rho, geo.max_blocks)
    q_sk = torch.empty((hq, geo.total_blocks, cfg.k), dtype=torch.float32, device="cuda")
    k_sk = torch.empty((hkv, geo.total_blocks, cfg.k), dtype=torch.float32, device="cuda")
    idx = torch.empty((hq, geo.total_blocks, width), dtype=torch.int32, device="cuda")
    cnt = torch.empty((hq, geo.total_blocks), dtype=torch.int32, device="cuda")
    out = torch.empty_like(layers[0][0])
    ws = torch.empty(sws.prefill_workspace_size(sws.BF16, geo.total_blocks, hkv, d, B),
                     dtype=torch.uint8, device="cuda")
    R = torch.empty(geo.walk_numel(hq), dtype=torch.float32, device="cuda")
    T = timer_cls(torch)

    def step(i, first, timed):
        q, k, v = layers[i % distinct]
        ev = [T.ev()] if timed else None
        sws.sketch(q, geo, cfg.k, signs_d, cols_d, out=q_sk)
        sws.sketch(k, geo, cfg.k, signs_d, cols_d, out=k_sk)
        sws.walk_update(q_sk, k_sk, geo, cfg.s, None if first else R, R_out=R)
        sws.select_topk(R, hq, geo, cfg.rho, idx=idx, cnt=cnt)
        if timed: ev.append(T.ev())
        sws.sparse_attn_prefill(q, k, v, geo, idx, cnt, out=out, ws=ws)
        if timed:
            ev.append(T.ev())
            T.add("layer", ev[0], ev[2])
            T.add("select_chain", ev[0], ev[1])
            T.add("attention", ev[1], ev[2])

    for i in range(warmup):
        step(i, i == 0, False)
    for i in range(steps):
        step(warmup + i, False, True)
    torch.cuda.synchronize()
    pairs = int(cnt.long().sum().item())
    ms = T.ms("layer")
    causal_pairs = hq * sum(b * (b + 1) // 2 for b in geo.blocks)
    dense_flops = 4.0 * d * hq * sum(n * (n + 1) / 2.0 for n in geo.seqlens)
    res = {"workload": cfg.name, "seqlens": list(geo.seqlens), "heads": f"{hq}q/{hkv}kv",
           "B": B, "k": cfg.k, "rho": cfg.rho, "ms_per_layer": ms,
           "ms_per_stack": ms * cfg.layers,
           "select_chain_us": T.ms("select_chain") * 1e3, "attn_ms": T.ms("attention"),
           "dense_equiv_tflops": dense_flops / (ms * 1e-3) / 1e12,
           "attn_exec_tflops": 4.0 * B * B * d * pairs / (T.ms("attention") * 1e-3) / 1e12,
           "executed_causal_density": pairs / causal_pairs,
           "note": (f"one sparse layer per step, {steps} timed after {warmup} warm-up; "
                    f"ms_per_stack = ms_per_layer x {cfg.layers} layers")}
    del layers
    return res


def bench_tiny(torch, sws, gen, reps=50):
    """Latency of the tiny fp32 stack (1 head, n = 1024, d = 64, B = 64,
    k = 16, 4 layers, the first two dense): all four layers (sketch, walk,
    select, attention each), timed with HIP events over `reps` runs."""
    cfg = gen.CONFIGS["C1"]
    geo = sws.Geometry(list(cfg.seqlens), cfg.B)
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    sd, cd = torch.from_numpy(signs).cuda(), torch.from_numpy(cols).cuda()
    layers = [gen.layer_inputs(cfg, l, device="cuda")[:3] for l in range(cfg.layers)]
    R = torch.empty(geo.walk_numel(cfg.hq), dtype=torch.float32, device="cuda")

    def stack():
        for l, (q, k, v) in enumerate(layers):
            sws.prefill_layer(q, k, v, geo, cfg.k, sd, cd, cfg.s, cfg.rho, l < cfg.n_dense, R,
                              first_layer=l == 0)

    for _ in range(3):
        stack()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        stack()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    return {"workload": cfg.name, "us_per_stack": us, "us_per_layer": us / cfg.layers,
            "layers": cfg.layers, "dtype": "f32",
            "note": "eager launches (5 per layer, outputs allocated by the binding); the host launches take most of the time"}


def bench_decode(args, torch, sws, gen, timer_cls):
    cfg = gen.CONFIGS["C4"]
    ns, P, steps = cfg.decode_batch, cfg.decode_prefix, args.decode_steps
    Lyr = args.decode_layers
    hq, hkv, d, B, kd = cfg.hq, cfg.hkv, cfg.d, cfg.B, cfg.k
    max_ctx = P + steps
    b_max = -(-max_ctx // B)
    signs, cols = gen.hadamard_tables(d, kd)
    signs_d = torch.from_numpy(signs).cuda()
    cols_d = torch.from_numpy(cols).cuda()
    t_setup = time.perf_counter()
    head_major = args.kv_layout == "head"
    geo_p = sws.Geometry([P], B)
    state = []
    for l in range(Lyr):
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
        del qpre
        knew = kc[:, P:].permute(1, 0, 2, 3).contiguous()       # [steps, ns, hkv, d]
        if head_major:
            kc = kc.permute(0, 2, 1, 3).contiguous()             # [ns, hkv, ctx, d]
            vc = vc.permute(0, 2, 1, 3).contiguous()
        if l % 8 == 7:
            print(f"[bench] decode setup: {l + 1}/{Lyr} layers", file=sys.stderr, flush=True)
        state.append({"qst": qst, "knew": knew, "kc": kc, "vc": vc, "qsk": qsk, "ksk": ksk,
                      "rq": rq, "rk": rk, "out": torch.empty((ns, hq, d), dtype=qst.dtype,
                                                             device="cuda")})
    # every layer's new-token q and k in one tensor each, so one copy stages a
    # step's inputs for all layers (the graph replay below)
    q_all = torch.stack([st_["qst"] for st_ in state])            # [L, steps, ns, hq, d]
    k_all = torch.stack([st_["knew"] for st_ in state])           # [L, steps, ns, hkv, d]
    for l, st_ in enumerate(state):
        st_["qst"], st_["knew"] = q_all[l], k_all[l]
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    pos = torch.arange(P, P + steps, dtype=torch.int32, device="cuda")[:, None].expand(steps, ns).contiguous()
    cur = (pos // B).contiguous()
    ctx_len = (pos + 1).contiguous()
    snap = [{k_: st_[k_].clone() for k_ in ("qsk", "ksk", "rq", "rk")} for st_ in state]
    uw = sws.union_width(cfg.rho, b_max, hq // hkv)
    ubufs = (torch.empty((ns, hkv, uw), dtype=torch.int32, device="cuda"),
             torch.empty((ns, hkv), dtype=torch.int32, device="cuda"),
             torch.empty((ns, hkv, uw), dtype=torch.int32, device="cuda"), None, None)
    dbufs = (torch.empty((ns, hkv, b_max), dtype=torch.int32, device="cuda"),
             torch.empty((ns, hkv), dtype=torch.int32, device="cuda"),
             torch.empty((ns, hkv, b_max), dtype=torch.int32, device="cuda"), None, None)
    ws = torch.empty(sws.decode_workspace_size(ns, hq, hkv, d, B, b_max), dtype=torch.uint8,
                     device="cuda")
    r = torch.empty((ns, hq, b_max), dtype=torch.float32, device="cuda")

    def one_step(t, T=None):
        for l, st in enumerate(state):
            dense = l < cfg.n_dense
            a = T.ev() if T else None
            sws.sketch_append_qk(st["qst"][t], st["knew"][t], pos[t], B, kd, signs_d, cols_d,
                                 st["rq"], st["rk"], st["qsk"], st["ksk"])
            sws.walk_update_row(st["qsk"], st["ksk"], cur[t], cfg.s, None if l == 0 else r, r)
            uidx, ucnt, umask, _, _ = sws.select_topk_row(r, hq, hkv, cur[t], b_max, cfg.rho,
                                                          dense=dense,
                                                          out=dbufs if dense else ubufs)
            b_ = T.ev() if T else None
            sws.sparse_attn_decode(st["qst"][t], st["kc"], st["vc"], ctx_len[t], B, uidx, ucnt,
                                   umask, out=st["out"], ws=ws, head_major=head_major)
            if T:
                c_ = T.ev()
                T.add("dense_layer" if dense else "sparse_layer", a, c_)
                T.add("dense_attn" if dense else "sparse_attn", b_, c_)
                T.add("dense_select_chain" if dense else "sparse_select_chain", a, b_)

    def restore(sn):
        for st_, x in zip(state, sn):
            for k_, v_ in x.items():
                st_[k_].copy_(v_)

    # The decode steps run in order (the sketch caches and running sums are
    # state).  An untimed pass over every step first (it warms up and
    # records the union size of every sparse layer-step: the algorithmic
    # bytes of the attention), then the state is restored and all steps are
    # timed.
    n_sparse = Lyr - min(Lyr, cfg.n_dense)
    union_sum = torch.zeros((steps, max(1, n_sparse)), dtype=torch.int64, device="cuda")
    for t in range(steps):
        for l, st in enumerate(state):
            dense = l < cfg.n_dense
            sws.sketch_append_qk(st["qst"][t], st["knew"][t], pos[t], B, kd, signs_d, cols_d,
                                 st["rq"], st["rk"], st["qsk"], st["ksk"])
            sws.walk_update_row(st["qsk"], st["ksk"], cur[t], cfg.s, None if l == 0 else r, r)
            u = sws.select_topk_row(r, hq, hkv, cur[t], b_max, cfg.rho, dense=dense,
                                    out=dbufs if dense else ubufs)
            sws.sparse_attn_decode(st["qst"][t], st["kc"], st["vc"], ctx_len[t], B, u[0], u[1],
                                   u[2], out=st["out"], ws=ws, head_major=head_major)
            if not dense:
                union_sum[t, l - cfg.n_dense] = u[1].sum()
        if (t + 1) % 64 == 0 or t + 1 == steps:
            torch.cuda.synchronize()
            print(f"[bench] decode recording pass: step {t + 1}/{steps}", file=sys.stderr,
                  flush=True)
    torch.cuda.synchronize()
    union_blocks = float(union_sum.double().mean()) if n_sparse else 0.0
    restore(snap)
    T = timer_cls(torch)
    e0 = T.ev()
    for t in range(steps):
        one_step(t, T)
        if (t + 1) % 64 == 0 and t + 1 < steps:
            print(f"[bench] decode eager pass: step {t + 1}/{steps} launched", file=sys.stderr,
                  flush=True)
    e1 = T.ev()
    torch.cuda.synchronize()
    print(f"[bench] decode eager pass: {steps} steps", file=sys.stderr, flush=True)
    timed = steps
    us_step = e0.elapsed_time(e1) * 1e3 / timed
    tok_read = union_blocks * B            # the open block is partial; counted whole
    attn_bytes = tok_read * d * 2 * 2 + ns * hq * d * 2 * 2
    sp_attn_us = T.ms("sparse_attn") * 1e3
    res = {
        "batch": ns, "context": P, "steps_timed": timed, "layers": Lyr,
        "us_per_step": us_step,
        "us_per_sparse_layer_step": T.ms("sparse_layer") * 1e3,
        "us_per_dense_layer_step": T.ms("dense_layer") * 1e3,
        "sparse_attn_us": sp_attn_us,
        "sparse_select_chain_us": T.ms("sparse_select_chain") * 1e3,
        "dense_attn_us": T.ms("dense_attn") * 1e3,
        "sparse_attn_bytes": attn_bytes,
        "sparse_attn_gbs": attn_bytes / (sp_attn_us * 1e-6) / 1e9,
        "dense_attn_gbs": (ns * (P + steps // 2) * hkv * d * 4) / (T.ms("dense_attn") * 1e-3) / 1e9,
        "union_blocks_per_group": union_blocks / (ns * hkv),
        "union_note": ("algorithmic bytes per sparse layer-step: the mean over every "
                       "sparse layer-step of the union blocks, K and V rows of whole blocks, "
                       "plus q and out"),
        "per_head_blocks": cfg.rho * (b_max - 1) // 100 + 1,
        "setup_s": setup_s,
        "kv_layout": ("head-major [seq][kv head][ctx][d]" if head_major
                      else "token-major [seq][ctx][kv head][d]"),
    }
    if not args.no_graph:
        # The same steps again from the same starting state, each step one
        # HIP graph replay of all layers' kernels (captured once on static
        # buffers) after one copy of the step's q, k and positions into them.
        restore(snap)
        del snap
        q_buf = torch.empty_like(q_all[:, 0])
        k_buf = torch.empty_like(k_all[:, 0])
        pcc_all = torch.stack([pos, cur, ctx_len], dim=1).contiguous()   # [steps, 3, ns]
        pcc = torch.empty_like(pcc_all[0])

        snap2 = [{k_: st_[k_].clone() for k_ in ("qsk", "ksk", "rq", "rk")} for st_ in state]

        def chain(l, st, sl):
            dense = l < cfg.n_dense
            bufs = dbufs if dense else ubufs
            sws.sketch_append_qk(q_buf[l][sl], k_buf[l][sl], pcc[0][sl], B, kd, signs_d, cols_d,
                                 st["rq"][sl], st["rk"][sl], st["qsk"][sl], st["ksk"][sl])
            sws.walk_update_row(st["qsk"][sl], st["ksk"][sl], pcc[1][sl], cfg.s,
                                None if l == 0 else r[sl], r[sl])
            return sws.select_topk_row(r[sl], hq, hkv, pcc[1][sl], b_max, cfg.rho, dense=dense,
                                       out=tuple(None if x is None else x[sl] for x in bufs))

        def attend(l, st, u, sl, ws_):
            sws.sparse_attn_decode(q_buf[l][sl], st["kc"][sl], st["vc"][sl], pcc[2][sl], B, u[0],
                                   u[1], u[2], out=st["out"][sl], ws=ws_, head_major=head_major)

        whole = slice(0, ns)

        def graph_step():
            for l, st in enumerate(state):
                attend(l, st, chain(l, st, whole), whole, ws)

        # Two micro-batches, the two halves of the batch, on two streams: each
        # half runs every layer in order (its select chain, then its
        # attention), exactly the dependencies of a model whose layer l + 1
        # reads layer l's output; the halves are independent, so one half's
        # select chain (vector ALU and latency bound) can run beside the other
        # half's attention (HBM bound).  Each half has its own workspace.
        nmb = max(1, min(args.microbatches, ns))
        sides = [torch.cuda.Stream() for _ in range(nmb - 1)]
        parts = [slice(ns * i // nmb, ns * (i + 1) // nmb) for i in range(nmb)]
        ws_part = [ws] + [torch.empty_like(ws) for _ in range(nmb - 1)]

        def graph_step_2s():
            main = torch.cuda.current_stream()
            for sd in sides:
                sd.wait_stream(main)
            for sl, strm, ws_ in zip(parts, [main] + sides, ws_part):
                with torch.cuda.stream(strm):
                    for l, st in enumerate(state):
                        attend(l, st, chain(l, st, sl), sl, ws_)
            for sd in sides:
                main.wait_stream(sd)

        def stage(t):
            q_buf.copy_(q_all[:, t])
            k_buf.copy_(k_all[:, t])
            pcc.copy_(pcc_all[t])

        def time_graph(fn):
            for st_, sn in zip(state, snap2):
                for k_, v_ in sn.items():
                    st_[k_].copy_(v_)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn()
            stage(0)
            graph.replay()
            torch.cuda.synchronize()
            for st_, sn in zip(state, snap2):
                for k_, v_ in sn.items():
                    st_[k_].copy_(v_)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for t in range(steps):
                stage(t)
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            del graph
            return e0.elapsed_time(e1) * 1e3 / timed

        res["us_per_step_eager"] = res["us_per_step"]
        res["us_per_step_graph_1stream"] = time_graph(graph_step)
        res["us_per_step"] = res["us_per_step_graph_microbatches"] = time_graph(graph_step_2s)
        res["graph"] = ("one HIP graph per step (all layers), inputs staged by 3 copies; "
                        f"us_per_step: the batch as {nmb} micro-batches on {nmb} streams, "
                        "each running the layers in order")
        del snap2
    if not args.no_serving:
        res["serving_layouts"] = serving_layouts(torch, sws, gen, state[-1], ubufs, ctx_len[-1],
                                                 B, steps - 1, head_major)
    return res


def serving_layouts(torch, sws, gen, st, ubufs, ctx, B, t, head_major, reps=20):
    """Decode attention of one sparse layer at the last decode step on the
    same union lists, over the contiguous cache, a paged copy (pages of one
    block in a random order) and an fp8 e4m3 paged copy (per-tensor scales),
    each token-major and head-major ("_hm"), sparse and dense.  Bytes are the
    KV rows the lists name (K and V) plus q and out; GB/s is those bytes over
    the average call time."""
    kc, vc = st["kc"], st["vc"]
    if head_major:
        kc, vc = (x.permute(0, 2, 1, 3).contiguous() for x in (kc, vc))
    ns, max_ctx, hkv, d = kc.shape
    q = st["qst"][t]
    hq = q.shape[1]
    nb = -(-max_ctx // B)
    table, num_pages = gen.page_table([max_ctx] * ns, B, spare_pages=0)
    tab = torch.from_numpy(table).cuda()
    dst = tab.reshape(-1).long()

    def to_pages(x):
        pad = nb * B - max_ctx
        xp = torch.nn.functional.pad(x, (0, 0, 0, 0, 0, pad)) if pad else x
        pages = torch.empty((num_pages, B, hkv, d), dtype=x.dtype, device=x.device)
        pages[dst] = xp.reshape(ns * nb, B, hkv, d)
        return pages

    kp, vp = to_pages(kc), to_pages(vc)
    ksc = float(kc.float().abs().amax()) / 448.0
    vsc = float(vc.float().abs().amax()) / 448.0
    kp8 = gen.to_fp8_e4m3(kp, ksc).view(torch.float8_e4m3fn)
    vp8 = gen.to_fp8_e4m3(vp, vsc).view(torch.float8_e4m3fn)
    hm = lambda x: x.permute(0, 2, 1, 3).contiguous()
    kch, vch, kph, vph = hm(kc), hm(vc), hm(kp), hm(vp)
    kph8 = hm(kp8.view(torch.uint8)).view(torch.float8_e4m3fn)
    vph8 = hm(vp8.view(torch.uint8)).view(torch.float8_e4m3fn)
    uidx, ucnt, umask = ubufs[0], ubufs[1], ubufs[2]
    ws = torch.empty(sws.decode_workspace_size(ns, hq, hkv, d, B, nb), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(q)
    union_rows = int(ucnt.long().sum().item()) * B
    dense_rows = int(ctx.long().sum().item()) * hkv
    qo = ns * hq * d * 2 * 2
    runs = {
        "contiguous_bf16": (lambda u: sws.sparse_attn_decode(q, kc, vc, ctx, B, *u, out=out,
                                                             ws=ws), 2),
        "paged_bf16": (lambda u: sws.sparse_attn_decode_paged(q, kp, vp, tab, ctx, *u, out=out,
                                                              ws=ws), 2),
        "paged_fp8": (lambda u: sws.sparse_attn_decode_paged(q, kp8, vp8, tab, ctx, *u,
                                                             k_scale=ksc, v_scale=vsc, out=out,
                                                             ws=ws), 1),
        "contiguous_bf16_hm": (lambda u: sws.sparse_attn_decode(q, kch, vch, ctx, B, *u, out=out,
                                                                ws=ws, head_major=True), 2),
        "paged_bf16_hm": (lambda u: sws.sparse_attn_decode_paged(q, kph, vph, tab, ctx, *u,
                                                                 out=out, ws=ws,
                                                                 head_major=True), 2),
        "paged_fp8_hm": (lambda u: sws.sparse_attn_decode_paged(q, kph8, vph8, tab, ctx, *u,
                                                                k_scale=ksc, v_scale=vsc,
                                                                out=out, ws=ws,
                                                                head_major=True), 1),
    }
    res = {"batch": ns, "context": int(ctx[0]), "reps": reps}
    for mode, u, rows in (("sparse", (uidx, ucnt, umask), union_rows),
                          ("dense", (None, None, None), dense_rows)):
        for name, (fn, eb) in runs.items():
            fn(u)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn(u)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            nbytes = rows * d * eb * 2 + qo
            res[f"{mode}_{name}_us"] = round(us, 2)
            res[f"{mode}_{name}_gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
    del kp, vp, kp8, vp8, kch, vch, kph, vph, kph8, vph8
    return res


# ---------------------------------------------------------------------------
# Exact-score references of the selection diagnostics (torch on the device;
# tests/test_bench_reference.py checks each against the oracle on small
# inputs on the CPU)
# ---------------------------------------------------------------------------

def ref_block_means(torch, x, B):
    """Mean of each block's token rows of x [n, d] in fp64, the last block over
    the tokens it holds."""
    n, d = x.shape
    b = -(-n // B)
    xx = torch.nn.functional.pad(x.double(), (0, 0, 0, b * B - n)).view(b, B, d).sum(1)
    cnt = torch.full((b, 1), float(B), dtype=torch.float64, device=x.device)
    cnt[-1, 0] = n - (b - 1) * B
    return xx / cnt


def ref_walk_sets(torch, qm, km, s, rho, floor=2.0 ** -64):
    """Selected sets of the walk on exact block scores: M = tril(qm km^T) /
    sqrt(d) (a sketch of dimension d is exact), s hops from the identity with
    each hop's rows cut below floor times their largest magnitude, then per
    query block i the tau = floor(rho b / 100) earlier blocks of largest score
    (ties by index) plus block i (all of 0..i when i <= tau)."""
    b, d = qm.shape
    M = torch.tril(qm.double() @ km.double().T) / math.sqrt(d)
    X = torch.eye(b, dtype=torch.float64, device=qm.device)
    for _ in range(s):
        X = X @ M
        mx = X.abs().amax(dim=1, keepdim=True)
        X = torch.where(X.abs() < floor * mx, torch.zeros_like(X), X)
    X = X / X.abs().amax(dim=1, keepdim=True).clamp_min(1e-300)
    tau = (rho * b) // 100
    Xc = X.cpu().numpy() + 0.0
    sets = []
    for i in range(b):
        if i <= tau:
            sets.append(set(range(i + 1)))
            continue
        order = np.lexsort((np.arange(i), -Xc[i, :i]))[:tau]
        sets.append(set(order.tolist()) | {i})
    return sets


def ref_captured_mass(torch, q, k, B, selections, rhos=(), chunk=8):
    """Exact attention mass that block selections capture, per query row, for
    one head: q, k [n, d] (computed in fp32, scale 1/sqrt(d), token-causal).
    selections: name -> list over query blocks of key-block collections.  For
    each rho in rhos also the best block selection of that density: for query
    block i, the tau = floor(rho b / 100) earlier key blocks of largest total
    exact mass over the block's queries, plus block i.  Returns name (or
    'best rho=..') -> numpy array of the per-row captured mass."""
    n, d = q.shape
    b = -(-n // B)
    qf, kf = q.float(), k.float()
    res = {nm: [] for nm in selections}
    res.update({f"best rho={r}": [] for r in rhos})
    for c0 in range(0, b, chunk):
        c1 = min(b, c0 + chunk)
        r0, r1 = c0 * B, min(n, c1 * B)
        S = (qf[r0:r1] @ kf[:r1].T.contiguous()) / math.sqrt(d)
        keys = torch.arange(r1, device=q.device)
        rows = torch.arange(r0, r1, device=q.device)
        S = S.masked_fill(keys[None, :] > rows[:, None], float("-inf"))
        P = torch.softmax(S, dim=1)
        P = torch.nn.functional.pad(P, (0, c1 * B - r1))
        Mrow = P.view(r1 - r0, c1, B).sum(2).double().cpu().numpy()
        for i in range(c0, c1):
            a, e = i * B - r0, min(n, (i + 1) * B) - r0
            Mi = Mrow[a:e, :i + 1]
            for nm, sel in selections.items():
                res[nm].append(Mi[:, np.asarray(sorted(sel[i]), dtype=np.int64)].sum(1))
            tot = Mi[:, :i].sum(0)
            for r in rhos:
                tau = (r * b) // 100
                if i <= tau:
                    keep = np.arange(i + 1)
                else:
                    keep = np.concatenate([np.lexsort((np.arange(i), -tot))[:tau], [i]])
                res[f"best rho={r}"].append(Mi[:, keep].sum(1))
    return {nm: np.concatenate(v) for nm, v in res.items()}


def diagnostics(args, torch, sws, gen, ctx):
    """Sweeps over the walk degree s, the sketch dimension k, the block size B
    and the density rho on one 128K layer (walk started from the identity), with
    the time split per stage, plus selection-quality diagnostics on the planted
    data:
    * agreement (Jaccard) of each configuration's selected sets with the
      selection of the exact block scores (k = d: the sketch is then exact, so
      the reference walks tril(qbar kbar^T)/sqrt(d) itself, computed here with
      plain torch fp64 on sampled heads);
    * attention mass captured by the selected blocks, exp(lse_sparse -
      lse_dense) per query row, from the kernels' log-sum-exp outputs;
    * recall of the planted multi-hop chains i -> j -> m: how often the far
      block m (and the near block j) is among block i's selection, for the
      multi-hop walk (s = 8) against a one-hop walk (s = 1)."""
    from gen import synth
    cfg, geo = ctx["cfg"], ctx["geo"]
    q, k, v = ctx["layers"][0]
    layer_id = 2                          # ctx layers are generator layers 2, 3, ...
    hq, hkv, d, B = cfg.hq, cfg.hkv, cfg.d, cfg.B
    grp = hq // hkv
    n = geo.total_tokens
    dev = q.device

    def tables(kk):
        sg, cl = gen.hadamard_tables(d, kk)
        return torch.from_numpy(sg).to(dev), torch.from_numpy(cl).to(dev)

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def run(geo_, kk, s, rho, attn=True, lse=None, mode=0):
        sd, cd = tables(kk)
        R = torch.empty(geo_.walk_numel(hq), dtype=torch.float32, device=dev)
        wws = (torch.empty(sws.walk_variant_workspace_size(geo_.walk_numel(hq)),
                           dtype=torch.uint8, device=dev) if mode else None)
        ts = [ev()]
        q_sk = sws.sketch(q, geo_, kk, sd, cd)
        k_sk = sws.sketch(k, geo_, kk, sd, cd)
        ts.append(ev())
        if mode:
            sws.walk_update_variant(q_sk, k_sk, geo_, s, mode, None, R_out=R, ws=wws)
        else:
            sws.walk_update(q_sk, k_sk, geo_, s, None, R_out=R)
        ts.append(ev())
        idx, cnt = sws.select_topk(R, hq, geo_, rho)
        ts.append(ev())
        if attn:
            ws = torch.empty(sws.prefill_workspace_size(sws.BF16, geo_.total_blocks, hkv, d,
                                                        geo_.B), dtype=torch.uint8, device=dev)
            sws.sparse_attn_prefill(q, k, v, geo_, idx, cnt, lse=lse, ws=ws)
            ts.append(ev())
        torch.cuda.synchronize()
        names = ("sketch", "walk", "select", "attention")
        t = {nm: ts[i].elapsed_time(ts[i + 1]) * 1e3 for i, nm in enumerate(names[:len(ts) - 1])}
        return idx, cnt, t

    # exact-score reference selection on sampled heads (torch fp64)
    b = geo.max_blocks
    tau = (20 * b) // 100
    ref_heads = [0, 13, 26]
    ref = {h: ref_walk_sets(torch, ref_block_means(torch, q[:, h], B),
                            ref_block_means(torch, k[:, h // grp], B), 8, 20)
           for h in ref_heads}

    def jaccard(idx, cnt, heads=ref_heads):
        idx_h = idx.cpu().numpy()
        cnt_h = cnt.cpu().numpy()
        js = []
        for h in heads:
            for i in range(tau + 1, b):
                got = set(idx_h[h, i, :cnt_h[h, i]].tolist())
                want = ref[h][i]
                js.append(len(got & want) / len(got | want))
        return float(np.mean(js))

    sweep = []
    for (kk, s, rho) in [(32, 1, 20), (32, 2, 20), (32, 4, 20), (32, 8, 20), (32, 16, 20),
                         (16, 8, 20), (64, 8, 20), (32, 8, 10), (32, 8, 30)]:
        run(geo, kk, s, rho)                                # warm-up (first launches)
        idx, cnt, t = run(geo, kk, s, rho)
        rec = {"B": B, "k": kk, "s": s, "rho": rho, "stage_us": t,
               "executed_block_pairs": int(cnt.long().sum()),
               "dense_equiv_tflops": 4.0 * d * hq * n * (n + 1) / 2.0 / (sum(t.values()) * 1e-6) / 1e12}
        if rho == 20:
            rec["jaccard_vs_exact_scores"] = jaccard(idx, cnt)
        sweep.append(rec)
        print(f"[diag] sweep B={B} k={kk} s={s} rho={rho}: {sum(t.values()) / 1e3:.2f} ms",
              file=sys.stderr, flush=True)
    for mode, name in ((sws.WALK_POWER, "power"), (sws.WALK_SOFTMAX, "softmax")):
        run(geo, 32, 8, 20, attn=False, mode=mode)          # warm-up
        idx, cnt, t = run(geo, 32, 8, 20, attn=False, mode=mode)
        sweep.append({"B": B, "k": 32, "s": 8, "rho": 20, "walk_mode": name, "stage_us": t,
                      "executed_block_pairs": int(cnt.long().sum()),
                      "jaccard_vs_exact_scores": jaccard(idx, cnt)})
        print(f"[diag] walk variant {name}: walk {t['walk'] / 1e3:.2f} ms", file=sys.stderr,
              flush=True)
    geo64 = sws.Geometry([n], 64)
    run(geo64, 32, 8, 20)                                   # warm-up (first launches)
    idx, cnt, t = run(geo64, 32, 8, 20)
    sweep.append({"B": 64, "k": 32, "s": 8, "rho": 20, "stage_us": t,
                  "executed_block_pairs": int(cnt.long().sum()),
                  "dense_equiv_tflops": 4.0 * d * hq * n * (n + 1) / 2.0 / (sum(t.values()) * 1e-6) / 1e12})
    del idx, cnt

    # attention mass captured by the selection
    lse_d = torch.empty((hq, n), dtype=torch.float32, device=dev)
    ws = torch.empty(sws.prefill_workspace_size(sws.BF16, geo.total_blocks, hkv, d, B),
                     dtype=torch.uint8, device=dev)
    sws.sparse_attn_prefill(q, k, v, geo, None, None, lse=lse_d, ws=ws)
    captured = {}
    for rho in (10, 20, 30):
        lse_s = torch.empty_like(lse_d)
        run(geo, 32, 8, rho, lse=lse_s)
        frac = torch.exp((lse_s - lse_d).double())
        captured[str(rho)] = {"mean": float(frac.mean()), "p5": float(frac.quantile(0.05)),
                              "min": float(frac.min()),
                              "mean_sampled_heads": float(frac[ref_heads].mean())}

    # The same mass from exact fp32 attention on the sampled heads, for the
    # kernels' selections and for the best block selection of each density
    # (the ceiling of any block-sparse selection at that density).
    sel_runs = {"s=8 rho=10": (8, 0, 10), "s=8 rho=20": (8, 0, 20), "s=8 rho=30": (8, 0, 30),
                "s=1 rho=20": (1, 0, 20), "power s=8 rho=20": (8, sws.WALK_POWER, 20),
                "softmax s=8 rho=20": (8, sws.WALK_SOFTMAX, 20)}
    sel_lists = {}
    for nm, (s_, mode, rho) in sel_runs.items():
        idx, cnt, _ = run(geo, 32, s_, rho, attn=False, mode=mode)
        sel_lists[nm] = (idx[ref_heads].cpu().numpy(), cnt[ref_heads].cpu().numpy())
        del idx, cnt
    per_name = {}
    for hi, h in enumerate(ref_heads):
        sels = {nm: [ix[hi, i, :ct[hi, i]] for i in range(b)] for nm, (ix, ct) in sel_lists.items()}
        got = ref_captured_mass(torch, q[:, h], k[:, h // grp], B, sels, rhos=(10, 20, 30))
        for nm, a in got.items():
            per_name.setdefault(nm, []).append(a)
    exact_mass = {}
    for nm, vs in per_name.items():
        a = np.concatenate(vs)
        exact_mass[nm] = {"mean": float(a.mean()), "p5": float(np.quantile(a, 0.05)),
                          "min": float(a.min())}
    print(f"[diag] exact captured mass: " + ", ".join(f"{nm} {v_['mean']:.3f}"
                                                      for nm, v_ in exact_mass.items()),
          file=sys.stderr, flush=True)

    # planted chain recall: multi-hop walk against a one-hop walk
    recall = {}
    for s, mode, key in ((1, 0, "s=1"), (8, 0, "s=8"), (8, sws.WALK_POWER, "power s=8"),
                         (8, sws.WALK_SOFTMAX, "softmax s=8")):
        idx, cnt, _ = run(geo, 32, s, 20, attn=False, mode=mode)
        idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
        hit_j = hit_m = tot = 0
        for g in range(hkv):
            z = synth._band(cfg.cfg_id, 0, g, b, d)
            m_hat = synth._unit(z.mean(axis=0))
            for trip, _, _ in synth.chain_draws(cfg, layer_id, 0, g, b, m_hat):
                for (i, j, m) in trip.tolist():
                    for h in range(g * grp, (g + 1) * grp):
                        sel = set(idx_h[h, i, :cnt_h[h, i]].tolist())
                        hit_j += j in sel
                        hit_m += m in sel
                        tot += 1
        recall[key] = {"near_block_j": hit_j / tot, "far_block_m": hit_m / tot,
                       "chains_x_heads": tot}
    return {"layer": "128K prefill layer (generator layer 2), walk from the identity",
            "sweep": sweep, "captured_attention_mass": captured,
            "exact_captured_mass_sampled_heads": exact_mass, "planted_chain_recall": recall,
            "exact_reference_heads": ref_heads}


def cpu_baseline(ctx, torch, budget_s=12.0):
    """The oracle (fp64 NumPy) on a bounded sample of one sparse 128K layer:
    the query heads of KV head 0 sketched, walked from the identity and
    selected in full, then the attention of as many query blocks (spread over
    the sequence) as fit in the time budget; the time is scaled to the whole
    layer (32 query heads, 8 KV heads, every executed block pair)."""
    import oracle as O
    cfg, geo = ctx["cfg"], ctx["geo"]
    q, k, v = ctx["layers"][0]
    n = geo.total_tokens
    grp = cfg.hq // cfg.hkv
    K = k[:, 0].double().cpu().numpy()
    V = v[:, 0].double().cpu().numpy()
    Qs = [q[:, h].double().cpu().numpy() for h in range(grp)]
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    ks = O.sketch(K, cfg.B, ctx["signs"], ctx["cols"])
    t_k = time.perf_counter() - t0
    per_head = []
    all_lists = []
    for Q in Qs:
        a = time.perf_counter()
        qs = O.sketch(Q, cfg.B, ctx["signs"], ctx["cols"])
        R = O.walk_update(None, O.sketched_scores(qs, ks), cfg.s)
        lists = O.select(R, 20)
        per_head.append(time.perf_counter() - a)
        all_lists.append(lists)
    b = len(all_lists[0])
    rng = np.random.default_rng(0)
    order = [b - 1] + rng.permutation(b - 1).tolist()
    t_attn = 0.0
    pairs_sample = 0
    n_rows = 0
    scale = 1.0 / math.sqrt(cfg.d)
    while n_rows < len(order) and t_attn < budget_s:
        i = order[n_rows]
        a = time.perf_counter()
        O.sparse_attention_rows(Qs[0], K, V, all_lists[0], cfg.B, scale, [i])
        t_attn += time.perf_counter() - a
        pairs_sample += len(all_lists[0][i])
        n_rows += 1
    total = time.perf_counter() - t0
    attn_per_pair = t_attn / pairs_sample
    pairs_layer = sum(len(x) for x in all_lists[0]) * cfg.hq
    est = cfg.hkv * t_k + cfg.hq * (sum(per_head) / len(per_head)) + attn_per_pair * pairs_layer
    dense_flops = 4.0 * cfg.d * cfg.hq * n * (n + 1) / 2.0
    return {
        "value": dense_flops / est / 1e12, "unit": "TFLOP/s (dense-equivalent, extrapolated)",
        "cores": cores, "kind": "oracle",
        "ms_per_layer_extrapolated": est * 1e3,
        "sample": (f"fp64 NumPy oracle on one sparse layer of the 128K workload: KV head 0 and its "
                   f"{grp} query heads sketched, walked (s={cfg.s}) from the identity and "
                   f"top-tau selected over all {b} rows; attention of {n_rows} query blocks "
                   f"({pairs_sample} block pairs); scaled to {cfg.hq} query heads, {cfg.hkv} KV "
                   f"heads and {pairs_layer} block pairs"),
        "sample_seconds": total,
    }


def cpu_tiny_single_thread(gen):
    """The oracle on the whole tiny stack (4 layers, every block, attention of
    every query block) with one BLAS thread."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    cfg = gen.CONFIGS["C1"]
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    layers = [tuple(x.double().numpy()[:, :, :] for x in gen.layer_inputs(cfg, l)[:3])
              for l in range(cfg.layers)]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.prefill(layers, signs, cols, cfg.B, cfg.s, cfg.rho, cfg.n_dense)
        dt = time.perf_counter() - t0
    return {"us_per_stack": dt * 1e6, "cores": 1, "kind": "oracle",
            "sample": "fp64 NumPy oracle, tiny stack (1 head, n=1024, 4 layers), one thread, whole"}


def cpu_decode_sample(torch, gen):
    """The oracle's decode of one sequence of the 16 x 64K decode workload at
    its first step (row p of the prefill of the first p + 1 tokens, every
    query head), one sparse layer with the walk row started from the open
    block; the time is scaled to the whole batch and all layers of a step."""
    import oracle as O
    cfg = gen.CONFIGS["C4"]
    qpre, qst, kc, vc = gen.decode_layer_inputs(cfg, cfg.n_dense, device="cpu", n_seqs=1,
                                                prefix=cfg.decode_prefix, steps=1)
    Q = torch.cat([qpre[0], qst[:, 0]], 0).double().numpy()
    K = kc[0].double().numpy()
    V = vc[0].double().numpy()
    del qpre, qst, kc, vc
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    t0 = time.perf_counter()
    O.decode_step([(Q, K, V)], signs, cols, cfg.B, cfg.s, cfg.rho, n_dense=0)
    dt = time.perf_counter() - t0
    return {"us_per_step_extrapolated": dt * 1e6 * cfg.decode_batch * cfg.layers,
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": (f"fp64 NumPy oracle decode of 1 of {cfg.decode_batch} sequences at its "
                       f"first step ({cfg.decode_prefix + 1} tokens, {cfg.hq} query heads), one "
                       f"sparse layer; scaled x{cfg.decode_batch} sequences x{cfg.layers} layers"),
            "sample_seconds": dt}


def copy_calibration(torch, nbytes=1 << 30, reps=3):
    """A plain device copy of known size, for scaling the HBM counters."""
    x = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "reps": reps}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(json.dumps({"error": "bench.py measures one GPU only; run with --gpus 1",
                          "n_gpus": max(args.gpus, world)}))
        sys.exit(2)
    import torch
    import dynamic_block_sparse_sws_amd as sws
    import gen
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    sws.lib()
    torch.cuda.init()
    if args.copy_calib:
        copy_calibration(torch)
    pre, ctx = bench_prefill(args, torch, sws, gen, Timer)
    print(f"[bench] prefill: {pre['ms_per_layer']:.3f} ms/layer, "
          f"{pre['dense_equiv_tflops']:.1f} dense-equiv TFLOP/s, attention "
          f"{pre['attn_exec_tflops']:.1f} TFLOP/s executed", file=sys.stderr, flush=True)
    diag = None
    if args.diag:
        diag = diagnostics(args, torch, sws, gen, ctx)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(ctx, torch)
        print(f"[bench] cpu oracle sample {cpu['sample_seconds']:.1f}s", file=sys.stderr, flush=True)
    del ctx
    torch.cuda.empty_cache()
    others = None
    if not args.no_other_workloads:
        others = {}
        for name, key in (("C2", "prefill_32k"), ("C5", "prefill_ragged")):
            others[key] = bench_prefill_workload(torch, sws, gen, Timer, name)
            torch.cuda.empty_cache()
            print(f"[bench] {key}: {others[key]['ms_per_layer']:.3f} ms/layer", file=sys.stderr,
                  flush=True)
        others["tiny_stack"] = bench_tiny(torch, sws, gen)
        print(f"[bench] tiny stack: {others['tiny_stack']['us_per_stack']:.1f} us",
              file=sys.stderr, flush=True)
        if cpu is not None:
            cpu["tiny_stack_single_thread"] = cpu_tiny_single_thread(gen)
    dec = None
    if not args.no_decode:
        dec = bench_decode(args, torch, sws, gen, Timer)
        print(f"[bench] decode: {dec['us_per_step']:.1f} us/step", file=sys.stderr, flush=True)
        if cpu is not None:
            cpu["decode_step"] = cpu_decode_sample(torch, gen)
            print(f"[bench] cpu oracle decode sample {cpu['decode_step']['sample_seconds']:.1f}s",
                  file=sys.stderr, flush=True)
    attn_bytes = traffic_for("attn_prefill.hip", "attn_prefill_bf16_128k_rho20")
    line = {
        "metric": METRIC,
        "value": round(pre["dense_equiv_tflops"], 3),
        "unit": "TFLOP/s (dense-equivalent, 128K prefill layer at 20% density)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_layer"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": ("long_128k_prefill: one sparse layer per step, 32 query / 8 KV "
                                f"heads, d=128, n={pre['n']}, B=128, k=32, s=8, rho={args.rho}% "
                                "(also rho = 10/30/100); decode_64k_b16: 16 x 64K-token context, "
                                "32 layers (2 dense), B=64, k=32, rho=20%, 256 steps; "
                                "other_workloads: 32K prefill (B=64), ragged 8-sequence prefill "
                                "(40q/8kv), tiny fp32 stack"),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(pre["attn_exec_tflops"], 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(pre["attn_exec_tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": attn_bytes,
                     "kernel": "attn_prefill_bf16_kernel<128, 128, 1>",
                     "flops_per_launch": pre["attn_flops_per_launch"],
                     "avg_launch_ms": round(pre["attn_ms"], 4),
                     "target_frac": TARGET_PREFILL_MFMA_FRAC,
                     "target_met": pre["attn_exec_tflops"] / PEAK_BF16_TFLOPS >= TARGET_PREFILL_MFMA_FRAC},
        "cpu_baseline": cpu,
        "prefill": pre,
        "decode": dec,
    }
    if others:
        line["other_workloads"] = others
    if dec:
        gbs = dec["sparse_attn_gbs"]
        line["roofline_decode"] = {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "kernel": "decode_mfma_kernel + decode_combine_kernel (sparse layer-step)",
            "bytes_per_launch": dec["sparse_attn_bytes"],
            "avg_launch_us": round(dec["sparse_attn_us"], 2),
            "traffic": traffic_for("attn_decode.hip", "decode_sparse_64k_b16"),
            "target_frac": TARGET_DECODE_HBM_FRAC,
            "target_met": gbs / PEAK_HBM_GBS >= TARGET_DECODE_HBM_FRAC}
    if diag:
        line["diagnostics"] = diag
    if dec:
        line["decode_us_per_step"] = round(dec["us_per_step"], 2)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
