"""Decode steps captured once as a HIP graph (torch.cuda.CUDAGraph over the
library's launches on static buffers) and replayed step after step, with
eager work and synchronisations between the replays: every replay's outputs
equal the eager calls' bit for bit (token-major and head-major caches; one
stream, or the batch as two micro-batches on two streams)."""
import pytest
import torch

import dynamic_block_sparse_sws_amd as sws
import gen

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("two_streams", [False, True])
def test_decode_step_graph_replays_equal_eager(two_streams):
    """two_streams: the batch as two micro-batches (one sequence each) on two
    streams, each running every layer in order; each has its own decode
    workspace."""
    cfg = gen.CONFIGS["C4"].with_(d=128, B=64, hq=8, hkv=2, k=32)
    B, d, kd, hq, hkv = cfg.B, cfg.d, cfg.k, cfg.hq, cfg.hkv
    prefixes, steps, rho = (190, 250), 8, 30
    ns, n_layers = len(prefixes), 4
    max_ctx = max(prefixes) + steps
    b_max = -(-max_ctx // B)
    signs, cols = gen.hadamard_tables(d, kd)
    sd, cd = torch.from_numpy(signs).cuda(), torch.from_numpy(cols).cuda()
    layers = []
    for l in range(n_layers):
        full = [{w: gen.seq_tensor(cfg, l, s, w, prefixes[s] + steps, "cuda") for w in "qkv"}
                for s in range(ns)]
        kc = torch.zeros((ns, max_ctx, hkv, d), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        st = {"qsk": torch.zeros((ns, hq, b_max, kd), device="cuda"),
              "ksk": torch.zeros((ns, hkv, b_max, kd), device="cuda"),
              "rq": torch.zeros((ns, hq, d), device="cuda"),
              "rk": torch.zeros((ns, hkv, d), device="cuda")}
        for s, P in enumerate(prefixes):
            kc[s, :P + steps] = full[s]["k"]
            vc[s, :P + steps] = full[s]["v"]
            geo = sws.Geometry([P], B)
            sq = torch.empty((hq, geo.total_blocks, d), device="cuda")
            sk = torch.empty((hkv, geo.total_blocks, d), device="cuda")
            sws.sketch(full[s]["q"][:P].contiguous(), geo, kd, sd, cd, out=st["qsk"][s],
                       ld_head=b_max * kd, sum_out=sq)
            sws.sketch(full[s]["k"][:P].contiguous(), geo, kd, sd, cd, out=st["ksk"][s],
                       ld_head=b_max * kd, sum_out=sk)
            if P % B:
                st["rq"][s] = sq[:, -1]
                st["rk"][s] = sk[:, -1]
        qn = torch.stack([torch.stack([full[s]["q"][prefixes[s] + t] for s in range(ns)])
                          for t in range(steps)]).contiguous()
        kn = torch.stack([torch.stack([full[s]["k"][prefixes[s] + t] for s in range(ns)])
                          for t in range(steps)]).contiguous()
        hm = l % 2 == 1                  # odd layers keep head-major caches
        if hm:
            kc, vc = (x.permute(0, 2, 1, 3).contiguous() for x in (kc, vc))
        layers.append({"kc": kc, "vc": vc, "hm": hm, "st": st, "qn": qn, "kn": kn,
                       "out": torch.empty((ns, hq, d), dtype=torch.bfloat16, device="cuda")})
    snap = [{k: v.clone() for k, v in L["st"].items()} for L in layers]
    P_t = torch.tensor(prefixes, dtype=torch.int32, device="cuda")
    uw = sws.union_width(rho, b_max, hq // hkv)
    # list buffers alternate between layers (sparse lists "u", dense "d")
    bufs = [{"u": (torch.empty((ns, hkv, uw), dtype=torch.int32, device="cuda"),
                   torch.empty((ns, hkv), dtype=torch.int32, device="cuda"),
                   torch.empty((ns, hkv, uw), dtype=torch.int32, device="cuda"), None, None),
             "d": (torch.empty((ns, hkv, b_max), dtype=torch.int32, device="cuda"),
                   torch.empty((ns, hkv), dtype=torch.int32, device="cuda"),
                   torch.empty((ns, hkv, b_max), dtype=torch.int32, device="cuda"), None, None)}
            for _ in range(2)]
    ws = torch.empty(sws.decode_workspace_size(ns, hq, hkv, d, B, b_max), dtype=torch.uint8,
                     device="cuda")
    r = torch.empty((ns, hq, b_max), device="cuda")
    lse = [torch.empty((ns, hq), device="cuda") for _ in layers]

    ws2 = torch.empty_like(ws)

    def chain(l, q_of, k_of, pos, cur, sl):
        st = layers[l]["st"]
        out = tuple(None if x is None else x[sl] for x in bufs[l % 2]["d" if l == 0 else "u"])
        sws.sketch_append_qk(q_of(l)[sl], k_of(l)[sl], pos[sl], B, kd, sd, cd, st["rq"][sl],
                             st["rk"][sl], st["qsk"][sl], st["ksk"][sl])
        sws.walk_update_row(st["qsk"][sl], st["ksk"][sl], cur[sl], cfg.s,
                            None if l == 0 else r[sl], r[sl])
        return sws.select_topk_row(r[sl], hq, hkv, cur[sl], b_max, rho, dense=l == 0, out=out)

    def attend(l, q_of, ctx, u, sl, ws_):
        L = layers[l]
        sws.sparse_attn_decode(q_of(l)[sl], L["kc"][sl], L["vc"][sl], ctx[sl], B, u[0], u[1],
                               u[2], out=L["out"][sl], lse=lse[l][sl], ws=ws_,
                               head_major=L["hm"])

    whole = slice(0, ns)

    def step(q_of, k_of, pos, cur, ctx):
        for l in range(n_layers):
            attend(l, q_of, ctx, chain(l, q_of, k_of, pos, cur, whole), whole, ws)

    side = torch.cuda.Stream()

    def step_2s(q_of, k_of, pos, cur, ctx, eager=False):
        # (the eager reference runs the same micro-batch calls on one stream:
        # a micro-batch's split-KV ranges differ from the whole batch's, so
        # its rounding does too)
        main = torch.cuda.current_stream()
        other = main if eager else side
        other.wait_stream(main)
        for sl, strm, ws_ in zip((slice(0, 1), slice(1, 2)), (main, other), (ws, ws2)):
            with torch.cuda.stream(strm):
                for l in range(n_layers):
                    attend(l, q_of, ctx, chain(l, q_of, k_of, pos, cur, sl), sl, ws_)
        main.wait_stream(other)

    def outputs():
        out = []
        for ub in (bufs[0]["u"], bufs[1]["u"]):          # layers 2 and 3
            n_u = ub[1].clone()
            out += [n_u] + [ub[0][s, g, :n_u[s, g]].clone() for s in range(ns)
                            for g in range(hkv)]
        lists = out
        return [r.clone(), *lists, *[L["out"].clone() for L in layers],
                *[x.clone() for x in lse], *[L["st"]["qsk"].clone() for L in layers]]

    eager = []
    for t in range(steps):
        pos = P_t + t
        if two_streams:
            step_2s(lambda l: layers[l]["qn"][t], lambda l: layers[l]["kn"][t], pos, pos // B,
                    pos + 1, eager=True)
        else:
            step(lambda l: layers[l]["qn"][t], lambda l: layers[l]["kn"][t], pos, pos // B,
                 pos + 1)
        eager.append(outputs())
    torch.cuda.synchronize()

    # graph on static buffers, replayed from the same starting state
    for L, sn in zip(layers, snap):
        for k, v in sn.items():
            L["st"][k].copy_(v)
    q_buf = torch.empty_like(torch.stack([L["qn"][0] for L in layers]))
    k_buf = torch.empty_like(torch.stack([L["kn"][0] for L in layers]))
    pcc = torch.empty((3, ns), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        (step_2s if two_streams else step)(lambda l: q_buf[l], lambda l: k_buf[l], pcc[0],
                                           pcc[1], pcc[2])
    for t in range(steps):
        pos = P_t + t
        for l, L in enumerate(layers):
            q_buf[l].copy_(L["qn"][t])
            k_buf[l].copy_(L["kn"][t])
        pcc.copy_(torch.stack([pos, pos // B, pos + 1]))
        graph.replay()
        junk = torch.randn(1000, device="cuda").sum()        # eager work between replays
        torch.cuda.synchronize()
        got = outputs()
        for a, b in zip(got, eager[t]):
            assert torch.equal(a, b), t
        del junk
