"""GPU parity of the decode chain (sketch append -> walk row -> select row +
GQA union -> split-KV attention) against the oracle, stage by stage, at steps
that open, fill and complete blocks."""
import math

import numpy as np
import pytest
import torch

import dynamic_block_sparse_sws_amd as sws
import gen
import oracle as O
from gpu_util import f64, rowwise_rel_err, TOL_ATTN_BF16, TOL_ATTN_F32, TOL_SKETCH, TOL_WALK

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def run_decode_case(cfg, prefixes, steps, n_layers, rho, n_dense, check_steps, dense_null=False):
    ns = len(prefixes)
    B, d, kd, hq, hkv = cfg.B, cfg.d, cfg.k, cfg.hq, cfg.hkv
    grp = hq // hkv
    max_ctx = max(prefixes) + steps
    b_max = -(-max_ctx // B)
    signs, cols = gen.hadamard_tables(d, kd)
    signs_d = torch.from_numpy(signs).cuda()
    cols_d = torch.from_numpy(cols).cuda()
    dt = cfg.torch_dtype
    layers = []
    for l in range(n_layers):
        full = [{w: gen.seq_tensor(cfg, l, s, w, prefixes[s] + steps, "cuda") for w in "qkv"}
                for s in range(ns)]
        kc = torch.zeros((ns, max_ctx, hkv, d), dtype=dt, device="cuda")
        vc = torch.zeros_like(kc)
        qsk = torch.zeros((ns, hq, b_max, kd), dtype=torch.float32, device="cuda")
        ksk = torch.zeros((ns, hkv, b_max, kd), dtype=torch.float32, device="cuda")
        rq = torch.zeros((ns, hq, d), dtype=torch.float32, device="cuda")
        rk = torch.zeros((ns, hkv, d), dtype=torch.float32, device="cuda")
        for s in range(ns):
            P = prefixes[s]
            n_all = P + steps
            kc[s, :n_all] = full[s]["k"]
            vc[s, :n_all] = full[s]["v"]
            geo = sws.Geometry([P], B)
            sq = torch.empty((hq, geo.total_blocks, d), dtype=torch.float32, device="cuda")
            sk = torch.empty((hkv, geo.total_blocks, d), dtype=torch.float32, device="cuda")
            sws.sketch(full[s]["q"][:P].contiguous(), geo, kd, signs_d, cols_d, out=qsk[s],
                       ld_head=b_max * kd, sum_out=sq)
            sws.sketch(full[s]["k"][:P].contiguous(), geo, kd, signs_d, cols_d, out=ksk[s],
                       ld_head=b_max * kd, sum_out=sk)
            if P % B:
                rq[s] = sq[:, -1]
                rk[s] = sk[:, -1]
        host = [{w: f64(full[s][w]) for w in "qkv"} for s in range(ns)]
        layers.append({"full": full, "host": host, "kc": kc, "vc": vc, "qsk": qsk, "ksk": ksk,
                       "rq": rq, "rk": rk, "r": torch.zeros((ns, hq, b_max), device="cuda")})
    P_t = torch.tensor(prefixes, dtype=torch.int32, device="cuda")
    worst = {"sketch": 0.0, "walk": 0.0, "attn": 0.0}
    last = None
    tol_attn = TOL_ATTN_F32 if cfg.dtype == "f32" else TOL_ATTN_BF16
    for t in range(steps):
        pos = P_t + t
        cur = pos // B
        ctx = pos + 1
        recs = []
        for l, L in enumerate(layers):
            dense = l < n_dense
            qn = torch.stack([L["full"][s]["q"][prefixes[s] + t] for s in range(ns)]).contiguous()
            kn = torch.stack([L["full"][s]["k"][prefixes[s] + t] for s in range(ns)]).contiguous()
            sws.sketch_append(qn, pos, B, kd, signs_d, cols_d, L["rq"], L["qsk"])
            sws.sketch_append(kn, pos, B, kd, signs_d, cols_d, L["rk"], L["ksk"])
            r_prev = None if l == 0 else layers[l - 1]["r"]
            sws.walk_update_row(L["qsk"], L["ksk"], cur, cfg.s, r_prev, L["r"])
            uidx, ucnt, umask, idx, cnt = sws.select_topk_row(L["r"], hq, hkv, cur, b_max, rho,
                                                              dense=dense, per_head=True)
            lse = torch.empty((ns, hq), dtype=torch.float32, device="cuda")
            if dense and dense_null:
                out = sws.sparse_attn_decode(qn, L["kc"], L["vc"], ctx, B, None, None, None, lse=lse)
            else:
                out = sws.sparse_attn_decode(qn, L["kc"], L["vc"], ctx, B, uidx, ucnt, umask,
                                             lse=lse)
            if t in check_steps:
                torch.cuda.synchronize()
                recs.append({"qsk": f64(L["qsk"]), "ksk": f64(L["ksk"]), "r": f64(L["r"]),
                             "uidx": uidx.cpu().numpy(), "ucnt": ucnt.cpu().numpy(),
                             "umask": umask.cpu().numpy().astype(np.uint32),
                             "idx": idx.cpu().numpy(), "cnt": cnt.cpu().numpy(),
                             "out": f64(out), "lse": f64(lse)})
        if t not in check_steps:
            continue
        for l, (L, rec) in enumerate(zip(layers, recs)):
            dense = l < n_dense
            for s in range(ns):
                p = prefixes[s] + t
                c = p // B
                H = L["host"][s]
                # sketch rows 0..c against the oracle on the first p+1 tokens
                for h in range(hq):
                    want = O.sketch(H["q"][:p + 1, h], B, signs, cols)
                    e = rowwise_rel_err(rec["qsk"][s, h, :c + 1], want)
                    worst["sketch"] = max(worst["sketch"], e)
                    assert e <= TOL_SKETCH, (t, l, s, h, "q sketch", e)
                for g in range(hkv):
                    want = O.sketch(H["k"][:p + 1, g], B, signs, cols)
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
                           else O.select_row(rg, c, O.n_select(rho, c + 1)))
                    got = rec["idx"][s, h, :rec["cnt"][s, h]]
                    assert got.tolist() == lst.tolist(), (t, l, s, h, got, lst)
                    # attention of token p over the selected blocks
                    o_want, lse_want = O.query_attention(H["q"][p, h], H["k"][:, g], H["v"][:, g],
                                                         lst, B, p, 1.0 / math.sqrt(d))
                    e = float(np.abs(rec["out"][s, h] - o_want).max())
                    worst["attn"] = max(worst["attn"], e)
                    assert e <= tol_attn, (t, l, s, h, "attn", e)
                    assert abs(rec["lse"][s, h] - lse_want) <= max(tol_attn, 1e-4)
                # union list and masks of every group
                for g in range(hkv):
                    want = {}
                    for h in range(g * grp, (g + 1) * grp):
                        for m in rec["idx"][s, h, :rec["cnt"][s, h]]:
                            want[int(m)] = want.get(int(m), 0) | (1 << (h - g * grp))
                    n_u = rec["ucnt"][s, g]
                    got_idx = rec["uidx"][s, g, :n_u].tolist()
                    got_mask = rec["umask"][s, g, :n_u].tolist()
                    assert got_idx == sorted(want), (t, l, s, g)
                    assert got_mask == [want[m] for m in sorted(want)], (t, l, s, g)
        last = recs
    return worst, [L["host"] for L in layers], last


@pytest.mark.parametrize("d,B,hq,hkv,prefixes,steps", [
    (128, 64, 8, 2, (1000, 64, 2000), 70),
    (64, 128, 10, 2, (700, 1000), 40),
])
def test_decode_bf16(d, B, hq, hkv, prefixes, steps):
    cfg = gen.CONFIGS["C4"].with_(d=d, B=B, hq=hq, hkv=hkv, k=32)
    checks = {0, 1, 23, 24, 25, 47, 48, 63, 64, steps - 1} & set(range(steps))
    _print("decode bf16", d, B, hq, hkv, prefixes, steps)
    w, _, _ = run_decode_case(cfg, prefixes, steps, 3, 30, 1, checks)
    _print("worst", w)


def test_decode_fp32_and_dense_null():
    cfg = gen.CONFIGS["C4"].with_(d=64, B=64, hq=4, hkv=4, k=16, dtype="f32")
    _print("decode fp32")
    w, _, _ = run_decode_case(cfg, (65, 127), 10, 2, 25, 1, {0, 1, 9}, dense_null=True)
    _print("worst", w)


def test_decode_matches_prefix_prefill_definition():
    """End to end: the state-carrying decode equals the oracle's stateless
    definition (row p of the prefill on the first p+1 tokens, every layer's walk
    carried from the previous layer in fp64) on every selection, except where
    an fp32-versus-fp64 near-tie separates the tau-th and next candidate."""
    cfg = gen.CONFIGS["C4"].with_(d=128, B=64, hq=4, hkv=2, k=32)
    prefixes, steps, n_layers, rho = (190, 300), 3, 4, 30
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    _, hosts, recs = run_decode_case(cfg, prefixes, steps, n_layers, rho, 1, {steps - 1})
    for s in range(len(prefixes)):
        p = prefixes[s] + steps - 1
        c = p // cfg.B
        lay = [(H[s]["q"][:p + 1], H[s]["k"][:p + 1], H[s]["v"][:p + 1]) for H in hosts]
        dec = O.decode_step(lay, signs, cols, cfg.B, cfg.s, rho, n_dense=1)
        for l in range(n_layers):
            for h in range(cfg.hq):
                want = dec[l][h]
                r_gpu = recs[l]["r"][s, h, :c + 1]
                e = rowwise_rel_err(r_gpu, want["r"])
                _print("e2e", s, l, h, "walk drift", e)
                assert e <= 1e-4
                got = recs[l]["idx"][s, h, :recs[l]["cnt"][s, h]]
                if got.tolist() != want["lst"].tolist():
                    tau = O.n_select(rho, c + 1)
                    row = want["r"][:c]
                    kth = np.sort(row)[::-1][tau - 1]
                    diff = set(got.tolist()) ^ set(want["lst"].tolist())
                    gap = max(abs(row[m] - kth) for m in diff)
                    assert gap <= 1e-4 * np.abs(row).max(), (s, l, h, diff, gap)
                else:
                    assert np.abs(recs[l]["out"][s, h] - want["o"]).max() <= TOL_ATTN_BF16


def test_decode_other_walk_degree_and_sketch_dim():
    """Decode chain with s = 2 hops and k = 64 sketch components."""
    cfg = gen.CONFIGS["C4"].with_(d=128, B=64, hq=4, hkv=2, k=64, s=2)
    _print("decode s=2 k=64")
    w, _, _ = run_decode_case(cfg, (300, 129), 6, 2, 25, 0, {0, 2, 5})
    _print("worst", w)


def test_decode_group_shared_selection():
    """Decode with one shared list per KV group: every head keeps the list the
    oracle selects on the group's fp32-summed walk rows, the union is that
    list with every head's bit set, and the attention matches."""
    cfg = gen.CONFIGS["C4"].with_(d=128, B=64, hq=8, hkv=2, k=32)
    ns, P, B = 2, 900, cfg.B
    hq, hkv, kd, grp = cfg.hq, cfg.hkv, cfg.k, cfg.hq // cfg.hkv
    b_max = -(-(P + 1) // B)
    signs, cols = gen.hadamard_tables(cfg.d, kd)
    sd, cd = torch.from_numpy(signs).cuda(), torch.from_numpy(cols).cuda()
    full = [{w: gen.seq_tensor(cfg, 0, s, w, P + 1, "cuda") for w in "qkv"} for s in range(ns)]
    geo = sws.Geometry([P + 1], B)
    qsk = torch.zeros((ns, hq, b_max, kd), dtype=torch.float32, device="cuda")
    ksk = torch.zeros((ns, hkv, b_max, kd), dtype=torch.float32, device="cuda")
    for s in range(ns):
        sws.sketch(full[s]["q"].contiguous(), geo, kd, sd, cd, out=qsk[s], ld_head=b_max * kd)
        sws.sketch(full[s]["k"].contiguous(), geo, kd, sd, cd, out=ksk[s], ld_head=b_max * kd)
    cur = torch.full((ns,), P // B, dtype=torch.int32, device="cuda")
    r = torch.zeros((ns, hq, b_max), dtype=torch.float32, device="cuda")
    sws.walk_update_row(qsk, ksk, cur, cfg.s, None, r)
    rho = 30
    uidx, ucnt, umask, idx, cnt = sws.select_topk_row(r, hq, hkv, cur, b_max, rho, per_head=True,
                                                      group=True)
    kc = torch.stack([full[s]["k"] for s in range(ns)]).contiguous()
    vc = torch.stack([full[s]["v"] for s in range(ns)]).contiguous()
    qn = torch.stack([full[s]["q"][P] for s in range(ns)]).contiguous()
    ctx = torch.full((ns,), P + 1, dtype=torch.int32, device="cuda")
    out = sws.sparse_attn_decode(qn, kc, vc, ctx, B, uidx, ucnt, umask)
    torch.cuda.synchronize()
    c = P // B
    rh = r.cpu().numpy()
    for s in range(ns):
        for g in range(hkv):
            score = O.group_scores([rh[s, h, :c + 1] for h in range(g * grp, (g + 1) * grp)])
            want = O.select_row(score, c, O.n_select(rho, c + 1)).tolist()
            for h in range(g * grp, (g + 1) * grp):
                assert idx[s, h, :cnt[s, h]].tolist() == want, (s, h)
            n_u = int(ucnt[s, g])
            assert uidx[s, g, :n_u].tolist() == want
            assert (umask[s, g, :n_u].cpu().numpy().astype(np.uint32) == (1 << grp) - 1).all()
            H = {w: f64(full[s][w]) for w in "qkv"}
            for h in range(g * grp, (g + 1) * grp):
                o_want, _ = O.query_attention(H["q"][P, h], H["k"][:, g], H["v"][:, g],
                                              np.array(want), B, P, 1.0 / math.sqrt(cfg.d))
                assert np.abs(f64(out[s, h]) - o_want).max() <= TOL_ATTN_BF16, (s, h)


@pytest.mark.parametrize("mode,s", [(sws.WALK_POWER, 8), (sws.WALK_SOFTMAX, 8), (sws.WALK_POWER, 3)])
def test_decode_walk_variants(mode, s):
    """Decode row walk of the variants against the oracle's row form, two
    layers carried, for sequences whose open block is partial and full."""
    cfg = gen.CONFIGS["C4"].with_(d=128, B=64, hq=4, hkv=2, k=32)
    B, kd, hq, hkv = cfg.B, cfg.k, cfg.hq, cfg.hkv
    grp = hq // hkv
    name = {sws.WALK_POWER: "power", sws.WALK_SOFTMAX: "softmax"}[mode]
    lens = (530, 640)                      # open block partial / just completed
    ns = len(lens)
    b_max = -(-max(lens) // B)
    signs, cols = gen.hadamard_tables(cfg.d, kd)
    sd, cd = torch.from_numpy(signs).cuda(), torch.from_numpy(cols).cuda()
    cur = torch.tensor([(n - 1) // B for n in lens], dtype=torch.int32, device="cuda")
    r_prev = None
    for l in range(2):
        qsk = torch.zeros((ns, hq, b_max, kd), dtype=torch.float32, device="cuda")
        ksk = torch.zeros((ns, hkv, b_max, kd), dtype=torch.float32, device="cuda")
        for si, n in enumerate(lens):
            geo = sws.Geometry([n], B)
            sws.sketch(gen.seq_tensor(cfg, l, si, "q", n, "cuda"), geo, kd, sd, cd, out=qsk[si],
                       ld_head=b_max * kd)
            sws.sketch(gen.seq_tensor(cfg, l, si, "k", n, "cuda"), geo, kd, sd, cd, out=ksk[si],
                       ld_head=b_max * kd)
        r = torch.zeros((ns, hq, b_max), dtype=torch.float32, device="cuda")
        sws.walk_update_row(qsk, ksk, cur, s, r_prev, r, mode=mode)
        torch.cuda.synchronize()
        for si, n in enumerate(lens):
            c = (n - 1) // B
            for h in range(hq):
                M = O.sketched_scores(f64(qsk[si, h, :c + 1]), f64(ksk[si, h // grp, :c + 1]))
                rp = None if r_prev is None else f64(r_prev[si, h, :c + 1])
                want = O.walk_row_variant(rp, M, c, s, name)
                got = f64(r[si, h])
                assert np.all(got[c + 1:] == 0)
                e = rowwise_rel_err(got[:c + 1], want)
                assert e <= 1e-4, (name, s, l, si, h, e)
        r_prev = r


def _paged_inputs(cfg, lens, share, layer=0):
    """Per-sequence K/V (sequence 1 reusing sequence 0's first `share` blocks
    when share > 0), the new token's q, a contiguous cache and a page table."""
    ns, B = len(lens), cfg.B
    K, V, q = [], [], []
    for s, n in enumerate(lens):
        k = gen.seq_tensor(cfg, layer, s, "k", n, "cuda")
        v = gen.seq_tensor(cfg, layer, s, "v", n, "cuda")
        if s == 1 and share:
            k[:share * B] = K[0][:share * B]
            v[:share * B] = V[0][:share * B]
        K.append(k)
        V.append(v)
        q.append(gen.seq_tensor(cfg, layer, s, "q", n, "cuda")[n - 1])
    table, num_pages = gen.page_table(lens, B, share_prefix_blocks=share)
    return K, V, torch.stack(q).contiguous(), table, num_pages


def _fill_pages(X, table, num_pages, B, dtype, tail):
    """Scatter per-sequence rows X[s] [n, hkv, d] into pages; rows past each
    sequence's end and unused pages hold `tail` (NaN), which the kernel must
    never read."""
    hkv, d = X[0].shape[1:]
    pages = torch.full((num_pages, B, hkv, d), tail, dtype=dtype, device="cuda")
    for s, x in enumerate(X):
        for j in range(-(-x.shape[0] // B)):
            rows = x[j * B:(j + 1) * B]
            pages[int(table[s, j]), :rows.shape[0]] = rows
    return pages


def _check_decode_rows(out, lse, qh, Kh, Vh, lens, lists, B, d, grp, tol):
    for s, n in enumerate(lens):
        for h in range(out.shape[1]):
            g = h // grp
            o_want, lse_want = O.query_attention(qh[s, h], Kh[s][:, g], Vh[s][:, g],
                                                 np.asarray(lists(s, h)), B, n - 1,
                                                 1.0 / math.sqrt(d))
            e = float(np.abs(out[s, h] - o_want).max())
            assert e <= tol, (s, h, e)
            assert abs(lse[s, h] - lse_want) <= max(tol, 1e-4), (s, h)


@pytest.mark.parametrize("d,B,hq,hkv,lens,share", [
    (128, 64, 8, 2, (1000, 2049, 64), 7),
    (64, 128, 4, 4, (700, 1, 1280), 0),
    (128, 64, 16, 1, (333, 4100), 2),
])
def test_decode_paged_bf16(d, B, hq, hkv, lens, share):
    """Paged bf16 cache (random page order, a shared prefix, NaN in every
    unused row and page): the output and lse equal the contiguous kernel's bit
    for bit, and the oracle's attention over the pages gathered by the table."""
    cfg = gen.CONFIGS["C4"].with_(d=d, B=B, hq=hq, hkv=hkv)
    ns, grp = len(lens), hq // hkv
    _print("paged bf16", d, B, hq, hkv, lens, share)
    K, V, q, table, num_pages = _paged_inputs(cfg, lens, share)
    kp = _fill_pages(K, table, num_pages, B, torch.bfloat16, float("nan"))
    vp = _fill_pages(V, table, num_pages, B, torch.bfloat16, float("nan"))
    max_ctx = max(lens)
    kc = torch.zeros((ns, max_ctx, hkv, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for s, n in enumerate(lens):
        kc[s, :n] = K[s]
        vc[s, :n] = V[s]
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cur = (ctx - 1) // B
    b_max = -(-max_ctx // B)
    gr = torch.Generator(device="cuda")
    gr.manual_seed(gen.seed_for(11, d, B, hq))
    r = torch.rand((ns, hq, b_max), generator=gr, device="cuda")
    uidx, ucnt, umask, idx, cnt = sws.select_topk_row(r, hq, hkv, cur, b_max, 25, per_head=True)
    tab = torch.from_numpy(table).cuda()
    for sparse in (True, False):
        u = (uidx, ucnt, umask) if sparse else (None, None, None)
        lse_p = torch.empty((ns, hq), dtype=torch.float32, device="cuda")
        lse_c = torch.empty_like(lse_p)
        out_p = sws.sparse_attn_decode_paged(q, kp, vp, tab, ctx, *u, lse=lse_p)
        out_c = sws.sparse_attn_decode(q, kc, vc, ctx, B, *u, lse=lse_c)
        torch.cuda.synchronize()
        assert torch.equal(out_p, out_c) and torch.equal(lse_p, lse_c), sparse
        Kh = [O.gather_pages(f64(kp), table[s], n, B) for s, n in enumerate(lens)]
        Vh = [O.gather_pages(f64(vp), table[s], n, B) for s, n in enumerate(lens)]
        ih, ch = idx.cpu().numpy(), cnt.cpu().numpy()
        lists = ((lambda s, h: ih[s, h, :ch[s, h]]) if sparse
                 else (lambda s, h: np.arange(-(-lens[s] // B))))
        _check_decode_rows(f64(out_p), f64(lse_p), f64(q), Kh, Vh, lens, lists, B, d, grp,
                           TOL_ATTN_BF16)


@pytest.mark.parametrize("d,B,hq,hkv,lens,share", [
    (128, 64, 8, 2, (1000, 2049, 64), 7),
    (64, 128, 8, 1, (700, 1281), 3),
])
def test_decode_paged_fp8(d, B, hq, hkv, lens, share):
    """fp8 e4m3 pages with per-tensor scales: the kernel's attention against
    the oracle on the codes decoded from the format's definition and scaled
    (code NaN in every unused row and page)."""
    cfg = gen.CONFIGS["C4"].with_(d=d, B=B, hq=hq, hkv=hkv)
    ns, grp = len(lens), hq // hkv
    _print("paged fp8", d, B, hq, hkv, lens, share)
    K, V, q, table, num_pages = _paged_inputs(cfg, lens, share)
    ks, vs = 0.0625, 0.02
    kp = _fill_pages([gen.to_fp8_e4m3(k, ks) for k in K], table, num_pages, B, torch.uint8, 0x7F)
    vp = _fill_pages([gen.to_fp8_e4m3(v, vs) for v in V], table, num_pages, B, torch.uint8, 0x7F)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cur = (ctx - 1) // B
    b_max = -(-max(lens) // B)
    gr = torch.Generator(device="cuda")
    gr.manual_seed(gen.seed_for(12, d, B, hq))
    r = torch.rand((ns, hq, b_max), generator=gr, device="cuda")
    uidx, ucnt, umask, idx, cnt = sws.select_topk_row(r, hq, hkv, cur, b_max, 25, per_head=True)
    tab = torch.from_numpy(table).cuda()
    kph, vph = kp.cpu().numpy(), vp.cpu().numpy()
    Kh = [O.fp8_e4m3_value(O.gather_pages(kph, table[s], n, B)) * ks for s, n in enumerate(lens)]
    Vh = [O.fp8_e4m3_value(O.gather_pages(vph, table[s], n, B)) * vs for s, n in enumerate(lens)]
    ih, ch = idx.cpu().numpy(), cnt.cpu().numpy()
    for sparse in (True, False):
        u = (uidx, ucnt, umask) if sparse else (None, None, None)
        lse = torch.empty((ns, hq), dtype=torch.float32, device="cuda")
        out = sws.sparse_attn_decode_paged(q, kp.view(torch.float8_e4m3fn),
                                           vp.view(torch.float8_e4m3fn), tab, ctx, *u,
                                           k_scale=ks, v_scale=vs, lse=lse)
        torch.cuda.synchronize()
        lists = ((lambda s, h: ih[s, h, :ch[s, h]]) if sparse
                 else (lambda s, h: np.arange(-(-lens[s] // B))))
        _check_decode_rows(f64(out), f64(lse), f64(q), Kh, Vh, lens, lists, B, d, grp,
                           TOL_ATTN_BF16)


@pytest.mark.parametrize("d,B,hq,hkv,lens,share", [
    (128, 64, 8, 2, (1000, 2049, 64), 7),
    (64, 128, 12, 3, (700, 1, 1281), 0),
])
def test_decode_head_major_layouts(d, B, hq, hkv, lens, share):
    """Head-major caches and pages (rows of one KV head contiguous) give the
    token-major result bit for bit: bf16 and fp32 contiguous caches, bf16 and
    fp8 pages (NaN in every unused row and page); the bf16 head-major output
    also against the oracle."""
    cfg = gen.CONFIGS["C4"].with_(d=d, B=B, hq=hq, hkv=hkv)
    ns, grp = len(lens), hq // hkv
    _print("head-major", d, B, hq, hkv, lens, share)
    K, V, q, table, num_pages = _paged_inputs(cfg, lens, share)
    max_ctx = max(lens)
    kc = torch.zeros((ns, max_ctx, hkv, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for s, n in enumerate(lens):
        kc[s, :n] = K[s]
        vc[s, :n] = V[s]
    hm = lambda x: x.permute(0, 2, 1, 3).contiguous()
    kp = _fill_pages(K, table, num_pages, B, torch.bfloat16, float("nan"))
    vp = _fill_pages(V, table, num_pages, B, torch.bfloat16, float("nan"))
    kp8 = _fill_pages([gen.to_fp8_e4m3(k, 0.0625) for k in K], table, num_pages, B, torch.uint8,
                      0x7F)
    vp8 = _fill_pages([gen.to_fp8_e4m3(v, 0.02) for v in V], table, num_pages, B, torch.uint8,
                      0x7F)
    f8 = lambda x: x.view(torch.float8_e4m3fn)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cur = (ctx - 1) // B
    b_max = -(-max_ctx // B)
    gr = torch.Generator(device="cuda")
    gr.manual_seed(gen.seed_for(13, d, B, hq))
    r = torch.rand((ns, hq, b_max), generator=gr, device="cuda")
    uidx, ucnt, umask, idx, cnt = sws.select_topk_row(r, hq, hkv, cur, b_max, 25, per_head=True)
    tab = torch.from_numpy(table).cuda()
    q32 = q.float()
    for sparse in (True, False):
        u = (uidx, ucnt, umask) if sparse else (None, None, None)
        pairs = [
            (lambda m: sws.sparse_attn_decode(q, hm(kc) if m else kc, hm(vc) if m else vc, ctx, B,
                                              *u, lse=lse_of(), head_major=m)),
            (lambda m: sws.sparse_attn_decode(q32, (hm(kc) if m else kc).float(),
                                              (hm(vc) if m else vc).float(), ctx, B, *u,
                                              lse=lse_of(), head_major=m)),
            (lambda m: sws.sparse_attn_decode_paged(q, hm(kp) if m else kp, hm(vp) if m else vp,
                                                    tab, ctx, *u, lse=lse_of(), head_major=m)),
            (lambda m: sws.sparse_attn_decode_paged(q, f8(hm(kp8) if m else kp8),
                                                    f8(hm(vp8) if m else vp8), tab, ctx, *u,
                                                    k_scale=0.0625, v_scale=0.02, lse=lse_of(),
                                                    head_major=m)),
        ]
        for n_call, call in enumerate(pairs):
            lses = []
            lse_of = lambda: lses.append(torch.empty((ns, hq), dtype=torch.float32,
                                                     device="cuda")) or lses[-1]
            o_t = call(False)
            o_h = call(True)
            torch.cuda.synchronize()
            assert torch.equal(o_t, o_h) and torch.equal(lses[0], lses[1]), (sparse, n_call)
            if n_call == 0:
                Kh = [K[s].double().cpu().numpy() for s in range(ns)]
                Vh = [V[s].double().cpu().numpy() for s in range(ns)]
                ih, ch = idx.cpu().numpy(), cnt.cpu().numpy()
                lists = ((lambda s, h: ih[s, h, :ch[s, h]]) if sparse
                         else (lambda s, h: np.arange(-(-lens[s] // B))))
                _check_decode_rows(f64(o_h), f64(lses[1]), f64(q), Kh, Vh, lens, lists, B, d,
                                   grp, TOL_ATTN_BF16)


def test_decode_paged_continuous_batching():
    """Continuous batching over one page pool: between two calls a sequence
    leaves (its pages go back to the pool), a new one joins on pages taken
    from the pool (some of them the leaver's, overwritten), the others grow
    by one token (the second crossing into a fresh page), and the batch
    slots are reordered; only the block table and ctx_len change.  Every
    pool page no sequence maps holds NaN.  Both calls equal the contiguous
    kernel on the gathered caches bit for bit, and the oracle."""
    cfg = gen.CONFIGS["C4"].with_(d=128, B=64, hq=8, hkv=2)
    B, d, hq, hkv = cfg.B, cfg.d, cfg.hq, cfg.hkv
    grp = hq // hkv
    num_pages = 40
    rng = np.random.default_rng(gen.seed_for(15, d, B, hq))
    free = list(rng.permutation(num_pages))
    kp = torch.full((num_pages, B, hkv, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    seqs = {}                                   # name -> dict(K, V, q, pages)

    def add_tokens(name, n_new, layer):
        st = seqs[name]
        n0 = st["K"].shape[0] if st["K"] is not None else 0
        k = gen.seq_tensor(cfg, layer, st["sid"], "k", n0 + n_new, "cuda")
        v = gen.seq_tensor(cfg, layer, st["sid"], "v", n0 + n_new, "cuda")
        st["K"], st["V"] = k, v
        st["q"] = gen.seq_tensor(cfg, layer, st["sid"], "q", n0 + n_new, "cuda")[-1]
        for j in range(-(-(n0 + n_new) // B)):
            if j >= len(st["pages"]):
                st["pages"].append(int(free.pop(0)))
            pg = st["pages"][j]
            rows = slice(j * B, min((j + 1) * B, n0 + n_new))
            kp[pg, :rows.stop - rows.start] = k[rows]
            vp[pg, :rows.stop - rows.start] = v[rows]

    def run(order, layer_seed):
        lens = [seqs[n]["K"].shape[0] for n in order]
        width = max(len(seqs[n]["pages"]) for n in order) + 2
        table = np.full((len(order), width), -1, dtype=np.int32)
        for s, n in enumerate(order):
            table[s, :len(seqs[n]["pages"])] = seqs[n]["pages"]
        tab = torch.from_numpy(table).cuda()
        ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
        q = torch.stack([seqs[n]["q"] for n in order]).contiguous()
        cur = (ctx - 1) // B
        b_max = width
        gr = torch.Generator(device="cuda")
        gr.manual_seed(layer_seed)
        r = torch.rand((len(order), hq, b_max), generator=gr, device="cuda")
        uidx, ucnt, umask, idx, cnt = sws.select_topk_row(r, hq, hkv, cur, b_max, 25,
                                                          per_head=True)
        lse_p = torch.empty((len(order), hq), dtype=torch.float32, device="cuda")
        out_p = sws.sparse_attn_decode_paged(q, kp, vp, tab, ctx, uidx, ucnt, umask, lse=lse_p)
        kc = torch.zeros((len(order), max(lens), hkv, d), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        for s, n in enumerate(order):
            kc[s, :lens[s]] = seqs[n]["K"]
            vc[s, :lens[s]] = seqs[n]["V"]
        lse_c = torch.empty_like(lse_p)
        out_c = sws.sparse_attn_decode(q, kc, vc, ctx, B, uidx, ucnt, umask, lse=lse_c)
        torch.cuda.synchronize()
        assert torch.equal(out_p, out_c) and torch.equal(lse_p, lse_c)
        Kh = [O.gather_pages(f64(kp), table[s], n, B) for s, n in enumerate(lens)]
        Vh = [O.gather_pages(f64(vp), table[s], n, B) for s, n in enumerate(lens)]
        ih, ch = idx.cpu().numpy(), cnt.cpu().numpy()
        _check_decode_rows(f64(out_p), f64(lse_p), f64(q), Kh, Vh, lens,
                           lambda s, h: ih[s, h, :ch[s, h]], B, d, grp, TOL_ATTN_BF16)

    _print("continuous batching")
    for sid, (name, n) in enumerate((("A", 300), ("B", 500), ("C", 2 * B))):
        seqs[name] = {"sid": sid, "K": None, "V": None, "q": None, "pages": []}
        add_tokens(name, n, 0)
    run(["A", "B", "C"], 101)
    # A leaves: its pages return to the pool (and are poisoned until reused)
    for pg in seqs.pop("A")["pages"]:
        kp[pg] = float("nan")
        vp[pg] = float("nan")
        free.insert(0, pg)
    seqs["D"] = {"sid": 3, "K": None, "V": None, "q": None, "pages": []}
    add_tokens("D", 200, 0)                     # takes the leaver's pages first
    add_tokens("B", 1, 0)
    add_tokens("C", 1, 0)                       # crosses into a new page
    assert len(seqs["C"]["pages"]) == 3
    run(["C", "D", "B"], 102)


@pytest.mark.parametrize("dtype,d,B,kd,hq,hkv", [
    (torch.bfloat16, 128, 64, 32, 12, 3),
    (torch.float32, 64, 128, 16, 4, 4),
])
def test_sketch_append_qk_matches_two_appends(dtype, d, B, kd, hq, hkv):
    """The fused query / key append leaves the running sums and both sketch
    caches bit for bit where two separate appends leave them, over steps that
    open, fill and complete blocks."""
    _print("append_qk", dtype, d, B, kd, hq, hkv)
    ns, steps = 3, 2 * B + 5
    pos0 = torch.tensor([0, B - 1, B + 7], dtype=torch.int32, device="cuda")
    b_max = int((pos0.max() + steps) // B) + 1
    gr = torch.Generator(device="cuda")
    gr.manual_seed(gen.seed_for(14, d, B, hq))
    q = torch.randn((steps, ns, hq, d), generator=gr, device="cuda").to(dtype)
    k = torch.randn((steps, ns, hkv, d), generator=gr, device="cuda").to(dtype)
    signs, cols = gen.hadamard_tables(d, kd)
    sd, cd = torch.from_numpy(signs).cuda(), torch.from_numpy(cols).cuda()
    st = [[torch.zeros((ns, h, d), device="cuda"), torch.zeros((ns, h, b_max, kd), device="cuda")]
          for _ in range(2) for h in (hq, hkv)]
    for t in range(steps):
        pos = pos0 + t
        sws.sketch_append(q[t], pos, B, kd, sd, cd, st[0][0], st[0][1])
        sws.sketch_append(k[t], pos, B, kd, sd, cd, st[1][0], st[1][1])
        sws.sketch_append_qk(q[t], k[t], pos, B, kd, sd, cd, st[2][0], st[3][0], st[2][1],
                             st[3][1])
        if t % 17 == 0 or t == steps - 1:
            torch.cuda.synchronize()
            for a, b in ((st[0], st[2]), (st[1], st[3])):
                assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), t


def test_decode_snapshot_resume_bit_identical():
    """The decode state (sketch caches, running block sums, walk rows) is plain
    device memory: a copy taken after some steps, restored, and stepped again
    reproduces every later output bit for bit (no order-dependent atomics or
    hidden state in the kernels)."""
    cfg = gen.CONFIGS["C4"].with_(d=128, B=64, hq=8, hkv=2, k=32)
    B, d, kd, hq, hkv = cfg.B, cfg.d, cfg.k, cfg.hq, cfg.hkv
    prefixes, steps, n_layers, rho = (190, 250), 20, 2, 30
    ns = len(prefixes)
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
              "rk": torch.zeros((ns, hkv, d), device="cuda"),
              "r": torch.zeros((ns, hq, b_max), device="cuda")}
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
        layers.append({"full": full, "kc": kc, "vc": vc, "st": st})
    P_t = torch.tensor(prefixes, dtype=torch.int32, device="cuda")

    def step(t):
        pos = P_t + t
        cur = pos // B
        outs = []
        for l, L in enumerate(layers):
            st = L["st"]
            qn = torch.stack([L["full"][s]["q"][prefixes[s] + t] for s in range(ns)]).contiguous()
            kn = torch.stack([L["full"][s]["k"][prefixes[s] + t] for s in range(ns)]).contiguous()
            sws.sketch_append(qn, pos, B, kd, sd, cd, st["rq"], st["qsk"])
            sws.sketch_append(kn, pos, B, kd, sd, cd, st["rk"], st["ksk"])
            sws.walk_update_row(st["qsk"], st["ksk"], cur, cfg.s,
                                None if l == 0 else layers[l - 1]["st"]["r"], st["r"])
            u = sws.select_topk_row(st["r"], hq, hkv, cur, b_max, rho, per_head=True)
            lse = torch.empty((ns, hq), device="cuda")
            out = sws.sparse_attn_decode(qn, L["kc"], L["vc"], pos + 1, B, u[0], u[1], u[2],
                                         lse=lse)
            # list entries past each count are unspecified: keep the defined ones
            uidx, ucnt, umask, idx, cnt = [x.cpu() for x in u]
            lists = [(uidx[s_, g, :ucnt[s_, g]], umask[s_, g, :ucnt[s_, g]])
                     for s_ in range(ns) for g in range(hkv)]
            lists += [idx[s_, h, :cnt[s_, h]] for s_ in range(ns) for h in range(hq)]
            outs.append([st["r"].clone(), ucnt, cnt, out, lse,
                         *[x for pair in lists[:ns * hkv] for x in pair], *lists[ns * hkv:]])
        return outs

    for t in range(8):
        step(t)
    snap = [{k: v.clone() for k, v in L["st"].items()} for L in layers]
    first = [step(t) for t in range(8, steps)]
    for L, sn in zip(layers, snap):
        for k, v in sn.items():
            L["st"][k].copy_(v)
    second = [step(t) for t in range(8, steps)]
    torch.cuda.synchronize()
    for a_t, b_t in zip(first, second):
        for a_l, b_l in zip(a_t, b_t):
            for x, y in zip(a_l, b_l):
                assert torch.equal(x, y)


@pytest.mark.parametrize("dtype,d,B,hq,hkv,lens", [
    ("bf16", 128, 64, 8, 2, (1000, 2049, 64)),
    ("bf16", 128, 128, 4, 4, (700, 1, 1280)),
    ("f32", 64, 64, 4, 2, (1000, 333)),
])
def test_decode_large_scores_across_splits(dtype, d, B, hq, hkv, lens):
    """Decode attention when the scores are far outside the usual range: key
    magnitudes grow along the context so single scores pass 2^128 above the
    first keys' (in log2 units), with a 1.5x jump in one 16-key half of every
    32 keys, for KV head 0; KV head 1 starts above 64 and grows.  The split
    workgroups' partial states and the combine's rescaling must still give
    the exact softmax: every (sequence, head) against the oracle, dense
    lists.  scale * log2(e) = 1/8, so the scores are exact up to fp32
    accumulation."""
    ns = len(lens)
    max_ctx = max(lens)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda")
    g.manual_seed(gen.seed_for(16, d, B, hq))
    pos = torch.arange(max_ctx, dtype=torch.float32, device="cuda")
    half = ((pos.long() % 32) // 16) == 1
    mag0 = (0.5 + 45.0 * (pos / max_ctx) ** 2) * torch.where(half, 1.5, 1.0)
    mag1 = (60.0 + 60.0 * pos / max_ctx) * torch.where(half, 1.5, 1.0)
    # (scaled by 128 / d so the score range does not shrink with d)
    mags = torch.stack([mag0, mag1] + [mag0] * max(0, hkv - 2), 1)[:, :hkv] * (128.0 / d)
    kc = (torch.randn((ns, max_ctx, hkv, d), generator=g, device="cuda") * mags[None, :, :, None]).to(tdt)
    vc = torch.randn((ns, max_ctx, hkv, d), generator=g, device="cuda").to(tdt)
    q = torch.randn((ns, hq, d), generator=g, device="cuda").to(tdt)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 0.125 * math.log(2.0)
    lse = torch.empty((ns, hq), dtype=torch.float32, device="cuda")
    out = sws.sparse_attn_decode(q, kc, vc, ctx, B, None, None, None, scale=scale, lse=lse)
    torch.cuda.synchronize()
    Q, K, V, Og, Lg = f64(q), f64(kc), f64(vc), f64(out), f64(lse)
    # fp32: scores in the hundreds carry fp32 rounding of about 1e-5 (natural
    # units), a relative error of that size in every weight; 1e-3 still
    # rejects any wrong rescale (an O(1) error)
    tol = TOL_ATTN_BF16 if dtype == "bf16" else 1e-3
    grp = hq // hkv
    worst = 0.0
    for s, n in enumerate(lens):
        for h in range(hq):
            gg = h // grp
            nb = -(-n // B)
            o_want, lse_want = O.query_attention(Q[s, h], K[s, :, gg], V[s, :, gg],
                                                 np.arange(nb), B, n - 1, scale)
            assert np.isfinite(Og[s, h]).all(), (s, h)
            e = float(np.abs(Og[s, h] - o_want).max())
            # the log-sum-exp is large here (hundreds); fp32 keeps it to ~1e-5 relative
            e2 = abs(Lg[s, h] - lse_want)
            worst = max(worst, e)
            assert e <= tol, (s, h, e)
            assert e2 <= max(tol, 1e-5 * abs(lse_want)), (s, h, e2, lse_want)
    # the inputs do reach scores far apart within one context (log2 units)
    sl = int(np.argmax(lens))
    s2 = (Q[sl, 0] / 8.0) @ K[sl, :lens[sl], 0].T
    assert s2.max() - np.abs(s2[:32]).max() > 128
    _print("decode large scores", dtype, d, B, hq, hkv, lens, "worst", worst)


def test_decode_at_the_pair_limit():
    """The largest decode batch the C ABI takes: 1024 sequences x 8 KV heads
    = 8192 (sequence, KV head) pairs (the split kernels' plan fills its whole
    LDS table), short contexts of 1 to 200 tokens, random union lists with
    random head masks (every head keeps the open block): every (sequence,
    head) against the oracle.  One pair more is rejected on the host."""
    ns, hq, hkv, d, B = 1024, 16, 8, 64, 64
    grp = hq // hkv
    rng = np.random.default_rng(2048)
    lens = rng.integers(1, 201, size=ns)
    max_ctx = int(lens.max())
    uw = -(-max_ctx // B)
    uidx = np.zeros((ns, hkv, uw), np.int32)
    ucnt = np.zeros((ns, hkv), np.int32)
    umask = np.zeros((ns, hkv, uw), np.int32)
    for s in range(ns):
        nb = -(-int(lens[s]) // B)
        for g in range(hkv):
            keep = [j for j in range(nb - 1) if rng.random() < 0.5] + [nb - 1]
            ucnt[s, g] = len(keep)
            uidx[s, g, :len(keep)] = keep
            for e in range(len(keep)):
                umask[s, g, e] = (1 << grp) - 1 if e == len(keep) - 1 else int(rng.integers(1, 1 << grp))
    g_ = torch.Generator(device="cuda")
    g_.manual_seed(gen.seed_for(17, ns, hkv))
    kc = torch.randn((ns, max_ctx, hkv, d), generator=g_, device="cuda").to(torch.bfloat16)
    vc = torch.randn((ns, max_ctx, hkv, d), generator=g_, device="cuda").to(torch.bfloat16)
    q = torch.randn((ns, hq, d), generator=g_, device="cuda").to(torch.bfloat16)
    ctx = torch.from_numpy(lens.astype(np.int32)).cuda()
    lse = torch.empty((ns, hq), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    out = sws.sparse_attn_decode(q, kc, vc, ctx, B, torch.from_numpy(uidx).cuda(),
                                 torch.from_numpy(ucnt).cuda(), torch.from_numpy(umask).cuda(),
                                 scale=scale, lse=lse)
    torch.cuda.synchronize()
    Q, K, V, Og, Lg = f64(q), f64(kc), f64(vc), f64(out), f64(lse)
    worst = 0.0
    for s in range(ns):
        n = int(lens[s])
        for h in range(hq):
            g, hb = h // grp, 1 << (h % grp)
            lst = [int(uidx[s, g, e]) for e in range(ucnt[s, g]) if umask[s, g, e] & hb]
            o_want, lse_want = O.query_attention(Q[s, h], K[s, :, g], V[s, :, g], lst, B, n - 1,
                                                 scale)
            e = float(np.abs(Og[s, h] - o_want).max())
            worst = max(worst, e)
            assert e <= TOL_ATTN_BF16, (s, h, e)
            assert abs(Lg[s, h] - lse_want) <= TOL_ATTN_BF16, (s, h)
    # one pair past the limit (8193 sequences x 1 KV head): rejected before any launch
    q1 = torch.zeros((8193, hq, d), dtype=torch.bfloat16, device="cuda")
    k1 = torch.zeros((8193, 1, 1, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sws.SwsError) as ei:
        sws.sparse_attn_decode(q1, k1, k1, torch.ones(8193, dtype=torch.int32, device="cuda"), B,
                               None, None, None, scale=scale)
    assert ei.value.code == 3
    _print("decode pair limit", ns * hkv, "worst", worst)
