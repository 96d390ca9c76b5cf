"""GPU edge cases: empty batches, the largest rows the decode kernels accept
(4096 blocks, the streaming form of the row walk, group size 16), sketch
dimensions that are not a power of two, prefill selection over more than
1024 blocks per sequence, and prefill attention on a sequence whose K and V
span more than 2^31 elements.  Everything is checked against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import dynamic_block_sparse_sws_amd as sws
import gen
import oracle as O
from gpu_util import f64, rowwise_rel_err, TOL_ATTN_BF16, TOL_WALK

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _rand(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(gen.seed_for(31, seed))
    return torch.randn(shape, generator=g, device="cuda")


def test_empty_batches_launch_nothing():
    """n_seqs = 0 (or no blocks) is a valid call for every entry point: it
    returns SWS_OK and leaves the outputs untouched."""
    L = sws.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    x = torch.zeros((4, 2, 128), dtype=torch.bfloat16, device="cuda")
    i32 = torch.zeros(8, dtype=torch.int32, device="cuda")
    signs = torch.ones(128, dtype=torch.int8, device="cuda")
    cols = torch.arange(32, dtype=torch.int32, device="cuda")
    sentinel = torch.full((4096,), 7.0, device="cuda")
    isent = torch.full((4096,), 7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(1 << 20, L.sws_decode_workspace_size(0, 4, 2, 128, 64, 0)),
                     dtype=torch.uint8, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    f = ctypes.c_float
    assert L.sws_sketch(P(x), 1, P(i32), P(i32), 0, 0, 2, 128, 64, 32, P(signs), P(cols),
                        P(sentinel), 64 * 32, None, st) == 0
    assert L.sws_sketch_append(P(x), 1, P(i32), 0, 2, 128, 64, 32, P(signs), P(cols),
                               P(sentinel), P(sentinel), 4, st) == 0
    assert L.sws_walk_update(P(sentinel), P(sentinel), 4, 2, 32, P(i32), 0, 0, 0, 8, None,
                             P(sentinel), st) == 0
    assert L.sws_walk_update_row(P(sentinel), P(sentinel), 4, 2, 32, 0, P(i32), 4, 8, None,
                                 P(sentinel), st) == 0
    assert L.sws_select_topk(P(sentinel), 4, P(i32), 0, 0, 0, 20, 0, 4, P(isent), P(isent),
                             st) == 0
    assert L.sws_select_topk_row(P(sentinel), 4, 2, 0, P(i32), 4, 20, 0, 4, P(isent), P(isent),
                                 P(isent), P(isent), P(isent), 4, st) == 0
    assert L.sws_sparse_attn_prefill(P(x), P(x), P(x), 1, P(i32), P(i32), 0, 0, 0, 4, 2, 128, 64,
                                     None, None, 0, f(0.1), P(x), None, P(ws), ws.numel(),
                                     st) == 0
    assert L.sws_sparse_attn_decode(P(x), P(x), P(x), 1, P(i32), 0, 64, 4, 2, 128, 64, None,
                                    None, None, 0, f(0.1), P(x), None, P(ws), ws.numel(),
                                    st) == 0
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all()) and bool((isent == 7).all())


@pytest.mark.parametrize("b,k,s,hq,hkv", [
    (4096, 32, 3, 4, 2),     # rows past 1280 blocks: sketches streamed every hop
    (2600, 24, 4, 4, 1),     # k not a power of two (padded to 32)
    (700, 64, 2, 2, 2),      # k = 64 past 512 blocks
    (1280, 32, 8, 4, 2),     # the largest rows held in registers (5 per segment)
    (768, 32, 8, 4, 2),      # four-wave form: its largest rows at k = 32 (12 per lane)
    (384, 64, 5, 4, 4),      # four-wave form at k = 64 (6 per lane)
    (1024, 16, 8, 8, 2),     # four-wave form at k = 16 (16 per lane)
    (37, 32, 8, 2, 1),       # short rows: most lanes hold no row
])
def test_walk_row_long_and_odd_rows(b, k, s, hq, hkv):
    _print("walk row", b, k, s, hq, hkv)
    ns = 2
    qsk = _rand((ns, hq, b, k), b + k)
    ksk = _rand((ns, hkv, b, k), b + k + 1)
    cur = torch.tensor([b - 1, b // 2 + 3], dtype=torch.int32, device="cuda")
    rp = _rand((ns, hq, b), b + 2).abs()
    rp /= rp.amax(dim=2, keepdim=True)
    out = torch.empty((ns, hq, b), device="cuda")
    for with_prev in (False, True):
        sws.walk_update_row(qsk, ksk, cur, s, rp if with_prev else None, out)
        torch.cuda.synchronize()
        qh, kh, rph, oh = f64(qsk), f64(ksk), f64(rp), f64(out)
        grp = hq // hkv
        for si in range(ns):
            c = int(cur[si])
            for h in (0, hq - 1):
                M = O.sketched_scores(qh[si, h, :c + 1], kh[si, h // grp, :c + 1])
                want = O.walk_row(rph[si, h, :c + 1] if with_prev else None, M, c, s)
                e = rowwise_rel_err(oh[si, h, :c + 1], want)
                assert e <= TOL_WALK, (b, k, si, h, with_prev, e)
                assert np.all(oh[si, h, c + 1:] == 0)


@pytest.mark.parametrize("b,hq,hkv,rho", [(4096, 32, 2, 20), (2049, 8, 8, 7), (3000, 16, 4, 50)])
def test_select_row_long_rows(b, hq, hkv, rho):
    """Decode selection and GQA union on the largest rows (E = 64 keys per
    lane), groups of 16, 1 and 4 query heads, bit-exact on the same fp32 row."""
    _print("select row", b, hq, hkv, rho)
    ns = 2
    r = _rand((ns, hq, b), b + hq)
    r[:, :, 0:b - 1:97] = r[:, :, 1:b:97]     # planted ties
    cur = torch.tensor([b - 1, b - 200], dtype=torch.int32, device="cuda")
    uidx, ucnt, umask, idx, cnt = sws.select_topk_row(r, hq, hkv, cur, b, rho, per_head=True)
    torch.cuda.synchronize()
    rh = r.cpu().numpy()
    grp = hq // hkv
    for si in range(ns):
        c = int(cur[si])
        tau = O.n_select(rho, c + 1)
        for g in range(hkv):
            want = {}
            for hh in range(grp):
                h = g * grp + hh
                lst = O.select_row(rh[si, h], c, tau).tolist()
                assert idx[si, h, :cnt[si, h]].tolist() == lst, (si, h)
                for m in lst:
                    want[m] = want.get(m, 0) | (1 << hh)
            n_u = int(ucnt[si, g])
            assert uidx[si, g, :n_u].tolist() == sorted(want)
            got_mask = umask[si, g, :n_u].cpu().numpy().astype(np.uint32).tolist()
            assert got_mask == [want[m] for m in sorted(want)]


def test_prefill_select_more_than_1024_blocks():
    """Prefill selection for sequences of 2048 and 1500 blocks (E = 64 keys
    per lane), bit-exact against the oracle on the same fp32 walk state."""
    B, hq, rho = 64, 2, 20
    geo = sws.Geometry([2048 * B, 1500 * B - 17], B)
    R = _rand((geo.walk_numel(hq),), 77)
    idx, cnt = sws.select_topk(R, hq, geo, rho)
    torch.cuda.synchronize()
    Rh = R.cpu().numpy()
    for si, nb in enumerate(geo.blocks):
        off = geo.walk_offset(si, hq)
        for h in range(hq):
            Rm = Rh[off + h * nb * nb: off + (h + 1) * nb * nb].reshape(nb, nb)
            tau = O.n_select(rho, nb)
            for i in list(range(0, nb, 97)) + [nb - 1]:
                gb = geo.cu_blocks_host[si] + i
                want = (np.arange(i + 1) if i <= tau else O.select_row(Rm[i], i, tau)).tolist()
                assert idx[h, gb, :cnt[h, gb]].tolist() == want, (si, h, i)


def test_prefill_attention_offsets_past_2_31():
    """Prefill attention on a sequence whose K and V span more than 2^31
    elements (n * hkv * d > 2^31: 64 KV heads, d = 128, 262,545 tokens), with
    every query block keeping block 0, the block farthest from the sequence's
    end, plus blocks i // 2, i - 1 and itself: sampled query blocks (first,
    middle, the partial last one) of the first and last head against the
    oracle."""
    d, B, hq, hkv = 128, 128, 64, 64
    n = (1 << 31) // (hkv * d) + 3 * B + 17
    geo = sws.Geometry([n], B)
    b = geo.blocks[0]
    _print("offsets past 2^31: n", n, "blocks", b)

    def bf16_rand(heads, seed):
        x = torch.empty((n, heads, d), dtype=torch.bfloat16, device="cuda")
        g = torch.Generator(device="cuda")
        g.manual_seed(gen.seed_for(31, seed))
        for t0 in range(0, n, 65536):
            t1 = min(n, t0 + 65536)
            x[t0:t1] = torch.randn((t1 - t0, heads, d), generator=g, device="cuda").bfloat16()
        return x

    q, k, v = bf16_rand(hq, 91), bf16_rand(hkv, 92), bf16_rand(hkv, 93)
    lists = [sorted({0, i // 2, max(i - 1, 0), i}) for i in range(b)]
    width = 4
    idx_h = np.zeros((hq, b, width), dtype=np.int32)
    cnt_h = np.zeros((hq, b), dtype=np.int32)
    for i, lst in enumerate(lists):
        idx_h[:, i, :len(lst)] = lst
        cnt_h[:, i] = len(lst)
    idx = torch.from_numpy(idx_h).cuda()
    cnt = torch.from_numpy(cnt_h).cuda()
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    out = sws.sparse_attn_prefill(q, k, v, geo, idx, cnt, lse=lse)
    torch.cuda.synchronize()
    rows = [0, 1, b // 2, b - 1]
    scale = 1.0 / np.sqrt(d)
    for h in (0, hq - 1):
        want = O.sparse_attention_rows(f64(q[:, h]), f64(k[:, h]), f64(v[:, h]), lists, B,
                                       scale, rows)
        for i in rows:
            a, e = i * B, min((i + 1) * B, n)
            o_w, lse_w = want[i]
            err = float(np.abs(f64(out[a:e, h]) - o_w).max())
            lerr = float(np.abs(f64(lse[h, a:e]) - lse_w).max())
            assert err <= TOL_ATTN_BF16, (h, i, err)
            assert lerr <= TOL_ATTN_BF16, (h, i, lerr)
        _print("head", h, "ok")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_malformed_lists_are_clamped(dtype):
    """Index lists with entries above the query block, past the sequence or
    negative, and counts above the list width: the kernels clamp each entry to
    [0, i] and the count to [0, min(width, i + 1)], so the result is the
    attention over the clamped list (the oracle on that list), never a stray
    access."""
    B, d, hq, hkv = 64, 128, 4, 2
    lens = [700, 300]
    geo = sws.Geometry(lens, B)
    q = _rand((geo.total_tokens, hq, d), 1).to(dtype)
    k = _rand((geo.total_tokens, hkv, d), 2).to(dtype)
    v = _rand((geo.total_tokens, hkv, d), 3).to(dtype)
    width = 4
    rng = np.random.default_rng(7)
    idx = np.zeros((hq, geo.total_blocks, width), np.int32)
    cnt = np.zeros((hq, geo.total_blocks), np.int32)
    for h in range(hq):
        for gb in range(geo.total_blocks):
            idx[h, gb] = rng.integers(-3, 20, size=width)
            cnt[h, gb] = rng.integers(1, width + 4)
    lse = torch.empty((hq, geo.total_tokens), dtype=torch.float32, device="cuda")
    out = sws.sparse_attn_prefill(q, k, v, geo, torch.from_numpy(idx).cuda(),
                                  torch.from_numpy(cnt).cuda(), lse=lse)
    torch.cuda.synchronize()
    Q, K, V, O_, L_ = (f64(t) for t in (q, k, v, out, lse))
    tol = TOL_ATTN_BF16 if dtype == torch.bfloat16 else 1e-5
    grp = hq // hkv
    for s, n in enumerate(lens):
        t0, b0, b = int(geo.cu_seqlens_host[s]), int(geo.cu_blocks_host[s]), geo.blocks[s]
        for h in range(hq):
            g = h // grp
            lists = []
            for i in range(b):
                nb = min(max(int(cnt[h, b0 + i]), 0), min(width, i + 1))
                lists.append(np.clip(idx[h, b0 + i, :nb].astype(np.int64), 0, i))
            res = O.sparse_attention_rows(Q[t0:t0 + n, h], K[t0:t0 + n, g], V[t0:t0 + n, g],
                                          lists, B, 1 / np.sqrt(d), range(b))
            for i in range(b):
                o_w, lse_w = res[i]
                a = t0 + i * B
                assert np.abs(O_[a:a + o_w.shape[0], h] - o_w).max() <= tol, (s, h, i)
                assert np.abs(L_[h, a:a + o_w.shape[0]] - lse_w).max() <= max(tol, 1e-4)


def test_decode_context_past_the_cache_and_long_union_counts_are_clamped():
    """A context length past the cache's rows is read as the whole cache, and
    a union count above the list width as the width: the result is the
    oracle's attention of the cache's last row over the clamped list."""
    B, d, hq, hkv, max_ctx = 64, 128, 8, 2, 1000
    ns = 2
    q = _rand((ns, hq, d), 4).to(torch.bfloat16)
    kc = _rand((ns, max_ctx, hkv, d), 5).to(torch.bfloat16)
    vc = _rand((ns, max_ctx, hkv, d), 6).to(torch.bfloat16)
    last = (max_ctx - 1) // B
    uw = 6
    rng = np.random.default_rng(8)
    uidx = rng.integers(-2, last + 5, size=(ns, hkv, uw)).astype(np.int32)
    ucnt = np.full((ns, hkv), uw + 3, np.int32)
    umask = rng.integers(1, 1 << (hq // hkv), size=(ns, hkv, uw)).astype(np.int32)
    ctx = torch.tensor([max_ctx + 100, max_ctx + 1], dtype=torch.int32, device="cuda")
    lse = torch.empty((ns, hq), dtype=torch.float32, device="cuda")
    out = sws.sparse_attn_decode(q, kc, vc, ctx, B, torch.from_numpy(uidx).cuda(),
                                 torch.from_numpy(ucnt).cuda(), torch.from_numpy(umask).cuda(),
                                 lse=lse)
    torch.cuda.synchronize()
    Qh, Kh, Vh, Oh, Lh = (f64(t) for t in (q, kc, vc, out, lse))
    grp = hq // hkv
    for s in range(ns):
        for h in range(hq):
            g, bit = h // grp, h % grp
            lst = np.array([min(max(int(e), 0), last)
                            for e, m in zip(uidx[s, g], umask[s, g]) if (m >> bit) & 1],
                           np.int64)
            if len(lst) == 0:
                continue
            o_w, lse_w = O.query_attention(Qh[s, h], Kh[s, :, g], Vh[s, :, g], lst, B,
                                           max_ctx - 1, 1 / np.sqrt(d))
            assert np.abs(Oh[s, h] - o_w).max() <= TOL_ATTN_BF16, (s, h)
            assert abs(Lh[s, h] - lse_w) <= TOL_ATTN_BF16, (s, h)


def test_prefill_walk_at_every_row_alignment():
    """The prefill walk on sequences of 200, 201, 202 and 131 blocks (walk-state
    rows of every length modulo 4, so rows that are and are not 16-byte
    aligned; partial last row tiles) plus a one-tile sequence of 40 blocks,
    two layers (the second carries the walk state), every stage against the
    oracle."""
    from gpu_util import PrefillRun, check_prefill_run
    cfg = gen.CONFIGS["C2"].with_(d=128, B=64, hq=4, hkv=2, k=32, s=8)
    seqlens = (200 * 64 - 5, 201 * 64, 202 * 64 - 63, 130 * 64 + 3, 40 * 64)
    _print("walk alignment", seqlens)
    run = PrefillRun(cfg, seqlens, 2, 20, n_dense=0)
    assert [b % 4 for b in run.geo.blocks] == [0, 1, 2, 3, 0]
    w = check_prefill_run(run, attn_rows_per_head=2, attn_heads=[0])
    _print("worst", w)


@pytest.mark.parametrize("hq", [2, 3])
def test_head_pairing_equals_one_head_form(hq):
    """At B = 64 a KV group of two or more query heads runs two heads per
    workgroup over the merge of their lists (three heads: a pair and a lone
    head).  Each head's output and log-sum-exp equal, bit for bit, what the
    one-head form computes for that head alone (one query head on the KV
    head), on random ascending lists that differ between the heads."""
    B, d = 64, 128
    lens = [900, 333]
    geo = sws.Geometry(lens, B)
    T = geo.total_tokens
    q = _rand((T, hq, d), 41).to(torch.bfloat16)
    k = _rand((T, 1, d), 42).to(torch.bfloat16)
    v = _rand((T, 1, d), 43).to(torch.bfloat16)
    rng = np.random.default_rng(44)
    width = 6
    idx = np.zeros((hq, geo.total_blocks, width), np.int32)
    cnt = np.zeros((hq, geo.total_blocks), np.int32)
    for h in range(hq):
        for s, b in enumerate(geo.blocks):
            for i in range(b):
                gb = int(geo.cu_blocks_host[s]) + i
                pick = np.sort(rng.choice(i, size=min(i, width - 1), replace=False)) if i else []
                lst = list(pick) + [i]
                idx[h, gb, :len(lst)] = lst
                cnt[h, gb] = len(lst)
    idx_d, cnt_d = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    lse = torch.empty((hq, T), dtype=torch.float32, device="cuda")
    out = sws.sparse_attn_prefill(q, k, v, geo, idx_d, cnt_d, lse=lse)
    for h in range(hq):
        lse1 = torch.empty((1, T), dtype=torch.float32, device="cuda")
        out1 = sws.sparse_attn_prefill(q[:, h:h + 1].contiguous(), k, v, geo,
                                       idx_d[h:h + 1].contiguous(), cnt_d[h:h + 1].contiguous(),
                                       lse=lse1)
        torch.cuda.synchronize()
        assert torch.equal(out1[:, 0], out[:, h]), h
        assert torch.equal(lse1[0], lse[h]), h


@pytest.mark.parametrize("B,hq,hkv,jump", [(128, 4, 2, 1), (128, 4, 2, 0), (64, 4, 2, 1),
                                           (64, 2, 2, 0)])
def test_prefill_softmax_reference_and_rescale(B, hq, hkv, jump):
    """The bf16 prefill fixes each query's softmax reference after its first
    32-key step (0 when that step's maximum is within +-64 in log2 units, else
    the maximum) and rescales the running state only when the running sum
    nears 2^100.  Here scale * log2(e) = 1/8, so the kernel's bf16 pre-scaled Q
    is exactly Q / 8 and the scores are exact up to fp32 accumulation.  KV
    head 0's key magnitudes start small (reference 0) and grow along the
    sequence until single scores pass 100 (repeated rescales); KV head 1's
    scores pass 64 in the first step (a nonzero reference) and grow past it by
    far more than 2^128 (an overflowing step).  Inside every 32-key step one
    16-key half is 1.5x larger (`jump` picks which), so the first overflow of a
    step can come in either half.  Dense lists on one ragged sequence; every
    query block against the oracle's exact softmax."""
    d = 128
    n = 5 * B + 17
    geo = sws.Geometry([n], B)
    scale = 0.125 * np.log(2.0)                     # scale * log2(e) = 1/8
    pos = torch.arange(n, dtype=torch.float32, device="cuda")
    half = ((pos.long() % 32) // 16) == jump
    mag0 = (0.5 + 30.0 * (pos / n) ** 2) * torch.where(half, 1.5, 1.0)
    mag1 = (60.0 + 60.0 * pos / n) * torch.where(half, 1.5, 1.0)
    mags = torch.stack([mag0, mag1], 1)[:, :hkv]
    q = _rand((n, hq, d), 51).to(torch.bfloat16)
    k = (_rand((n, hkv, d), 52) * mags[:, :, None]).to(torch.bfloat16)
    v = _rand((n, hkv, d), 53).to(torch.bfloat16)
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    out = sws.sparse_attn_prefill(q, k, v, geo, None, None, scale=scale, lse=lse)
    torch.cuda.synchronize()
    Q, K, V, Og, Lg = f64(q), f64(k), f64(v), f64(out), f64(lse)
    G = hq // hkv
    b = geo.blocks[0]
    lists = [np.arange(i + 1) for i in range(b)]
    worst = 0.0
    for h in range(hq):
        g = h // G
        # the inputs reach the paths named above (scores in log2 units)
        s2 = (Q[:, h] / 8.0) @ K[:, g].T
        first = s2[32:, :32].max(axis=1)           # first-step maxima of queries 32..
        late = np.tril(s2).max()
        if g == 0:
            assert np.abs(first).max() < 64 and late > 110, (first, late)
        else:
            assert first.min() > 64 and late - first.max() > 128, (first.min(), late)
        res = O.sparse_attention_rows(Q[:, h], K[:, g], V[:, g], lists, B, scale, range(b))
        for i in range(b):
            o_want, lse_want = res[i]
            a = i * B
            e = float(np.abs(Og[a:a + o_want.shape[0], h] - o_want).max())
            e2 = float(np.abs(Lg[h, a:a + o_want.shape[0]] - lse_want).max())
            worst = max(worst, e)
            assert e <= TOL_ATTN_BF16, (h, i, "attn", e)
            assert e2 <= TOL_ATTN_BF16, (h, i, "lse", e2)
    _print("softmax paths", B, hq, hkv, jump, "worst", worst)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_zero_length_sequences(dtype):
    """Sequences of no tokens inside a ragged batch: every stage (sketches,
    walk state over two layers, lists, attention and lse) equals, bit for
    bit, the same call on the batch without them, on the same tensors (the
    empty sequences own no blocks and no walk rows); the sketches of the
    others also match the oracle."""
    cfg = gen.CONFIGS["C2"].with_(hq=4, hkv=2, B=64, k=32, dtype=dtype)
    lens_with = [0, 300, 0, 129, 0, 64]
    lens_without = [n for n in lens_with if n > 0]
    signs, cols = gen.hadamard_tables(cfg.d, cfg.k)
    sd, cd = torch.from_numpy(signs).cuda(), torch.from_numpy(cols).cuda()
    layers = [gen.layer_inputs(cfg, l, device="cuda", seqlens=lens_without)[:3] for l in range(2)]
    results = []
    for lens in (lens_with, lens_without):
        geo = sws.Geometry(lens, cfg.B)
        R = torch.empty(geo.walk_numel(cfg.hq), dtype=torch.float32, device="cuda")
        per_layer = []
        for li, (q, k, v) in enumerate(layers):
            lse = torch.empty((cfg.hq, geo.total_tokens), dtype=torch.float32, device="cuda")
            r = sws.prefill_layer(q, k, v, geo, cfg.k, sd, cd, cfg.s, cfg.rho, False, R,
                                  first_layer=li == 0)
            r["out"] = sws.sparse_attn_prefill(q, k, v, geo, r["idx"], r["cnt"], lse=lse)
            torch.cuda.synchronize()
            per_layer.append({key: r[key].float().cpu().numpy() if key != "idx" and key != "cnt"
                              else r[key].cpu().numpy()
                              for key in ("q_sk", "k_sk", "R", "idx", "cnt", "out")}
                             | {"lse": lse.cpu().numpy()})
        results.append(per_layer)
    for li in range(2):
        a, b = results[0][li], results[1][li]
        for key in ("q_sk", "k_sk", "R", "cnt", "out", "lse"):
            assert np.array_equal(a[key], b[key]), (dtype, li, key)
        # list entries up to each count (past it the lists are not defined)
        for h in range(cfg.hq):
            for g in range(a["cnt"].shape[1]):
                c = int(a["cnt"][h, g])
                assert np.array_equal(a["idx"][h, g, :c], b["idx"][h, g, :c]), (dtype, li, h, g)
    # the remaining sequences' sketches against the oracle (first layer)
    geo = sws.Geometry(lens_without, cfg.B)
    q = f64(layers[0][0])
    for s, n in enumerate(lens_without):
        t0, b0, nb = int(geo.cu_seqlens_host[s]), int(geo.cu_blocks_host[s]), geo.blocks[s]
        for h in range(cfg.hq):
            want = O.sketch(q[t0:t0 + n, h], cfg.B, signs, cols)
            got = results[0][0]["q_sk"][h, b0:b0 + nb]
            assert rowwise_rel_err(got, want) <= 1e-4, (dtype, s, h)
    _print("zero-length sequences", dtype, "ok")
