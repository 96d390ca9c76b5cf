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
