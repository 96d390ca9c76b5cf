"""sws_sparse_attn_decode_noalloc (split-KV records in the library's fixed
device array) against sws_sparse_attn_decode (caller workspace): two calls in
a row, the second smaller, each bit for bit the workspace form's output and
log-sum-exp, and the oracle's single-query attention on sampled heads."""
import math

import numpy as np
import pytest
import torch

import dynamic_block_sparse_sws_amd as sws
import oracle as O
from gpu_util import TOL_ATTN_BF16

pytestmark = pytest.mark.gpu


def _case(ns, hq, hkv, ctx_lens, B, d, seed, head_major):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    max_ctx = max(ctx_lens)
    b_max = -(-max_ctx // B)
    q = torch.randn((ns, hq, d), generator=g, device="cuda").to(torch.bfloat16)
    kc = torch.randn((ns, max_ctx, hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((ns, max_ctx, hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    ctx = torch.tensor(ctx_lens, dtype=torch.int32, device="cuda")
    cur = (ctx - 1) // B
    r = torch.rand((ns, hq, b_max), generator=g, device="cuda")
    uidx, ucnt, umask, idx, cnt = sws.select_topk_row(r, hq, hkv, cur, b_max, 20, per_head=True)
    if head_major:
        kc_l, vc_l = (x.permute(0, 2, 1, 3).contiguous() for x in (kc, vc))
    else:
        kc_l, vc_l = kc, vc
    return q, kc, vc, kc_l, vc_l, ctx, uidx, ucnt, umask, idx, cnt


@pytest.mark.parametrize("head_major", [False, True])
def test_noalloc_decode_equals_workspace_form(head_major):
    calls = [
        # (n_seqs, hq, hkv, context lengths, B, d) - the second call smaller
        (8, 32, 8, [4100, 9000, 65, 7777, 8192, 3000, 12345, 64], 64, 128),
        (3, 8, 2, [700, 129, 1500], 64, 128),
    ]
    for n, (ns, hq, hkv, lens, B, d) in enumerate(calls):
        print(f"no-alloc decode call {n}: n_seqs={ns} hq={hq} hkv={hkv} B={B} d={d} "
              f"head_major={head_major}", flush=True)
        q, kc, vc, kc_l, vc_l, ctx, uidx, ucnt, umask, idx, cnt = _case(
            ns, hq, hkv, lens, B, d, 100 + n, head_major)
        assert sws.decode_workspace_size(ns, hq, hkv, d, B, uidx.shape[2]) <= \
            sws.DECODE_NOALLOC_SCRATCH_BYTES
        lse_a = torch.empty((ns, hq), dtype=torch.float32, device="cuda")
        lse_b = torch.empty_like(lse_a)
        out_a = sws.sparse_attn_decode(q, kc_l, vc_l, ctx, B, uidx, ucnt, umask, lse=lse_a,
                                       head_major=head_major)
        out_b = sws.sparse_attn_decode_noalloc(q, kc_l, vc_l, ctx, B, uidx, ucnt, umask,
                                               lse=lse_b, head_major=head_major)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), n
        assert torch.equal(lse_a, lse_b), n
        # and the oracle, on one head of every KV group of every sequence
        Kh, Vh = kc.double().cpu().numpy(), vc.double().cpu().numpy()
        qh = q.double().cpu().numpy()
        idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
        ob = out_b.double().cpu().numpy()
        grp = hq // hkv
        for s in range(ns):
            for g in range(hkv):
                h = g * grp + (s + g) % grp
                lst = idx_h[s, h, :cnt_h[s, h]].astype(np.int64)
                o_w, _ = O.query_attention(qh[s, h], Kh[s, :, g], Vh[s, :, g], lst, B,
                                           lens[s] - 1, 1.0 / math.sqrt(d))
                assert np.abs(ob[s, h] - o_w).max() <= TOL_ATTN_BF16, (n, s, h)
