"""The C ABI library loads, exports every symbol include/sws.h declares, and
rejects bad arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest
import torch

import dynamic_block_sparse_sws_amd as sws

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "sws.h")) as f:
        txt = f.read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sws_[a-z_0-9]+)\s*\(", txt)))


def test_header_symbols_exported():
    names = _declared()
    assert len(names) == 20
    L = sws.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(sws.EXPORTED_SYMBOLS)


def test_version_and_status_strings():
    L = sws.lib()
    assert L.sws_version() == 100
    assert L.sws_status_string(0) == b"SWS_OK"
    assert L.sws_status_string(4) == b"SWS_ERR_WORKSPACE"
    assert L.sws_status_string(99) == b"SWS_ERR_UNKNOWN"


# Host-side validation: every call below must fail validation, so nothing is
# launched and the fake pointers are never dereferenced.  On a machine with a
# GPU these are skipped (they are covered there by the GPU tests' error cases).
cpu_only = pytest.mark.skipif(torch.cuda.is_available(), reason="host-validation probes run without a GPU")
P = ctypes.c_void_p(4096)
N = None


@cpu_only
@pytest.mark.parametrize("args,code", [
    # x NULL
    ((N, 1, P, P, 1, 4, 8, 128, 64, 32, P, P, P, 128, N, N), 1),
    # d unsupported
    ((P, 1, P, P, 1, 4, 8, 96, 64, 32, P, P, P, 128, N, N), 3),
    # B unsupported
    ((P, 1, P, P, 1, 4, 8, 128, 32, 32, P, P, P, 128, N, N), 3),
    # k > 64
    ((P, 1, P, P, 1, 4, 8, 128, 64, 65, P, P, P, 4 * 65, N, N), 3),
    # bad dtype
    ((P, 7, P, P, 1, 4, 8, 128, 64, 32, P, P, P, 128, N, N), 3),
    # ld_head too small
    ((P, 1, P, P, 1, 4, 8, 128, 64, 32, P, P, P, 100, N, N), 2),
    # misaligned x
    ((ctypes.c_void_p(4098), 1, P, P, 1, 4, 8, 128, 64, 32, P, P, P, 128, N, N), 2),
])
def test_sketch_validation(args, code):
    assert sws.lib().sws_sketch(*args) == code
    assert sws.lib().sws_last_error_detail().startswith(b"sws_sketch")


@cpu_only
def test_other_entry_points_validation():
    L = sws.lib()
    # walk: hq not a multiple of hkv; s = 0; k = 0
    assert L.sws_walk_update(P, P, 6, 4, 32, P, 1, 4, 4, 8, N, P, N) == 2
    assert L.sws_walk_update(P, P, 8, 4, 32, P, 1, 4, 4, 0, N, P, N) == 2
    assert L.sws_walk_update(P, P, 8, 4, 0, P, 1, 4, 4, 8, N, P, N) == 3
    assert L.sws_walk_update(N, P, 8, 4, 32, P, 1, 4, 4, 8, N, P, N) == 1
    assert L.sws_walk_update_row(P, P, 8, 4, 32, 2, P, 5000, 8, N, P, N) == 2
    # select: width too small, rho out of range, too many blocks
    assert L.sws_select_topk(P, 8, P, 1, 1024, 1024, 20, 0, 204, P, P, N) == 2
    assert L.sws_select_topk(P, 8, P, 1, 1024, 1024, 101, 0, 1024, P, P, N) == 2
    assert L.sws_select_topk(P, 8, P, 1, 8192, 8192, 20, 0, 8192, P, P, N) == 3
    assert L.sws_select_topk(P, 8, P, 1, 16, 16, 100, 1, 15, P, P, N) == 2
    # walk variants: unknown mode, workspace too small, walk_numel too small
    assert L.sws_walk_update_variant(P, P, 8, 4, 32, P, 1, 4, 4, 8, 7, N, P, 128, P, 1 << 20, N) == 3
    need = L.sws_walk_variant_workspace_size(128)
    assert need == 128 * 3 * 4
    assert L.sws_walk_update_variant(P, P, 8, 4, 32, P, 1, 4, 4, 8, 2, N, P, 128, P, need - 4, N) == 4
    assert L.sws_walk_update_variant(P, P, 8, 4, 32, P, 1, 4, 4, 8, 1, N, P, 100, P, 1 << 20, N) == 2
    assert L.sws_walk_update_row_variant(P, P, 8, 4, 32, 2, P, 5000, 8, 1, N, P, N) == 2
    assert L.sws_walk_update_row_variant(P, P, 8, 4, 32, 2, P, 50, 8, 9, N, P, N) == 3
    # select with flags: unknown flag bits, group size not dividing hq, R NULL
    assert L.sws_select_topk_flags(P, 8, 4, P, 1, 16, 16, 20, 8, 16, P, P, N) == 2
    assert L.sws_select_topk_flags(P, 8, 3, P, 1, 16, 16, 20, 4, 16, P, P, N) == 2
    assert L.sws_select_topk_flags(N, 8, 4, P, 1, 16, 16, 20, 6, 16, P, P, N) == 1
    assert L.sws_select_topk_row(P, 32, 8, 2, P, 1029, 20, 16, 206, N, N, P, P, P, 1029, N) == 2
    # select row: union too narrow; group too large; idx without cnt
    assert L.sws_select_topk_row(P, 32, 8, 2, P, 1029, 20, 0, 206, N, N, P, P, P, 800, N) == 2
    assert L.sws_select_topk_row(P, 64, 2, 2, P, 1029, 20, 0, 206, N, N, P, P, P, 1029, N) == 3
    assert L.sws_select_topk_row(P, 32, 8, 2, P, 1029, 20, 0, 206, P, N, P, P, P, 1029, N) == 1
    # prefill attention: bad d, bad dtype, misaligned out, idx without cnt
    assert L.sws_sparse_attn_prefill(P, P, P, 1, P, P, 1, 8, 8, 32, 8, 80, 64, P, P, 3,
                                     ctypes.c_float(0.1), P, N, P, 1 << 30, N) == 3
    assert L.sws_sparse_attn_prefill(P, P, P, 5, P, P, 1, 8, 8, 32, 8, 128, 64, P, P, 3,
                                     ctypes.c_float(0.1), P, N, P, 1 << 30, N) == 3
    assert L.sws_sparse_attn_prefill(P, P, P, 1, P, P, 1, 8, 8, 32, 8, 128, 64, P, P, 3,
                                     ctypes.c_float(0.1), ctypes.c_void_p(4100), N, P, 1 << 30, N) == 2
    assert L.sws_sparse_attn_prefill(P, P, P, 1, P, P, 1, 8, 8, 32, 8, 128, 64, P, N, 3,
                                     ctypes.c_float(0.1), P, N, P, 1 << 30, N) == 1
    need = L.sws_prefill_workspace_size(1, 8, 8, 128, 64)
    assert need == 8 * 8 * 128 * 64 * 2 and L.sws_prefill_workspace_size(0, 8, 8, 128, 64) == 0
    assert L.sws_sparse_attn_prefill(P, P, P, 1, P, P, 1, 8, 8, 32, 8, 128, 64, P, P, 3,
                                     ctypes.c_float(0.1), P, N, P, need - 16, N) == 4
    assert L.sws_sparse_attn_prefill(P, P, P, 1, P, P, 1, 8, 8, 32, 8, 128, 64, P, P, 3,
                                     ctypes.c_float(0.1), P, N, N, need, N) == 4
    # decode attention: workspace too small, group too large
    need = L.sws_decode_workspace_size(16, 32, 8, 128, 64, 821)
    assert need > 0
    assert L.sws_sparse_attn_decode(P, P, P, 1, P, 16, 65792, 32, 8, 128, 64, P, P, P, 821,
                                    ctypes.c_float(0.1), P, N, P, need - 1, N) == 4
    assert L.sws_sparse_attn_decode(P, P, P, 1, P, 16, 65792, 32, 8, 128, 64, P, P, P, 821,
                                    ctypes.c_float(0.1), P, N, N, need, N) == 4
    assert L.sws_sparse_attn_decode(P, P, P, 1, P, 16, 65792, 64, 2, 128, 64, P, P, P, 821,
                                    ctypes.c_float(0.1), P, N, P, 1 << 40, N) == 3
    # paged decode: bad kv dtype, table NULL, table_width 0, workspace too small
    need = L.sws_decode_workspace_size(16, 32, 8, 128, 64, 821)
    f = ctypes.c_float
    assert L.sws_sparse_attn_decode_paged(P, P, P, 0, f(1), f(1), P, 1029, 4096, P, 16, 32, 8, 128,
                                          64, P, P, P, 821, f(0.1), P, N, P, need, N) == 3
    assert L.sws_sparse_attn_decode_paged(P, P, P, 2, f(1), f(1), N, 1029, 4096, P, 16, 32, 8, 128,
                                          64, P, P, P, 821, f(0.1), P, N, P, need, N) == 1
    assert L.sws_sparse_attn_decode_paged(P, P, P, 2, f(1), f(1), P, 0, 4096, P, 16, 32, 8, 128,
                                          64, P, P, P, 821, f(0.1), P, N, P, need, N) == 2
    assert L.sws_sparse_attn_decode_paged(P, P, P, 1, f(1), f(1), P, 1029, 4096, P, 16, 32, 8, 128,
                                          64, P, P, P, 821, f(0.1), P, N, P, need - 1, N) == 4
    assert L.sws_sparse_attn_decode_paged(P, P, P, 2, f(float("inf")), f(1), P, 1029, 4096, P, 16,
                                          32, 8, 128, 64, P, P, P, 821, f(0.1), P, N, P, need, N) == 2
    # the head-major layout flag does not make an unknown dtype valid
    assert L.sws_sparse_attn_decode_paged(P, P, P, 0x100 | 0, f(1), f(1), P, 1029, 4096, P, 16, 32,
                                          8, 128, 64, P, P, P, 821, f(0.1), P, N, P, need, N) == 3
    assert L.sws_sparse_attn_decode_paged(P, P, P, 0x100 | 1, f(1), f(1), P, 1029, 4096, P, 16, 32,
                                          8, 128, 64, P, P, P, 821, f(0.1), P, N, P, need - 1, N) == 4
    assert L.sws_sparse_attn_decode(P, P, P, 0x100 | 7, P, 16, 65536, 32, 8, 128, 64, P, P, P, 821,
                                    f(0.1), P, N, P, need, N) == 3
    # append: b_max 0
    assert L.sws_sketch_append(P, 1, P, 2, 8, 128, 64, 32, P, P, P, P, 0, N) == 2
    # fused query / key append: k_new NULL, hkv 0, bad k, misaligned run sum
    assert L.sws_sketch_append_qk(P, N, 1, P, 2, 32, 8, 128, 64, 32, P, P, P, P, P, P, 9, N) == 1
    assert L.sws_sketch_append_qk(P, P, 1, P, 2, 32, 0, 128, 64, 32, P, P, P, P, P, P, 9, N) == 2
    assert L.sws_sketch_append_qk(P, P, 1, P, 2, 32, 8, 128, 64, 65, P, P, P, P, P, P, 9, N) == 3
    assert L.sws_sketch_append_qk(P, P, 1, P, 2, 32, 8, 128, 64, 32, P, P, P,
                                  ctypes.c_void_p(4100), P, P, 9, N) == 2


@cpu_only
def test_decode_noalloc_validation():
    """The no-allocation decode call validates like the workspace form and
    rejects calls whose split-KV records exceed its fixed device array, all
    on the host (no device symbol is looked up for a rejected call)."""
    L = sws.lib()
    f = ctypes.c_float
    # 8192 (sequence, KV head) pairs x 16 heads per group x (d + 2) floats > 32 MiB
    assert L.sws_decode_workspace_size(1024, 128, 8, 128, 64, 821) > sws.DECODE_NOALLOC_SCRATCH_BYTES
    assert L.sws_sparse_attn_decode_noalloc(P, P, P, 1, P, 1024, 65792, 128, 8, 128, 64, P, P, P,
                                            821, f(0.1), P, N, N) == 4
    assert L.sws_last_error_detail().startswith(b"sws_sparse_attn_decode_noalloc")
    # the bench's decode shape fits
    assert L.sws_decode_workspace_size(16, 32, 8, 128, 64, 821) <= sws.DECODE_NOALLOC_SCRATCH_BYTES
    # argument errors as in the workspace form: q NULL, bad d, group too large
    assert L.sws_sparse_attn_decode_noalloc(N, P, P, 1, P, 16, 65792, 32, 8, 128, 64, P, P, P, 821,
                                            f(0.1), P, N, N) == 1
    assert L.sws_sparse_attn_decode_noalloc(P, P, P, 1, P, 16, 65792, 32, 8, 96, 64, P, P, P, 821,
                                            f(0.1), P, N, N) == 3
    assert L.sws_sparse_attn_decode_noalloc(P, P, P, 1, P, 16, 65792, 64, 2, 128, 64, P, P, P, 821,
                                            f(0.1), P, N, N) == 3


def test_binding_rejects_strided_host_and_mistyped_tensors():
    """The binding passes dense row-major GPU arrays only: a strided view, a
    host tensor or an index tensor of the wrong dtype raises SwsError before
    any call reaches the library."""
    x = torch.zeros((4, 6, 8))
    with pytest.raises(sws.SwsError, match="not contiguous"):
        sws._ptr(x.transpose(0, 1))
    with pytest.raises(sws.SwsError, match="not on a GPU"):
        sws._ptr(x)
    with pytest.raises(sws.SwsError, match="must be torch.int32"):
        sws._typed(torch.zeros(3, dtype=torch.int64), torch.int32, "ctx_len")
    with pytest.raises(sws.SwsError, match="must be torch.int8"):
        sws._typed(torch.zeros(3, dtype=torch.int32), torch.int8, "signs")
    assert sws._ptr(None) is None and sws._typed(None, torch.int32, "idx") is None
    # a whole call: host tensors never reach the C ABI
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16)
    kc = torch.zeros((2, 64, 2, 128), dtype=torch.bfloat16)
    ctx = torch.full((2,), 64, dtype=torch.int32)
    with pytest.raises(sws.SwsError, match="not on a GPU"):
        sws.sparse_attn_decode(q, kc, kc, ctx, 64, None, None, None,
                               ws=torch.zeros(1 << 20, dtype=torch.uint8))
