"""Sketch&Walk sparse attention for AMD MI355X: Python binding of libsws.so.

Every function here only marshals arguments (tensor pointers, sizes, the
current HIP stream) into the C ABI declared in include/sws.h; all computation
runs in the HIP kernels.  If the library is missing or fails to load, every
call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "SwsError", "lib", "F32", "BF16", "FP8_E4M3", "KV_HEAD_MAJOR", "WALK_DEFAULT", "WALK_POWER", "WALK_SOFTMAX",
    "SELECT_DENSE", "SELECT_ROW_TAU", "SELECT_GROUP", "Geometry", "geometry", "walk_state_numel",
    "sketch", "sketch_append", "sketch_append_qk", "walk_update", "walk_update_row", "walk_update_variant",
    "walk_variant_workspace_size", "select_topk",
    "select_topk_row", "sparse_attn_prefill", "sparse_attn_decode", "decode_workspace_size",
    "sparse_attn_decode_paged", "sparse_attn_decode_noalloc", "DECODE_NOALLOC_SCRATCH_BYTES",
    "prefill_layer", "EXPORTED_SYMBOLS", "version",
]

F32 = 0
BF16 = 1
FP8_E4M3 = 2   # KV pages only
KV_HEAD_MAJOR = 0x100   # layout flag for the decode calls: [.., hkv, rows, d] caches

# walk modes and selection flags (include/sws.h)
WALK_DEFAULT = 0
WALK_POWER = 1
WALK_SOFTMAX = 2
SELECT_DENSE = 1
SELECT_ROW_TAU = 2
SELECT_GROUP = 4

_HERE = os.path.dirname(os.path.abspath(__file__))
# SWS_LIBRARY selects another build of the same library (the host-sanitizer
# build, libsws_asan.so); by default the in-tree libsws.so
LIB_PATH = os.environ.get("SWS_LIBRARY") or os.path.join(_HERE, "libsws.so")

EXPORTED_SYMBOLS = (
    "sws_version", "sws_status_string", "sws_last_error_detail", "sws_sketch",
    "sws_sketch_append", "sws_sketch_append_qk", "sws_walk_update", "sws_walk_update_row", "sws_select_topk",
    "sws_select_topk_row", "sws_sparse_attn_prefill", "sws_sparse_attn_decode",
    "sws_decode_workspace_size", "sws_prefill_workspace_size", "sws_select_topk_flags",
    "sws_walk_update_variant", "sws_walk_variant_workspace_size", "sws_walk_update_row_variant",
    "sws_sparse_attn_decode_paged", "sws_sparse_attn_decode_noalloc",
)

# include/sws.h SWS_DECODE_NOALLOC_SCRATCH_BYTES
DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20


class SwsError(RuntimeError):
    def __init__(self, fn: str, code: int, detail: str):
        super().__init__(f"{fn} failed: {code} ({detail})")
        self.code = code
        self.detail = detail


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGS = {
    "sws_version": ([], ctypes.c_int),
    "sws_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "sws_last_error_detail": ([], ctypes.c_char_p),
    "sws_sketch": ([_P, ctypes.c_int, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I64, _P, _P],
                   ctypes.c_int),
    "sws_sketch_append": ([_P, ctypes.c_int, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P],
                          ctypes.c_int),
    "sws_sketch_append_qk": ([_P, _P, ctypes.c_int, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P,
                              _P, _P, _I, _P], ctypes.c_int),
    "sws_walk_update": ([_P, _P, _I, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P], ctypes.c_int),
    "sws_walk_update_row": ([_P, _P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P], ctypes.c_int),
    "sws_walk_update_variant": ([_P, _P, _I, _I, _I, _P, _I, _I, _I, _I, _I, _P, _P, _I64, _P,
                                 _SZ, _P], ctypes.c_int),
    "sws_walk_variant_workspace_size": ([_I64], _SZ),
    "sws_walk_update_row_variant": ([_P, _P, _I, _I, _I, _I, _P, _I, _I, _I, _P, _P, _P],
                                    ctypes.c_int),
    "sws_select_topk": ([_P, _I, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P], ctypes.c_int),
    "sws_select_topk_flags": ([_P, _I, _I, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P],
                              ctypes.c_int),
    "sws_select_topk_row": ([_P, _I, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P],
                            ctypes.c_int),
    "sws_sparse_attn_prefill": ([_P, _P, _P, ctypes.c_int, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                 _P, _P, _I, _F, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "sws_prefill_workspace_size": ([ctypes.c_int, _I, _I, _I, _I], _SZ),
    "sws_sparse_attn_decode": ([_P, _P, _P, ctypes.c_int, _P, _I, _I, _I, _I, _I, _I, _P, _P,
                                _P, _I, _F, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "sws_decode_workspace_size": ([_I, _I, _I, _I, _I, _I], _SZ),
    "sws_sparse_attn_decode_noalloc": ([_P, _P, _P, ctypes.c_int, _P, _I, _I, _I, _I, _I, _I, _P,
                                        _P, _P, _I, _F, _P, _P, _P], ctypes.c_int),
    "sws_sparse_attn_decode_paged": ([_P, _P, _P, ctypes.c_int, _F, _F, _P, _I, _I, _P, _I, _I,
                                      _I, _I, _I, _P, _P, _P, _I, _F, _P, _P, _P, _SZ, _P],
                                     ctypes.c_int),
}


def lib():
    """Load libsws.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m dynamic_block_sparse_sws_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def version() -> int:
    return lib().sws_version()


def _ptr(t: Optional[torch.Tensor]):
    """Device pointer of a tensor for the C ABI, which takes dense row-major
    arrays on the GPU: a strided view (e.g. a slice of a fused qkv tensor) or
    a host tensor would be read with the wrong layout, so both are rejected."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise SwsError("argument", 2, f"tensor of shape {tuple(t.shape)} is not contiguous "
                                      f"(strides {t.stride()}); pass .contiguous()")
    if not t.is_cuda:
        raise SwsError("argument", 2, f"tensor of shape {tuple(t.shape)} is on {t.device}, "
                                      "not on a GPU")
    return ctypes.c_void_p(t.data_ptr())


def _typed(t: Optional[torch.Tensor], dtype, what: str):
    """_ptr of an index / table tensor that must have the given dtype."""
    if t is not None and t.dtype != dtype:
        raise SwsError("argument", 3, f"{what} must be {dtype}, not {t.dtype}")
    return _ptr(t)


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    if torch.cuda.is_available():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return None


def _check(fn: str, code: int):
    if code != 0:
        L = lib()
        raise SwsError(fn, code, L.sws_last_error_detail().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise SwsError("dtype", 3, f"unsupported tensor dtype {t.dtype}")


class Geometry:
    """Block geometry of a (possibly ragged) batch: host copies of the offsets
    and their device copies for the kernels."""

    def __init__(self, seqlens: Sequence[int], B: int, device="cuda"):
        self.seqlens = [int(n) for n in seqlens]
        self.B = int(B)
        self.n_seqs = len(self.seqlens)
        cu = np.zeros(self.n_seqs + 1, np.int64)
        cu[1:] = np.cumsum(self.seqlens)
        nb = [-(-n // self.B) for n in self.seqlens]
        cb = np.zeros(self.n_seqs + 1, np.int64)
        cb[1:] = np.cumsum(nb)
        self.cu_seqlens_host = cu.astype(np.int32)
        self.cu_blocks_host = cb.astype(np.int32)
        self.blocks = nb
        self.total_tokens = int(cu[-1])
        self.total_blocks = int(cb[-1])
        self.max_blocks = max(nb) if nb else 0
        self.cu_seqlens = torch.from_numpy(self.cu_seqlens_host).to(device)
        self.cu_blocks = torch.from_numpy(self.cu_blocks_host).to(device)

    def walk_numel(self, hq: int) -> int:
        return walk_state_numel(self.blocks, hq)

    def walk_offset(self, seq: int, hq: int) -> int:
        return hq * sum(b * b for b in self.blocks[:seq])


def geometry(seqlens, B, device="cuda") -> Geometry:
    return Geometry(seqlens, B, device)


def walk_state_numel(blocks: Sequence[int], hq: int) -> int:
    return int(hq * sum(int(b) * int(b) for b in blocks))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI without the sws_ prefix)
# ---------------------------------------------------------------------------

def sketch(x: torch.Tensor, geo: Geometry, k: int, signs: torch.Tensor, cols: torch.Tensor,
           out: Optional[torch.Tensor] = None, ld_head: Optional[int] = None,
           sum_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    T, H, d = x.shape
    if ld_head is None:
        ld_head = geo.total_blocks * k
    if out is None:
        if ld_head != geo.total_blocks * k:
            raise ValueError("pass `out` when ld_head differs from total_blocks * k")
        out = torch.empty((H, geo.total_blocks, k), dtype=torch.float32, device=x.device)
    _check("sws_sketch", lib().sws_sketch(
        _ptr(x), _dtype_code(x), _ptr(geo.cu_seqlens), _ptr(geo.cu_blocks), geo.n_seqs,
        geo.total_blocks, H, d, geo.B, k, _typed(signs, torch.int8, "signs"),
        _typed(cols, torch.int32, "cols"), _ptr(out), ld_head, _ptr(sum_out), _stream(stream)))
    return out


def sketch_append(x_new: torch.Tensor, pos: torch.Tensor, B: int, k: int, signs, cols,
                  run_sum: torch.Tensor, sketch_cache: torch.Tensor, stream=None):
    n_seqs, H, d = x_new.shape
    b_max = sketch_cache.shape[2]
    _check("sws_sketch_append", lib().sws_sketch_append(
        _ptr(x_new), _dtype_code(x_new), _typed(pos, torch.int32, "pos"), n_seqs, H, d, B, k,
        _typed(signs, torch.int8, "signs"), _typed(cols, torch.int32, "cols"), _ptr(run_sum),
        _ptr(sketch_cache), b_max, _stream(stream)))


def sketch_append_qk(q_new: torch.Tensor, k_new: torch.Tensor, pos: torch.Tensor, B: int, k: int,
                     signs, cols, run_q: torch.Tensor, run_k: torch.Tensor, q_cache: torch.Tensor,
                     k_cache: torch.Tensor, stream=None):
    """sketch_append of the query rows and of the key rows in one launch."""
    n_seqs, hq, d = q_new.shape
    hkv = k_new.shape[1]
    if k_new.dtype != q_new.dtype:
        raise TypeError("q_new and k_new must share a dtype")
    b_max = q_cache.shape[2]
    if k_cache.shape[2] != b_max:
        raise ValueError("q_cache and k_cache differ in b_max")
    _check("sws_sketch_append_qk", lib().sws_sketch_append_qk(
        _ptr(q_new), _ptr(k_new), _dtype_code(q_new), _typed(pos, torch.int32, "pos"), n_seqs,
        hq, hkv, d, B, k, _typed(signs, torch.int8, "signs"), _typed(cols, torch.int32, "cols"),
        _ptr(run_q), _ptr(run_k), _ptr(q_cache), _ptr(k_cache), b_max, _stream(stream)))


def walk_update(q_sk: torch.Tensor, k_sk: torch.Tensor, geo: Geometry, s: int,
                R_prev: Optional[torch.Tensor], R_out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    hq, _, k = q_sk.shape
    hkv = k_sk.shape[0]
    if R_out is None:
        R_out = torch.empty(geo.walk_numel(hq), dtype=torch.float32, device=q_sk.device)
    _check("sws_walk_update", lib().sws_walk_update(
        _ptr(q_sk), _ptr(k_sk), hq, hkv, k, _ptr(geo.cu_blocks), geo.n_seqs, geo.total_blocks,
        geo.max_blocks, s, _ptr(R_prev), _ptr(R_out), _stream(stream)))
    return R_out


def walk_update_row(q_cache: torch.Tensor, k_cache: torch.Tensor, cur_block: torch.Tensor,
                    s: int, r_prev: Optional[torch.Tensor], r_out: torch.Tensor, stream=None,
                    mode: int = WALK_DEFAULT):
    n_seqs, hq, b_max, k = q_cache.shape
    hkv = k_cache.shape[1]
    if mode == WALK_DEFAULT:
        _check("sws_walk_update_row", lib().sws_walk_update_row(
            _ptr(q_cache), _ptr(k_cache), hq, hkv, k, n_seqs,
            _typed(cur_block, torch.int32, "cur_block"), b_max, s, _ptr(r_prev), _ptr(r_out),
            _stream(stream)))
    else:
        _check("sws_walk_update_row_variant", lib().sws_walk_update_row_variant(
            _ptr(q_cache), _ptr(k_cache), hq, hkv, k, n_seqs,
            _typed(cur_block, torch.int32, "cur_block"), b_max, s, mode, _ptr(r_prev),
            _ptr(r_out), _stream(stream)))
    return r_out


def walk_variant_workspace_size(walk_numel: int) -> int:
    return int(lib().sws_walk_variant_workspace_size(walk_numel))


def walk_update_variant(q_sk: torch.Tensor, k_sk: torch.Tensor, geo: Geometry, s: int,
                        mode: int, R_prev: Optional[torch.Tensor],
                        R_out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """Walk update with a walk mode (WALK_POWER, WALK_SOFTMAX)."""
    hq, _, k = q_sk.shape
    hkv = k_sk.shape[0]
    numel = geo.walk_numel(hq)
    if R_out is None:
        R_out = torch.empty(numel, dtype=torch.float32, device=q_sk.device)
    if ws is None:
        ws = torch.empty(max(1, walk_variant_workspace_size(numel)), dtype=torch.uint8,
                         device=q_sk.device)
    _check("sws_walk_update_variant", lib().sws_walk_update_variant(
        _ptr(q_sk), _ptr(k_sk), hq, hkv, k, _ptr(geo.cu_blocks), geo.n_seqs, geo.total_blocks,
        geo.max_blocks, s, mode, _ptr(R_prev), _ptr(R_out), numel, _ptr(ws), ws.numel(),
        _stream(stream)))
    return R_out


def select_width(rho: int, max_blocks: int, dense: bool = False) -> int:
    if dense:
        return max(1, max_blocks)
    return max(1, min(max_blocks, (rho * max_blocks) // 100 + 1))


def select_topk(R: Optional[torch.Tensor], hq: int, geo: Geometry, rho: int, dense: bool = False,
                width: Optional[int] = None, idx=None, cnt=None, stream=None,
                row_tau: bool = False, group_hkv: Optional[int] = None):
    """Top-tau lists per (query head, block).  row_tau / group_hkv select the
    variants SELECT_ROW_TAU and SELECT_GROUP (one shared list per KV group of
    hq / group_hkv heads)."""
    width = width or select_width(rho, geo.max_blocks, dense)
    dev = geo.cu_blocks.device
    if idx is None:
        idx = torch.empty((hq, geo.total_blocks, width), dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.empty((hq, geo.total_blocks), dtype=torch.int32, device=dev)
    if not row_tau and group_hkv is None:
        _check("sws_select_topk", lib().sws_select_topk(
            _ptr(R), hq, _ptr(geo.cu_blocks), geo.n_seqs, geo.total_blocks, geo.max_blocks, rho,
            int(dense), width, _typed(idx, torch.int32, "idx"), _typed(cnt, torch.int32, "cnt"),
            _stream(stream)))
        return idx, cnt
    flags = ((SELECT_DENSE if dense else 0) | (SELECT_ROW_TAU if row_tau else 0)
             | (SELECT_GROUP if group_hkv is not None else 0))
    _check("sws_select_topk_flags", lib().sws_select_topk_flags(
        _ptr(R), hq, group_hkv or hq, _ptr(geo.cu_blocks), geo.n_seqs, geo.total_blocks,
        geo.max_blocks, rho, flags, width, _typed(idx, torch.int32, "idx"),
        _typed(cnt, torch.int32, "cnt"), _stream(stream)))
    return idx, cnt


def union_width(rho: int, b_max: int, group: int, dense: bool = False) -> int:
    if dense:
        return b_max
    return min(b_max, group * ((rho * b_max) // 100) + 1)


def select_topk_row(r: Optional[torch.Tensor], hq: int, hkv: int, cur_block: torch.Tensor,
                    b_max: int, rho: int, dense: bool = False, per_head: bool = False,
                    out=None, stream=None, group: bool = False):
    """Returns (union_idx, union_cnt, union_mask, idx, cnt); idx/cnt are None
    unless per_head.  `out` may supply the five buffers.  group selects the
    SELECT_GROUP variant (one shared list per KV group)."""
    n_seqs = cur_block.shape[0]
    dev = cur_block.device
    uw = union_width(rho, b_max, hq // hkv, dense)
    w = select_width(rho, b_max, dense)
    if out is None:
        uidx = torch.empty((n_seqs, hkv, uw), dtype=torch.int32, device=dev)
        ucnt = torch.empty((n_seqs, hkv), dtype=torch.int32, device=dev)
        umask = torch.empty((n_seqs, hkv, uw), dtype=torch.int32, device=dev)
        idx = torch.empty((n_seqs, hq, w), dtype=torch.int32, device=dev) if per_head else None
        cnt = torch.empty((n_seqs, hq), dtype=torch.int32, device=dev) if per_head else None
    else:
        uidx, ucnt, umask, idx, cnt = out
        uw = uidx.shape[2]
        if idx is not None:
            w = idx.shape[2]
    _check("sws_select_topk_row", lib().sws_select_topk_row(
        _ptr(r), hq, hkv, n_seqs, _typed(cur_block, torch.int32, "cur_block"), b_max, rho,
        (SELECT_DENSE if dense else 0) | (SELECT_GROUP if group else 0), w,
        _typed(idx, torch.int32, "idx"), _typed(cnt, torch.int32, "cnt"),
        _typed(uidx, torch.int32, "union_idx"), _typed(ucnt, torch.int32, "union_cnt"),
        _typed(umask, torch.int32, "union_mask"), uw, _stream(stream)))
    return uidx, ucnt, umask, idx, cnt


def prefill_workspace_size(dtype_code: int, total_blocks: int, hkv: int, d: int, B: int) -> int:
    return int(lib().sws_prefill_workspace_size(dtype_code, total_blocks, hkv, d, B))


def sparse_attn_prefill(q, k, v, geo: Geometry, idx: Optional[torch.Tensor],
                        cnt: Optional[torch.Tensor], scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None, stream=None):
    T, hq, d = q.shape
    hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    need = prefill_workspace_size(_dtype_code(q), geo.total_blocks, hkv, d, geo.B)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    width = idx.shape[-1] if idx is not None else 0
    _check("sws_sparse_attn_prefill", lib().sws_sparse_attn_prefill(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(geo.cu_seqlens), _ptr(geo.cu_blocks),
        geo.n_seqs, geo.total_blocks, geo.max_blocks, hq, hkv, d, geo.B,
        _typed(idx, torch.int32, "idx"), _typed(cnt, torch.int32, "cnt"), width, float(scale),
        _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))
    return out


def decode_workspace_size(n_seqs, hq, hkv, d, B, uwidth) -> int:
    return int(lib().sws_decode_workspace_size(n_seqs, hq, hkv, d, B, uwidth))


def sparse_attn_decode(q, k_cache, v_cache, ctx_len, B: int, union_idx, union_cnt, union_mask,
                       scale: Optional[float] = None, out=None, lse=None, ws=None, stream=None,
                       head_major: bool = False):
    """Decode attention over a contiguous cache [n_seqs][max_ctx][hkv][d], or
    [n_seqs][hkv][max_ctx][d] with head_major=True."""
    n_seqs, hq, d = q.shape
    if head_major:
        _, hkv, max_ctx, _ = k_cache.shape
    else:
        _, max_ctx, hkv, _ = k_cache.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    uw = union_idx.shape[2] if union_idx is not None else -(-max_ctx // B)
    if ws is None:
        ws = torch.empty(max(1, decode_workspace_size(n_seqs, hq, hkv, d, B, uw)),
                         dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _check("sws_sparse_attn_decode", lib().sws_sparse_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q) | (KV_HEAD_MAJOR if head_major else 0),
        _typed(ctx_len, torch.int32, "ctx_len"), n_seqs, max_ctx, hq,
        hkv, d, B, _typed(union_idx, torch.int32, "union_idx"),
        _typed(union_cnt, torch.int32, "union_cnt"), _typed(union_mask, torch.int32, "union_mask"),
        uw, float(scale), _ptr(out),
        _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def sparse_attn_decode_noalloc(q, k_cache, v_cache, ctx_len, B: int, union_idx, union_cnt,
                               union_mask, scale: Optional[float] = None, out=None, lse=None,
                               stream=None, head_major: bool = False):
    """sparse_attn_decode with the split-KV records in the library's fixed
    device array (no workspace argument; the C call allocates nothing)."""
    n_seqs, hq, d = q.shape
    if head_major:
        _, hkv, max_ctx, _ = k_cache.shape
    else:
        _, max_ctx, hkv, _ = k_cache.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    uw = union_idx.shape[2] if union_idx is not None else -(-max_ctx // B)
    if out is None:
        out = torch.empty_like(q)
    _check("sws_sparse_attn_decode_noalloc", lib().sws_sparse_attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q) | (KV_HEAD_MAJOR if head_major else 0),
        _typed(ctx_len, torch.int32, "ctx_len"), n_seqs, max_ctx, hq, hkv, d, B,
        _typed(union_idx, torch.int32, "union_idx"), _typed(union_cnt, torch.int32, "union_cnt"),
        _typed(union_mask, torch.int32, "union_mask"), uw, float(scale), _ptr(out), _ptr(lse),
        _stream(stream)))
    return out


def sparse_attn_decode_paged(q, k_pages, v_pages, block_table, ctx_len, union_idx, union_cnt,
                             union_mask, k_scale: float = 1.0, v_scale: float = 1.0,
                             scale: Optional[float] = None, out=None, lse=None, ws=None,
                             stream=None, head_major: bool = False):
    """Decode attention over a paged cache: k_pages / v_pages [num_pages][B][hkv][d]
    ([num_pages][hkv][B][d] with head_major=True) in bf16 or torch.float8_e4m3fn
    (value = code * k_scale / v_scale), block_table [n_seqs][width] int32 pages of each
    sequence's logical blocks; q and out bf16."""
    n_seqs, hq, d = q.shape
    if head_major:
        num_pages, hkv, B, _ = k_pages.shape
    else:
        num_pages, B, hkv, _ = k_pages.shape
    width = block_table.shape[1]
    if k_pages.dtype == torch.bfloat16:
        kv = BF16
    elif k_pages.dtype == torch.float8_e4m3fn:
        kv = FP8_E4M3
    else:
        raise TypeError(f"KV pages must be bf16 or float8_e4m3fn, not {k_pages.dtype}")
    if v_pages.dtype != k_pages.dtype or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages and v_pages differ in dtype or shape")
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bf16")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    uw = union_idx.shape[2] if union_idx is not None else width
    if ws is None:
        ws = torch.empty(max(1, decode_workspace_size(n_seqs, hq, hkv, d, B, uw)),
                         dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _check("sws_sparse_attn_decode_paged", lib().sws_sparse_attn_decode_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), kv | (KV_HEAD_MAJOR if head_major else 0),
        float(k_scale), float(v_scale),
        _typed(block_table, torch.int32, "block_table"), width, num_pages,
        _typed(ctx_len, torch.int32, "ctx_len"), n_seqs, hq, hkv, d, B,
        _typed(union_idx, torch.int32, "union_idx"), _typed(union_cnt, torch.int32, "union_cnt"),
        _typed(union_mask, torch.int32, "union_mask"), uw, float(scale), _ptr(out),
        _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def prefill_layer(q, k, v, geo: Geometry, kdim: int, signs, cols, s: int, rho: int, dense: bool,
                  R: Optional[torch.Tensor], first_layer: bool, bufs: Optional[dict] = None,
                  stream=None) -> dict:
    """One layer of the hot path: sketch Q, sketch K, walk update (in place on
    R), top-tau selection, block-sparse attention.  `bufs` may hold
    preallocated outputs (q_sk, k_sk, idx, cnt, out)."""
    bufs = {} if bufs is None else bufs
    hq, hkv = q.shape[1], k.shape[1]
    q_sk = sketch(q, geo, kdim, signs, cols, out=bufs.get("q_sk"), stream=stream)
    k_sk = sketch(k, geo, kdim, signs, cols, out=bufs.get("k_sk"), stream=stream)
    R = walk_update(q_sk, k_sk, geo, s, None if first_layer else R, R_out=R, stream=stream)
    idx, cnt = select_topk(R, hq, geo, rho, dense=dense, idx=bufs.get("idx"),
                           cnt=bufs.get("cnt"), stream=stream)
    o = sparse_attn_prefill(q, k, v, geo, idx, cnt, out=bufs.get("out"), ws=bufs.get("ws"),
                            stream=stream)
    return {"q_sk": q_sk, "k_sk": k_sk, "R": R, "idx": idx, "cnt": cnt, "out": o}
