"""Seeded synthetic workloads shaped like the long-context prefill and decode runs
of "Scout Before You Attend: Sketch-and-Walk Sparse Attention" (the deep-reading
blog page, section 7: Llama-3.1-8B-like head layouts, contexts up to 128K,
block 64, density 20%).

The public evaluation suites the page names (LongBench, RULER) and trained
weights are not used: plain Gaussian activations stand in for them, with three
planted structures so that block selection has something to find:

* a block latent shared by the query and key tokens of a block (the block
  coherence model of the page's section 6.1: token = block mean + noise);
* for the GQA configurations: an attention-sink direction on key block 0, a
  local AR(1) band (neighbouring blocks correlate, 0.9 per block) and
  multi-hop chains i -> j -> m where block i's queries align with block j's
  keys and block j's queries with block m's keys, while i and m share nothing
  (the one-hop versus multi-hop example of the page's section 1).

Nothing here computes any part of the method.  Random numbers the method
itself consumes (the Hadamard sign vector and column subset) are drawn here
and passed to both sides as inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from functools import lru_cache

import numpy as np
import torch

ROOT_SEED = 20260207

_TENSOR_ID = {"q": 0, "k": 1, "v": 2, "mu": 3, "band": 4, "chain": 5, "tables": 6, "lens": 7}


def seed_for(*parts: int) -> int:
    """64-bit seed derived from a tuple of small integers."""
    ss = np.random.SeedSequence([ROOT_SEED] + [int(p) & 0xFFFFFFFF for p in parts])
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    hq: int
    hkv: int
    d: int
    B: int
    k: int
    layers: int
    dtype: str                      # "f32" or "bf16"
    rho: int                        # density in percent
    s: int = 8                      # walk degree (hops per layer)
    n_dense: int = 2                # leading layers attended densely
    seqlens: tuple = ()             # prefill sequence lengths (ragged allowed)
    structure: str = "planted"      # "planted" or "blocklatent"
    decode_batch: int = 0
    decode_prefix: int = 0
    decode_steps: int = 0
    rho_sweep: tuple = field(default=())

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


def ragged_lengths(n_seqs: int, lo: int, hi: int, seed_parts=(5,)) -> tuple:
    rng = np.random.default_rng(seed_for(*seed_parts, _TENSOR_ID["lens"]))
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=n_seqs))


CONFIGS = {
    # tiny stack: 1 head, 4 layers, n=1024, d=64, B=64 (b=16), k=16, 20% (tau=3 + diagonal), fp32
    "C1": Config("tiny", 1, hq=1, hkv=1, d=64, B=64, k=16, layers=4, dtype="f32", rho=20,
                 seqlens=(1024,), structure="blocklatent"),
    # Llama-3-8B-shaped 32K prefill
    "C2": Config("llama8b_32k_prefill", 2, hq=32, hkv=8, d=128, B=64, k=32, layers=32,
                 dtype="bf16", rho=20, seqlens=(32768,)),
    # long 128K prefill, density sweep 10/20/30/100
    "C3": Config("long_128k_prefill", 3, hq=32, hkv=8, d=128, B=128, k=32, layers=32,
                 dtype="bf16", rho=20, seqlens=(131072,), rho_sweep=(10, 20, 30, 100)),
    # decode: batch 16, 64K-token prefix, 256 steps
    "C4": Config("decode_64k_b16", 4, hq=32, hkv=8, d=128, B=64, k=32, layers=32,
                 dtype="bf16", rho=20, decode_batch=16, decode_prefix=65536, decode_steps=256),
    # ragged batch prefill: 8 sequences of 4096..65536 tokens, 40q/8kv, 40 layers
    "C5": Config("ragged_prefill", 5, hq=40, hkv=8, d=128, B=64, k=32, layers=40,
                 dtype="bf16", rho=20, seqlens=ragged_lengths(8, 4096, 65536)),
}


def cu_offsets(lengths) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


def hadamard_tables(d: int, k: int, seed_parts=(0,)):
    """Rademacher sign vector (int8, +-1) of length d and k distinct column
    indices of the d x d Sylvester matrix, ascending (int32)."""
    if k > d:
        raise ValueError("sketch dimension k must not exceed d")
    rng = np.random.default_rng(seed_for(*seed_parts, _TENSOR_ID["tables"], d, k))
    signs = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    cols = np.sort(rng.choice(d, size=k, replace=False)).astype(np.int32)
    return signs, cols


def _unit(x: np.ndarray) -> np.ndarray:
    return x / max(np.linalg.norm(x), 1e-30)


@lru_cache(maxsize=512)
def _band(cfg_id: int, seq: int, group: int, b: int, d: int) -> np.ndarray:
    """Local AR(1) band latent z [b, d] (0.9 correlation per block), shared by
    every layer."""
    rng = np.random.default_rng(seed_for(cfg_id, _TENSOR_ID["band"], seq, group))
    eps = rng.normal(0.0, 0.5, size=(b, d))
    z = np.empty((b, d))
    z[0] = eps[0]
    a = 0.9
    c = math.sqrt(1.0 - a * a)
    for i in range(1, b):
        z[i] = a * z[i - 1] + c * eps[i]
    z.setflags(write=False)
    return z


def chain_draws(cfg: Config, layer: int, seq: int, group: int, b: int, m_hat: np.ndarray):
    """Multi-hop chains of one (sequence, KV group, layer): block triples
    (i > j > m) and unit directions e1, e2 orthogonal to each other and to the
    sink direction.  The first half of the chains is the same in every layer,
    the second half is redrawn per layer."""
    d = cfg.d
    n_ch = -(-b // 16)
    out = []
    for persistent, n in ((True, n_ch // 2), (False, n_ch - n_ch // 2)):
        if n == 0:
            continue
        lay = 0xFFFF if persistent else layer
        r = np.random.default_rng(seed_for(cfg.cfg_id, _TENSOR_ID["chain"], seq, group, lay))
        trip = np.argpartition(r.random((n, b)), 2, axis=1)[:, :3]
        trip = -np.sort(-trip, axis=1)                         # i > j > m
        e1 = r.normal(size=(n, d))
        e1 -= np.outer(e1 @ m_hat, m_hat)
        e1 /= np.linalg.norm(e1, axis=1, keepdims=True)
        e2 = r.normal(size=(n, d))
        e2 -= np.outer(e2 @ m_hat, m_hat)
        e2 -= (np.sum(e2 * e1, axis=1, keepdims=True)) * e1
        e2 /= np.linalg.norm(e2, axis=1, keepdims=True)
        out.append((trip, e1, e2))
    return out


@lru_cache(maxsize=64)
def block_latents(cfg: Config, layer: int, seq: int, group: int, seqlen: int):
    """Per-block latent offsets (fp64, [b, d]) added to every query token and
    every key token of a block, for one (sequence, KV group)."""
    b = -(-seqlen // cfg.B)
    d = cfg.d
    if cfg.structure == "blocklatent":
        rng = np.random.default_rng(seed_for(cfg.cfg_id, _TENSOR_ID["mu"], seq, group))
        mu = rng.normal(0.0, 0.5, size=(b, d))
        return mu, mu.copy()
    z = _band(cfg.cfg_id, seq, group, b, d)
    lat_q = z.copy()
    lat_k = z.copy()
    # attention sink on key block 0, along the mean query-latent direction
    m_hat = _unit(z.mean(axis=0))
    lat_k[0] += 0.5 * math.sqrt(d) * m_hat
    if b >= 3:
        beta = 0.5 * math.sqrt(d)
        for trip, e1, e2 in chain_draws(cfg, layer, seq, group, b, m_hat):
            np.add.at(lat_q, trip[:, 0], beta * e1)
            np.add.at(lat_k, trip[:, 1], beta * e1)
            np.add.at(lat_q, trip[:, 1], beta * e2)
            np.add.at(lat_k, trip[:, 2], beta * e2)
    return lat_q, lat_k


def seq_tensor(cfg: Config, layer: int, seq: int, which: str, seqlen: int, device="cpu",
               out_dtype=None) -> torch.Tensor:
    """One sequence's activations, token-major [seqlen, H, d] (H = hq for 'q',
    hkv for 'k'/'v'), Gaussian noise plus the block latents of its group."""
    heads = cfg.hq if which == "q" else cfg.hkv
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed_for(cfg.cfg_id, _TENSOR_ID[which], layer, seq))
    x = torch.randn((seqlen, heads, cfg.d), generator=g, device=dev, dtype=torch.float32)
    if which in ("q", "k"):
        b = -(-seqlen // cfg.B)
        lat = np.empty((b, heads, cfg.d), dtype=np.float32)
        for grp in range(cfg.hkv):
            lq, lk = block_latents(cfg, layer, seq, grp, seqlen)
            if which == "q":
                lat[:, grp * cfg.group:(grp + 1) * cfg.group, :] = lq[:, None, :]
            else:
                lat[:, grp, :] = lk
        lat_t = torch.from_numpy(lat).to(dev)
        blk = torch.arange(seqlen, device=dev) // cfg.B
        x += lat_t[blk]
    return x.to(out_dtype or cfg.torch_dtype)


def layer_inputs(cfg: Config, layer: int, device="cpu", seqlens=None):
    """Token-major packed Q [T, hq, d], K and V [T, hkv, d] of one layer over
    the sequences `seqlens` (default: the config's), plus cu_seqlens (int32)."""
    lens = tuple(seqlens if seqlens is not None else cfg.seqlens)
    qs, ks, vs = [], [], []
    for si, n in enumerate(lens):
        qs.append(seq_tensor(cfg, layer, si, "q", n, device))
        ks.append(seq_tensor(cfg, layer, si, "k", n, device))
        vs.append(seq_tensor(cfg, layer, si, "v", n, device))
    cat = (lambda xs: xs[0]) if len(lens) == 1 else (lambda xs: torch.cat(xs, 0))
    return cat(qs), cat(ks), cat(vs), cu_offsets(lens)


def decode_layer_inputs(cfg: Config, layer: int, device="cpu", n_seqs=None, prefix=None,
                        steps=None, want_prefix_q=True):
    """Decode workload of one layer: every sequence holds `prefix` tokens and
    then receives `steps` new tokens one at a time.

    Returns q_prefix [n_seqs, prefix, hq, d] (or None), q_steps
    [steps, n_seqs, hq, d], and the KV caches k_cache, v_cache
    [n_seqs, prefix + steps, hkv, d] already holding every token the steps will
    append (position prefix + t is step t's token)."""
    n_seqs = n_seqs or cfg.decode_batch
    prefix = cfg.decode_prefix if prefix is None else prefix
    steps = cfg.decode_steps if steps is None else steps
    total = prefix + steps
    dev = torch.device(device)
    kc = torch.empty((n_seqs, total, cfg.hkv, cfg.d), dtype=cfg.torch_dtype, device=dev)
    vc = torch.empty_like(kc)
    qst = torch.empty((steps, n_seqs, cfg.hq, cfg.d), dtype=cfg.torch_dtype, device=dev)
    qpre = (torch.empty((n_seqs, prefix, cfg.hq, cfg.d), dtype=cfg.torch_dtype, device=dev)
            if want_prefix_q else None)
    for si in range(n_seqs):
        q = seq_tensor(cfg, layer, si, "q", total, dev)
        if want_prefix_q:
            qpre[si] = q[:prefix]
        qst[:, si] = q[prefix:]
        del q
        kc[si] = seq_tensor(cfg, layer, si, "k", total, dev)
        vc[si] = seq_tensor(cfg, layer, si, "v", total, dev)
    return qpre, qst, kc, vc


def page_table(ctx_lens, B: int, spare_pages: int = 3, share_prefix_blocks: int = 0,
               seed_parts=(9,)):
    """A paged-KV layout for sequences of `ctx_lens` tokens with pages of B
    tokens: a seeded random page for every logical block, `spare_pages` pages
    that no sequence uses, and, when share_prefix_blocks > 0, sequence 1
    reusing sequence 0's first pages (a shared prompt prefix).  Returns
    (table [n_seqs][width] int32, num_pages); unused entries hold -1."""
    rng = np.random.default_rng(seed_for(_TENSOR_ID["tables"], *seed_parts))
    nb = [-(-int(n) // B) for n in ctx_lens]
    width = max(nb)
    shared = min(share_prefix_blocks, nb[0], nb[1] if len(nb) > 1 else 0)
    need = sum(nb) - (shared if len(nb) > 1 else 0)
    num_pages = need + spare_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((len(nb), width), -1, dtype=np.int32)
    nxt = 0
    for s, n in enumerate(nb):
        for j in range(n):
            if s == 1 and j < shared:
                table[1, j] = table[0, j]
            else:
                table[s, j] = perm[nxt]
                nxt += 1
    return table, num_pages


def to_fp8_e4m3(x: torch.Tensor, scale: float) -> torch.Tensor:
    """Store x as OCP fp8 e4m3 codes of x / scale (torch's round-to-nearest
    cast), returned as raw bytes (uint8)."""
    return (x.float() / scale).to(torch.float8_e4m3fn).view(torch.uint8)
