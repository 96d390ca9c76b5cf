"""Plain, slow fp64 reference of the Sketch&Walk sparse-attention hot path.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py.  It shares no code with the HIP library.

Sources (all on the deep-reading blog page "Scout Before You Attend:
Sketch-and-Walk Sparse Attention for Efficient LLM Inference", arXiv
2602.07397, unless stated):

* section 2      - blocking b = ceil(n/B) and the exact block score A_true;
* section 3.1    - token-space sketch: per-block means of Q and K;
* section 3.2    - feature-space sketch with a subsampled randomized Hadamard
                   projection H_d (d -> k) and the sketched score
                   A_SWS = (Qbar H_d)(Kbar H_d)^T / sqrt(k);
* section 4      - walk state R^0 = (A^0)^s, R^l = R^(l-1) (A^l)^s, and the
                   top-tau key blocks per query block taken from R^l's row;
* sections 4, 5  - block-sparse attention on the original Q/K/V over the
                   selected blocks, the same selection rule for prefill and for
                   each decode step;
* section 7      - defaults: block 64, sketch dim 64, walk degree 8, the first
                   two layers dense, density 20%.

Readings taken where the page is silent or ambiguous (each is listed with its
reason in the design notes of this repository):

* the walk runs on the raw signed sketched scores, causally masked
  (M[i, j] = 0 for j > i), with (.)^s the s-th matrix power (s hops);
* R^(-1) = I; each row of R^l is divided by its largest magnitude after every
  layer (positive row scaling commutes with right-multiplication, so rankings
  are unchanged);
* the walk state has a finite dynamic range: after every hop, entries smaller
  in magnitude than WALK_FLOOR = 2^-64 times their row's largest magnitude are
  set to zero.  Without it the walk over many layers is not computable in any
  fixed floating-point format: row entries fall hundreds of binary orders of
  magnitude below the row maximum and grow back to dominate the row several
  layers later, so the result depends on the format's exponent range;
* the Hadamard projection is H_d[r, c] = sign[r] * H_syl[r, cols[c]] / sqrt(k)
  with H_syl the natural-order Sylvester matrix; sign and cols are inputs;
* a partial last block is averaged over the tokens it holds;
* tau = floor(rho * b / 100) off-diagonal blocks chosen among the earlier
  blocks by (score descending, index ascending), and the diagonal block is
  always kept; lists are ascending;
* attention is the causal softmax renormalised over the allowed keys, scale
  1/sqrt(d); GQA query head h reads KV head h // (Hq / Hkv); ragged batches
  are handled per sequence.

No function here is pinned by a worked example from the pages (they print
none); each is pinned by closed forms, invariants, brute force or a library
routine in tests/test_oracle_*.py.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "n_blocks", "block_ranges", "block_sums", "block_means", "a_true", "a_true_bruteforce",
    "sylvester", "fwht", "hadamard_projection", "sketch_from_means", "sketch", "sketched_scores",
    "rownorm", "WALK_FLOOR", "floor_rows", "walk_update", "walk_row", "n_select", "select_row", "select", "n_select_row",
    "select_rows_tau", "group_scores", "transition", "walk_update_variant",
    "walk_row_variant", "sparse_attention",
    "sparse_attention_rows", "query_attention", "prefill_layer", "prefill", "decode_step", "SeqPrefill",
    "fp8_e4m3_value", "gather_pages",
]


# ---------------------------------------------------------------------------
# Section 2: blocking and the exact block score
# ---------------------------------------------------------------------------

def n_blocks(n: int, B: int) -> int:
    """b = ceil(n / B) (blog page, section 2)."""
    return -(-int(n) // int(B))


def block_ranges(n: int, B: int):
    """Token ranges [iB, min((i+1)B, n)) of the b blocks."""
    return [(i * B, min((i + 1) * B, n)) for i in range(n_blocks(n, B))]


def block_sums(X: np.ndarray, B: int) -> np.ndarray:
    """Sum of the token rows of each block; X is [n, d]."""
    X = np.asarray(X, dtype=np.float64)
    return np.stack([X[a:e].sum(axis=0) for a, e in block_ranges(X.shape[0], B)])


def block_means(X: np.ndarray, B: int) -> np.ndarray:
    """Token-space sketch (section 3.1): the mean of each block's token rows,
    over the tokens the block holds."""
    X = np.asarray(X, dtype=np.float64)
    return np.stack([X[a:e].mean(axis=0) for a, e in block_ranges(X.shape[0], B)])


def a_true(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """A_true[i, j] = qbar_i . kbar_j / sqrt(d): the section 2 double sum over
    the B x B token pairs factorises into the product of the block means."""
    d = qbar.shape[1]
    return (np.asarray(qbar, np.float64) @ np.asarray(kbar, np.float64).T) / math.sqrt(d)


def a_true_bruteforce(Q: np.ndarray, K: np.ndarray, B: int) -> np.ndarray:
    """Section 2 as printed: (1/sqrt d)(1/(c_i c_j)) sum_s sum_t Q_i[s] . K_j[t],
    summed over every token pair (c_i = tokens in block i)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    d = Q.shape[1]
    rq = block_ranges(Q.shape[0], B)
    rk = block_ranges(K.shape[0], B)
    out = np.zeros((len(rq), len(rk)))
    for i, (a, e) in enumerate(rq):
        for j, (a2, e2) in enumerate(rk):
            acc = 0.0
            for s in range(a, e):
                for t in range(a2, e2):
                    acc += float(Q[s] @ K[t])
            out[i, j] = acc / ((e - a) * (e2 - a2) * math.sqrt(d))
    return out


# ---------------------------------------------------------------------------
# Section 3.2: Hadamard projection and the sketched block score
# ---------------------------------------------------------------------------

def sylvester(d: int) -> np.ndarray:
    """Natural-order Sylvester-Hadamard matrix, entry (-1)^popcount(r & c)."""
    r = np.arange(d)[:, None]
    c = np.arange(d)[None, :]
    bits = np.vectorize(lambda x: bin(int(x)).count("1"))(r & c)
    return np.where(bits % 2 == 0, 1.0, -1.0)


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis (natural
    order): returns x @ sylvester(d)."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def hadamard_projection(signs: np.ndarray, cols: np.ndarray, d: int) -> np.ndarray:
    """H_d in R^{d x k} (section 3.2), subsampled randomized Hadamard:
    H_d[r, c] = signs[r] * (-1)^popcount(r & cols[c]) / sqrt(k)."""
    signs = np.asarray(signs, np.float64)
    cols = np.asarray(cols, np.int64)
    k = cols.shape[0]
    return signs[:, None] * sylvester(d)[:, cols] / math.sqrt(k)


def sketch_from_means(Xbar: np.ndarray, signs, cols) -> np.ndarray:
    """Feature-space sketch of block means: Xbar @ H_d."""
    Xbar = np.asarray(Xbar, np.float64)
    return Xbar @ hadamard_projection(signs, cols, Xbar.shape[1])


def sketch(X: np.ndarray, B: int, signs, cols) -> np.ndarray:
    """Block means then the Hadamard projection: [b, k] (sections 3.1 and 3.2)."""
    return sketch_from_means(block_means(X, B), signs, cols)


def sketched_scores(qs: np.ndarray, ks: np.ndarray) -> np.ndarray:
    """M = tril(Qtilde Ktilde^T) / sqrt(k): the sketched block attention of
    section 3.2, with causal blocks (key block after query block) set to 0."""
    qs = np.asarray(qs, np.float64)
    ks = np.asarray(ks, np.float64)
    k = qs.shape[1]
    return np.tril(qs @ ks.T) / math.sqrt(k)


# ---------------------------------------------------------------------------
# Section 4: the walk state
# ---------------------------------------------------------------------------

def rownorm(X: np.ndarray) -> np.ndarray:
    """Divide each row by its largest magnitude; an all-zero row stays zero."""
    X = np.asarray(X, np.float64)
    m = np.abs(X).max(axis=1, keepdims=True)
    return np.where(m > 0, X / np.where(m > 0, m, 1.0), 0.0)


WALK_FLOOR = 2.0 ** -64


def floor_rows(X: np.ndarray, floor: float = WALK_FLOOR) -> np.ndarray:
    """Entries smaller in magnitude than floor times their row's largest
    magnitude set to zero (the walk state's dynamic range; floor = 0 keeps
    every entry)."""
    X = np.atleast_2d(np.asarray(X, np.float64))
    m = np.abs(X).max(axis=1, keepdims=True)
    return np.where(np.abs(X) < floor * m, 0.0, X)


def walk_update(R_prev: Optional[np.ndarray], M: np.ndarray, s: int,
                floor: float = WALK_FLOOR) -> np.ndarray:
    """R^l = rownorm(R^(l-1) M^s) with R^(-1) = I (section 4): s successive
    right-multiplications by the layer's sketched score matrix, each hop's
    rows cut to the walk state's dynamic range (floor_rows)."""
    M = np.asarray(M, np.float64)
    X = np.eye(M.shape[0]) if R_prev is None else np.asarray(R_prev, np.float64).copy()
    for _ in range(s):
        X = floor_rows(X @ M, floor)
    return rownorm(X)


def walk_row(r_prev: Optional[np.ndarray], M: np.ndarray, i: int, s: int,
             floor: float = WALK_FLOOR) -> np.ndarray:
    """Row i of walk_update, computed as a row vector (decode): r <- r M, s times."""
    M = np.asarray(M, np.float64)
    if r_prev is None:
        x = np.zeros(M.shape[0])
        x[i] = 1.0
    else:
        x = np.asarray(r_prev, np.float64).copy()
    for _ in range(s):
        x = floor_rows(x @ M, floor)[0]
    m = np.abs(x).max()
    return x / m if m > 0 else x


# ---------------------------------------------------------------------------
# Section 4: top-tau selection
# ---------------------------------------------------------------------------

def n_select(rho: int, b: int) -> int:
    """tau = floor(rho * b / 100) (density rho percent of the b blocks)."""
    return (int(rho) * int(b)) // 100


def select_row(row: np.ndarray, i: int, tau: int) -> np.ndarray:
    """Blocks kept for query block i: the tau best earlier blocks m < i ordered
    by (row[m] descending, m ascending), plus block i itself; ascending."""
    cand = np.arange(i, dtype=np.int64)
    if i > tau:
        vals = np.asarray(row[:i], np.float64) + 0.0        # -0.0 -> +0.0
        # lexsort orders by its last key first: value descending, then index
        order = np.lexsort((cand, -vals))
        cand = np.sort(cand[order[:tau]])
    return np.concatenate([cand, [i]]).astype(np.int64)


def select(R: np.ndarray, rho: int, dense: bool = False):
    """Per-row lists for a b x b walk-state matrix (dense: every block <= i)."""
    b = R.shape[0]
    if dense:
        return [np.arange(i + 1, dtype=np.int64) for i in range(b)]
    tau = n_select(rho, b)
    return [select_row(R[i], i, tau) for i in range(b)]


# ---------------------------------------------------------------------------
# Walk variants for readings the page leaves open (kept behind a mode)
# ---------------------------------------------------------------------------

def transition(M: np.ndarray, mode: str, s: int) -> np.ndarray:
    """The block transition matrix T of a walk variant, from the causal
    sketched scores M (entries above the diagonal are not part of the graph):
    * "power"   - the exponent read elementwise: T[i, j] = M[i, j] ** s;
    * "softmax" - the scores turned into transition probabilities: row i of T
                  is the softmax of M[i, 0..i] (0 above the diagonal)."""
    M = np.asarray(M, np.float64)
    b = M.shape[0]
    lower = np.tril(np.ones((b, b), dtype=bool))
    if mode == "power":
        return np.where(lower, M ** s, 0.0)
    if mode == "softmax":
        Z = np.where(lower, M, -np.inf)
        Z = Z - Z.max(axis=1, keepdims=True)
        E = np.exp(Z)
        return E / E.sum(axis=1, keepdims=True)
    raise ValueError(mode)


def walk_update_variant(R_prev: Optional[np.ndarray], M: np.ndarray, s: int,
                        mode: str) -> np.ndarray:
    """Walk state of a variant: "power" takes one step with the elementwise
    power, R = rownorm(R_prev T); "softmax" takes s steps with the transition
    probabilities, R = rownorm(R_prev T^s).  R_prev = None is the identity."""
    T = transition(M, mode, s)
    X = np.eye(T.shape[0]) if R_prev is None else np.asarray(R_prev, np.float64).copy()
    for _ in range(1 if mode == "power" else s):
        X = X @ T
    return rownorm(X)


def walk_row_variant(r_prev: Optional[np.ndarray], M: np.ndarray, i: int, s: int,
                     mode: str) -> np.ndarray:
    """Row i of walk_update_variant, as a row vector (decode)."""
    T = transition(M, mode, s)
    if r_prev is None:
        x = np.zeros(T.shape[0])
        x[i] = 1.0
    else:
        x = np.asarray(r_prev, np.float64).copy()
    for _ in range(1 if mode == "power" else s):
        x = x @ T
    m = np.abs(x).max()
    return x / m if m > 0 else x


# ---------------------------------------------------------------------------
# Selection variants for readings the page leaves open (kept behind flags)
# ---------------------------------------------------------------------------

def n_select_row(rho: int, i: int) -> int:
    """Per-row budget: query block i keeps tau_i = floor(rho * (i + 1) / 100)
    earlier blocks, the same density of its own causal prefix (the decode
    rule, where the open block is the last of the prefix, applied to every
    prefill row)."""
    return (int(rho) * (int(i) + 1)) // 100


def select_rows_tau(R: np.ndarray, rho: int, dense: bool = False):
    """Per-row lists with the per-row budget tau_i of n_select_row."""
    b = R.shape[0]
    if dense:
        return [np.arange(i + 1, dtype=np.int64) for i in range(b)]
    return [select_row(R[i], i, n_select_row(rho, i)) for i in range(b)]


def group_scores(Rs) -> np.ndarray:
    """Shared walk score of a KV group (GQA): the walk states of the group's
    query heads added up, in fp32 and in ascending head order.  The score only
    decides an integer result (which blocks are kept), so it is formed in the
    precision and order the kernels use, and the selections compare exactly."""
    acc = np.asarray(Rs[0], np.float32).copy()
    for R in Rs[1:]:
        acc = (acc + np.asarray(R, np.float32)).astype(np.float32)
    return acc


# ---------------------------------------------------------------------------
# Sections 4-5: block-sparse attention on the original Q, K, V
# ---------------------------------------------------------------------------

def sparse_attention_rows(Q, K, V, lists, B: int, scale: float, rows: Sequence[int]):
    """Attention for the query blocks in `rows` only (single head, one
    sequence).  Token t of block i attends to every key u <= t lying in a block
    of lists[i]; the softmax is renormalised over those keys.
    Returns {i: (O_block [c_i, d], lse [c_i])}."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n = Q.shape[0]
    out = {}
    for i in rows:
        a, e = i * B, min((i + 1) * B, n)
        keys = np.concatenate([np.arange(j * B, min((j + 1) * B, n)) for j in lists[i]])
        Z = (Q[a:e] @ K[keys].T) * scale
        allowed = keys[None, :] <= np.arange(a, e)[:, None]
        Z = np.where(allowed, Z, -np.inf)
        zmax = Z.max(axis=1, keepdims=True)
        P = np.exp(Z - zmax)
        l = P.sum(axis=1, keepdims=True)
        out[i] = ((P @ V[keys]) / l, (zmax + np.log(l))[:, 0])
    return out


def query_attention(q, K, V, lst, B: int, p: int, scale: float):
    """Attention of the single query token at position p (a decode step) over
    the keys u <= p that lie in the blocks of `lst`: the softmax of
    q . K[u] * scale renormalised over those keys, applied to V.  This is row p
    of sparse_attention_rows for the block holding p, without the block's
    other rows.  Returns (o [d], lse)."""
    q = np.asarray(q, np.float64)
    keys = np.concatenate([np.arange(j * B, min((j + 1) * B, p + 1)) for j in lst])
    Kr = np.asarray(K[keys], np.float64)
    Vr = np.asarray(V[keys], np.float64)
    z = (Kr @ q) * scale
    zmax = z.max()
    w = np.exp(z - zmax)
    return (w @ Vr) / w.sum(), float(zmax + math.log(w.sum()))


def sparse_attention(Q, K, V, lists, B: int, scale: Optional[float] = None):
    """Full single-head attention output O [n, d] and log-sum-exp [n]."""
    Q = np.asarray(Q, np.float64)
    n, d = Q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    res = sparse_attention_rows(Q, K, V, lists, B, scale, range(n_blocks(n, B)))
    O = np.concatenate([res[i][0] for i in sorted(res)])
    lse = np.concatenate([res[i][1] for i in sorted(res)])
    return O, lse


# ---------------------------------------------------------------------------
# One layer / a stack of layers (prefill), GQA and ragged batches
# ---------------------------------------------------------------------------

class SeqPrefill:
    """State of the oracle prefill for one sequence: the walk state per query
    head, carried from layer to layer."""

    def __init__(self, hq: int):
        self.R = [None] * hq


def prefill_layer(Q, K, V, state: SeqPrefill, signs, cols, B: int, s: int, rho: int,
                  dense: bool, attn_rows=None, with_attention=True):
    """One layer for one sequence.  Q [n, Hq, d], K and V [n, Hkv, d].
    Updates state.R and returns per-head dicts with qs, ks, M, R, lists and
    (if requested) the attention output / lse (for attn_rows blocks only when
    given)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n, hq, d = Q.shape
    hkv = K.shape[1]
    grp = hq // hkv
    ks_all = [sketch(K[:, g, :], B, signs, cols) for g in range(hkv)]
    out = []
    for h in range(hq):
        g = h // grp
        qs = sketch(Q[:, h, :], B, signs, cols)
        M = sketched_scores(qs, ks_all[g])
        R = walk_update(state.R[h], M, s)
        state.R[h] = R
        lists = select(R, rho, dense)
        rec = {"qs": qs, "ks": ks_all[g], "M": M, "R": R, "lists": lists}
        if with_attention:
            scale = 1.0 / math.sqrt(d)
            rows = range(len(lists)) if attn_rows is None else attn_rows
            rec["attn"] = sparse_attention_rows(Q[:, h, :], K[:, g, :], V[:, g, :], lists, B,
                                                scale, rows)
        out.append(rec)
    return out


def prefill(layers, signs, cols, B: int, s: int, rho: int, n_dense: int = 2,
            attn_rows=None, with_attention=True):
    """Whole stack for one sequence; `layers` is a list of (Q, K, V)."""
    hq = np.asarray(layers[0][0]).shape[1]
    st = SeqPrefill(hq)
    return [prefill_layer(Q, K, V, st, signs, cols, B, s, rho, l < n_dense, attn_rows,
                          with_attention)
            for l, (Q, K, V) in enumerate(layers)]


# ---------------------------------------------------------------------------
# Section 5: decode - the same selection rule for one new token
# ---------------------------------------------------------------------------

def decode_step(layers_prefix, signs, cols, B: int, s: int, rho: int, n_dense: int = 2):
    """Decode of the token at position p = len(prefix) - 1 for one sequence.

    Defined as row p of the prefill over the first p + 1 tokens: for every
    layer the open block c = floor(p / B) is averaged over the tokens it holds
    so far, and only row c of the walk state is carried (a row vector).
    `layers_prefix` is a list of (Q, K, V) with p + 1 tokens each.
    Returns per layer a list over query heads of dicts with qs, ks, r (the
    row), lst and o (attention output [d]) and lse."""
    out = []
    hq = np.asarray(layers_prefix[0][0]).shape[1]
    r = [None] * hq
    for l, (Q, K, V) in enumerate(layers_prefix):
        Q = np.asarray(Q, np.float64)
        K = np.asarray(K, np.float64)
        V = np.asarray(V, np.float64)
        n, _, d = Q.shape
        p = n - 1
        c = p // B
        hkv = K.shape[1]
        grp = hq // hkv
        ks_all = [sketch(K[:, g, :], B, signs, cols) for g in range(hkv)]
        heads = []
        for h in range(hq):
            g = h // grp
            qs = sketch(Q[:, h, :], B, signs, cols)
            M = sketched_scores(qs, ks_all[g])
            r[h] = walk_row(r[h], M, c, s)
            b = c + 1
            lst = (np.arange(b, dtype=np.int64) if l < n_dense
                   else select_row(r[h], c, n_select(rho, b)))
            o, lse = query_attention(Q[p, h, :], K[:, g, :], V[:, g, :], lst, B, p,
                                     1.0 / math.sqrt(d))
            heads.append({"qs": qs, "ks": ks_all[g], "r": r[h].copy(), "lst": lst, "o": o,
                          "lse": lse})
        out.append(heads)
    return out


# ---------------------------------------------------------------------------
# Section 11.4 (serving integration): paged KV caches and low-precision KV
# ---------------------------------------------------------------------------

def fp8_e4m3_value(codes) -> np.ndarray:
    """Value of OCP 8-bit floating-point E4M3 codes (OCP "8-bit Floating Point
    Specification (OFP8)"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent field 0 is subnormal (m / 8 * 2^-6); S.1111.111 is NaN and
    there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def gather_pages(pages, table_row, n: int, B: int) -> np.ndarray:
    """The contiguous cache rows of one sequence of n tokens held in pages of B
    tokens: token t lives in row t % B of page table_row[t // B]."""
    pages = np.asarray(pages)
    return np.stack([pages[int(table_row[t // B]), t % B] for t in range(n)])
