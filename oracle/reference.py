"""Float64 reference for GQA decode attention (TEST INFRASTRUCTURE).

Only tests/, the entry file's smoke() and the bench's cpu_baseline leg may use
this module.  It shares no code with the HIP path.

Definition followed (decode-long page, "Local attention" and "Final normalise
+ store"; kernel-map page, ``paged_attention_v1``): for sequence s, query head
i, KV head j = floor(i / G) with G = h_q / h_kv, and logical tokens
t in [0, L_s):

    x_t   = scale * <q[s, i, :], K_s[t, :]>
    w_t   = exp(x_t - max_u x_u) / sum_u exp(x_u - max_u x_u)
    out   = sum_t w_t V_s[t, :]

Every stored fp16/bf16 operand is upcast exactly to float64 first, so input
quantisation is not part of any error measured against this module.

Readings where the pages are silent or loose:
  * ``scale`` multiplies the logits (the decode-long page's ``tl.dot`` carries
    no softmax scale; the workloads use 1/sqrt(d)).
  * K enters as a true transpose (the page's reshape-not-transpose load is a
    simulator caveat, not the mathematics).
  * query head i reads KV head floor(i / G) (consecutive groups).
  * max / sum / normalise act per query row.
  * L_s = 0 yields a zero output row.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

Triple = Tuple[np.ndarray, np.ndarray, np.ndarray]   # (m, l, O)


# ---------------------------------------------------------------- storage ---

def upcast(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of fp16 ("f16") or bf16 ("bf16") storage bits."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------- gather ---

def kv_head(i: int, group: int) -> int:
    """KV head read by query head i: the G consecutive query heads share one."""
    return i // group


def gather_contiguous(k: np.ndarray, v: np.ndarray, s: int, j: int, L: int):
    """K_s, V_s rows [0, L) of KV head j from a [num_seqs, S, h_kv, d] cache."""
    return k[s, :L, j, :], v[s, :L, j, :]


def gather_paged(k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray,
                 s: int, j: int, L: int, block_size: int):
    """K_s, V_s for logical tokens t < L of a [num_blocks, bs, h_kv, d] pool.

    Token t lives in physical block block_table[s, t // bs], slot t % bs.
    Table entries past ceil(L / bs) and slots past L are never touched.
    """
    rows_k, rows_v = [], []
    for t in range(L):
        b = int(block_table[s, t // block_size])
        rows_k.append(k_pool[b, t % block_size, j, :])
        rows_v.append(v_pool[b, t % block_size, j, :])
    d = k_pool.shape[-1]
    if not rows_k:
        return (np.zeros((0, d), k_pool.dtype), np.zeros((0, d), v_pool.dtype))
    return np.stack(rows_k), np.stack(rows_v)


def gather_paged_xsplit(k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray,
                        s: int, j: int, L: int, block_size: int):
    """K_s, V_s for logical tokens t < L of an x-split pool.

    Kernel-map page, ``paged_attention_v1``: the key cache is
    [num_blocks, num_kv_heads, head_dim // x, block_size, x], so element d of
    the token in slot o of block b is k_pool[b, j, d // x, o, d % x] (x is the
    pool's last extent).  The page gives no value-cache layout; the reading
    used here is [num_blocks, num_kv_heads, head_dim, block_size], element
    v_pool[b, j, d, o].
    """
    x = k_pool.shape[-1]
    d = k_pool.shape[2] * x
    K = np.zeros((L, d), dtype=k_pool.dtype)
    V = np.zeros((L, d), dtype=v_pool.dtype)
    for t in range(L):
        b = int(block_table[s, t // block_size])
        o = t % block_size
        # the [d // x, d % x] slice read in C order is d = (d // x) * x + d % x
        K[t, :] = k_pool[b, j, :, o, :].reshape(d)
        V[t, :] = v_pool[b, j, :, o]
    return K, V


def sequence_kv(case, s: int, j: int):
    """Float64 K_s, V_s of (sequence s, KV head j) for a workloads.DecodeCase."""
    L = int(case.ctx_lens[s])
    if case.layout == "contiguous":
        K, V = gather_contiguous(case.k, case.v, s, j, L)
    elif case.layout == "paged_xsplit":
        K, V = gather_paged_xsplit(case.k, case.v, case.block_table, s, j, L, case.block_size)
    else:
        K, V = gather_paged(case.k, case.v, case.block_table, s, j, L, case.block_size)
    return upcast(K, case.dtype), upcast(V, case.dtype)


# ------------------------------------------------------------- definition ---

def logits(q_row: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """x_t = scale * sum_d q[d] * K[t, d]   (true K transpose)."""
    return scale * (K @ q_row)


def softmax(x: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the token axis."""
    M = np.max(x)
    e = np.exp(x - M)
    return e / np.sum(e)


def attend(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for one query row; zero row when there are no tokens."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[-1], dtype=np.float64)
    return softmax(logits(q_row, K, scale)) @ V


def decode(case, heads: Optional[Iterable[Tuple[int, int]]] = None) -> np.ndarray:
    """Reference output in float64: [num_seqs, h_q, d], or [num_seqs, T_q, h_q, d]
    for a case with T_q query tokens per sequence (a 4-D q).  Only the listed
    (s, i) rows are computed (for every query token); the others stay NaN.

    T_q > 1 (decode-long page, tensor-layout docstring: Q is (T_q, h_q * d_head)
    per sequence and O has the same shape; the page applies no mask): every
    query token of sequence s attends to all L_s keys of the cache.
    """
    G = case.h_q // case.h_kv
    q = case.q if case.q.ndim == 4 else case.q[:, None]        # [B, T_q, h_q, d]
    out = np.full((case.num_seqs, q.shape[1], case.h_q, case.d), np.nan, dtype=np.float64)
    if heads is None:
        heads = [(s, i) for s in range(case.num_seqs) for i in range(case.h_q)]
    by_pair = {}
    for s, i in heads:
        by_pair.setdefault((s, kv_head(i, G)), []).append(i)
    for (s, j), idx in sorted(by_pair.items()):
        K, V = sequence_kv(case, s, j)
        for tau in range(q.shape[1]):
            for i in idx:
                out[s, tau, i] = attend(upcast(q[s, tau, i], case.dtype), K, V, case.scale)
    return out if case.q.ndim == 4 else out[:, 0]


# ------------------------------------------------- partial triples, merge ---

def partial(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> Triple:
    """(m, l, O) of one token range, O un-normalised.

    decode-long page, "Local attention" tile step: m = max of the scores,
    l = sum exp(scores - m), O = exp(scores - m) @ V.  An empty range is the
    merge identity (-inf, 0, 0).
    """
    d = V.shape[-1]
    if K.shape[0] == 0:
        return (np.float64(-np.inf), np.float64(0.0), np.zeros(d, dtype=np.float64))
    x = logits(q_row, K, scale)
    m = np.max(x)
    e = np.exp(x - m)
    return (np.float64(m), np.float64(np.sum(e)), e @ V)


def merge(a: Triple, b: Triple) -> Triple:
    """decode-long page, ``_merge_running``: rescale both sides to the larger max.

    m = max(m_a, m_b); l = l_a e^{m_a - m} + l_b e^{m_b - m};
    O = O_a e^{m_a - m} + O_b e^{m_b - m}.  When both maxima are -inf (two
    empty ranges) the page's formula would form -inf - (-inf); the identity is
    returned instead.
    """
    m_a, l_a, O_a = a
    m_b, l_b, O_b = b
    m = max(m_a, m_b)
    if m == -np.inf:
        return (np.float64(-np.inf), np.float64(0.0), np.zeros_like(O_a))
    sa = math.exp(m_a - m)
    sb = math.exp(m_b - m)
    return (np.float64(m), l_a * sa + l_b * sb, O_a * sa + O_b * sb)


def normalize(t: Triple) -> np.ndarray:
    """decode-long page, "Final normalise + store": O / l (zero row if l = 0)."""
    m, l, O = t
    if l == 0:
        return np.zeros_like(O)
    return O / l


# ---------------------------------------------------- work decomposition ---

def partition_bounds(L: int, partition_size: int, v1_max_ctx: int) -> List[Tuple[int, int]]:
    """Token ranges one sequence is cut into.

    kernel-map page, ``paged_attention_v1`` / ``v2`` and policy page,
    ``AttentionConfig``: a sequence of at most ``v1_max_ctx`` tokens is one
    range (single pass); a longer one is cut into ceil(L / partition_size)
    ranges of ``partition_size`` tokens, the last one shorter.  No range is
    empty and no token is dropped.
    """
    if L <= v1_max_ctx:
        return [(0, L)]
    return [(t0, min(t0 + partition_size, L)) for t0 in range(0, L, partition_size)]


def split_attend(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                 bounds: Sequence[Tuple[int, int]]) -> np.ndarray:
    """The method's split form: a partial triple per range, merged left to right
    (the order of the page's chain), then normalised once."""
    acc = partial(q_row, K[:0], V[:0], scale)
    for t0, t1 in bounds:
        acc = merge(acc, partial(q_row, K[t0:t1], V[t0:t1], scale))
    return normalize(acc)
