"""Seeded synthetic inputs for single-query GQA decode attention.

This module is shared by the CPU oracle's tests and by the GPU path (tests,
bench, smoke).  It holds no attention arithmetic: only random draws, the
rounding of float32 draws to fp16/bf16 storage, sequence-length draws and the
two K/V cache layouts.

Layouts (all row-major):
  q               [num_seqs, h_q, d]                      fp16/bf16 bits (uint16)
                  [num_seqs, t_q, h_q, d] with t_q > 1 query tokens per sequence
  contiguous k,v  [num_seqs, s_kv, h_kv, d]               one (S_kv, h_kv*d) slab per
                                                          sequence, as the decode-long
                                                          page lays K and V out
  paged k,v pool  [num_blocks, block_size, h_kv, d]       the same rows cut into blocks
  x-split k pool  [num_blocks, h_kv, d/8, block_size, 8]  the kernel-map page's key_cache
  x-split v pool  [num_blocks, h_kv, d, block_size]       (layout "paged_xsplit")
  block_table     [num_seqs, max_blocks_per_seq] int32    padded with -1
  ctx_lens        [num_seqs] int32

Every case is drawn from ``numpy.random.SeedSequence(seed)`` spawned into five
independent streams (ctx, perm, q, k, v), each fed to ``default_rng``.  Values
are standard normals drawn in float32 and rounded to nearest-even into the
storage dtype.  Unused slots of a sequence's last block and every pool block
no sequence references are filled with NaN, so a read of them poisons the
output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F16 = "f16"
BF16 = "bf16"
DTYPES = (F16, BF16)

NAN_BITS = {F16: np.uint16(0x7E00), BF16: np.uint16(0x7FC0)}

_CHUNK = 1 << 24  # elements drawn per batch, bounds float32 temporaries


def f32_to_storage_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to fp16/bf16 (nearest-even); return the uint16 bits."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = x.view(np.uint32).astype(np.uint64)
        rnd = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
        out = ((u + rnd) >> np.uint64(16)).astype(np.uint16)
        out[np.isnan(x)] = NAN_BITS[BF16]
        return out
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        out[lo:hi] = f32_to_storage_bits(
            rng.standard_normal(hi - lo, dtype=np.float32), dtype)
    return out.reshape(shape)


@dataclasses.dataclass
class DecodeCase:
    """One batch of decode-attention inputs (storage bits + metadata)."""
    name: str
    dtype: str
    layout: str                 # "contiguous", "paged" or "paged_xsplit"
    q: np.ndarray               # uint16 [num_seqs, h_q, d]
    k: np.ndarray               # uint16, layout-dependent (see module doc)
    v: np.ndarray
    ctx_lens: np.ndarray        # int32 [num_seqs]
    block_table: Optional[np.ndarray]  # int32 [num_seqs, max_blocks] or None
    h_q: int
    h_kv: int
    d: int
    scale: float
    block_size: int = 16
    s_kv: int = 0               # contiguous only

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def t_q(self) -> int:
        return int(self.q.shape[1]) if self.q.ndim == 4 else 1

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def max_blocks(self) -> int:
        return 0 if self.block_table is None else int(self.block_table.shape[1])

    @property
    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode step reads: sum_s L_s*h_kv*d*2 (K and V)*2 B."""
        return int(self.ctx_lens.astype(np.int64).sum()) * self.h_kv * self.d * 2 * 2


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.default_rng(c) for c in ss.spawn(5)]


def _q_shape(num_seqs: int, t_q: int, h_q: int, d: int):
    return (num_seqs, h_q, d) if t_q == 1 else (num_seqs, t_q, h_q, d)


def contiguous_case(name: str, seed: int, num_seqs: int, h_q: int, h_kv: int,
                    d: int, s_kv: int, dtype: str = F16,
                    scale: Optional[float] = None, t_q: int = 1) -> DecodeCase:
    """Contiguous cache: every sequence holds ``s_kv`` tokens."""
    _, _, rq, rk, rv = _streams(seed)
    q = _normal_bits(rq, _q_shape(num_seqs, t_q, h_q, d), dtype)
    k = _normal_bits(rk, (num_seqs, s_kv, h_kv, d), dtype)
    v = _normal_bits(rv, (num_seqs, s_kv, h_kv, d), dtype)
    return DecodeCase(name=name, dtype=dtype, layout="contiguous", q=q, k=k, v=v,
                      ctx_lens=np.full(num_seqs, s_kv, dtype=np.int32),
                      block_table=None, h_q=h_q, h_kv=h_kv, d=d,
                      scale=float(1.0 / math.sqrt(d) if scale is None else scale),
                      s_kv=s_kv)


def paged_case(name: str, seed: int, ctx_lens, h_q: int, h_kv: int, d: int,
               dtype: str = F16, block_size: int = 16,
               max_blocks: Optional[int] = None, extra_blocks: int = 0,
               scale: Optional[float] = None, poison: bool = True,
               t_q: int = 1) -> DecodeCase:
    """Paged cache with a seeded random permutation of physical blocks.

    The pool holds ``sum_s ceil(L_s/bs) + extra_blocks`` blocks; sequence s gets
    the next ceil(L_s/bs) entries of a random permutation of all block ids.
    With ``poison`` the unused tail slots of each last block and the extra blocks
    are NaN.
    """
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    _, rperm, rq, rk, rv = _streams(seed)
    num_seqs = int(ctx.shape[0])
    nblk = (ctx.astype(np.int64) + block_size - 1) // block_size
    used = int(nblk.sum())
    num_blocks = used + int(extra_blocks)
    if max_blocks is None:
        max_blocks = max(1, int(nblk.max()) if num_seqs else 1)
    assert max_blocks >= (int(nblk.max()) if num_seqs else 0)
    perm = rperm.permutation(num_blocks).astype(np.int32)
    table = np.full((num_seqs, max_blocks), -1, dtype=np.int32)
    off = 0
    for s in range(num_seqs):
        table[s, :nblk[s]] = perm[off:off + nblk[s]]
        off += int(nblk[s])
    q = _normal_bits(rq, _q_shape(num_seqs, t_q, h_q, d), dtype)
    pool_shape = (num_blocks, block_size, h_kv, d)
    k = _normal_bits(rk, pool_shape, dtype)
    v = _normal_bits(rv, pool_shape, dtype)
    if poison:
        nan = NAN_BITS[dtype]
        for s in range(num_seqs):
            L = int(ctx[s])
            if L % block_size and nblk[s]:
                b = table[s, nblk[s] - 1]
                k[b, L % block_size:] = nan
                v[b, L % block_size:] = nan
        if extra_blocks:
            spare = perm[used:]
            k[spare] = nan
            v[spare] = nan
    return DecodeCase(name=name, dtype=dtype, layout="paged", q=q, k=k, v=v,
                      ctx_lens=ctx, block_table=table, h_q=h_q, h_kv=h_kv, d=d,
                      scale=float(1.0 / math.sqrt(d) if scale is None else scale),
                      block_size=block_size)


XSPLIT_X = 8   # elements per 16-byte vector of fp16/bf16


def xsplit_case(case: DecodeCase) -> DecodeCase:
    """The same logical cache as a paged case, in the x-split pool layout:
    k[b, j, d // 8, o, d % 8] and v[b, j, d, o] hold element d of slot o of KV
    head j in block b (a pure rearrangement; NaN poison moves with its slot)."""
    assert case.layout == "paged"
    nb, bs, h_kv, d = case.k.shape
    assert d % XSPLIT_X == 0
    k = np.ascontiguousarray(
        case.k.reshape(nb, bs, h_kv, d // XSPLIT_X, XSPLIT_X).transpose(0, 2, 3, 1, 4))
    v = np.ascontiguousarray(case.v.transpose(0, 2, 3, 1))
    return dataclasses.replace(case, name=case.name + "_xsplit", layout="paged_xsplit", k=k, v=v)


# ---------------------------------------------------------------------------
# The five named workloads.  Lengths for the two paged ones are drawn from the
# "ctx" stream of the same seed.
# ---------------------------------------------------------------------------

WORKLOADS = {
    # name: (index, description)
    "tiny_contig": (0, "B=1, h_q=4, h_kv=1, d=64, S_kv=256, fp16, contiguous"),
    "contig_b8": (1, "B=8, h_q=32, h_kv=8, d=128, S_kv=4096, fp16, contiguous"),
    "paged_b64": (2, "B=64, h_q=32, h_kv=8, d=128, bs=16, L~U{512..8192}, fp16, paged"),
    "long_128k": (3, "B=1, h_q=64, h_kv=8, d=128, S_kv=131072, bf16, contiguous"),
    "mixed_b256": (4, "B=256, h_q=32, h_kv=4, d=128, bs=16, L=clip(lognormal(ln 2048, 1), 64, 32768), fp16, paged"),
    # head dimension 256 (a shape of its own, beside the five above)
    "contig_d256": (5, "B=2, h_q=32, h_kv=8, d=256, S_kv=32768, bf16, contiguous"),
    # four query tokens per sequence (T_q = 4, G * T_q = 16)
    "paged_b64_t4": (6, "B=64, T_q=4, h_q=32, h_kv=8, d=128, bs=16, L~U{512..8192}, fp16, paged"),
}


def uniform_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    rctx = _streams(seed)[0]
    return rctx.integers(lo, hi + 1, size=n).astype(np.int32)


def lognormal_lengths(seed: int, n: int, median: float, sigma: float,
                      lo: int, hi: int) -> np.ndarray:
    rctx = _streams(seed)[0]
    z = rctx.standard_normal(n)
    return np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int32)


def workload(name: str, poison: bool = True) -> DecodeCase:
    """Build one of the named workloads (seed = 1000 + index)."""
    idx = WORKLOADS[name][0]
    seed = 1000 + idx
    if name == "tiny_contig":
        return contiguous_case(name, seed, 1, 4, 1, 64, 256, F16)
    if name == "contig_b8":
        return contiguous_case(name, seed, 8, 32, 8, 128, 4096, F16)
    if name == "paged_b64":
        ctx = uniform_lengths(seed, 64, 512, 8192)
        return paged_case(name, seed, ctx, 32, 8, 128, F16, 16, poison=poison)
    if name == "long_128k":
        return contiguous_case(name, seed, 1, 64, 8, 128, 131072, BF16)
    if name == "mixed_b256":
        ctx = lognormal_lengths(seed, 256, 2048.0, 1.0, 64, 32768)
        return paged_case(name, seed, ctx, 32, 4, 128, F16, 16, poison=poison)
    if name == "contig_d256":
        return contiguous_case(name, seed, 2, 32, 8, 256, 32768, BF16)
    if name == "paged_b64_t4":
        ctx = uniform_lengths(seed, 64, 512, 8192)
        return paged_case(name, seed, ctx, 32, 8, 128, F16, 16, poison=poison, t_q=4)
    raise KeyError(name)
