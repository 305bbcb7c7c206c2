"""The seeded generators: determinism, shapes, storage rounding, paging structure."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e-40, 3.3e38, -1.00390625, 1.00390625], np.float32)])
    ours = W.f32_to_storage_bits(x, W.BF16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    ours16 = W.f32_to_storage_bits(x, W.F16)
    ref16 = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours16, ref16)


def test_contiguous_deterministic_and_shaped():
    a = W.contiguous_case("a", 5, 2, 8, 2, 64, 33)
    b = W.contiguous_case("a", 5, 2, 8, 2, 64, 33)
    assert a.q.shape == (2, 8, 64) and a.k.shape == (2, 33, 2, 64)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v) and np.array_equal(a.q, b.q)
    assert not np.array_equal(a.k, a.v)
    assert a.kv_bytes == 2 * 33 * 2 * 64 * 4
    c = W.contiguous_case("a", 6, 2, 8, 2, 64, 33)
    assert not np.array_equal(a.k, c.k)


def test_paged_structure_and_poison():
    ctx = [17, 16, 1, 0, 40]
    c = W.paged_case("p", 3, ctx, 4, 2, 8, W.F16, 16, extra_blocks=3)
    nblk = [(L + 15) // 16 for L in ctx]
    assert c.k.shape == (sum(nblk) + 3, 16, 2, 8)
    used = []
    for s, L in enumerate(ctx):
        row = c.block_table[s]
        assert np.all(row[nblk[s]:] == -1)
        used += row[:nblk[s]].tolist()
        for t in range(L):                      # every live slot is finite
            f = c.k[row[t // 16], t % 16].view(np.float16)
            assert np.all(np.isfinite(f))
        if L % 16:                              # tail slots poisoned
            tail = c.k[row[nblk[s] - 1], L % 16:].view(np.float16)
            assert np.all(np.isnan(tail))
    assert sorted(used) == sorted(set(used))    # no block shared
    spare = sorted(set(range(c.k.shape[0])) - set(used))
    assert len(spare) == 3 and np.all(np.isnan(c.v[spare].view(np.float16)))


def test_named_workloads_small_and_lengths():
    t = W.workload("tiny_contig")
    assert (t.num_seqs, t.h_q, t.h_kv, t.d, t.s_kv, t.dtype) == (1, 4, 1, 64, 256, W.F16)
    assert t.kv_bytes == 65536
    L3 = W.uniform_lengths(1002, 64, 512, 8192)
    assert L3.min() >= 512 and L3.max() <= 8192
    L5 = W.lognormal_lengths(1004, 256, 2048.0, 1.0, 64, 32768)
    assert L5.min() >= 64 and L5.max() <= 32768
    assert (L5 > 8192).any() and (L5 <= 8192).any()     # both single pass and split fire
    assert np.array_equal(L5, W.lognormal_lengths(1004, 256, 2048.0, 1.0, 64, 32768))


def test_xsplit_case_is_a_rearrangement():
    rows = W.paged_case("xr", 5, [20, 3, 16], h_q=4, h_kv=2, d=16, dtype=W.F16,
                        block_size=16, extra_blocks=1)
    xs = W.xsplit_case(rows)
    nb, bs, h_kv, d = rows.k.shape
    assert xs.layout == "paged_xsplit"
    assert xs.k.shape == (nb, h_kv, d // 8, bs, 8) and xs.v.shape == (nb, h_kv, d, bs)
    for b in range(nb):
        for o in range(bs):
            for j in range(h_kv):
                for dd in range(d):
                    assert xs.k[b, j, dd // 8, o, dd % 8] == rows.k[b, o, j, dd]
                    assert xs.v[b, j, dd, o] == rows.v[b, o, j, dd]
    # poison moves with its slot: sequence 0's last block holds 4 live slots of 16
    b = rows.block_table[0, 1]
    assert np.all(xs.k[b, :, :, 4:, :] == W.NAN_BITS[W.F16])
    assert np.all(xs.v[b, :, :, 4:] == W.NAN_BITS[W.F16])
    assert np.array_equal(xs.q, rows.q) and np.array_equal(xs.block_table, rows.block_table)


def test_multi_token_query_shape():
    c = W.paged_case("mt", 6, [10, 40], h_q=8, h_kv=2, d=64, dtype=W.BF16, t_q=3)
    assert c.q.shape == (2, 3, 8, 64) and c.t_q == 3
    one = W.paged_case("mt1", 6, [10, 40], h_q=8, h_kv=2, d=64, dtype=W.BF16)
    assert one.q.shape == (2, 8, 64) and one.t_q == 1
    assert np.array_equal(c.k, one.k) and np.array_equal(c.v, one.v)   # K/V streams independent of q
    cc = W.contiguous_case("mtc", 7, 2, 4, 1, 64, 33, W.F16, t_q=2)
    assert cc.q.shape == (2, 2, 4, 64)
