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
