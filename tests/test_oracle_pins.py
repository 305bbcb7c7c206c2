"""Pins of the float64 oracle against facts fixed outside its own code.

Each pin is a function of no arguments that raises AssertionError when the
oracle disagrees with: the hand-derived closed forms in tests/golden, a
40-digit Decimal brute force, closed forms (one token, zero query, two
tokens), invariances of softmax attention, the merge identity of the
decode-long page's ``_merge_running``, a library routine
(torch scaled_dot_product_attention in float64 on the CPU) and the paged
gather against the contiguous layout.

``test_planted_mistakes`` then plants plausible mistakes in the oracle (on the
CPU) and checks that at least one pin fails for each, so the pins are known to
bite.
"""
import dataclasses
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute
from oracle import reference as R
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form.json")


# ------------------------------------------------------------ helpers ---

def _case_from_json(c):
    """Build a DecodeCase (f16 storage) from a golden fixture entry."""
    def bits(a):
        arr = np.array([[np.nan if x is None else x for x in _flat(a)]], dtype=np.float64)
        return W.f32_to_storage_bits(arr.astype(np.float32), W.F16).reshape(_shape(a))
    q = bits(c["q"])
    k = bits(c["k"])
    v = bits(c["v"])
    table = None if c["layout"] == "contiguous" else np.array(c["block_table"], np.int32)
    return W.DecodeCase(name=c["name"], dtype=W.F16, layout=c["layout"], q=q, k=k, v=v,
                        ctx_lens=np.array(c["ctx_lens"], np.int32), block_table=table,
                        h_q=c["h_q"], h_kv=c["h_kv"], d=c["d"], scale=math.log(2.0),
                        block_size=c.get("block_size", 16),
                        s_kv=(len(c["k"][0]) if c["layout"] == "contiguous" else 0))


def _flat(a):
    if isinstance(a, list):
        for x in a:
            yield from _flat(x)
    else:
        yield a


def _shape(a):
    s = []
    while isinstance(a, list):
        s.append(len(a))
        a = a[0]
    return tuple(s)


def _closed_form(c, s, i):
    """Exact rational output of (s, i): weights 2^n_t / sum 2^n_u, n_t = <q, k_t>."""
    G = c["h_q"] // c["h_kv"]
    j = i // G
    L = c["ctx_lens"][s]
    rows_k, rows_v = [], []
    for t in range(L):
        if c["layout"] == "contiguous":
            rows_k.append(c["k"][s][t][j])
            rows_v.append(c["v"][s][t][j])
        else:
            bs = c["block_size"]
            b = c["block_table"][s][t // bs]
            rows_k.append(c["k"][b][t % bs][j])
            rows_v.append(c["v"][b][t % bs][j])
    q = c["q"][s][i]
    n = [sum(a * b for a, b in zip(q, kr)) for kr in rows_k]
    wts = [Fraction(2) ** x for x in n]
    den = sum(wts)
    return [sum(w * Fraction(vr[col]) for w, vr in zip(wts, rows_v)) / den
            for col in range(c["d"])]


def _rand_case(rng, L, d, dtype=np.float64):
    q = rng.standard_normal(d)
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    return q, K, V


# --------------------------------------------------------------- pins ---

def pin_golden_closed_form():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        case = _case_from_json(c)
        out = R.decode(case)
        for s in range(case.num_seqs):
            for i in range(case.h_q):
                exact = _closed_form(c, s, i)
                got = out[s, i]
                assert np.all(np.isfinite(got)), (c["name"], s, i, got)
                err = max(abs(float(e) - g) for e, g in zip(exact, got))
                assert err <= 1e-12, (c["name"], s, i, got, [str(e) for e in exact])
        for key, vals in c["hand_checked"].items():
            s, i = int(key[1]), int(key.split("_h")[1])
            assert [str(x) for x in _closed_form(c, s, i)] == vals, key


def pin_brute_force_tiny():
    rng = np.random.default_rng(7)
    for _ in range(12):
        L = int(rng.integers(1, 9))
        d = int(rng.integers(1, 9))
        scale = float(rng.uniform(0.2, 2.0))
        q, K, V = _rand_case(rng, L, d)
        ref = R.attend(q, K, V, scale)
        bf = np.array(brute.attend_decimal(q.tolist(), K.tolist(), V.tolist(), scale))
        assert np.max(np.abs(ref - bf)) <= 1e-13, (ref, bf)


def pin_brute_force_gqa_paged():
    """Whole decode over a tiny paged GQA case vs brute force per (s, i)."""
    case = W.paged_case("tiny_paged", 11, [5, 1, 8], h_q=4, h_kv=2, d=8,
                        dtype=W.BF16, block_size=4, extra_blocks=1)
    out = R.decode(case)
    G = case.h_q // case.h_kv
    for s in range(case.num_seqs):
        L = int(case.ctx_lens[s])
        for i in range(case.h_q):
            j = i // G
            Ks, Vs = [], []
            for t in range(L):
                b = int(case.block_table[s, t // case.block_size])
                Ks.append(R.upcast(case.k[b, t % case.block_size, j], case.dtype).tolist())
                Vs.append(R.upcast(case.v[b, t % case.block_size, j], case.dtype).tolist())
            qv = R.upcast(case.q[s, i], case.dtype).tolist()
            bf = np.array(brute.attend_decimal(qv, Ks, Vs, case.scale))
            assert np.max(np.abs(out[s, i] - bf)) <= 1e-13, (s, i)


def pin_single_token():
    """S_kv = 1 gives O = v_0 exactly."""
    rng = np.random.default_rng(3)
    for d in (1, 4, 64, 128):
        q, K, V = _rand_case(rng, 1, d)
        assert np.array_equal(R.attend(q, K, V, 0.7), V[0])


def pin_zero_query_mean():
    """q = 0 gives the mean of the V rows (uniform weights)."""
    rng = np.random.default_rng(4)
    for L in (1, 2, 7, 300):
        _, K, V = _rand_case(rng, L, 16)
        got = R.attend(np.zeros(16), K, V, 1.0)
        assert np.max(np.abs(got - V.mean(axis=0))) <= 1e-14


def pin_identical_keys_mean():
    rng = np.random.default_rng(5)
    q, K, V = _rand_case(rng, 9, 8)
    K[:] = K[0]
    assert np.max(np.abs(R.attend(q, K, V, 2.0) - V.mean(axis=0))) <= 1e-14


def pin_weights_simplex():
    rng = np.random.default_rng(6)
    for L in (1, 3, 1000):
        x = rng.standard_normal(L) * 5
        w = R.softmax(x)
        assert np.all(w >= 0) and abs(np.sum(w) - 1.0) <= 1e-15 * max(1, L) ** 0.5 + 1e-15
        assert int(np.argmax(w)) == int(np.argmax(x))


def pin_two_token_closed_form():
    rng = np.random.default_rng(8)
    for _ in range(5):
        q, K, V = _rand_case(rng, 2, 6)
        sc = 0.9
        x0, x1 = sc * float(q @ K[0]), sc * float(q @ K[1])
        sig = lambda z: 1.0 / (1.0 + math.exp(-z))
        want = sig(x0 - x1) * V[0] + sig(x1 - x0) * V[1]
        assert np.max(np.abs(R.attend(q, K, V, sc) - want)) <= 1e-14


def pin_invariances():
    rng = np.random.default_rng(9)
    q, K, V = _rand_case(rng, 40, 12)
    base = R.attend(q, K, V, 0.5)
    w = rng.standard_normal(12)
    assert np.max(np.abs(R.attend(q, K + w, V, 0.5) - base)) <= 1e-13   # key shift
    a, b = -1.7, rng.standard_normal(12)
    assert np.max(np.abs(R.attend(q, K, a * V + b, 0.5) - (a * base + b))) <= 1e-13
    perm = rng.permutation(40)
    assert np.max(np.abs(R.attend(q, K[perm], V[perm], 0.5) - base)) <= 1e-14


def pin_merge_split():
    """Merging the partial triples of any split equals the unsplit result."""
    rng = np.random.default_rng(10)
    for L in (1, 2, 17, 100, 513):
        q, K, V = _rand_case(rng, L, 8)
        K *= 3.0
        whole = R.attend(q, K, V, 1.0)
        cuts = sorted(set(rng.integers(1, L, size=min(L - 1, 6)).tolist())) if L > 1 else []
        edges = [0] + cuts + [L]
        bounds = list(zip(edges[:-1], edges[1:]))
        assert np.max(np.abs(R.split_attend(q, K, V, 1.0, bounds) - whole)) <= 1e-13
        # every single-token split, and the policy's partitions
        ones = [(t, t + 1) for t in range(L)]
        assert np.max(np.abs(R.split_attend(q, K, V, 1.0, ones) - whole)) <= 1e-13
        for P_, T_ in ((512, 8192), (16, 0), (32, 16)):
            b = R.partition_bounds(L, P_, T_)
            assert b[0][0] == 0 and b[-1][1] == L and all(t0 < t1 for t0, t1 in b)
            assert all(b[n][1] == b[n + 1][0] for n in range(len(b) - 1))
            assert np.max(np.abs(R.split_attend(q, K, V, 1.0, b) - whole)) <= 1e-13
    # identity, commutativity, associativity
    q, K, V = _rand_case(rng, 30, 8)
    a = R.partial(q, K[:10], V[:10], 1.3)
    b = R.partial(q, K[10:22], V[10:22], 1.3)
    c = R.partial(q, K[22:], V[22:], 1.3)
    e = R.partial(q, K[:0], V[:0], 1.3)
    for x in (R.merge(a, e), R.merge(e, a)):
        assert x[0] == a[0] and x[1] == a[1] and np.array_equal(x[2], a[2])
    ab, ba = R.merge(a, b), R.merge(b, a)
    assert abs(ab[1] - ba[1]) <= 1e-13 and np.max(np.abs(ab[2] - ba[2])) <= 1e-13
    l1, l2 = R.merge(R.merge(a, b), c), R.merge(a, R.merge(b, c))
    assert np.max(np.abs(R.normalize(l1) - R.normalize(l2))) <= 1e-13
    assert np.max(np.abs(R.normalize(l1) - R.attend(q, K, V, 1.3))) <= 1e-13
    # partial's own closed form on one token: (x, 1, v)
    t = R.partial(q, K[:1], V[:1], 1.3)
    assert t[1] == 1.0 and np.array_equal(t[2], V[0])


def pin_stability_and_argmax_limit():
    rng = np.random.default_rng(12)
    q, K, V = _rand_case(rng, 64, 16)
    out = R.attend(q, K, V, 1e4)
    assert np.all(np.isfinite(out))
    x = 1e4 * (K @ q)
    top2 = np.sort(x)[-2:]
    assert top2[1] - top2[0] > 50
    assert np.max(np.abs(out - V[int(np.argmax(x))])) <= 1e-12
    t = R.partial(q, K, V, 1e4)
    assert np.isfinite(t[0]) and np.all(np.isfinite(t[2]))


def pin_sdpa_library_routine():
    """Contiguous GQA equals torch SDPA (float64, CPU) with KV heads repeated G times."""
    import torch
    case = W.contiguous_case("sdpa", 21, num_seqs=2, h_q=8, h_kv=2, d=16, s_kv=37,
                             dtype=W.F16)
    out = R.decode(case)
    G = case.h_q // case.h_kv
    q = torch.from_numpy(R.upcast(case.q, case.dtype))                 # [B, hq, d]
    k = torch.from_numpy(R.upcast(case.k, case.dtype)).permute(0, 2, 1, 3)  # [B, hkv, S, d]
    v = torch.from_numpy(R.upcast(case.v, case.dtype)).permute(0, 2, 1, 3)
    k = k.repeat_interleave(G, dim=1).contiguous()
    v = v.repeat_interleave(G, dim=1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.unsqueeze(2), k, v, scale=case.scale).squeeze(2).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-13


def pin_paged_equals_contiguous():
    """The same logical tokens behind a random block table give the same output."""
    ctx = [33, 16, 1, 50]
    paged = W.paged_case("p", 31, ctx, h_q=4, h_kv=2, d=8, dtype=W.F16, block_size=16,
                         extra_blocks=2)
    S = max(ctx)
    k = np.zeros((len(ctx), S, 2, 8), np.uint16)
    v = np.zeros_like(k)
    for s, L in enumerate(ctx):
        for t in range(L):
            b = paged.block_table[s, t // 16]
            k[s, t] = paged.k[b, t % 16]
            v[s, t] = paged.v[b, t % 16]
    contig = W.DecodeCase("c", W.F16, "contiguous", paged.q, k, v,
                          np.array(ctx, np.int32), None, 4, 2, 8, paged.scale, s_kv=S)
    a, b = R.decode(paged), R.decode(contig)
    assert np.all(np.isfinite(a))
    assert np.array_equal(a, b)


def pin_xsplit_gather_coded():
    """x-split pools whose every element holds its own (block, head, d, slot)
    code, laid out as the kernel-map page's key cache
    [num_blocks, h_kv, d / x, block_size, x] (and V as [num_blocks, h_kv, d,
    block_size]): the gather must return code(table[s, t // bs], j, d, t % bs)."""
    nb, h_kv, d, bs, x = 3, 2, 16, 16, 8

    def code(b, j, dd, o):
        return ((b * h_kv + j) * d + dd) * bs + o

    k = np.zeros((nb, h_kv, d // x, bs, x), np.int64)
    v = np.zeros((nb, h_kv, d, bs), np.int64)
    for b in range(nb):
        for j in range(h_kv):
            for dd in range(d):
                for o in range(bs):
                    k[b, j, dd // x, o, dd % x] = code(b, j, dd, o)
                    v[b, j, dd, o] = code(b, j, dd, o) + 7
    table = np.array([[2, 0, -1], [1, -1, -1]], np.int32)
    for s, L in ((0, 20), (1, 16)):
        for j in range(h_kv):
            K, V = R.gather_paged_xsplit(k, v, table, s, j, L, bs)
            assert K.shape == (L, d) and V.shape == (L, d)
            for t in range(L):
                for dd in range(d):
                    want = code(int(table[s, t // bs]), j, dd, t % bs)
                    assert K[t, dd] == want and V[t, dd] == want + 7, (s, j, t, dd)


def pin_xsplit_equals_rows():
    """The same logical cache in the x-split layout decodes bit-identically."""
    rows = W.paged_case("xr", 43, [33, 16, 1, 50, 0], h_q=8, h_kv=2, d=16, dtype=W.BF16,
                        block_size=16, extra_blocks=2)
    xs = W.xsplit_case(rows)
    a, b = R.decode(rows), R.decode(xs)
    assert np.all(np.isfinite(a))
    assert np.array_equal(a, b)


def pin_multi_token_rows():
    """T_q query tokens per sequence: token tau gives exactly what a one-token
    case with q[:, tau] gives, and the whole batch matches torch's
    scaled_dot_product_attention with query length T_q and no mask."""
    import torch
    T, G, h_kv, d = 3, 2, 2, 8
    case = W.paged_case("mt", 47, [5, 40, 17], h_q=G * h_kv, h_kv=h_kv, d=d, dtype=W.BF16,
                        t_q=T, extra_blocks=1)
    out = R.decode(case)
    assert out.shape == (3, T, G * h_kv, d) and np.all(np.isfinite(out))
    for tau in range(T):
        one = dataclasses.replace(case, q=np.ascontiguousarray(case.q[:, tau]))
        assert np.array_equal(out[:, tau], R.decode(one)), tau
    for s, L in enumerate(case.ctx_lens):
        K = np.stack([R.sequence_kv(case, s, j)[0] for j in range(h_kv)])   # [h_kv, L, d]
        V = np.stack([R.sequence_kv(case, s, j)[1] for j in range(h_kv)])
        q = torch.from_numpy(R.upcast(case.q[s], case.dtype)).permute(1, 0, 2)  # [h_q, T, d]
        k = torch.from_numpy(K).repeat_interleave(G, dim=0)
        v = torch.from_numpy(V).repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=case.scale)
        assert np.max(np.abs(out[s] - ref.permute(1, 0, 2).numpy())) <= 1e-13, s


def pin_empty_sequence_zero():
    case = W.paged_case("e", 41, [0, 3], h_q=2, h_kv=1, d=4, dtype=W.F16, block_size=16)
    out = R.decode(case)
    assert np.array_equal(out[0], np.zeros((2, 4)))
    assert np.all(np.isfinite(out[1]))


def pin_upcast_known_bits():
    """Storage decoding against the formats' definitions and torch's converters."""
    import torch
    f16 = {0x3C00: 1.0, 0xC000: -2.0, 0x3555: 0.333251953125, 0x7BFF: 65504.0,
           0x0001: 2.0 ** -24, 0x8000: -0.0}
    bf16 = {0x3F80: 1.0, 0xC000: -2.0, 0x3FC0: 1.5, 0x3EAB: 0.333984375,
            0x7F7F: 3.3895313892515355e38, 0x0001: 2.0 ** -133}
    for table, dt in ((f16, "f16"), (bf16, "bf16")):
        bits = np.array(list(table), np.uint16)
        got = R.upcast(bits, dt)
        assert got.tolist() == list(table.values()), (dt, got)
    rng = np.random.default_rng(13)
    raw = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    raw = raw[(raw & 0x7F80) != 0x7F80]           # finite bf16 only
    t = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    assert np.array_equal(R.upcast(raw, "bf16"), t.numpy())
    raw = raw[(raw & 0x7C00) != 0x7C00]           # finite fp16 only
    t = torch.from_numpy(raw.view(np.int16)).view(torch.float16).to(torch.float64)
    assert np.array_equal(R.upcast(raw, "f16"), t.numpy())


PINS = [pin_upcast_known_bits, pin_golden_closed_form, pin_brute_force_tiny, pin_brute_force_gqa_paged,
        pin_single_token, pin_zero_query_mean, pin_identical_keys_mean,
        pin_weights_simplex, pin_two_token_closed_form, pin_invariances,
        pin_merge_split, pin_stability_and_argmax_limit, pin_sdpa_library_routine,
        pin_paged_equals_contiguous, pin_xsplit_gather_coded, pin_xsplit_equals_rows,
        pin_multi_token_rows, pin_empty_sequence_zero]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------- planted mistakes ---

def _m_no_scale(q_row, K, scale):
    return K @ q_row


def _m_transposed_slot(k_pool, v_pool, block_table, s, j, L, block_size):
    rows_k = [k_pool[int(block_table[s, t % block_size]) if t % block_size < block_table.shape[1] else 0,
                     t // block_size, j, :] for t in range(L)]
    rows_v = [v_pool[int(block_table[s, t % block_size]) if t % block_size < block_table.shape[1] else 0,
                     t // block_size, j, :] for t in range(L)]
    return np.stack(rows_k), np.stack(rows_v)


def _m_xsplit_chunks_transposed(k_pool, v_pool, block_table, s, j, L, block_size):
    x = k_pool.shape[-1]
    d = k_pool.shape[2] * x
    K = np.zeros((L, d), dtype=k_pool.dtype)
    V = np.zeros((L, d), dtype=v_pool.dtype)
    for t in range(L):
        b = int(block_table[s, t // block_size])
        K[t, :] = k_pool[b, j, :, t % block_size, :].T.reshape(d)
        V[t, :] = v_pool[b, j, :, t % block_size]
    return K, V


def _m_decode_first_token(case, heads=None):
    if case.q.ndim == 4:
        case = dataclasses.replace(case, q=np.ascontiguousarray(
            np.repeat(case.q[:, :1], case.q.shape[1], axis=1)))
    return _ORIG_DECODE(case, heads)


def _m_kv_interleaved(i, group):
    return i % group


def _m_softmax_no_max(x):
    e = np.exp(x)
    return e / np.sum(e)


def _m_softmax_unnormalised(x):
    return np.exp(x - np.max(x))


def _m_merge_sign(a, b):
    m_a, l_a, O_a = a
    m_b, l_b, O_b = b
    m = max(m_a, m_b)
    if m == -np.inf:
        return (np.float64(-np.inf), np.float64(0.0), np.zeros_like(O_a))
    sa, sb = math.exp(m - m_a), math.exp(m_b - m)
    return (np.float64(m), l_a * sa + l_b * sb, O_a * sa + O_b * sb)


def _m_merge_drop_l(a, b):
    m_a, l_a, O_a = a
    m_b, l_b, O_b = b
    m = max(m_a, m_b)
    if m == -np.inf:
        return (np.float64(-np.inf), np.float64(0.0), np.zeros_like(O_a))
    sa, sb = math.exp(m_a - m), math.exp(m_b - m)
    return (np.float64(m), l_a * sa, O_a * sa + O_b * sb)


def _m_partial_drop_last(q_row, K, V, scale):
    return _ORIG_PARTIAL(q_row, K[:-1] if K.shape[0] > 1 else K,
                         V[:-1] if V.shape[0] > 1 else V, scale)


def _m_bounds_drop_tail(L, P, T):
    if L <= T:
        return [(0, L)]
    return [(t0, t0 + P) for t0 in range(0, L - P + 1, P)] or [(0, L)]


def _m_upcast_bf16_shift(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


_ORIG_PARTIAL = R.partial
_ORIG_DECODE = R.decode

MUTANTS = {
    "logits_without_scale": ("logits", _m_no_scale),
    "paged_block_and_slot_swapped": ("gather_paged", _m_transposed_slot),
    "xsplit_chunks_transposed": ("gather_paged_xsplit", _m_xsplit_chunks_transposed),
    "kv_head_interleaved": ("kv_head", _m_kv_interleaved),
    "every_query_token_reads_the_first": ("decode", _m_decode_first_token),
    "softmax_without_max_shift": ("softmax", _m_softmax_no_max),
    "softmax_unnormalised": ("softmax", _m_softmax_unnormalised),
    "merge_wrong_sign": ("merge", _m_merge_sign),
    "merge_drops_l_term": ("merge", _m_merge_drop_l),
    "partial_drops_last_token": ("partial", _m_partial_drop_last),
    "partitions_drop_tail": ("partition_bounds", _m_bounds_drop_tail),
    "bf16_upcast_wrong_shift": ("upcast", _m_upcast_bf16_shift),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(R, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:      # AssertionError, or a crash the mistake causes
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} slipped past every pin"
