"""GPU parity: the HIP library through its C ABI against the float64 oracle.

Tolerances are those in tests/parity.py.  Small cases are compared element by
element over every output; the five named workloads at full size are compared
on sampled (sequence, query head) rows the oracle computes one by one, in the
launch configuration the bench times (default policy) and under the pages'
policy (partition 512, single pass up to 8192).
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from oracle import reference as R
from tests.parity import assert_close, bits_to_device, case_to_device, run_case

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def gq():
    import decode_attention_08_amd as m
    return m


def _policies(gq):
    return {
        "default": None,                                           # balanced, v1_max 256
        "balanced_all_split": gq.policy_default(v1_max_ctx=0),
        "balanced_no_split": gq.policy_default(v1_max_ctx=1 << 30),
        "pages": gq.policy_pages(),
        "all_split_p32": gq.policy_pages(partition_size=32, v1_max_ctx=0),
        "all_split_p96": gq.policy_pages(partition_size=96, v1_max_ctx=0),
        "all_single": gq.policy_pages(v1_max_ctx=1 << 30),
    }


EDGE_LENGTHS = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 511, 512, 513, 1000, 8192, 8193]


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_edge_lengths_all_policies(gq, dtype, d):
    case = W.paged_case(f"edges_{dtype}_{d}", 100 + d, EDGE_LENGTHS, h_q=16, h_kv=2, d=d,
                        dtype=dtype, extra_blocks=3)
    ref = R.decode(case)
    dev = case_to_device(case, DEV)
    for name, pol in _policies(gq).items():
        print(f"edges dtype={dtype} d={d} policy={name}", flush=True)
        got = run_case(dev, policy=pol)
        assert_close(got, ref, dtype, what=f"edges {dtype} d={d} {name}")


@pytest.mark.parametrize("layout", ["paged", "contiguous"])
def test_d256_every_tile_count(gq, layout):
    """At d = 256 the token loop keeps K two tiles ahead and walks the tiles in
    groups of six with a ragged end: whole sequences of 1 to 14 tiles (and a
    ragged last tile), one wave per KV head and no split, reach every end of
    that loop; the all-split policies cut the same sequences into segments of
    every short length."""
    lengths = [32 * n + r for n in range(15) for r in (0, 5) if 32 * n + r > 0]
    if layout == "paged":
        case = W.paged_case("d256_tiles", 700, lengths, h_q=8, h_kv=4, d=256, dtype=W.BF16,
                            extra_blocks=2)
    else:
        case = W.contiguous_case("d256_tiles_c", 701, 2, 8, 4, 256, 32 * 13 + 5, W.BF16)
    ref = R.decode(case)
    dev = case_to_device(case, DEV)
    for name in ("balanced_no_split", "balanced_all_split", "all_single", "all_split_p96"):
        print(f"d256 tile counts {layout} policy={name}", flush=True)
        got = run_case(dev, policy=_policies(gq)[name])
        assert_close(got, ref, W.BF16, what=f"d256 tile counts {layout} {name}")


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 16])
def test_group_sizes(gq, G):
    h_kv = 2
    case = W.paged_case(f"group{G}", 200 + G, [700, 33, 1], h_q=G * h_kv, h_kv=h_kv, d=128,
                        dtype=W.F16)
    ref = R.decode(case)
    dev = case_to_device(case, DEV)
    for name in ("default", "balanced_all_split", "all_split_p96"):
        got = run_case(dev, policy=_policies(gq)[name])
        assert_close(got, ref, W.F16, what=f"G={G} {name}")


@pytest.mark.parametrize("bs", [16, 32, 64, 256])
def test_block_sizes(gq, bs):
    case = W.paged_case(f"bs{bs}", 300 + bs, [1, bs - 1, bs, bs + 1, 3 * bs + 5, 700],
                        h_q=8, h_kv=1, d=64, dtype=W.BF16, block_size=bs, extra_blocks=1)
    ref = R.decode(case)
    dev = case_to_device(case, DEV)
    for name in ("default", "balanced_all_split", "pages", "all_split_p32"):
        got = run_case(dev, policy=_policies(gq)[name])
        assert_close(got, ref, W.BF16, what=f"bs={bs} {name}")


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_contiguous_small(gq, dtype):
    case = W.contiguous_case(f"contig_{dtype}", 400, 3, 32, 8, 128, 1000, dtype)
    ref = R.decode(case)
    dev = case_to_device(case, DEV)
    for name, pol in _policies(gq).items():
        got = run_case(dev, policy=pol)
        assert_close(got, ref, dtype, what=f"contig {dtype} {name}")


def test_zero_length_gives_zeros(gq):
    case = W.paged_case("zeros", 500, [0, 5, 0, 40], h_q=8, h_kv=2, d=128, dtype=W.F16)
    dev = case_to_device(case, DEV)
    ref = R.decode(case)
    for name, pol in _policies(gq).items():
        got = run_case(dev, policy=pol)
        assert np.array_equal(got[0], np.zeros((8, 128))) and np.array_equal(got[2], got[0]), name
        assert_close(got, ref, W.F16, what=f"zeros {name}")
    c0 = W.contiguous_case("s0", 501, 2, 4, 1, 64, 0)
    got = run_case(case_to_device(c0, DEV))
    assert np.array_equal(got, np.zeros_like(got))


def test_single_token_is_exact(gq):
    """S_kv = 1: the output is v_0 bit for bit (p = 1, l = 1)."""
    for dtype in (W.F16, W.BF16):
        case = W.contiguous_case("s1", 600, 4, 16, 4, 128, 1, dtype)
        got = run_case(case_to_device(case, DEV))
        want = R.upcast(case.v[:, 0], dtype)                      # [B, h_kv, d]
        want = np.repeat(want, 4, axis=1)                          # query head i -> kv i // 4
        assert np.array_equal(got, want), dtype


def test_zero_query_is_mean(gq):
    case = W.contiguous_case("q0", 700, 2, 8, 2, 64, 777, W.F16)
    case.q[:] = 0
    got = run_case(case_to_device(case, DEV))
    Vf = R.upcast(case.v, case.dtype)                              # [B, S, h_kv, d]
    want = np.repeat(Vf.mean(axis=1), 4, axis=1)
    assert_close(got, want, W.F16, what="q=0 mean")


def test_large_logits_stable(gq):
    case = W.paged_case("big", 800, [300, 2000], h_q=8, h_kv=1, d=128, dtype=W.BF16, scale=25.0)
    ref = R.decode(case)
    for name, pol in _policies(gq).items():
        got = run_case(case_to_device(case, DEV), policy=pol)
        assert_close(got, ref, W.BF16, what=f"large logits {name}")


def test_paged_bitwise_equals_contiguous(gq):
    """A random block table and the contiguous layout of the same tokens agree bit
    for bit under the balanced policies (same segments, same reduction order).
    Under the fixed policies a paged cache goes through the planner's work list
    (four-wave workgroups) and a contiguous one through an exact grid, so their
    reduction orders differ: there both must match the oracle, and a paged cache
    must decode bit for bit the same under any placement of its blocks."""
    S = 1500
    paged = W.paged_case("pc", 900, [S] * 3, h_q=16, h_kv=2, d=128, dtype=W.F16, extra_blocks=2)
    k = np.zeros((3, S, 2, 128), np.uint16)
    v = np.zeros_like(k)
    for s in range(3):
        for t in range(S):
            b = paged.block_table[s, t // 16]
            k[s, t] = paged.k[b, t % 16]
            v[s, t] = paged.v[b, t % 16]
    contig = W.DecodeCase("c", W.F16, "contiguous", paged.q, k, v, paged.ctx_lens, None,
                          16, 2, 128, paged.scale, s_kv=S)
    # the same logical cache with every physical block moved (block b -> nb - 1 - b)
    nb = paged.k.shape[0]
    moved = dataclasses.replace(
        paged, name="pc_moved", k=np.ascontiguousarray(paged.k[::-1]),
        v=np.ascontiguousarray(paged.v[::-1]),
        block_table=np.where(paged.block_table >= 0, nb - 1 - paged.block_table, -1).astype(np.int32))
    ref = R.decode(paged)
    for name, pol in _policies(gq).items():
        a = run_case(case_to_device(paged, DEV), policy=pol)
        b = run_case(case_to_device(contig, DEV), policy=pol)
        c = run_case(case_to_device(moved, DEV), policy=pol)
        assert np.array_equal(a, c), name
        if pol is None or pol.partition_size == 0:
            assert np.array_equal(a, b), name
        else:
            assert_close(a, ref, W.F16, what=f"paged {name}")
            assert_close(b, ref, W.F16, what=f"contiguous {name}")


def test_deterministic(gq):
    case = W.workload("paged_b64")
    dev = case_to_device(case, DEV)
    for pol in (None, gq.policy_pages(v1_max_ctx=0)):
        a = run_case(dev, policy=pol)
        for _ in range(2):
            assert np.array_equal(a, run_case(dev, policy=pol))


def test_phases_split_equals_whole(gq):
    case = W.paged_case("ph", 1000, [5000, 100, 9000], h_q=32, h_kv=4, d=128, dtype=W.F16)
    dev = case_to_device(case, DEV)
    for base in (gq.policy_pages(), gq.policy_default()):
        whole = run_case(dev, policy=base)
        ws = torch.empty(gq.workspace_size(3, 32, 4, 128, case.max_blocks * 16, base),
                         dtype=torch.uint8, device=DEV)
        out = torch.empty_like(dev["q"])
        p1 = gq.Policy(base.partition_size, base.v1_max_ctx, 1, 0)
        p2 = gq.Policy(base.partition_size, base.v1_max_ctx, 2, 0)
        run_case(dev, policy=p1, out=out, workspace=ws)
        got = run_case(dev, policy=p2, out=out, workspace=ws)
        assert np.array_equal(whole, got), base


def test_reused_workspace_and_changing_lengths(gq):
    """The same workspace serves consecutive calls whose lengths differ (records are
    rewritten each call; nothing needs clearing)."""
    lens_a = [3000, 17, 900, 12000]
    lens_b = [5, 12000, 300, 1]
    ca = W.paged_case("wa", 1100, lens_a, h_q=16, h_kv=2, d=128, dtype=W.F16)
    cb = W.paged_case("wb", 1101, lens_b, h_q=16, h_kv=2, d=128, dtype=W.F16,
                      max_blocks=ca.max_blocks)
    pol = gq.policy_default(v1_max_ctx=0)
    ws = torch.empty(gq.workspace_size(4, 16, 2, 128, ca.max_blocks * 16, pol),
                     dtype=torch.uint8, device=DEV)
    for c in (ca, cb, ca):
        got = run_case(case_to_device(c, DEV), policy=pol, workspace=ws)
        assert_close(got, R.decode(c), W.F16, what=f"reuse {c.name}")


def _sample_heads(case, rng, n_seq, per_seq):
    seqs = sorted(set([0, case.num_seqs - 1] +
                      rng.choice(case.num_seqs, size=min(n_seq, case.num_seqs), replace=False).tolist()))
    if case.layout == "paged":                  # always include the longest sequence
        seqs = sorted(set(seqs + [int(np.argmax(case.ctx_lens))]))
    heads = []
    for s in seqs:
        idx = sorted(set([0, case.h_q - 1] + rng.choice(case.h_q, size=per_seq, replace=False).tolist()))
        heads += [(s, i) for i in idx]
    return heads


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_named_workloads_sampled(gq, name):
    case = W.workload(name)
    rng = np.random.default_rng(12345)
    heads = ([(s, i) for s in range(case.num_seqs) for i in range(case.h_q)]
             if case.kv_bytes <= (1 << 27) else _sample_heads(case, rng, 6, 6))
    ref = R.decode(case, heads=heads)
    dev = case_to_device(case, DEV)
    pols = dict(_policies(gq), fused=gq.policy_default(flags=gq.GQA_POLICY_FUSED_MERGE))
    for pname in ("default", "balanced_all_split", "pages", "fused"):
        print(f"workload {name} policy={pname} rows={len(heads)}", flush=True)
        got = run_case(dev, policy=pols[pname])   # (a fused call's own workspace starts zeroed)
        assert np.all(np.isfinite(got)), pname
        assert_close(got, ref, case.dtype, what=f"{name} {pname}")


@pytest.mark.parametrize("h_kv,G,d", [(12, 2, 64), (16, 1, 128), (6, 3, 128), (2, 16, 64),
                                      (4, 3, 256), (8, 2, 256), (6, 1, 256), (2, 16, 256)])
def test_head_groups(gq, h_kv, G, d):
    """KV heads per workgroup = largest divisor of h_kv up to 4 (12 -> 4, 16 -> 4,
    6 -> 3, 2 -> 2, 4 -> 4, 8 -> 4); groups of one or two heads give each head
    several waves."""
    case = W.paged_case(f"hg{h_kv}", 1200 + h_kv, [1300, 5, 333], h_q=G * h_kv, h_kv=h_kv, d=d,
                        dtype=W.BF16, extra_blocks=1)
    ref = R.decode(case)
    dev = case_to_device(case, DEV)
    for name in ("default", "balanced_all_split", "pages", "all_split_p96"):
        got = run_case(dev, policy=_policies(gq)[name])
        assert_close(got, ref, W.BF16, what=f"h_kv={h_kv} G={G} d={d} {name}")


@pytest.mark.parametrize("d", [128, 256])
def test_most_sequences_balanced(gq, d):
    """The largest batch the balanced scheduler takes (7168 sequences, whose prefix
    shares the workgroup's LDS with its V tiles), one KV head, so that each head
    gets several waves: mostly short sequences and a few long, split ones."""
    rng = np.random.default_rng(7 + d)
    lens = rng.integers(0, 48, size=7168).astype(np.int32)
    lens[[5, 3000, 7167]] = [2500, 40000, 700]
    case = W.paged_case(f"most{d}", 1310 + d, lens, h_q=8, h_kv=1, d=d, dtype=W.BF16)
    heads = [(s, i) for s in list(range(0, 7168, 211)) + [5, 3000, 7167] for i in (0, 7)]
    ref = R.decode(case, heads=heads)
    got = run_case(case_to_device(case, DEV))
    assert_close(got, ref, W.BF16, what=f"7168 sequences d={d}")


def test_many_sequences_fallback(gq):
    """More sequences than the balanced scheduler keeps in LDS: fixed 512-token partitions."""
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 40, size=8200).astype(np.int32)
    lens[17] = 1500                               # one sequence long enough to split
    case = W.paged_case("many", 1300, lens, h_q=2, h_kv=1, d=64, dtype=W.F16)
    heads = [(s, i) for s in list(range(0, 8200, 97)) + [17, 8199] for i in range(2)]
    ref = R.decode(case, heads=heads)
    got = run_case(case_to_device(case, DEV))
    assert_close(got, ref, W.F16, what="8200 sequences")


def test_long_sequence_many_segments(gq):
    """One sequence spread over every workgroup: hundreds of partials per head."""
    case = W.contiguous_case("long1", 1400, 1, 8, 1, 128, 70001, W.F16)
    ref = R.decode(case)
    got = run_case(case_to_device(case, DEV), policy=gq.policy_default(v1_max_ctx=0))
    assert_close(got, ref, W.F16, what="S=70001")
    got = run_case(case_to_device(case, DEV), policy=gq.policy_pages(partition_size=64))
    assert_close(got, ref, W.F16, what="S=70001 fixed 64")


def test_million_token_sequence(gq):
    """One paged sequence of 2^20 + 5 tokens (the balanced shares cut it into
    hundreds of partials per head; the pages' 512-token partitions into 2049)."""
    n = (1 << 20) + 5
    case = W.paged_case("mega", 1500, [n, 3], h_q=8, h_kv=1, d=64, dtype=W.F16)
    ref = R.decode(case)
    dev = case_to_device(case, DEV)
    for name in ("default", "pages"):
        print(f"million-token sequence policy={name}", flush=True)
        got = run_case(dev, policy=_policies(gq)[name])
        assert_close(got, ref, W.F16, what=f"2^20 tokens {name}")


@pytest.mark.parametrize("pname", ["default", "pages"])
def test_graph_replay_matches_eager(gq, pname):
    """Decode steps captured in a HIP graph: every replay, with eager work and
    synchronisations in between, equals the eager result bit for bit."""
    case = W.paged_case("graph", 1500, [3000, 70, 9000, 1], h_q=16, h_kv=4, d=128, dtype=W.F16)
    dev = case_to_device(case, DEV)
    pol = _policies(gq)[pname]
    stream = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(stream):
        out = torch.empty_like(dev["q"])
        call = gq.prepare(dev["q"], dev["k"], dev["v"], block_table=dev["block_table"],
                          ctx_lens=dev["ctx_lens"], scale=case.scale, out=out, policy=pol,
                          stream=stream)
        call(phases=3)
        torch.cuda.synchronize()
        eager = out.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            call(phases=3)
        for rep in range(4):
            out.zero_()
            junk = torch.randn(1 << 20, device=DEV).sum()       # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {rep}"
            del junk
    assert_close(eager.float().cpu().numpy().astype(np.float64), R.decode(case), W.F16,
                 what=f"graph {pname}")


def _merge_case(kind):
    """Fixed 32-token partitions shaped so that the merge runs 1, 4, 16 and 64
    slots per head: (heads, partials per head) = (4200, 16), (1200, 64), (64, 200),
    (16, 625); the last two with d sliced (few merge blocks), and (256, 625) unsliced."""
    rng = np.random.default_rng(1600)
    if kind == "slots1":
        lens = rng.integers(0, 513, size=2100)
        lens[:3] = [512, 0, 33]
        return W.paged_case(kind, 1601, lens, h_q=2, h_kv=1, d=128, dtype=W.BF16)
    if kind == "slots4":
        lens = rng.integers(0, 2049, size=600)
        lens[:3] = [2048, 1, 65]
        return W.paged_case(kind, 1602, lens, h_q=2, h_kv=1, d=64, dtype=W.F16)
    if kind == "slots16":
        return W.paged_case(kind, 1603, [6400, 3000, 31, 0], h_q=16, h_kv=2, d=128,
                            dtype=W.BF16, extra_blocks=1)
    if kind == "slots64_unsliced":                 # 256 heads x 625 partials: 256 merge blocks
        lens = rng.integers(1, 20001, size=16)
        lens[0] = 20000
        return W.paged_case(kind, 1605, lens, h_q=16, h_kv=2, d=64, dtype=W.BF16)
    return W.paged_case(kind, 1604, [20000, 777], h_q=8, h_kv=1, d=128, dtype=W.F16)


@pytest.mark.parametrize("kind", ["slots1", "slots4", "slots16", "slots64", "slots64_unsliced"])
def test_merge_widths(gq, kind):
    case = _merge_case(kind)
    heads = [(s, i) for s in range(min(case.num_seqs, 40)) for i in range(case.h_q)]
    heads += [(s, 0) for s in range(40, case.num_seqs, 37)]
    ref = R.decode(case, heads=heads)
    got = run_case(case_to_device(case, DEV),
                   policy=gq.policy_pages(partition_size=32, v1_max_ctx=0))
    assert_close(got, ref, case.dtype, what=f"merge {kind}")


@pytest.mark.parametrize("nseq", [1, 4, 16, 64])
def test_balanced_merge_spread(gq, nseq):
    """Balanced scheduler, every range split: about grid / nseq partials per head."""
    case = W.paged_case(f"mwb{nseq}", 1700 + nseq, [9000 - 37 * s for s in range(nseq)],
                        h_q=32, h_kv=8, d=64, dtype=W.F16)
    heads = [(s, i) for s in range(min(nseq, 4)) for i in range(32)]
    got = run_case(case_to_device(case, DEV), policy=gq.policy_default(v1_max_ctx=0))
    assert_close(got, R.decode(case, heads=heads), W.F16, what=f"balanced nseq={nseq}")


def test_concurrent_streams(gq):
    """Calls on two streams with their own workspaces and outputs may overlap."""
    a = W.paged_case("cs_a", 1800, [5000, 300, 9000], h_q=32, h_kv=8, d=128, dtype=W.F16)
    b = W.contiguous_case("cs_b", 1801, 4, 16, 4, 64, 3000, W.BF16)
    da, db = case_to_device(a, DEV), case_to_device(b, DEV)
    want_a, want_b = run_case(da), run_case(db)
    sa, sb = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    outs = []
    for _ in range(3):
        oa, ob = torch.empty_like(da["q"]), torch.empty_like(db["q"])
        ca = gq.prepare(da["q"], da["k"], da["v"], block_table=da["block_table"],
                        ctx_lens=da["ctx_lens"], scale=a.scale, out=oa, stream=sa)
        cb = gq.prepare(db["q"], db["k"], db["v"], scale=b.scale, out=ob, stream=sb)
        torch.cuda.synchronize()
        for _ in range(4):
            ca()
            cb()
        torch.cuda.synchronize()
        outs.append((oa, ob))
    for oa, ob in outs:
        assert np.array_equal(oa.float().cpu().numpy().astype(np.float64), want_a)
        assert np.array_equal(ob.float().cpu().numpy().astype(np.float64), want_b)


def test_checked_block_ids_same_result(gq):
    """check_blocks=True only adds the host check: same output bit for bit."""
    case = W.paged_case("chk", 1900, [700, 1, 9000], h_q=16, h_kv=4, d=128, dtype=W.F16,
                        extra_blocks=2)
    dev = case_to_device(case, DEV)
    want = run_case(dev)
    got = gq.decode(dev["q"], dev["k"], dev["v"], dev["block_table"], dev["ctx_lens"],
                    scale=case.scale, check_blocks=True)
    torch.cuda.synchronize()
    assert np.array_equal(got.float().cpu().numpy().astype(np.float64), want)
    bad = dev["block_table"].clone()
    bad[2, 3] = case.k.shape[0]
    with pytest.raises(ValueError, match="outside the pool"):
        gq.decode(dev["q"], dev["k"], dev["v"], bad, dev["ctx_lens"], check_blocks=True)


def test_side_stream_calls_keep_their_workspace(gq):
    """One-shot calls on a side stream drop their workspace on return while the
    launch may still be queued.  The binding allocates it on the launch stream,
    so allocations and writes on the current stream meanwhile cannot reuse it."""
    case = W.paged_case("side", 2000, [9000, 4000, 300, 12000], h_q=32, h_kv=8, d=128,
                        dtype=W.F16)
    dev = case_to_device(case, DEV)
    want = run_case(dev)
    pol = gq.policy_default(v1_max_ctx=0)          # every range split: partials in the workspace
    want_split = run_case(dev, policy=pol)
    need = gq.workspace_size(case.num_seqs, case.h_q, case.h_kv, case.d,
                             case.max_blocks * case.block_size, pol)
    assert need > 0
    side = torch.cuda.Stream(device=DEV)
    outs = []
    for rep in range(4):
        with torch.cuda.stream(side):
            torch.cuda._sleep(20_000_000)            # keeps the side stream busy (bounded)
        outs.append(gq.decode(dev["q"], dev["k"], dev["v"], dev["block_table"], dev["ctx_lens"],
                              scale=case.scale, policy=pol, stream=side))
        junk = torch.empty(need, dtype=torch.uint8, device=DEV)   # current stream
        junk.fill_(0xFF)                             # NaN bit patterns if it aliased
        del junk
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(o.float().cpu().numpy().astype(np.float64), want_split)
    ref = R.decode(case)
    assert_close(want_split, ref, W.F16, what="side stream, all split")
    assert_close(want, ref, W.F16, what="side stream, default")
