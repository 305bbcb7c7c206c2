"""The allocation-free entry point gqa_decode_noalloc (static per-device
scratch instead of a workspace), through the C ABI.

CPU part: the header's scratch size matches the binding, and the host checks
that refuse a call before any HIP call.  GPU part: two calls in a row, the
second on a smaller input, each equal bit for bit to gqa_decode's output with
a caller-owned workspace on the same inputs (same kernels, same grid) and
within the oracle's tolerance; and a call captured in a HIP graph, replayed
several times."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import workloads as W
from oracle import reference as R
from tests.parity import assert_close, case_to_device, run_case

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def gq():
    import decode_attention_08_amd as m
    return m


def test_scratch_size_matches_header(gq):
    text = open(os.path.join(ROOT, "include", "gqa_decode.h")).read()
    m = re.search(r"#define GQA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == gq.NOALLOC_SCRATCH_BYTES


def _call(gq, policy, num_seqs=64, max_blocks=4096, h_q=32, h_kv=8, d=128):
    # fake, aligned device addresses: every call here is refused before any HIP call
    p = 1 << 20
    return gq.lib.gqa_decode_noalloc(p, p, p, p, p, p, num_seqs, max_blocks, h_q, h_kv, d, 16,
                                     0.1, gq.GQA_F16, ctypes.byref(policy), None)


def test_host_refusals(gq):
    WS, UNSUP = 5, 3
    # the fused merge's counters would need a zeroed scratch
    assert _call(gq, gq.policy_default(flags=gq.GQA_POLICY_FUSED_MERGE)) == UNSUP
    # fixed partitions of 512 over 64 sequences of up to 65536 tokens: 64*32*128 rows of
    # 520 B = 136 MB, more than the scratch
    assert _call(gq, gq.policy_pages(v1_max_ctx=0)) == WS
    assert _call(gq, gq.policy_pages(v1_max_ctx=0), num_seqs=0) == 0     # nothing to do
    # the usual argument checks still come first
    assert gq.lib.gqa_decode_noalloc(None, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 2, 4,
                                     8, 2, 128, 16, 0.1, 0, None, None) == 1


DEV = torch.device("cuda:0")


def _cases():
    big = W.paged_case("na_big", 2100, [9000, 33, 4100, 20000, 1, 700, 12000, 256, 257, 3000],
                       h_q=32, h_kv=4, d=128, dtype=W.F16, extra_blocks=2)
    small = W.paged_case("na_small", 2101, [300, 5000, 17], h_q=16, h_kv=2, d=64,
                         dtype=W.BF16, extra_blocks=1)
    return big, small


@pytest.mark.gpu
@pytest.mark.parametrize("pname", ["default", "all_split", "pages"])
def test_noalloc_equals_workspace_call(gq, pname):
    policy = {"default": None, "all_split": gq.policy_default(v1_max_ctx=0),
              "pages": gq.policy_pages()}[pname]
    for case in _cases():                       # the second call is on a smaller input
        print(f"noalloc {case.name} policy={pname}", flush=True)
        dev = case_to_device(case, DEV)
        want = run_case(dev, policy=policy)     # gqa_decode, workspace from torch
        out = torch.full_like(dev["q"], float("nan"))
        gq.decode_noalloc(dev["q"], dev["k"], dev["v"], dev["block_table"], dev["ctx_lens"],
                          out, scale=case.scale, policy=policy)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(got, want), f"{case.name} {pname}"
        assert_close(got, R.decode(case), case.dtype, what=f"noalloc {case.name} {pname}")


@pytest.mark.gpu
def test_noalloc_d256_and_phases(gq):
    """d = 256 (the largest partial rows), then a partition-only call followed by
    a merge-only call: the merge reads what the first left in the scratch."""
    case = W.paged_case("na_d256", 2102, [7000, 40, 30000], h_q=32, h_kv=8, d=256,
                        dtype=W.BF16)
    dev = case_to_device(case, DEV)
    pol = gq.policy_default(v1_max_ctx=0)
    want = run_case(dev, policy=pol)
    out = torch.zeros_like(dev["q"])
    args = (dev["q"], dev["k"], dev["v"], dev["block_table"], dev["ctx_lens"], out)
    gq.decode_noalloc(*args, scale=case.scale, policy=pol)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), want)
    out.zero_()
    gq.decode_noalloc(*args, scale=case.scale,
                      policy=gq.Policy(pol.partition_size, pol.v1_max_ctx, 1, 0))
    gq.decode_noalloc(*args, scale=case.scale,
                      policy=gq.Policy(pol.partition_size, pol.v1_max_ctx, 2, 0))
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), want)


@pytest.mark.gpu
@pytest.mark.parametrize("pname", ["default", "pages"])
def test_noalloc_graph_replay(gq, pname):
    """The callers this entry point is for include HIP-graph capture: a captured
    call, replayed several times with eager work and synchronisations between
    the replays, gives the eager call's bits every time (the graph holds the
    library's kernels only; nothing in it clears memory)."""
    policy = None if pname == "default" else gq.policy_pages()
    case = W.paged_case("na_graph", 2103, [6000, 1, 900, 15000, 64], h_q=32, h_kv=8, d=128,
                        dtype=W.F16, extra_blocks=1)
    dev = case_to_device(case, DEV)
    stream = torch.cuda.Stream(device=DEV)
    args = (dev["q"], dev["k"], dev["v"], dev["block_table"], dev["ctx_lens"])
    with torch.cuda.stream(stream):
        out = torch.zeros_like(dev["q"])
        gq.decode_noalloc(*args, out, scale=case.scale, policy=policy, stream=stream)
        torch.cuda.synchronize()
        eager = out.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            gq.decode_noalloc(*args, out, scale=case.scale, policy=policy, stream=stream)
        for rep in range(4):
            print(f"noalloc graph policy={pname} replay {rep}", flush=True)
            out.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {rep}"
    assert_close(eager.float().cpu().numpy().astype(np.float64), R.decode(case), W.F16,
                 what=f"noalloc graph {pname}")
