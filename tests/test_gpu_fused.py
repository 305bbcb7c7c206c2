"""GPU parity of the fused merge (policy flag GQA_POLICY_FUSED_MERGE): the last
workgroup to finish a split range merges it, and no merge kernel runs.

The counters live in the workspace, which must be zero before the first fused
call; every call leaves them zero again.  So repeated calls on one workspace
and HIP-graph replays must all give the same bits, matching the oracle.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import reference as R
from tests.parity import assert_close, case_to_device, run_case

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LENGTHS = [1, 17, 33, 64, 257, 700, 2000, 0, 9001, 513]


@pytest.fixture(scope="module")
def gq():
    import decode_attention_08_amd as m
    return m


def _fused(gq, **kw):
    return gq.policy_default(flags=gq.GQA_POLICY_FUSED_MERGE, **kw)


@pytest.mark.parametrize("layout,d,dtype,h_kv,G,T", [
    ("paged", 128, W.F16, 8, 4, 1),
    ("paged", 64, W.BF16, 2, 8, 1),
    ("xsplit", 128, W.BF16, 4, 2, 2),
    ("paged", 256, W.F16, 4, 3, 1),
    ("contiguous", 128, W.F16, 8, 4, 1),
])
def test_fused_matches_oracle_and_repeats(gq, layout, d, dtype, h_kv, G, T):
    if layout == "contiguous":
        case = W.contiguous_case("fz_c", 2400, 3, G * h_kv, h_kv, d, 6000, dtype)
    else:
        case = W.paged_case(f"fz_{layout}_{d}", 2400 + d, LENGTHS, h_q=G * h_kv, h_kv=h_kv,
                            d=d, dtype=dtype, t_q=T, extra_blocks=1)
        if layout == "xsplit":
            case = W.xsplit_case(case)
    ref = R.decode(case)
    dev = case_to_device(case, DEV)
    for v1 in (256, 0):
        # one prepared call owns one (zero-filled) workspace; call it repeatedly
        kw = ({} if layout == "contiguous" else
              dict(block_table=dev["block_table"], ctx_lens=dev["ctx_lens"]))
        call = gq.prepare(dev["q"], dev["k"], dev["v"], scale=case.scale,
                          policy=_fused(gq, v1_max_ctx=v1), xsplit=layout == "xsplit", **kw)
        out = call._keep[5]
        first = None
        for rep in range(3):
            print(f"fused {layout} d={d} v1={v1} rep={rep}", flush=True)
            out.zero_()
            call()
            torch.cuda.synchronize()
            got = out.float().cpu().numpy().astype(np.float64)
            assert_close(got, ref, dtype, what=f"fused {layout} d={d} v1={v1}")
            if first is None:
                first = got
            assert np.array_equal(got, first), f"repeat {rep} differs"


def test_fused_counters_reset(gq):
    case = W.paged_case("fz_cnt", 2500, [3000, 9000, 40, 5000], h_q=32, h_kv=8, d=128,
                        dtype=W.F16)
    dev = case_to_device(case, DEV)
    pol = _fused(gq, v1_max_ctx=0)
    need = gq.workspace_size(case.num_seqs, case.h_q, case.h_kv, case.d,
                             case.max_blocks * case.block_size, pol)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    run_case(dev, policy=pol, workspace=ws)
    # layout: records (num_seqs * n_groups * 16 bytes, 256-aligned), then the counters
    rec = ((case.num_seqs * 1 * 16 + 255) // 256) * 256
    counters = ws[rec:rec + case.num_seqs * 4].view(torch.int32)
    assert torch.count_nonzero(counters).item() == 0


def test_fused_graph_replay(gq):
    case = W.paged_case("fz_graph", 2600, [3000, 70, 9000, 1, 4500], h_q=16, h_kv=4, d=128,
                        dtype=W.BF16)
    dev = case_to_device(case, DEV)
    stream = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(stream):
        out = torch.empty_like(dev["q"])
        call = gq.prepare(dev["q"], dev["k"], dev["v"], block_table=dev["block_table"],
                          ctx_lens=dev["ctx_lens"], scale=case.scale, out=out,
                          policy=_fused(gq, v1_max_ctx=0), stream=stream)
        call(phases=3)
        torch.cuda.synchronize()
        eager = out.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            call(phases=3)
        for rep in range(4):
            out.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {rep}"
    assert_close(eager.float().cpu().numpy().astype(np.float64), R.decode(case), W.BF16,
                 what="fused graph")


@pytest.mark.parametrize("layout,dtype", [("contiguous", W.F16), ("paged", W.BF16)])
def test_fused_alternating_inputs_one_workspace(gq, layout, dtype):
    """Partials pass between workgroups, often on different XCDs, without a
    device-scope fence.  Alternate two queries on one workspace and check every
    call against its own oracle result: a merge that read a partial of the
    previous call (a stale cache line) would miss the tolerance by far, since
    the second query is the first one negated and doubled."""
    import dataclasses
    if layout == "contiguous":
        base = W.contiguous_case("fz_alt_c", 2700, 3, 32, 8, 128, 6000, dtype)
    else:
        base = W.paged_case("fz_alt_p", 2701, [6000, 900, 3000, 7000, 40, 2500], h_q=32,
                            h_kv=8, d=128, dtype=dtype)
    q32 = {W.F16: lambda b: b.view(np.float16).astype(np.float32)}.get(dtype)
    if q32 is None:
        def q32(b):
            return (b.astype(np.uint32) << 16).view(np.float32)
    other = dataclasses.replace(base, q=W.f32_to_storage_bits(-2.0 * q32(base.q), dtype))
    cases = [base, other]
    refs = [R.decode(c) for c in cases]
    qs = [case_to_device(c, DEV)["q"] for c in cases]
    dev = case_to_device(base, DEV)
    kw = ({} if layout == "contiguous" else
          dict(block_table=dev["block_table"], ctx_lens=dev["ctx_lens"]))
    call = gq.prepare(dev["q"], dev["k"], dev["v"], scale=base.scale,
                      policy=_fused(gq, v1_max_ctx=0), **kw)
    out = call.out
    for rep in range(6):
        i = rep % 2
        print(f"fused alternating {layout} rep={rep}", flush=True)
        dev["q"].copy_(qs[i])
        call()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        assert_close(got, refs[i], dtype, what=f"fused alternating {layout} rep {rep}")
