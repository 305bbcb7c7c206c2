"""GPU parity of multi-token decode (T_q > 1 query tokens per sequence, each
attending to every cached key) through gqa_decode_ex.

The G * T_q query rows of a KV head are the columns of the same matrix-core
products, and no column's arithmetic depends on another's, so query token tau
of a T_q-token call must equal, bit for bit, a one-token call on q[:, tau];
both must match the float64 oracle within the tolerance in tests/parity.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from oracle import reference as R
from tests.parity import assert_close, case_to_device, run_case

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LENGTHS = [1, 17, 32, 33, 300, 513, 2000, 0, 9000]


@pytest.fixture(scope="module")
def gq():
    import decode_attention_08_amd as m
    return m


def _policies(gq):
    return {"default": None,
            "balanced_all_split": gq.policy_default(v1_max_ctx=0),
            "pages": gq.policy_pages(),
            "all_split_p32": gq.policy_pages(partition_size=32, v1_max_ctx=0)}


def _case(layout, G, T, h_kv, d, dtype, seed):
    if layout == "contiguous":
        return W.contiguous_case(f"mt_c{G}_{T}", seed, 3, G * h_kv, h_kv, d, 1500, dtype, t_q=T)
    rows = W.paged_case(f"mt_p{G}_{T}", seed, LENGTHS, h_q=G * h_kv, h_kv=h_kv, d=d,
                        dtype=dtype, t_q=T, extra_blocks=2)
    return W.xsplit_case(rows) if layout == "xsplit" else rows


@pytest.mark.parametrize("layout", ["contiguous", "paged", "xsplit"])
@pytest.mark.parametrize("G,T,h_kv,d,dtype", [
    (4, 4, 2, 128, W.F16),     # 16 columns
    (8, 2, 2, 128, W.BF16),    # 16 columns
    (1, 16, 2, 64, W.F16),     # one head, 16 query tokens
    (3, 5, 2, 64, W.BF16),     # 15 columns, ragged
    (2, 3, 4, 256, W.F16),     # d = 256
])
def test_multitoken_parity(gq, layout, G, T, h_kv, d, dtype):
    case = _case(layout, G, T, h_kv, d, dtype, 3000 + 16 * G + T)
    ref = R.decode(case)
    dev = case_to_device(case, DEV)
    for name, pol in _policies(gq).items():
        print(f"multitoken {layout} G={G} T={T} d={d} policy={name}", flush=True)
        got = run_case(dev, policy=pol)
        assert got.shape == ref.shape
        assert_close(got, ref, dtype, what=f"T_q={T} G={G} {layout} {name}")


@pytest.mark.parametrize("layout", ["contiguous", "paged", "xsplit"])
def test_multitoken_equals_single_token_calls(gq, layout):
    case = _case(layout, 4, 3, 2, 128, W.F16, 3100)
    dev = case_to_device(case, DEV)
    for name, pol in _policies(gq).items():
        got = run_case(dev, policy=pol)
        for tau in range(3):
            one = dataclasses.replace(case, q=np.ascontiguousarray(case.q[:, tau]))
            d1 = dict(dev, case=one, q=dev["q"][:, tau].contiguous())
            assert np.array_equal(got[:, tau], run_case(d1, policy=pol)), (name, tau)


def test_one_token_through_ex_equals_legacy(gq):
    """A [B, 1, h_q, d] query goes through gqa_decode_ex; a [B, h_q, d] one through
    gqa_decode: same bits."""
    case = W.paged_case("mt1", 3200, LENGTHS, h_q=16, h_kv=2, d=128, dtype=W.BF16)
    dev = case_to_device(case, DEV)
    for name, pol in _policies(gq).items():
        legacy = run_case(dev, policy=pol)
        d4 = dict(dev, q=dev["q"][:, None].contiguous())
        ex = gq.decode(d4["q"], dev["k"], dev["v"], dev["block_table"], dev["ctx_lens"],
                       scale=case.scale, policy=pol)
        torch.cuda.synchronize()
        assert np.array_equal(ex[:, 0].float().cpu().numpy().astype(np.float64), legacy), name


def test_multitoken_unsupported_width(gq):
    case = W.paged_case("mtw", 3300, [40], h_q=8, h_kv=1, d=64, dtype=W.F16, t_q=3)  # 24 columns
    dev = case_to_device(case, DEV)
    with pytest.raises(gq.GqaError) as e:
        run_case(dev)
    assert e.value.status == 3


@pytest.mark.parametrize("layout", ["xsplit", "contiguous"])
def test_multitoken_graph_replay(gq, layout):
    """T_q = 2 steps captured in a HIP graph: every replay equals the eager result."""
    case = _case(layout, 4, 2, 2, 128, W.F16, 3400)
    dev = case_to_device(case, DEV)
    stream = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(stream):
        out = torch.empty_like(dev["q"])
        kw = ({} if layout == "contiguous" else
              dict(block_table=dev["block_table"], ctx_lens=dev["ctx_lens"]))
        call = gq.prepare(dev["q"], dev["k"], dev["v"], scale=case.scale, out=out,
                          policy=gq.policy_default(v1_max_ctx=0), stream=stream,
                          xsplit=layout == "xsplit", **kw)
        call(phases=3)
        torch.cuda.synchronize()
        eager = out.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            call(phases=3)
        for rep in range(3):
            out.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {rep}"
    assert_close(eager.float().cpu().numpy().astype(np.float64), R.decode(case), W.F16,
                 what=f"graph T_q=2 {layout}")
