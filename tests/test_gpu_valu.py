"""GPU parity of the vector-ALU partition variant (policy flag
GQA_POLICY_VALU_DOT2): both products as packed dot2 with fp32 accumulation
instead of MFMA, for d = 128, row layouts and G * T_q <= 8.

It must meet the same tolerance against the oracle as the matrix-core path,
over the edge lengths (empty, one token, ragged tails, split and unsplit
sequences), column counts that pad 4 or 8 columns (G * T_q = 1, 3, 4, 6, 8),
both dtypes, both row layouts, and at the two G = 8 workloads' full sizes on
sampled rows.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import reference as R
from tests.parity import assert_close, case_to_device, run_case

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LENGTHS = [1, 17, 33, 64, 257, 700, 2000, 0, 9001, 513, 31, 32]


@pytest.fixture(scope="module")
def gq():
    import decode_attention_08_amd as m
    return m


def _valu(gq, **kw):
    return gq.policy_default(flags=gq.GQA_POLICY_VALU_DOT2, **kw)


@pytest.mark.parametrize("layout,dtype,h_kv,G,T", [
    ("paged", W.F16, 8, 4, 1),        # 4 columns, two workgroups of 4 KV heads
    ("paged", W.BF16, 4, 8, 1),       # 8 columns
    ("paged", W.F16, 2, 1, 1),        # 1 column of 4; a group of two heads, one wave each
    ("paged", W.BF16, 3, 3, 2),       # 6 query rows of 8 (two tokens of three heads)
    ("paged", W.F16, 1, 2, 4),        # 8 query rows (four tokens of two heads)
    ("contiguous", W.BF16, 8, 8, 1),
    ("contiguous", W.F16, 6, 2, 2),
])
def test_valu_matches_oracle(gq, layout, dtype, h_kv, G, T):
    if layout == "contiguous":
        case = W.contiguous_case(f"vz_c{G}", 2600 + G, 3, G * h_kv, h_kv, 128, 5000, dtype, t_q=T)
    else:
        case = W.paged_case(f"vz_p{G}_{T}", 2700 + 10 * G + T, LENGTHS, h_q=G * h_kv, h_kv=h_kv,
                            d=128, dtype=dtype, t_q=T, extra_blocks=1)
    ref = R.decode(case)
    dev = case_to_device(case, DEV)
    for v1 in (256, 0, 1 << 20):
        print(f"valu {layout} {dtype} h_kv={h_kv} G={G} T={T} v1={v1}", flush=True)
        got = run_case(dev, policy=_valu(gq, v1_max_ctx=v1))
        assert np.all(np.isfinite(got))
        assert_close(got, ref, dtype, what=f"valu {layout} G={G} T={T} v1={v1}")


def test_valu_close_to_matrix_core_path(gq):
    """Same inputs through both units: the results differ only by rounding order."""
    case = W.paged_case("vz_cmp", 2800, [4000, 3, 1500, 8000], h_q=32, h_kv=4, d=128,
                        dtype=W.F16)
    dev = case_to_device(case, DEV)
    a = run_case(dev, policy=gq.policy_default())
    b = run_case(dev, policy=_valu(gq))
    assert np.max(np.abs(a - b)) <= 2e-3
    ref = R.decode(case)
    assert_close(b, ref, W.F16, what="valu vs oracle")


def test_valu_deterministic(gq):
    case = W.paged_case("vz_det", 2900, [3000, 9000, 40, 5000], h_q=32, h_kv=4, d=128,
                        dtype=W.BF16)
    dev = case_to_device(case, DEV)
    first = run_case(dev, policy=_valu(gq, v1_max_ctx=0))
    for _ in range(2):
        assert np.array_equal(run_case(dev, policy=_valu(gq, v1_max_ctx=0)), first)


def _sample(case, rng, n_seq, per_seq):
    seqs = sorted(set([0, case.num_seqs - 1] +
                      rng.choice(case.num_seqs, size=min(n_seq, case.num_seqs), replace=False).tolist()))
    if case.layout == "paged":
        seqs = sorted(set(seqs + [int(np.argmax(case.ctx_lens))]))
    heads = []
    for s in seqs:
        idx = sorted(set([0, case.h_q - 1] + rng.choice(case.h_q, size=per_seq, replace=False).tolist()))
        heads += [(s, i) for i in idx]
    return heads


@pytest.mark.parametrize("name", ["long_128k", "mixed_b256", "contig_b8", "paged_b64"])
def test_valu_named_workloads_sampled(gq, name):
    case = W.workload(name)
    rng = np.random.default_rng(777)
    heads = _sample(case, rng, 6, 6)
    ref = R.decode(case, heads=heads)
    dev = case_to_device(case, DEV)
    print(f"valu workload {name} rows={len(heads)}", flush=True)
    got = run_case(dev, policy=_valu(gq))
    assert np.all(np.isfinite(got))
    assert_close(got, ref, case.dtype, what=f"valu {name}")
