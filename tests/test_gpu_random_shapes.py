"""Seeded random shapes through every layout and policy family, each against
the float64 oracle on every output row (tolerance of tests/parity.py).

Each case draws: the cache layout (contiguous, paged rows, paged x-split), the
dtype, d_head, KV heads and group size with G * T_q <= 16, T_q, the block
size, 1-9 sequence lengths (zero, one token, block and tile edges, and lengths
past the pages' single-pass threshold), spare NaN blocks, a scale (kept
moderate for bf16 at d >= 128, see _draw), and a policy (balanced with a
random single-pass bound, or fixed partitions of a random multiple of 32).
The draws are printed before each case runs."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import reference as R
from tests.parity import assert_close, case_to_device, run_case

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
N_CASES = 40


@pytest.fixture(scope="module")
def gq():
    import decode_attention_08_amd as m
    return m


def _draw(i):
    rng = np.random.default_rng(9000 + i)
    layout = ["contiguous", "paged", "xsplit"][rng.integers(3)]
    dtype = [W.F16, W.BF16][rng.integers(2)]
    d = int(rng.choice([64, 128, 256]))
    h_kv = int(rng.choice([1, 2, 3, 4, 6, 8]))
    t_q = int(rng.choice([1, 1, 1, 2, 3, 4]))
    G = int(rng.integers(1, 16 // t_q + 1))
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    n = int(rng.integers(1, 10))
    edges = [0, 1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 8192, 8193, 9001]
    lens = [int(rng.choice(edges)) if rng.random() < 0.4 else int(rng.integers(0, 6000))
            for _ in range(n)]
    scale = float(rng.choice([1.0 / np.sqrt(d), 0.02, 0.3]))
    if dtype == W.BF16 and scale == 0.3 and d >= 128:
        # logits of spread 0.3 sqrt(d) make the softmax nearly one-hot, and an
        # output that is then a single V value in [4, 8) moves by up to 1.6e-2
        # when it is rounded to bf16, beyond the 1e-2 bound for any kernel
        scale = 1.0 / np.sqrt(d)
    if rng.random() < 0.5:
        pol = ("balanced", 0, int(rng.choice([0, 64, 256, 1000, 1 << 30])))
    else:
        pol = ("fixed", 32 * int(rng.integers(1, 33)), int(rng.choice([0, 96, 512, 8192, 1 << 30])))
    return dict(layout=layout, dtype=dtype, d=d, h_kv=h_kv, t_q=t_q, G=G, bs=bs, lens=lens,
                scale=scale, pol=pol, extra=int(rng.integers(0, 3)), seed=9500 + i)


def _case(c):
    if c["layout"] == "contiguous":
        return W.contiguous_case("rnd", c["seed"], len(c["lens"]), c["G"] * c["h_kv"], c["h_kv"],
                                 c["d"], max(c["lens"]), c["dtype"], scale=c["scale"], t_q=c["t_q"])
    # a paged pool holds at least one block: the library takes no NULL pool, even
    # when every sequence is empty
    extra = max(c["extra"], 1 if max(c["lens"]) == 0 else 0)
    case = W.paged_case("rnd", c["seed"], c["lens"], h_q=c["G"] * c["h_kv"], h_kv=c["h_kv"],
                        d=c["d"], dtype=c["dtype"], block_size=c["bs"], extra_blocks=extra,
                        scale=c["scale"], t_q=c["t_q"])
    return W.xsplit_case(case) if c["layout"] == "xsplit" else case


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(gq, i):
    c = _draw(i)
    print(f"random case {i}: {c}", flush=True)
    kind, part, v1 = c["pol"]
    pol = gq.policy_default(v1_max_ctx=v1) if kind == "balanced" else \
        gq.policy_pages(partition_size=part, v1_max_ctx=v1)
    case = _case(c)
    got = run_case(case_to_device(case, DEV), policy=pol)
    assert_close(got, R.decode(case), case.dtype, what=f"random case {i}")
