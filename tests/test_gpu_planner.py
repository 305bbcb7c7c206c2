"""The fixed decomposition's work list on a paged cache, read back from the
workspace after a partition-only call (phases = 1): every (KV head,
partition) of every sequence is listed exactly once, and the list runs from
the largest items to the smallest (by the size class the planner sorts on)."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import case_to_device

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def gq():
    import decode_attention_08_amd as m
    return m


def _list_from_workspace(gq, case, pol):
    dev = case_to_device(case, DEV)
    ws = torch.zeros(gq.workspace_size(case.num_seqs, case.h_q, case.h_kv, case.d,
                                       case.max_blocks * case.block_size, pol),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(dev["q"])
    call = gq.prepare(dev["q"], dev["k"], dev["v"], block_table=dev["block_table"],
                      ctx_lens=dev["ctx_lens"], scale=case.scale, out=out, workspace=ws,
                      policy=gq.Policy(pol.partition_size, pol.v1_max_ctx, 1, 0))
    call()
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    n = int(raw[:4].view(np.int32)[0])                 # header: items listed
    items = raw[256:256 + 8 * n].view(np.int32).reshape(n, 2)
    return n, items


@pytest.mark.parametrize("kind", ["pages", "split_p96"])
def test_work_list_covers_every_item_once_largest_first(gq, kind):
    rng = np.random.default_rng(42)
    lens = rng.integers(0, 12000, size=300).astype(np.int32)
    lens[:4] = [0, 1, 8192, 8193]
    case = W.paged_case("plan", 2200, lens, h_q=32, h_kv=8, d=64, dtype=W.F16)
    pol = gq.policy_pages() if kind == "pages" else gq.policy_pages(partition_size=96, v1_max_ctx=0)
    P, v1 = pol.partition_size, pol.v1_max_ctx
    n, items = _list_from_workspace(gq, case, pol)
    assert n == len(items) > 0
    s = items[:, 0] // case.h_kv
    j0 = items[:, 0] % case.h_kv
    p = items[:, 1] >> 2
    nh = 1 << (items[:, 1] & 3)
    assert set(np.unique(nh)) <= {1, 2, 4} and np.all(j0 % nh == 0)
    # coverage: each (sequence, KV head, partition) exactly once
    seen = {}
    for a, b, c, h in zip(s, j0, p, nh):
        for j in range(b, b + h):
            key = (int(a), int(j), int(c))
            assert key not in seen, key
            seen[key] = True
    want = set()
    for q, L in enumerate(case.ctx_lens.tolist()):
        parts = -(-L // P) if L > v1 else 1
        for j in range(case.h_kv):
            for c in range(parts):
                want.add((q, j, c))
    assert set(seen) == want
    # order: non-increasing size class (tiles x heads), at a class width no finer than
    # the planner's (its widest possible items have 4 heads)
    L = case.ctx_lens[s].astype(np.int64)
    tiles = np.where(L > v1, -(-P // 32), -(-L // 32))
    size = tiles * nh
    longest = max(-(-min(v1, case.max_blocks * case.block_size) // 32) * 4, -(-P // 32) * 4)
    shift = 0
    while (longest >> shift) >= 256:
        shift += 1
    cls = np.minimum(255, size >> shift)
    assert np.all(np.diff(cls) <= 0), "work list not largest first"
