"""Host-side parts of the Python binding (no GPU): the checked mode for block
ids rejects out-of-pool entries before anything is launched."""
import pytest
import torch

import decode_attention_08_amd as gq


def _paged_inputs(table, lens, num_blocks=6, bs=16):
    q = torch.zeros(len(lens), 4, 64, dtype=torch.float16)
    k = torch.zeros(num_blocks, bs, 1, 64, dtype=torch.float16)
    bt = torch.tensor(table, dtype=torch.int32)
    ctx = torch.tensor(lens, dtype=torch.int32)
    return q, k, k.clone(), bt, ctx


def test_out_of_pool_block_id_rejected_before_launch():
    q, k, v, bt, ctx = _paged_inputs([[0, 1, 6], [2, -1, -1]], [40, 3])
    with pytest.raises(ValueError, match=r"block_table\[0, 2\] = 6 is outside the pool of 6"):
        gq.decode(q, k, v, bt, ctx, check_blocks=True)


def test_negative_block_id_in_range_rejected():
    q, k, v, bt, ctx = _paged_inputs([[0, 1, 2], [-1, -1, -1]], [33, 1])
    with pytest.raises(ValueError, match=r"block_table\[1, 0\] = -1"):
        gq.check_block_table(bt, ctx, 6, 16)


def test_entries_past_the_length_are_not_checked():
    # sequence 0 reads ceil(17/16) = 2 blocks: the -1 and 99 after them are never read
    q, k, v, bt, ctx = _paged_inputs([[0, 1, 99], [2, -1, -1]], [17, 16])
    gq.check_block_table(bt, ctx, 6, 16)
    # a full table at the largest length is fine, one block short of the pool is not
    _, _, _, bt2, ctx2 = _paged_inputs([[0, 1, 2]], [48])
    gq.check_block_table(bt2, ctx2, 3, 16)
    with pytest.raises(ValueError, match="outside the pool of 2"):
        gq.check_block_table(bt2, ctx2, 2, 16)


def test_lengths_outside_the_table_rejected():
    """The kernels clamp ctx_lens to [0, max_blocks * block_size]; the checked
    mode reports such lengths instead."""
    _, _, _, bt, ctx = _paged_inputs([[0, 1, 2]], [49])
    with pytest.raises(ValueError, match=r"ctx_lens\[0\] = 49 is outside \[0, 48\]"):
        gq.check_block_table(bt, ctx, 3, 16)
    with pytest.raises(ValueError, match=r"ctx_lens\[1\] = -3"):
        gq.check_block_table(torch.tensor([[0], [1]], dtype=torch.int32),
                             torch.tensor([5, -3], dtype=torch.int32), 2, 16)


def test_valid_table_passes_the_check_then_needs_a_gpu():
    """With a valid table the checked call goes on to the ordinary argument
    checks (here: host tensors are refused), so nothing is launched either way."""
    q, k, v, bt, ctx = _paged_inputs([[0, 1, 2], [3, 4, -1]], [40, 20])
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        gq.decode(q, k, v, bt, ctx, check_blocks=True)


def test_xsplit_pool_block_size_taken_from_its_layout():
    # x-split k [num_blocks, h_kv, d/8, bs, 8]: bs = 32 here, so 33 tokens read 2 blocks
    q = torch.zeros(1, 4, 64, dtype=torch.float16)
    k = torch.zeros(3, 1, 8, 32, 8, dtype=torch.float16)
    v = torch.zeros(3, 1, 64, 32, dtype=torch.float16)
    bt = torch.tensor([[2, 3]], dtype=torch.int32)
    ctx = torch.tensor([33], dtype=torch.int32)
    with pytest.raises(ValueError, match=r"block_table\[0, 1\] = 3 is outside the pool of 3"):
        gq.decode_xsplit(q, k, v, bt, ctx, check_blocks=True)
