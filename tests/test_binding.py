"""The Python binding's own checks, on the CPU: argument errors are raised before the library is
called (no device memory is touched), and parameter objects carry the flags the C ABI expects."""

import pytest
import torch

import quantized_paged_kv_dgq_amd as Q
from quantized_paged_kv_dgq_amd import _lib


def test_params_flags_and_layout():
    p = Q.DGQParams(8, 32, 128, 16)
    assert p.group == 4 and not p.length_aware and not p.marker and p.c.flags == 0
    p = Q.DGQParams(8, 32, 128, 64, length_aware=True, min_var=1e-3, marker=True)
    assert p.length_aware and p.marker
    assert p.c.flags == _lib.DGQ_POLICY_LENGTH_AWARE | _lib.DGQ_FORMAT_MARKER
    assert p.c.min_var == 1e-3 and p.c.tau == 2.0 and p.c.win == 16 and p.c.seg_capacity == 16


def test_compress_rejects_bad_tensors_before_the_library():
    p = Q.DGQParams(2, 2, 64, 16)
    k32 = torch.zeros((4, 2, 64), dtype=torch.float32)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    table = torch.zeros((1, 1), dtype=torch.int32)
    with pytest.raises(ValueError, match="float16"):
        Q.dgq_compress(p, k32, k32, cu, table, None, 4, 4)
    k = torch.zeros((4, 2, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="int32"):
        Q.dgq_compress(p, k, k, cu.long(), table, None, 4, 4)
    with pytest.raises(ValueError, match="contiguous"):
        Q.dgq_compress(p, k.transpose(1, 2), k.transpose(1, 2), cu, table, None, 4, 4)


def test_decode_and_append_reject_bad_tensors():
    p = Q.DGQParams(2, 2, 64, 16)
    q32 = torch.zeros((1, 2, 64), dtype=torch.float32)
    lens = torch.zeros(1, dtype=torch.int32)
    table = torch.zeros((1, 1), dtype=torch.int32)
    with pytest.raises(ValueError, match="float16"):
        Q.paged_decode_attn_int8(p, q32, None, table, lens, 16)
    tok = torch.zeros((1, 2, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="int32"):
        Q.dgq_append(p, tok, tok, lens.long(), table, None)
    with pytest.raises(ValueError, match="float16"):
        Q.dgq_append_decode(p, tok, tok, lens, q32, table, None, 16)


def test_lifecycle_rejects_bad_ids():
    p = Q.DGQParams(2, 2, 64, 16)
    with pytest.raises(ValueError, match="differ in length"):
        Q.dgq_copy_blocks(p, None, torch.zeros(2, dtype=torch.int32), torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="int32"):
        Q.dgq_copy_seq_state(p, None, torch.zeros(1, dtype=torch.int64), torch.zeros(1, dtype=torch.int64))
    staging = torch.zeros(16, dtype=torch.float32)
    with pytest.raises(ValueError, match="uint8"):
        Q.dgq_swap_out(p, None, 0, torch.zeros(1, dtype=torch.int32), staging)


def test_block_pool_wrapper():
    pool = Q.BlockPool(4)
    ids = pool.alloc(2)
    assert ids == [0, 1] and pool.num_free == 2
    pool.share([ids[0]])
    assert pool.refcount(ids[0]) == 2
    new = pool.cow([ids[0]])
    assert new[0] != ids[0] and pool.refcount(ids[0]) == 1 and pool.refcount(new[0]) == 1
    with pytest.raises(Q.DGQError):
        pool.alloc(5)
    pool.free([ids[0], ids[1], new[0]])
    assert pool.num_free == 4
    pool.close()
