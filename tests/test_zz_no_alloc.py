"""paged_decode_attn_int8_noalloc (the allocation-free decode, partials in the library's fixed
per-device scratch array) against paged_decode_attn_int8 with a caller workspace: the same launch
plan and kernels, so the outputs must be bit-identical.  Two calls in a row, the second on a
smaller input (fewer sequences, shorter, other partition count), then the first again; each is
also within the decode tolerance of the oracle."""

import ctypes
import math

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q
from quantized_paged_kv_dgq_amd import _lib

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _case(cid, over, seed):
    cfg = dgq_data.get_config(cid, **over)
    lens = np.asarray(dgq_data.seq_lens(cfg, seed), np.int64)
    heads = {}
    for b in range(cfg.batch):
        for h in range(cfg.hkv):
            k, v = dgq_data.head_kv(cfg, seed, 0, b, h, int(lens[b]))
            heads[(b, h)] = O.compress_head(k[:lens[b]], v[:lens[b]])
    table, nblk = dgq_data.block_tables(cfg, seed, lens_total=np.maximum(lens, 1))
    params = H.params_for(cfg)
    cache = H.cache_from_oracle(params, heads, table, nblk, cfg.batch)
    q16 = dgq_data.queries(cfg, seed)
    return cfg, lens, heads, table, params, cache, q16


def _both(cfg, lens, heads, table, params, cache, q16):
    dq = torch.from_numpy(q16).cuda()
    dt = torch.from_numpy(table).cuda()
    dl = torch.from_numpy(lens.astype(np.int32)).cuda()
    max_len = int(max(lens.max(), 1))
    ref = Q.paged_decode_attn_int8(params, dq, cache, dt, dl, max_len)
    out = torch.full(dq.shape, float("nan"), dtype=torch.float32, device="cuda")
    # straight through the C ABI
    st = _lib.load().paged_decode_attn_int8_noalloc(
        ctypes.byref(params.c), dq.data_ptr(), ctypes.byref(cache.c), dt.data_ptr(), dt.shape[1], dl.data_ptr(),
        dq.shape[0], max_len, 1.0 / math.sqrt(cfg.head_dim), out.data_ptr(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.DGQ_OK, _lib.load().dgq_status_string(st)
    torch.cuda.synchronize()
    assert int(cache.status[2].item()) == 0
    ref, out = ref.cpu().numpy(), out.cpu().numpy()
    assert np.array_equal(ref.view(np.uint32), out.view(np.uint32))
    oracle = H.oracle_decode(q16, heads, lens, cfg.hkv, cfg.group)
    assert H.rel_err_rows(out, oracle) <= TOL
    return out


def test_noalloc_decode_equals_workspace_decode():
    big = _case(2, dict(batch=3, seq_len=3000), 11)          # 47 chunks per head: split and merged
    small = _case(4, dict(batch=2, seq_len=500, min_len=1), 12)   # MHA, shorter, fewer partitions
    H.say("noalloc decode: 3 x 3000 tokens, 8/32 heads")
    first = _both(*big)
    H.say("noalloc decode: 2 MHA sequences <= 500 tokens")
    _both(*small)
    H.say("noalloc decode: the first input again")
    again = _both(*big)
    assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
