"""The one-launch compress for short sequences (at most 256 tokens at head_dim 128, 512 at 64)
against the oracle and, byte for byte, against the separate stats / selection / encode launches
(DGQ_COMPRESS_MULTIPASS) on the same input: pools, boundary bits, segment table, nseg, append
state and status words, in both identifier formats and all three block sizes, for ragged batches that
reach the length limit, with the segment-count policies, non-finite inputs, an out-of-range
block id and a sequence longer than max_seq_len (DGQ article 2.2 for the method; 3.2 for
short-context compress latency)."""

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q
from test_gpu_compress import compress_and_check

pytestmark = pytest.mark.gpu

FIELDS = ("k_pool", "v_pool", "bits", "segs", "nseg", "tail", "status")


def _short_limit(d):
    return 32768 // d


def _lens(d):
    s = _short_limit(d)
    return np.array([0, 1, 15, 16, 31, 32, 33, 63, 64, 65, 100, 129, s - 1, s, s - 17, 200], np.int64)


def _data(lens, hkv, d, seed):
    """Piecewise-sigma Gaussian keys and values (0.03 / 0.15 / 0.47 runs of 16..96 tokens), with a
    constant run, a -0 run and exact ties in some sequences."""
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    k = np.zeros((total, hkv, d), np.float16)
    v = np.zeros_like(k)
    for b, L in enumerate(lens):
        L = int(L)
        for h in range(hkv):
            sig = np.empty(L, np.float32)
            t = 0
            while t < L:
                n = int(rng.integers(16, 97))
                sig[t:t + n] = rng.choice([0.03, 0.15, 0.47])
                t += n
            kk = rng.standard_normal((L, d)).astype(np.float32) * sig[:, None]
            vv = rng.standard_normal((L, d)).astype(np.float32) * sig[:, None]
            if L >= 96 and b % 3 == 0:
                kk[32:64] = 0.0
                vv[32:64] = -0.125
            if L >= 128 and b % 3 == 1:
                kk[64:96] = -0.0
            k[cu[b]:cu[b + 1], h] = kk.astype(np.float16)
            v[cu[b]:cu[b + 1], h] = vv.astype(np.float16)
    return k, v, cu


def _table(lens_cap, bs, max_len, seed):
    rng = np.random.default_rng(seed)
    mb = max(1, -(-max_len // bs))
    ids = rng.permutation(len(lens_cap) * mb) + 1
    return ids.reshape(len(lens_cap), mb).astype(np.int32), len(lens_cap) * mb + 1


def _run(params, k, v, cu, table, nblk, max_len, batch, total=None):
    cache = Q.DGQCache(params, nblk, batch)
    Q.dgq_compress(params, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(cu).cuda(),
                   torch.from_numpy(table).cuda(), cache, max_len, int(cu[-1]) if total is None else total)
    torch.cuda.synchronize()
    return cache


def _same(a, b, what):
    for f in FIELDS:
        x, y = getattr(a, f), getattr(b, f)
        if x is None:
            assert y is None
            continue
        assert torch.equal(x, y), (what, f)


@pytest.mark.parametrize("d,bs", [(64, 16), (64, 32), (64, 64), (128, 16), (128, 32), (128, 64)])
@pytest.mark.parametrize("marker", [False, True], ids=["bitmap", "marker"])
def test_short_path_equals_multipass_and_oracle(d, bs, marker):
    lens = _lens(d)
    hkv = 2
    k, v, cu = _data(lens, hkv, d, 100 + d + bs)
    max_len = _short_limit(d)
    table, nblk = _table(lens, bs, max_len, 7)
    kw = dict(marker=marker)
    one = Q.DGQParams(hkv, 2 * hkv, d, bs, **kw)
    multi = Q.DGQParams(hkv, 2 * hkv, d, bs, multipass=True, **kw)
    H.say("short compress vs multipass", d, bs, marker)
    a = _run(one, k, v, cu, table, nblk, max_len, len(lens))
    b = _run(multi, k, v, cu, table, nblk, max_len, len(lens))
    _same(a, b, (d, bs, marker))
    assert a.status.cpu().tolist() == [0, 0, 0, 0]
    # and the one-launch result against the oracle (segments, codes, bits, append state, decode)
    cfg = dgq_data.get_config(1, batch=len(lens), hkv=hkv, hq=2 * hkv, head_dim=d, block_size=bs, seq_len=max_len)
    H.say("short compress vs oracle", d, bs, marker)
    compress_and_check(cfg, 5, params=one, k=k, v=v, cu=cu, lens=lens)


@pytest.mark.parametrize("max_segments,tau,length_aware,min_var", [
    (8, 1.0, False, 0.0), (2, 2.0, False, 0.0), (5, 1.5, True, 0.0), (5, 2.0, False, 1e-3), (1, 2.0, False, 0.0)])
def test_short_path_policies(max_segments, tau, length_aware, min_var):
    d, bs = 128, 16
    lens = _lens(d)
    k, v, cu = _data(lens, 2, d, 311)
    max_len = _short_limit(d)
    table, nblk = _table(lens, bs, max_len, 8)
    kw = dict(max_segments=max_segments, seg_capacity=max(max_segments, 8), tau=tau, length_aware=length_aware,
              min_var=min_var)
    H.say("short compress policies", kw)
    a = _run(Q.DGQParams(2, 8, d, bs, **kw), k, v, cu, table, nblk, max_len, len(lens))
    b = _run(Q.DGQParams(2, 8, d, bs, multipass=True, **kw), k, v, cu, table, nblk, max_len, len(lens))
    _same(a, b, kw)
    nseg = a.nseg.cpu().numpy()
    for bb, L in enumerate(lens):
        for h in range(2):
            hc = O.compress_head(k[cu[bb]:cu[bb + 1], h], v[cu[bb]:cu[bb + 1], h], max_segments, tau, min_var,
                                 length_aware)
            assert nseg[bb, h] == len(hc.segs), (bb, h)
    if max_segments == 8 and tau == 1.0:
        assert nseg.max() >= 6       # the largest cut counts are reached


def test_short_path_status_words_match():
    """Non-finite inputs (counted per 16-token group), a block id past the pool (counted per
    16-channel key unit, its writes skipped) and a sequence longer than max_seq_len (clamped,
    counted once): both paths count the same and write the same bytes."""
    d, bs, hkv = 64, 16, 2
    lens = np.array([40, 300, 530, 17], np.int64)      # 530 > max_seq_len 512: clamped
    k, v, cu = _data(lens, hkv, d, 9)
    k[cu[0] + 3, 1, 5] = np.float16(np.nan)
    v[cu[1] + 250, 0, 63] = np.float16(np.inf)
    k[cu[1] + 251, 0, 0] = np.float16(-np.inf)           # same 16-token group: one count
    v[cu[3] + 16, 1, 2] = np.float16(np.nan)
    max_len = 512
    table, nblk = _table(lens, bs, max_len, 3)
    table[1, 5] = nblk + 10                               # not a pool block
    total = int(cu[-1])
    assert total <= len(lens) * max_len
    H.say("short compress status words")
    a = _run(Q.DGQParams(hkv, hkv, d, bs), k, v, cu, table, nblk, max_len, len(lens), total)
    b = _run(Q.DGQParams(hkv, hkv, d, bs, multipass=True), k, v, cu, table, nblk, max_len, len(lens), total)
    _same(a, b, "status")
    st = a.status.cpu().tolist()
    assert st[1] == 3, st
    # block 5 of sequence 1 holds 16 tokens x 4 key units x 2 heads; plus one clamped sequence
    assert st[2] == 16 * (d // 16) * hkv + 1, st
