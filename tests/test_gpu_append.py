"""dgq_append on the GPU against the oracle's AppendState: a compressed prefix followed by one
token per sequence per step; segment tables, codes, bits, tail state and decode checked along
the way."""

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
import paged_layout as PL
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q

pytestmark = pytest.mark.gpu


def run_stream(cfg, seed, steps, params=None, check_every=None, k=None, v=None, cu=None, lens=None):
    if k is None:
        k, v, cu, lens = dgq_data.batch_kv(cfg, seed)   # prefix + appended tokens
    lens = np.asarray(lens, np.int64)
    if params is None:
        params = H.params_for(cfg)
    p = params.c
    bsz, hkv, d = cfg.batch, cfg.hkv, cfg.head_dim
    # prefix-only packed copy for the compressor
    pk = np.concatenate([k[cu[b]:cu[b] + lens[b]] for b in range(bsz)])
    pv = np.concatenate([v[cu[b]:cu[b] + lens[b]] for b in range(bsz)])
    pcu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    table, nblk = dgq_data.block_tables(cfg, seed, lens_total=lens + steps)
    dtable = torch.from_numpy(table).cuda()
    cache = Q.DGQCache(params, nblk, bsz)
    max_total = int((lens + steps).max())
    Q.dgq_compress(params, torch.from_numpy(pk).cuda(), torch.from_numpy(pv).cuda(), torch.from_numpy(pcu).cuda(),
                   dtable, cache, int(lens.max()), int(pcu[-1]))
    states = {}
    for b in range(bsz):
        for h in range(hkv):
            kk = k[cu[b]:cu[b] + lens[b], h]
            vv = v[cu[b]:cu[b] + lens[b], h]
            states[(b, h)] = O.AppendState(O.compress_head(kk, vv, p.max_segments, p.tau, p.min_var,
                                                           params.length_aware, H.fmt_of(params)),
                                           kk, p.block_size, p.seg_capacity, p.tau, p.min_var)
    check_every = check_every or steps
    for s in range(steps):
        pos = lens + s
        ktok = np.stack([k[cu[b] + pos[b]] for b in range(bsz)])     # [B][H][D]
        vtok = np.stack([v[cu[b] + pos[b]] for b in range(bsz)])
        Q.dgq_append(params, torch.from_numpy(ktok).cuda(), torch.from_numpy(vtok).cuda(),
                     torch.from_numpy(pos.astype(np.int32)).cuda(), dtable, cache)
        for b in range(bsz):
            for h in range(hkv):
                states[(b, h)].append(ktok[b, h], vtok[b, h])
        if (s + 1) % check_every == 0 or s == steps - 1:
            torch.cuda.synchronize()
            check_state(cfg, params, cache, states, table, pos + 1, seed + s)
    return cache, states


def check_state(cfg, params, cache, states, table, cur_lens, qseed):
    p = params.c
    heads = {key: st.snapshot() for key, st in states.items()}
    H.compare_segments(cache, heads, cfg.batch, cfg.hkv)
    bits = H.identifier_bits(cache, table, cur_lens)
    tails = cache.tail.cpu().numpy()
    for (b, h), hc in heads.items():
        kc, vc = H.read_codes(cache, table, b, h, hc.length)
        H.compare_codes(kc, hc.kcodes, f"K codes b{b} h{h}")
        H.compare_codes(vc, hc.vcodes, f"V codes b{b} h{h}")
        if params.marker:
            H.compare_markers(kc, hc.kcodes, f"K markers b{b} h{h}")
        assert np.array_equal(PL.gather_bits(bits, table[b], h, hc.length, p.block_size), hc.bits), (b, h)
        st = states[(b, h)]
        tl = tails[b, h]
        assert tl[0] == st.r0 and tl[1] == len(st.ring_a) and tl[2] == int(st.span_own), (b, h, tl[:3])
        assert list(tl[4:4 + tl[1]]) == st.ring_a
        assert list(tl[20:52].view(np.int64)[:tl[1]]) == st.ring_b
    clamped = sum(st.clamped for st in states.values())
    assert int(cache.status[0].item()) == clamped
    q16 = dgq_data.queries(cfg, qseed)
    out = Q.paged_decode_attn_int8(params, torch.from_numpy(q16).cuda(), cache, torch.from_numpy(table).cuda(),
                                   torch.from_numpy(cur_lens.astype(np.int32)).cuda(), int(cur_lens.max()))
    ref = H.oracle_decode(q16, heads, cur_lens, cfg.hkv, cfg.group)
    err = H.rel_err_rows(out.cpu().numpy(), ref)
    assert err <= 2e-3, err


def test_stream_bs64_mid_block_prefix():
    cfg = dgq_data.get_config(5, batch=3, seq_len=200, append_steps=150)
    H.say("append stream bs64 prefix 200 + 150")
    run_stream(cfg, 0, 150, check_every=30)


def test_stream_bs16_block_aligned_prefix():
    cfg = dgq_data.get_config(2, batch=2, seq_len=256, append_steps=80)
    H.say("append stream bs16 prefix 256 + 80")
    run_stream(cfg, 1, 80, check_every=16)


def test_stream_bs32():
    """32-token blocks (two 16-token tiles each): prefix 300 + 100 appends, crossing blocks."""
    cfg = dgq_data.get_config(2, batch=2, seq_len=300, append_steps=100, block_size=32)
    H.say("append stream bs32 prefix 300 + 100")
    run_stream(cfg, 5, 100, check_every=25)


def test_stream_from_empty_and_short_prefixes():
    """Prefixes of 0, 5 and 40 tokens (no full window in the ring at first)."""
    cfg = dgq_data.get_config(1, batch=3, append_steps=100, block_size=16)
    rng = np.random.default_rng(3)
    d = cfg.head_dim
    lens = np.array([0, 5, 40])
    seqs = [(rng.standard_normal((n + 100, 2, d)) * rng.uniform(0.05, 0.5)).astype(np.float16) for n in lens]
    cu = np.concatenate([[0], np.cumsum(lens + 100)]).astype(np.int32)
    k = np.concatenate(seqs)
    v = (k * 0.7).astype(np.float16)
    H.say("append stream from short prefixes")
    run_stream(cfg, 2, 100, check_every=20, k=k, v=v, cu=cu, lens=lens)


@pytest.mark.parametrize("min_var", [1e-3, 0.03])
def test_stream_with_variance_floor_and_length_cap(min_var):
    """Appends under the variance floor (the window test ignores quiet window pairs) after a
    length-capped compress."""
    cfg = dgq_data.get_config(5, batch=3, seq_len=200, append_steps=150)
    H.say("append with floor", min_var)
    run_stream(cfg, 8, 150, params=H.params_for(cfg, length_aware=True, min_var=min_var), check_every=50)


def test_stream_table_full_clamps_and_counts():
    """A full segment table: the span joins, codes saturate, status[0] counts like the oracle."""
    cfg = dgq_data.get_config(2, batch=2, seq_len=128, append_steps=64)
    rng = np.random.default_rng(4)
    d = cfg.head_dim
    k = (rng.standard_normal((2 * 192, cfg.hkv, d)) * 0.2).astype(np.float16)
    k[128:192] *= np.float16(10.0)
    k[192 + 128:] *= np.float16(10.0)
    v = k.copy()
    cu = np.array([0, 192, 384], np.int32)
    lens = np.array([128, 128])
    params = H.params_for(cfg, max_segments=2, seg_capacity=2)
    H.say("append stream clamp")
    cache, states = run_stream(cfg, 3, 64, params=params, check_every=16, k=k, v=v, cu=cu, lens=lens)
    assert sum(st.clamped for st in states.values()) > 0
    st = cache.read_status()
    assert st["clamped_appends"] == sum(s.clamped for s in states.values())
    assert st["nonfinite_groups"] == 0 and st["inconsistencies"] == 0


@pytest.mark.parametrize("cid,over,steps", [
    (5, dict(batch=3, seq_len=200, append_steps=160), 160),
    (2, dict(batch=2, seq_len=250, append_steps=90), 90),
], ids=["bs64", "bs16"])
def test_stream_marker_format(cid, over, steps):
    """Appends in the marker format: every span that opens a segment writes its marker at r0,
    no bit tensor is touched; against the oracle's marker-format AppendState."""
    cfg = dgq_data.get_config(cid, **over)
    H.say("append marker format", cid, over)
    run_stream(cfg, 17, steps, params=H.params_for(cfg, marker=True), check_every=steps // 3)


def growing_values(cfg, prefix, steps, seed):
    """One sequence: keys N(0, 0.25), values whose standard deviation grows by 15 % per block, so
    that the span of almost every appended block leaves the range of the row before it and takes a
    row of its own, until the segment table is full."""
    rng = np.random.default_rng(seed)
    n = prefix + steps
    amp = 1.15 ** (np.arange(n) // cfg.block_size)
    k = (rng.standard_normal((n, cfg.hkv, cfg.head_dim)) * 0.5).astype(np.float16)
    v = (rng.standard_normal((n, cfg.hkv, cfg.head_dim)) * 0.5 * amp[:, None, None]).astype(np.float16)
    return k, v, np.array([0, n], np.int32), np.array([prefix], np.int64)


def test_stream_fills_largest_segment_table():
    """A 64-row segment table (the largest) filled by appended blocks, then the table-full clamp:
    rows, codes, bits, append state, the clamp count and the decode against the oracle."""
    cfg = dgq_data.get_config(1, batch=1, seq_len=64, append_steps=1100, block_size=16)
    H.say("append stream through a full 64-row segment table")
    params = H.params_for(cfg, max_segments=8, seg_capacity=64)
    k, v, cu, lens = growing_values(cfg, 64, 1100, 7)
    _, states = run_stream(cfg, 7, 1100, params=params, check_every=275, k=k, v=v, cu=cu, lens=lens)
    assert all(len(st.snapshot().segs) == 64 and st.clamped > 0 for st in states.values())
