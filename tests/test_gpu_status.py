"""The device status words driven by data, and decode's independence from bytes it must not read.

* Non-finite fp16 inputs (DGQ article 2.2 gives the method for finite values only): dgq_compress
  counts every 16-token group of one (sequence, head) that holds a NaN or an infinity in
  status[1], dgq_append counts every 64-channel wave of an appended token that holds one; the
  codes of those heads are unspecified, and every other head stays bit-exact against the oracle.
* Decode reads only the segment rows below nseg and only the blocks the table names: rows past
  nseg filled with NaN parameters and in-range starts, unused pool blocks holding random codes
  and all-ones boundary bits give the same bits as a clean cache (DGQ article 5.1's decode
  self-test: garbled output comes from reading the wrong min/max)."""

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
import paged_layout as PL
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _check_clean_heads(cfg, params, cache, table, heads, skip):
    p = params.c
    starts, prm, nseg = cache.segment_table()
    bits = cache.bits.cpu().numpy()
    for (b, h), hc in heads.items():
        if (b, h) in skip:
            continue
        assert nseg[b, h] == len(hc.segs), (b, h)
        for i, s in enumerate(hc.segs):
            assert starts[b, h, i] == s.start, (b, h, i)
            want = np.array([s.kmin, s.kmax, s.vmin, s.vmax, s.kscale, s.vscale], np.float32)
            assert np.array_equal(prm[b, h, i].view(np.int32), want.view(np.int32)), (b, h, i)
        kc, vc = H.read_codes(cache, table, b, h, hc.length)
        H.compare_codes(kc, hc.kcodes, f"K codes b{b} h{h}")
        H.compare_codes(vc, hc.vcodes, f"V codes b{b} h{h}")
        assert np.array_equal(PL.gather_bits(bits, table[b], h, hc.length, p.block_size), hc.bits), (b, h)


def _decode_clean_rows(cfg, params, cache, table, heads, lens, skip, seed):
    q16 = dgq_data.queries(cfg, seed)
    out = Q.paged_decode_attn_int8(params, torch.from_numpy(q16).cuda(), cache, torch.from_numpy(table).cuda(),
                                   torch.from_numpy(np.asarray(lens, np.int32)).cuda(), int(max(lens)))
    out = out.cpu().numpy()
    g = cfg.group
    for (b, h), hc in heads.items():
        if (b, h) in skip:
            continue
        ref = O.decode_attention(q16[b, h * g:(h + 1) * g], hc.khat(), hc.vhat())
        assert H.rel_err_rows(out[b, h * g:(h + 1) * g], ref) <= TOL, (b, h)


def test_nonfinite_compress_input_counted_other_heads_exact():
    cfg = dgq_data.get_config(2, batch=2, seq_len=1500)
    k, v, cu, lens, _, _ = H.upload_batch(cfg, 21)
    k, v = k.copy(), v.copy()
    plant = [(0, 1, 100, "k", 5, np.nan), (0, 1, 101, "v", 7, np.inf),
             (1, 3, 900, "k", 17, -np.inf), (1, 6, int(lens[1]) - 1, "v", 0, np.nan)]
    for b, h, t, which, d, val in plant:
        (k if which == "k" else v)[cu[b] + t, h, d] = np.float16(val)
    # one count per 16-token group of a (sequence, head) that holds a non-finite value
    want = len({(b, h, t // 16) for b, h, t, _, _, _ in plant})
    bad = {(b, h) for b, h, _, _, _, _ in plant}
    params = H.params_for(cfg)
    table, nblk = dgq_data.block_tables(cfg, 21, lens_total=lens)
    cache = Q.DGQCache(params, nblk, cfg.batch)
    H.say("compress with non-finite inputs", plant)
    Q.dgq_compress(params, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                   torch.from_numpy(np.asarray(cu, np.int32)).cuda(), torch.from_numpy(table).cuda(), cache,
                   int(lens.max()), int(cu[-1]))
    st = cache.read_status()
    assert st == {"clamped_appends": 0, "nonfinite_groups": want, "inconsistencies": 0}, st
    heads = {(b, h): O.compress_head(k[cu[b]:cu[b + 1], h], v[cu[b]:cu[b + 1], h])
             for b in range(cfg.batch) for h in range(cfg.hkv) if (b, h) not in bad}
    _check_clean_heads(cfg, params, cache, table, heads, bad)
    _decode_clean_rows(cfg, params, cache, table, heads, lens, bad, 21)


def test_nonfinite_appended_token_counted_other_heads_exact():
    cfg = dgq_data.get_config(5, batch=2, seq_len=150, append_steps=40)
    k, v, cu, lens = dgq_data.batch_kv(cfg, 22)
    k, v = k.copy(), v.copy()
    steps = 40
    # (b, h, step, which, channel, value): channel 70 is in the second 64-channel wave
    plant = [(0, 2, 3, "k", 70, np.nan), (1, 0, 7, "v", 3, np.inf), (1, 0, 8, "k", 0, -np.inf)]
    for b, h, s, which, d, val in plant:
        (k if which == "k" else v)[cu[b] + lens[b] + s, h, d] = np.float16(val)
    bad = {(b, h) for b, h, _, _, _, _ in plant}
    params = H.params_for(cfg)
    p = params.c
    pk = np.concatenate([k[cu[b]:cu[b] + lens[b]] for b in range(cfg.batch)])
    pv = np.concatenate([v[cu[b]:cu[b] + lens[b]] for b in range(cfg.batch)])
    pcu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    table, nblk = dgq_data.block_tables(cfg, 22, lens_total=lens + steps)
    dtable = torch.from_numpy(table).cuda()
    cache = Q.DGQCache(params, nblk, cfg.batch)
    H.say("append with non-finite tokens", plant)
    Q.dgq_compress(params, torch.from_numpy(pk).cuda(), torch.from_numpy(pv).cuda(), torch.from_numpy(pcu).cuda(),
                   dtable, cache, int(lens.max()), int(pcu[-1]))
    states = {}
    for b in range(cfg.batch):
        for h in range(cfg.hkv):
            if (b, h) in bad:
                continue
            kk, vv = k[cu[b]:cu[b] + lens[b], h], v[cu[b]:cu[b] + lens[b], h]
            states[(b, h)] = O.AppendState(O.compress_head(kk, vv), kk, p.block_size, p.seg_capacity)
    for s in range(steps):
        pos = lens + s
        ktok = np.stack([k[cu[b] + pos[b]] for b in range(cfg.batch)])
        vtok = np.stack([v[cu[b] + pos[b]] for b in range(cfg.batch)])
        Q.dgq_append(params, torch.from_numpy(ktok).cuda(), torch.from_numpy(vtok).cuda(),
                     torch.from_numpy(pos.astype(np.int32)).cuda(), dtable, cache)
        for key, stt in states.items():
            stt.append(ktok[key[0], key[1]], vtok[key[0], key[1]])
    st = cache.read_status()
    assert st == {"clamped_appends": 0, "nonfinite_groups": len(plant), "inconsistencies": 0}, st
    heads = {key: stt.snapshot() for key, stt in states.items()}
    _check_clean_heads(cfg, params, cache, table, heads, bad)
    _decode_clean_rows(cfg, params, cache, table, heads, lens + steps, bad, 22)


def test_decode_ignores_rows_past_nseg_and_unused_blocks():
    cfg = dgq_data.get_config(2, batch=3, seq_len=900)
    lens = np.array([900, 417, 64])
    heads = {}
    for b in range(cfg.batch):
        for h in range(cfg.hkv):
            kk, vv = dgq_data.head_kv(cfg, 23, 0, b, h, int(lens[b]))
            heads[(b, h)] = O.compress_head(kk[:lens[b]], vv[:lens[b]])
    table, nblk = dgq_data.block_tables(cfg, 23, lens_total=lens, spare_blocks=40)
    params = H.params_for(cfg)
    clean = H.cache_from_oracle(params, heads, table, nblk, cfg.batch, fill=0)
    dirty = H.cache_from_oracle(params, heads, table, nblk, cfg.batch, fill=None)   # random unused codes
    used = np.zeros(nblk, bool)
    for b in range(cfg.batch):
        used[table[b][:(lens[b] + cfg.block_size - 1) // cfg.block_size]] = True
    bits = dirty.bits.cpu().numpy()
    bits[~used] = 0xFF
    dirty.bits.copy_(torch.from_numpy(bits))
    segs = dirty.segs.cpu().numpy()
    nseg = dirty.nseg.cpu().numpy()
    rng = np.random.default_rng(5)
    nan_row = np.full(6, np.nan, np.float32).view(np.int32)
    for b in range(cfg.batch):
        for h in range(cfg.hkv):
            for i in range(nseg[b, h], params.c.seg_capacity):
                segs[b, h, i, 0] = rng.integers(0, lens[b])
                segs[b, h, i, 1:7] = nan_row
                segs[b, h, i, 7] = -1
    dirty.segs.copy_(torch.from_numpy(segs))
    q16 = torch.from_numpy(dgq_data.queries(cfg, 23)).cuda()
    dt = torch.from_numpy(table).cuda()
    dl = torch.from_numpy(lens.astype(np.int32)).cuda()
    H.say("decode with poisoned rows past nseg and unused blocks")
    o1 = Q.paged_decode_attn_int8(params, q16, clean, dt, dl, int(lens.max())).cpu().numpy()
    o2 = Q.paged_decode_attn_int8(params, q16, dirty, dt, dl, int(lens.max())).cpu().numpy()
    assert np.all(np.isfinite(o2))
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert int(dirty.status[2].item()) == 0
    ref = H.oracle_decode(dgq_data.queries(cfg, 23), heads, lens, cfg.hkv, cfg.group)
    assert H.rel_err_rows(o1, ref) <= TOL
