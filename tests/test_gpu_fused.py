"""The fused append + decode step (dgq_append_decode) against dgq_append followed by
paged_decode_attn_int8 on a second copy of the same cache: outputs bit-identical at every step,
and the two caches (segment rows, row counts, append state, codes, bits) identical at the end;
against the oracle's AppendState and attention at checkpoints."""

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
import paged_layout as PL
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q

pytestmark = pytest.mark.gpu


def _same_cache(c1, c2, table, lens, p):
    assert torch.equal(c1.nseg, c2.nseg)
    assert torch.equal(c1.segs, c2.segs)
    assert torch.equal(c1.tail, c2.tail)
    assert torch.equal(c1.status, c2.status)
    assert (c1.bits is None) == (c2.bits is None)
    k1, k2 = c1.k_pool.cpu().numpy(), c2.k_pool.cpu().numpy()
    v1, v2 = c1.v_pool.cpu().numpy(), c2.v_pool.cpu().numpy()
    b1, b2 = (None, None) if c1.bits is None else (c1.bits.cpu().numpy(), c2.bits.cpu().numpy())
    koff, voff = PL.k_offsets(p.block_size, p.head_dim), PL.v_offsets(p.block_size, p.head_dim)
    for b, n in enumerate(lens):
        for h in range(p.num_kv_heads):
            assert np.array_equal(PL.gather_head(k1, table[b], h, n, koff), PL.gather_head(k2, table[b], h, n, koff))
            assert np.array_equal(PL.gather_head(v1, table[b], h, n, voff), PL.gather_head(v2, table[b], h, n, voff))
            if b1 is not None:
                assert np.array_equal(PL.gather_bits(b1, table[b], h, n, p.block_size),
                                      PL.gather_bits(b2, table[b], h, n, p.block_size))


def run_fused(cfg, seed, steps, checks, params=None, data=None):
    k, v, cu, lens = data if data is not None else dgq_data.batch_kv(cfg, seed)
    lens = np.asarray(lens, np.int64)
    params = params or H.params_for(cfg)
    p = params.c
    bsz, hkv = cfg.batch, cfg.hkv
    pk = np.concatenate([k[cu[b]:cu[b] + lens[b]] for b in range(bsz)])
    pv = np.concatenate([v[cu[b]:cu[b] + lens[b]] for b in range(bsz)])
    pcu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    table, nblk = dgq_data.block_tables(cfg, seed, lens_total=lens + steps)
    dtable = torch.from_numpy(table).cuda()
    max_total = int((lens + steps).max())
    caches = [Q.DGQCache(params, nblk, bsz) for _ in range(2)]
    for c in caches:
        Q.dgq_compress(params, torch.from_numpy(pk).cuda(), torch.from_numpy(pv).cuda(), pcu, dtable, c,
                       int(lens.max()), int(pk.shape[0]))
    ws = [Q.workspace(Q.decode_workspace_size(params, bsz, max_total)) for _ in range(2)]
    states = {}
    for b in range(bsz):
        for h in range(hkv):
            kk, vv = k[cu[b]:cu[b] + lens[b], h], v[cu[b]:cu[b] + lens[b], h]
            states[(b, h)] = O.AppendState(O.compress_head(kk, vv, p.max_segments, p.tau, p.min_var,
                                                           params.length_aware, H.fmt_of(params)),
                                           kk, p.block_size, p.seg_capacity, p.tau, p.min_var)
    for s in range(steps):
        pos = lens + s
        dpos = torch.from_numpy(pos.astype(np.int32)).cuda()
        ktok = torch.from_numpy(np.stack([k[cu[b] + pos[b]] for b in range(bsz)])).cuda()
        vtok = torch.from_numpy(np.stack([v[cu[b] + pos[b]] for b in range(bsz)])).cuda()
        q16 = dgq_data.queries(cfg, seed, 0, s)
        dq = torch.from_numpy(q16).cuda()
        Q.dgq_append(params, ktok, vtok, dpos, dtable, caches[0])
        o_sep = Q.paged_decode_attn_int8(params, dq, caches[0], dtable, dpos + 1, max_total, ws=ws[0])
        o_fused = Q.dgq_append_decode(params, ktok, vtok, dpos, dq, dtable, caches[1], max_total, ws=ws[1])
        torch.cuda.synchronize()
        assert torch.equal(o_sep, o_fused), f"step {s}: fused output differs"
        for b in range(bsz):
            for h in range(hkv):
                states[(b, h)].append(k[cu[b] + pos[b], h], v[cu[b] + pos[b], h])
        if s in checks:
            heads = {key: st.snapshot() for key, st in states.items()}
            ref = H.oracle_decode(q16, heads, pos + 1, hkv, cfg.group)
            err = H.rel_err_rows(o_fused.cpu().numpy(), ref)
            print(f"step {s}: fused decode vs oracle {err:.3e}", flush=True)
            assert err <= 2e-3
            H.compare_segments(caches[1], heads, bsz, hkv)
    _same_cache(caches[0], caches[1], table, lens + steps, p)
    for w in ws:   # completion counters back at zero
        assert int(w[: bsz * hkv * 4].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("cid,over,steps,checks", [
    (5, dict(batch=3, seq_len=200, append_steps=150), 150, (0, 55, 64, 149)),
    (2, dict(batch=2, seq_len=256, append_steps=80), 80, (0, 15, 16, 79)),
    (1, dict(hq=4, block_size=64, seq_len=100, append_steps=60, batch=2), 60, (0, 59)),
    (2, dict(batch=2, seq_len=250, append_steps=70, block_size=32), 70, (0, 5, 6, 69)),
], ids=["bs64_stream", "bs16_block_aligned", "d64_g2", "bs32"])
def test_fused_matches_separate_and_oracle(cid, over, steps, checks):
    cfg = dgq_data.get_config(cid, **over)
    H.say("fused append+decode", cid, over)
    run_fused(cfg, 41, steps, checks)


def test_fused_many_partitions():
    """A long sequence split over many workgroups: the row count is published by the merging
    workgroup, not by the one that appended."""
    cfg = dgq_data.get_config(3, seq_len=20000, append_steps=70)
    H.say("fused many partitions", cfg.seq_len)
    run_fused(cfg, 42, 70, (0, 47, 48, 69))


def test_fused_with_policies():
    cfg = dgq_data.get_config(5, batch=2, seq_len=300, append_steps=100)
    H.say("fused with policies")
    run_fused(cfg, 43, 100, (0, 99), params=H.params_for(cfg, length_aware=True, min_var=1e-3))


def test_fused_marker_format():
    """The fused step in the marker format: the appending workgroup writes the marker and the decode
    uses the marker format's dequantization."""
    cfg = dgq_data.get_config(5, batch=2, seq_len=260, append_steps=90)
    H.say("fused marker format")
    run_fused(cfg, 44, 90, (0, 45, 89), params=H.params_for(cfg, marker=True))


def _fused_vs_separate(cfg, seed, steps, max_seq_len, corrupt=None):
    """Both paths on two copies of one compressed cache with the given max_seq_len (which may
    clamp the decode), optionally with one (sequence, head)'s append state made inconsistent in
    both copies; outputs, caches and status words must agree at every step."""
    k, v, cu, lens = dgq_data.batch_kv(cfg, seed)
    lens = np.asarray(lens, np.int64)
    params = H.params_for(cfg)
    p = params.c
    bsz = cfg.batch
    pk = np.concatenate([k[cu[b]:cu[b] + lens[b]] for b in range(bsz)])
    pv = np.concatenate([v[cu[b]:cu[b] + lens[b]] for b in range(bsz)])
    pcu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    table, nblk = dgq_data.block_tables(cfg, seed, lens_total=lens + steps)
    dtable = torch.from_numpy(table).cuda()
    caches = [Q.DGQCache(params, nblk, bsz) for _ in range(2)]
    for c in caches:
        Q.dgq_compress(params, torch.from_numpy(pk).cuda(), torch.from_numpy(pv).cuda(), pcu, dtable, c,
                       int(lens.max()), int(pk.shape[0]))
        if corrupt is not None:
            b, h = corrupt
            c.tail[b, h, 0] = int(lens[b]) + 1000   # r0 past every new token: the state does not fit
    ws = [Q.workspace(Q.decode_workspace_size(params, bsz, max_seq_len)) for _ in range(2)]
    for s in range(steps):
        pos = lens + s
        dpos = torch.from_numpy(pos.astype(np.int32)).cuda()
        ktok = torch.from_numpy(np.stack([k[cu[b] + pos[b]] for b in range(bsz)])).cuda()
        vtok = torch.from_numpy(np.stack([v[cu[b] + pos[b]] for b in range(bsz)])).cuda()
        dq = torch.from_numpy(dgq_data.queries(cfg, seed, 0, s)).cuda()
        Q.dgq_append(params, ktok, vtok, dpos, dtable, caches[0])
        o_sep = Q.paged_decode_attn_int8(params, dq, caches[0], dtable, dpos + 1, max_seq_len, ws=ws[0])
        o_fused = Q.dgq_append_decode(params, ktok, vtok, dpos, dq, dtable, caches[1], max_seq_len, ws=ws[1])
        torch.cuda.synchronize()
        assert torch.equal(o_sep, o_fused), f"step {s}: fused output differs"
        assert torch.equal(caches[0].status, caches[1].status), f"step {s}: status differs"
    _same_cache(caches[0], caches[1], table, lens + steps, p)
    return caches[1].read_status()


def test_fused_clamped_length_matches_separate():
    """A length past max_seq_len: the decode attends to max_seq_len tokens (counted in status[2])
    while the append still places the token at its position; the new token then lies outside
    every wave's tokens and a fixed wave writes it, as in the append kernel."""
    cfg = dgq_data.get_config(2, batch=2, seq_len=120, append_steps=8)
    lens = np.asarray(dgq_data.batch_kv(cfg, 45)[3], np.int64)
    max_seq_len = int(lens.max()) + 3
    H.say("fused clamped length", lens.tolist(), max_seq_len)
    st = _fused_vs_separate(cfg, 45, 8, max_seq_len)
    assert st["inconsistencies"] > 0, st


def test_fused_inconsistent_state_skipped_like_append():
    """An append state that does not fit the new position: nothing is appended for that (sequence,
    head) in either path, status[2] counts it once per step, and every other head is unchanged."""
    cfg = dgq_data.get_config(5, batch=2, seq_len=150, append_steps=20)
    H.say("fused inconsistent append state")
    st = _fused_vs_separate(cfg, 46, 20, 150 + 20, corrupt=(1, 3))
    assert st["inconsistencies"] == 20 and st["clamped_appends"] == 0, st


def test_fused_fills_largest_segment_table():
    """The fused step on a head whose appended blocks each take a row of their own, through the
    largest segment table (64 rows) and on into the table-full clamp."""
    from test_gpu_append import growing_values
    cfg = dgq_data.get_config(1, batch=1, seq_len=64, append_steps=1100, block_size=16)
    H.say("fused step through a full 64-row segment table")
    params = H.params_for(cfg, max_segments=8, seg_capacity=64)
    run_fused(cfg, 7, 1100, (0, 550, 1099), params=params, data=growing_values(cfg, 64, 1100, 7))
