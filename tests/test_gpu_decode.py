"""paged_decode_attn_int8 on the GPU against the oracle, fed with the oracle's own compression
(so decode is checked independently of the GPU compressor)."""

import math

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q

pytestmark = pytest.mark.gpu

TOL = 2e-3   # max relative error of the attention output in fp32


def _heads_for(cfg, seed, lens):
    heads = {}
    for b in range(cfg.batch):
        for h in range(cfg.hkv):
            k, v = dgq_data.head_kv(cfg, seed, 0, b, h, int(lens[b]))
            heads[(b, h)] = O.compress_head(k[:lens[b]], v[:lens[b]])
    return heads


def _run(cfg, seed, lens, heads=None, table=None, num_blocks=None, fill=None, seg_capacity=16):
    lens = np.asarray(lens, np.int64)
    if heads is None:
        heads = _heads_for(cfg, seed, lens)
    if table is None:
        table, num_blocks = dgq_data.block_tables(cfg, seed, lens_total=np.maximum(lens, 1))
    params = H.params_for(cfg, seg_capacity=seg_capacity)
    cache = H.cache_from_oracle(params, heads, table, num_blocks, cfg.batch, fill=fill)
    q16 = dgq_data.queries(cfg, seed)
    max_len = int(max(lens.max(), 1))
    out = Q.paged_decode_attn_int8(params, torch.from_numpy(q16).cuda(), cache,
                                   torch.from_numpy(table).cuda(), torch.from_numpy(lens.astype(np.int32)).cuda(),
                                   max_len)
    torch.cuda.synchronize()
    assert int(cache.status[2].item()) == 0
    return out.cpu().numpy(), H.oracle_decode(q16, heads, lens, cfg.hkv, cfg.group), heads, q16


CASES = [
    ("tiny", 1, {}, 0, None),
    ("llama_bs16_g4_ragged", 2, dict(batch=2, seq_len=1000), 1, None),
    ("long_bs64_g4_outliers", 3, dict(seq_len=3000), 2, None),
    ("mha_g1_bs16_mixed", 4, dict(batch=5, seq_len=700, min_len=1), 3, None),
    ("stream_bs64_g4", 5, dict(batch=3, seq_len=300, append_steps=0), 4, None),
    ("d64_g2_bs64", 1, dict(hq=4, block_size=64, seq_len=333), 5, None),
    ("llama_bs32_g4", 2, dict(batch=3, seq_len=1111, block_size=32), 7, None),
    ("mha_g1_bs32_mixed", 4, dict(batch=4, seq_len=600, min_len=1, block_size=32, hkv=4, hq=4), 8, None),
    ("short_and_empty", 2, dict(batch=4, seq_len=70), 6, [70, 1, 0, 17]),
]


@pytest.mark.parametrize("name,cid,over,seed,lens", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle(name, cid, over, seed, lens):
    cfg = dgq_data.get_config(cid, **over)
    if lens is None:
        lens = dgq_data.seq_lens(cfg, seed)
    H.say("decode", name, dict(over), "lens", list(np.asarray(lens)[:8]))
    out, ref, _, _ = _run(cfg, seed, lens)
    err = H.rel_err_rows(out, ref)
    print(f"{name}: max rel err vs oracle {err:.3e}")
    assert err <= TOL


def test_decode_many_segments_any_positions():
    """Eleven segments starting anywhere (mid-block, adjacent, last token): the per-token
    segment lookup path."""
    cfg = dgq_data.get_config(2, batch=1, seq_len=700)
    k, v = dgq_data.head_kv(cfg, 7, 0, 0, 0, 700)
    starts = [0, 5, 17, 64, 65, 100, 250, 251, 400, 640, 699]
    heads = {}
    for h in range(cfg.hkv):
        kk, vv = dgq_data.head_kv(cfg, 7, 0, 0, h, 700)
        segs = O.segment_params(kk, vv, starts)
        heads[(0, h)] = O.HeadCompressed(700, segs, O.encode_by_segment(kk, segs, "k"),
                                         O.encode_by_segment(vv, segs, "v"), O.boundary_bits(starts, 700))
    H.say("decode many segments")
    out, ref, _, _ = _run(cfg, 7, [700], heads=heads)
    assert H.rel_err_rows(out, ref) <= TOL


def test_decode_independent_of_physical_blocks_and_unused_bytes():
    """The same logical cache under two block permutations, and with unused pool bytes zero or
    random, gives bit-identical outputs."""
    cfg = dgq_data.get_config(2, batch=2, seq_len=500)
    lens = [500, 333]
    heads = _heads_for(cfg, 9, np.array(lens))
    t1, n = dgq_data.block_tables(cfg, 9, lens_total=np.array(lens), spare_blocks=7)
    rng = np.random.default_rng(1)
    perm = rng.permutation(n)
    t2 = np.where(t1 >= 0, perm[np.maximum(t1, 0)], -1).astype(np.int32)
    H.say("decode permutation invariance")
    o1, ref, _, _ = _run(cfg, 9, lens, heads=heads, table=t1, num_blocks=n, fill=0)
    o2, _, _, _ = _run(cfg, 9, lens, heads=heads, table=t2, num_blocks=n, fill=None)
    assert np.array_equal(o1, o2)
    assert H.rel_err_rows(o1, ref) <= TOL


def test_decode_vs_unquantized_fp16_reported():
    """Report (not gate) the error of quantized attention against fp16 attention."""
    cfg = dgq_data.get_config(2, batch=2, seq_len=2048)
    lens = dgq_data.seq_lens(cfg, 11)
    out, ref, heads, q16 = _run(cfg, 11, lens)
    exact = np.zeros_like(ref)
    for b in range(cfg.batch):
        for h in range(cfg.hkv):
            k, v = dgq_data.head_kv(cfg, 11, 0, b, h, int(lens[b]))
            g = cfg.group
            exact[b, h * g:(h + 1) * g] = O.decode_attention(q16[b, h * g:(h + 1) * g], k.astype(np.float64),
                                                             v.astype(np.float64))
    print(f"DGQ attention vs fp16 attention: max rel err {H.rel_err_rows(out, exact):.3e}; "
          f"oracle DGQ vs fp16 {H.rel_err_rows(ref, exact):.3e}")
    assert H.rel_err_rows(out, ref) <= TOL


@pytest.mark.parametrize("cid,over", [(2, dict(batch=4, seq_len=8192)), (3, dict(seq_len=32768))],
                         ids=["bs16_4x8192", "bs64_1x32768"])
def test_decode_split_merge_repeatable(cid, over):
    """Many workgroups per (sequence, head): the last one to finish merges the partials of the
    others.  Thirty calls on one workspace, alternating two query sets, give bit-identical outputs
    per query set that match the oracle: a merge that read a partial left by the previous call
    (the other query set) would not."""
    cfg = dgq_data.get_config(cid, **over)
    lens = dgq_data.seq_lens(cfg, 15)
    heads = _heads_for(cfg, 15, lens)
    table, nblk = dgq_data.block_tables(cfg, 15, lens_total=lens)
    params = H.params_for(cfg)
    cache = H.cache_from_oracle(params, heads, table, nblk, cfg.batch)
    qs = [dgq_data.queries(cfg, 15, 0, step) for step in (0, 1)]
    dqs = [torch.from_numpy(q).cuda() for q in qs]
    dt = torch.from_numpy(table).cuda()
    dl = torch.from_numpy(lens.astype(np.int32)).cuda()
    ws = Q.workspace(Q.decode_workspace_size(params, cfg.batch, int(lens.max())))
    H.say("decode split merge", cid, over)
    outs = [Q.paged_decode_attn_int8(params, dqs[i % 2], cache, dt, dl, int(lens.max()), ws=ws).clone()
            for i in range(30)]
    torch.cuda.synchronize()
    for i, o in enumerate(outs[2:], start=2):
        assert torch.equal(o, outs[i % 2]), i
    for i in (0, 1):
        ref = H.oracle_decode(qs[i], heads, lens, cfg.hkv, cfg.group)
        assert H.rel_err_rows(outs[i].cpu().numpy(), ref) <= TOL
    # the merge leaves its completion counters at zero
    assert int(ws[: cfg.batch * cfg.hkv * 4].view(torch.int32).abs().sum().item()) == 0


def test_decode_longest_workgroup_span():
    """The largest launch the plan makes: 65,536 chunks of 64 tokens in all (one kv head of
    4,194,304 tokens, head_dim 64, 64-token blocks permuted over the pool) gives every wave the
    most chunks a workgroup stages block ids for (64 per wave, 16,384 tokens per workgroup) and
    256 partitions to merge.  Random codes under five segments, against the oracle's float64
    attention over the same codes."""
    L = 1 << 22
    cfg = dgq_data.get_config(3, batch=1, hkv=1, hq=1, head_dim=64, block_size=64, seq_len=L, outlier_frac=0.0)
    rng = np.random.default_rng(91)
    starts = [0, 70001, 1500000, 2500017, 4000000]
    bounds = starts + [L]
    segs = []
    for j, s in enumerate(starts):
        lo_k, lo_v = -rng.uniform(0.1, 2.0), -rng.uniform(0.1, 2.0)
        segs.append(O.SegParams(s, np.float32(lo_k), np.float32(lo_k + rng.uniform(0.2, 4.0)),
                                np.float32(lo_v), np.float32(lo_v + rng.uniform(0.2, 4.0))))
    kc = rng.integers(-128, 128, (L, cfg.head_dim)).astype(np.int8)
    vc = rng.integers(-128, 128, (L, cfg.head_dim)).astype(np.int8)
    assert all(bounds[j] < bounds[j + 1] for j in range(len(starts)))
    hc = O.HeadCompressed(L, segs, kc, vc, O.boundary_bits(starts, L))
    H.say("decode longest span", L)
    out, ref, _, _ = _run(cfg, 92, [L], heads={(0, 0): hc})
    err = H.rel_err_rows(out, ref)
    print(f"4M-token decode: max rel err {err:.3e}")
    assert err <= 2e-3
