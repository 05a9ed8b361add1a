"""dgq_compress on the GPU against the oracle: segment starts and min/max bit-exact, scales
bit-exact, codes equal (the bound allows 1 LSB on <= 1e-4 of elements), boundary bits, append
state; then decode of the GPU-compressed cache against the oracle."""

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
import paged_layout as PL
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q

pytestmark = pytest.mark.gpu


def compress_and_check(cfg, seed, params=None, k=None, v=None, cu=None, lens=None, check_decode=True,
                       spare_blocks=0):
    if k is None:
        k, v, cu, lens, dk, dv = H.upload_batch(cfg, seed)
    else:
        dk, dv = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    lens = np.asarray(lens, np.int64)
    if params is None:
        params = H.params_for(cfg)
    p = params.c
    table, nblk = dgq_data.block_tables(cfg, seed, lens_total=np.maximum(lens, 1), spare_blocks=spare_blocks)
    cache = Q.DGQCache(params, nblk, cfg.batch)
    max_len = int(max(lens.max(), 1))
    dtable = torch.from_numpy(table).cuda()
    Q.dgq_compress(params, dk, dv, torch.from_numpy(np.asarray(cu, np.int32)).cuda(), dtable, cache,
                   max_len, int(cu[-1]))
    torch.cuda.synchronize()
    status = cache.status.cpu().numpy()
    assert status[2] == 0 and status[1] == 0, status

    heads = {}
    for b in range(cfg.batch):
        for h in range(cfg.hkv):
            kk = k[cu[b]:cu[b + 1], h]
            vv = v[cu[b]:cu[b + 1], h]
            heads[(b, h)] = O.compress_head(kk, vv, p.max_segments, p.tau, p.min_var, params.length_aware,
                                            H.fmt_of(params))
    H.compare_segments(cache, heads, cfg.batch, cfg.hkv)
    bits = H.identifier_bits(cache, table, lens)
    tails = cache.tail.cpu().numpy()
    for b in range(cfg.batch):
        for h in range(cfg.hkv):
            hc = heads[(b, h)]
            kc, vc = H.read_codes(cache, table, b, h, hc.length)
            H.compare_codes(kc, hc.kcodes, f"K codes b{b} h{h}")
            H.compare_codes(vc, hc.vcodes, f"V codes b{b} h{h}")
            if params.marker:
                H.compare_markers(kc, hc.kcodes, f"K markers b{b} h{h}")
                H.compare_markers(vc, hc.vcodes, f"V markers b{b} h{h}")
            got_bits = PL.gather_bits(bits, table[b], h, hc.length, p.block_size)
            assert np.array_equal(got_bits, hc.bits), (b, h)
            # append state: r0 = length, ring = moments of the last min(16, L) tokens
            tl = tails[b, h]
            assert tl[0] == hc.length and tl[1] == min(16, hc.length) and tl[2] == 0
            a_t, b_t = O.token_moments(k[cu[b]:cu[b + 1], h])
            rl = tl[1]
            assert np.array_equal(tl[4:4 + rl], a_t[hc.length - rl:])
            assert np.array_equal(tl[20:52].view(np.int64)[:rl], b_t[hc.length - rl:])
    if check_decode:
        q16 = dgq_data.queries(cfg, seed)
        out = Q.paged_decode_attn_int8(params, torch.from_numpy(q16).cuda(), cache, dtable,
                                       torch.from_numpy(lens.astype(np.int32)).cuda(), max_len)
        ref = H.oracle_decode(q16, heads, lens, cfg.hkv, cfg.group)
        err = H.rel_err_rows(out.cpu().numpy(), ref)
        print(f"decode after GPU compress: max rel err {err:.3e}")
        assert err <= 2e-3
    return cache, heads, table


CASES = [
    ("tiny", 1, {}, 0),
    ("llama_bs16", 2, dict(batch=2, seq_len=1500), 1),
    ("long_bs64_outliers", 3, dict(seq_len=4100), 2),
    ("mha_g1_mixed", 4, dict(batch=6, seq_len=900, min_len=1), 3),
    ("stream_prefix_bs64", 5, dict(batch=3, seq_len=200, append_steps=0), 4),
    ("d64_g2", 1, dict(hq=4, block_size=64, seq_len=1111, batch=2), 5),
    ("llama_bs32", 2, dict(batch=2, seq_len=1300, block_size=32), 6),
    ("d64_g2_bs32_ragged", 4, dict(batch=5, hkv=2, hq=4, head_dim=64, block_size=32, seq_len=1500, min_len=1), 7),
]


@pytest.mark.parametrize("name,cid,over,seed", CASES, ids=[c[0] for c in CASES])
def test_compress_matches_oracle(name, cid, over, seed):
    cfg = dgq_data.get_config(cid, **over)
    H.say("compress", name, over)
    compress_and_check(cfg, seed)


@pytest.mark.parametrize("max_segments,tau", [(1, 2.0), (2, 2.0), (8, 1.0), (5, 1.5)])
def test_compress_segment_policies(max_segments, tau):
    cfg = dgq_data.get_config(2, batch=2, seq_len=2000)
    H.say("compress policy", max_segments, tau)
    compress_and_check(cfg, 12, params=H.params_for(cfg, max_segments=max_segments, tau=tau))


POLICY_CASES = [
    ("mixed_lengths_capped", 4, dict(batch=6, seq_len=5000, min_len=300), True, 0.0),
    ("floor_1e-3", 2, dict(batch=2, seq_len=3000), False, 1e-3),
    ("floor_0.02_capped", 2, dict(batch=2, seq_len=3000), True, 0.02),
    ("long_path_floor_capped", 3, dict(seq_len=20000), True, 5e-3),
    ("d64_floor_capped", 1, dict(hq=4, block_size=64, seq_len=3000, batch=2), True, 0.01),
]


@pytest.mark.parametrize("name,cid,over,length_aware,min_var", POLICY_CASES, ids=[c[0] for c in POLICY_CASES])
def test_compress_length_cap_and_variance_floor(name, cid, over, length_aware, min_var):
    """The segment-count policies of the DGQ article (3.2: length-aware cap; 5.3: variance floor)
    on the short-sequence (fused) and long-sequence (tiled) selection paths."""
    cfg = dgq_data.get_config(cid, **over)
    H.say("compress policies", name, over, length_aware, min_var)
    params = H.params_for(cfg, length_aware=length_aware, min_var=min_var)
    cache, heads, _ = compress_and_check(cfg, 21, params=params)
    counts = np.bincount([len(hc.segs) for hc in heads.values()], minlength=6)
    print(f"{name}: segments per head {counts.tolist()}")


def test_compress_beyond_lds_tile_limit():
    """A 1.1M-token sequence (4,297 tiles of 256 candidates): more tile maxima than the selection
    keeps in LDS (4,096), so its greedy rounds read and update them in the workspace, and more tiles
    than one pass of its range reduction covers (1,024 per pass).  Segments, codes and bits against
    the oracle, then a decode over the whole sequence."""
    cfg = dgq_data.get_config(1, seq_len=1_100_000, block_size=64)
    assert (cfg.seq_len - 16) // 256 + 1 > 4096
    H.say("compress beyond the LDS tile limit", cfg.seq_len)
    params = H.params_for(cfg, max_segments=8, tau=1.5)
    _, heads, _ = compress_and_check(cfg, 51, params=params)
    nseg = [len(hc.segs) for hc in heads.values()]
    print(f"segments per head {nseg}")
    assert max(nseg) > 2


@pytest.mark.parametrize("marker", [False, True], ids=["bitmap", "marker"])
def test_compress_long_path_seven_cuts(marker):
    """The tiled selection with eight segments (tau = 1 takes a cut every round, as no score is
    below 1): seven cuts per head, some sharing a 256-token tile, so the range reduction's
    cut-tile groups span two waves and skip tiles an earlier cut already took."""
    cfg = dgq_data.get_config(3, seq_len=12000)
    H.say("compress long path seven cuts", marker)
    params = H.params_for(cfg, max_segments=8, tau=1.0, marker=marker)
    _, heads, _ = compress_and_check(cfg, 61, params=params)
    assert all(len(hc.segs) == 8 for hc in heads.values())


def test_compress_long_batch_with_empty_and_tiny_sequences():
    """The tiled selection (the batch's longest sequence has 9,000 tokens) on a batch that also
    holds an empty and a 5-token sequence: no tiles, and fewer tokens than one window."""
    cfg = dgq_data.get_config(3, batch=3, hkv=2, hq=8, seq_len=9000)
    k, v, cu, _ = dgq_data.batch_kv(cfg, 71)
    lens = np.array([0, 9000, 5], np.int64)
    kk = np.concatenate([k[cu[b]:cu[b] + lens[b]] for b in range(3)])
    vv = np.concatenate([v[cu[b]:cu[b] + lens[b]] for b in range(3)])
    cu2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    H.say("compress long batch with empty and tiny sequences")
    _, heads, _ = compress_and_check(cfg, 71, k=kk, v=vv, cu=cu2, lens=lens)
    assert len(heads[(0, 0)].segs) == 0 and len(heads[(2, 1)].segs) == 1


MARKER_CASES = [
    ("tiny", 1, {}),
    ("llama_bs16", 2, dict(batch=2, seq_len=1500)),
    ("long_path_bs64_outliers", 3, dict(seq_len=12000)),
    ("mha_g1_mixed", 4, dict(batch=5, seq_len=900, min_len=1)),
    ("d64_g2_bs64", 1, dict(hq=4, block_size=64, seq_len=1111, batch=2)),
    ("llama_bs32", 2, dict(batch=2, seq_len=900, block_size=32)),
    ("long_path_bs32", 3, dict(seq_len=9000, block_size=32)),
]


@pytest.mark.parametrize("name,cid,over", MARKER_CASES, ids=[c[0] for c in MARKER_CASES])
def test_compress_marker_format(name, cid, over):
    """The marker format (DGQ article 3.2): 254-level codes with the identifier in the key bytes,
    no bit tensor; codes, markers, scales and the read-back identifier against the oracle, then
    decode; on the fused short-sequence and the tiled long-sequence selection paths."""
    cfg = dgq_data.get_config(cid, **over)
    H.say("compress marker format", name, over)
    cache, heads, _ = compress_and_check(cfg, 31, params=H.params_for(cfg, marker=True))
    assert cache.bits is None
    assert sum(len(hc.segs) - 1 for hc in heads.values()) > 0


def _custom(cfg, seqs):
    """Pack explicit per-(b, h) arrays [L][D] into token-major K/V."""
    lens = np.array([s[0].shape[0] for s in seqs], np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    k = np.zeros((int(cu[-1]), cfg.hkv, cfg.head_dim), np.float16)
    v = np.zeros_like(k)
    for b, (kk, vv) in enumerate(seqs):
        k[cu[b]:cu[b + 1]] = kk
        v[cu[b]:cu[b + 1]] = vv
    return k, v, cu, lens


@pytest.mark.parametrize("marker", [False, True], ids=["bitmap", "marker"])
def test_compress_edge_cases(marker):
    """Lengths 0, 1, 31, 32, 33; constant runs (exact reconstruction); subnormals and signed
    zeros; exact score ties; values beyond the statistics clamp; in both identifier formats."""
    cfg = dgq_data.get_config(1, batch=10, hq=2)
    rng = np.random.default_rng(0)
    d = cfg.head_dim
    seqs = []
    for length in (0, 1, 31, 32, 33):
        x = (rng.standard_normal((length, 2, d)) * 0.2).astype(np.float16)
        seqs.append((x, (x * 0.5).astype(np.float16)))
    # constant run inside Gaussian data
    x = (rng.standard_normal((200, 2, d)) * 0.3).astype(np.float16)
    x[64:128] = np.float16(0.0)
    y = x.copy()
    y[64:128] = np.float16(-0.125)
    seqs.append((x, y))
    # a run of -0 keys and mixed +-0 values: ranges stored as +0 bit patterns
    x = (rng.standard_normal((200, 2, d)) * 0.3).astype(np.float16)
    x[64:128] = np.float16(-0.0)
    y = (rng.standard_normal((200, 2, d)) * 0.3).astype(np.float16)
    y[64:128] = np.where(rng.random((64, 2, d)) < 0.5, np.float16(-0.0), np.float16(0.0)).astype(np.float16)
    seqs.append((x, y))
    # subnormals, signed zeros
    x = (rng.standard_normal((150, 2, d)) * 1e-5).astype(np.float16)
    x[::7] = np.float16(-0.0)
    seqs.append((x, (-x).astype(np.float16)))
    # periodic data: many equal scores (ties broken by the smallest t)
    x = np.zeros((160, 2, d), np.float16)
    x[::2] = np.float16(0.5)
    x[40:80] = np.float16(0.0)
    x[120:] = np.float16(0.25)
    seqs.append((x, x.copy()))
    # beyond the +-32 statistics clamp, up to the fp16 limits
    x = (rng.standard_normal((100, 2, d)) * 40).astype(np.float16)
    x[50, 0, :4] = np.array([65504, -65504, 1000, -3000], np.float16)
    seqs.append((x, (x / 3).astype(np.float16)))
    k, v, cu, lens = _custom(cfg, seqs)
    H.say("compress edge cases", marker)
    cache, heads, table = compress_and_check(cfg, 13, k=k, v=v, cu=cu, lens=lens,
                                             params=H.params_for(cfg, marker=marker))
    hc = heads[(5, 0)]
    assert hc.starts[1:3] == [64, 128] or 64 in hc.starts
    if marker:
        # the constant run is exact on the GPU side too, its marker byte included
        kc, vc = H.read_codes(cache, table, 5, 0, hc.length)
        assert np.array_equal(kc[64:128], hc.kcodes[64:128]) and np.array_equal(vc[64:128], hc.vcodes[64:128])


def test_compress_repeatable():
    """Integer statistics make the result independent of scheduling: two runs are identical."""
    cfg = dgq_data.get_config(2, batch=2, seq_len=1024)
    k, v, cu, lens, dk, dv = H.upload_batch(cfg, 21)
    params = H.params_for(cfg)
    table, nblk = dgq_data.block_tables(cfg, 21)
    dtable = torch.from_numpy(table).cuda()
    dcu = torch.from_numpy(cu).cuda()
    outs = []
    for _ in range(2):
        cache = Q.DGQCache(params, nblk, cfg.batch)
        Q.dgq_compress(params, dk, dv, dcu, dtable, cache, 1024, int(cu[-1]))
        torch.cuda.synchronize()
        outs.append((cache.k_pool.cpu(), cache.v_pool.cpu(), cache.segs.cpu(), cache.bits.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_compress_strided_inputs():
    """The input is addressed through (stride_tok, stride_head): a head-major [H][T][D] tensor
    (passed as its [T][H][D] view) and the K and V slices of a fused QKV projection output
    [T][Hq + 2 Hkv][D] compress to the same bytes as contiguous token-major K and V, and the
    contiguous result matches the oracle's segments."""
    cfg = dgq_data.get_config(2, batch=3, seq_len=700)
    k, v, cu, lens, dk, dv = H.upload_batch(cfg, 33)
    params = H.params_for(cfg)
    table, nblk = dgq_data.block_tables(cfg, 33)
    dtable = torch.from_numpy(table).cuda()
    dcu = torch.from_numpy(cu).cuda()
    total = int(cu[-1])

    def run(kk, vv):
        cache = Q.DGQCache(params, nblk, cfg.batch)
        Q.dgq_compress(params, kk, vv, dcu, dtable, cache, cfg.seq_len, total)
        torch.cuda.synchronize()
        assert cache.status.cpu().numpy()[1:3].tolist() == [0, 0]
        return cache

    ref = run(dk, dv)
    heads = {(b, h): O.compress_head(k[cu[b]:cu[b + 1], h], v[cu[b]:cu[b + 1], h])
             for b in range(cfg.batch) for h in range(cfg.hkv)}
    H.compare_segments(ref, heads, cfg.batch, cfg.hkv)

    # head-major storage, handed over as a [T][H][D] view (stride_tok = D, stride_head = T * D)
    kh = dk.permute(1, 0, 2).contiguous()
    vh = dv.permute(1, 0, 2).contiguous()
    got_hm = run(kh.permute(1, 0, 2), vh.permute(1, 0, 2))
    # fused QKV output: K and V are head slices of one [T][Hq + 2 Hkv][D] tensor; the query part
    # holds a large value that would show up in the ranges if it were read
    qkv = torch.full((total, cfg.hq + 2 * cfg.hkv, cfg.head_dim), 30.0, dtype=torch.float16, device="cuda")
    qkv[:, cfg.hq:cfg.hq + cfg.hkv] = dk
    qkv[:, cfg.hq + cfg.hkv:] = dv
    got_qkv = run(qkv[:, cfg.hq:cfg.hq + cfg.hkv], qkv[:, cfg.hq + cfg.hkv:])
    for got in (got_hm, got_qkv):
        for name in ("k_pool", "v_pool", "segs", "nseg", "bits", "tail"):
            assert torch.equal(getattr(got, name), getattr(ref, name)), name


@pytest.mark.parametrize("max_segments", [5, 8])
def test_compress_ragged_batch_tile_map(max_segments):
    """A ragged batch whose padded grid (longest sequence's tiles for every sequence) is far above
    its real tiles, so the two passes over the input run on the list of real tiles: empty, 1-, 63-,
    64- and 65-token sequences beside 4000-token ones, against the oracle (segments, codes, bits,
    append state, decode).  max_segments 5 takes the 4096-token selection, 8 the 8192-token one."""
    lens = np.array([0, 1, 63, 64, 65, 4000, 17, 0, 128, 3999, 2, 640, 33, 0, 4000, 100], np.int64)
    cfg = dgq_data.get_config(4, batch=len(lens), hkv=2, hq=4, head_dim=64, seq_len=4000, min_len=1)
    rng = np.random.default_rng(55)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    sig = rng.choice([0.03, 0.15, 0.47], size=(total, cfg.hkv, 1))
    k = (rng.standard_normal((total, cfg.hkv, cfg.head_dim)) * sig).astype(np.float16)
    v = (rng.standard_normal((total, cfg.hkv, cfg.head_dim)) * sig).astype(np.float16)
    padded = -(-int(lens.max()) // 64) * len(lens)
    assert 5 * (-(-total // 64) + len(lens)) < 4 * padded      # the tile-list path is the one taken
    H.say("compress ragged tile map", lens.tolist(), max_segments)
    compress_and_check(cfg, 56, params=H.params_for(cfg, max_segments=max_segments), k=k, v=v, cu=cu, lens=lens)
