"""Checks that tie the CPU oracle to facts other than itself.

Each ``check_*`` function raises AssertionError when the oracle disagrees with a textbook or
library routine, a closed form, a different algorithm for the same definition, a high-precision
brute force, or a number the pages print.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutations.py`` plants plausible mistakes in the oracle (on the CPU) and checks that
some pin catches each one.
"""

from __future__ import annotations

import decimal
import math

import numpy as np

import dgq_data
from oracle import dgq_oracle as O

W = 16


# -- fixed point and moments ---------------------------------------------------------------------

def check_fixed_point():
    # values on the 2^-9 grid map to their integer exactly; halfway values go to the even neighbour
    k = np.arange(-4096, 4097, 37)
    x = (k / 512.0).astype(np.float16)
    assert np.array_equal(O.fixed_point(x), np.asarray(x, np.float64) * 512)
    half = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 7.5], dtype=np.float64) / 512.0
    got = O.fixed_point(half.astype(np.float16))
    assert list(got) == [0, 2, 2, 0, -2, 8], got
    # the statistics clamp at +-32
    big = np.array([40.0, -1000.0, 32.0, -32.0, 65504.0], dtype=np.float16)
    assert list(O.fixed_point(big)) == [16384, -16384, 16384, -16384, 16384]
    # -0 is +0
    assert O.fixed_point(np.array([-0.0], np.float16))[0] == 0


def check_window_q_against_variance(seed=0):
    """Q(s) / N^2 is the population variance of the window's fixed-point values (numpy.var)."""
    rng = np.random.default_rng(seed)
    for d in (4, 8, 64):
        length = 60
        x = (rng.standard_normal((length, d)) * rng.uniform(0.02, 3.0)).astype(np.float16)
        a, b = O.token_moments(x)
        q = O.window_q(a, b, d)
        assert len(q) == length - W + 1
        n = O.fixed_point(x).astype(np.float64)
        big_n = W * d
        for s in range(len(q)):
            ref = np.var(n[s:s + W]) * big_n * big_n
            assert abs(q[s] - ref) <= 1e-9 * max(1.0, ref), (d, s, q[s], ref)
    # exact closed forms: a constant window has Q = 0; a window of +-v halves has Q = N^2 v^2
    d = 8
    const = np.full((W, d), 0.25, np.float16)
    a, b = O.token_moments(const)
    assert O.window_q(a, b, d)[0] == 0
    pm = np.full((W, d), 0.5, np.float16)
    pm[::2] = -0.5
    a, b = O.token_moments(pm)
    v = 0.5 * 512
    assert O.window_q(a, b, d)[0] == (W * d) ** 2 * v * v


def check_scores_closed_form():
    # constant data: every candidate scores exactly 1
    x = np.full((64, 8), 0.1, np.float16)
    a, b = O.token_moments(x)
    sc = O.change_scores(O.window_q(a, b, 8), 64)
    assert len(sc) == 64 - 2 * W + 1 and np.all(sc == 1.0)
    # zeros then +-v rows from t = 40: the candidate at 40 sees Q = 0 on the left and the full
    # two-valued window on the right
    x = np.zeros((96, 8), np.float16)
    x[40:] = 0.5
    x[41::2] = -0.5
    a, b = O.token_moments(x)
    sc = O.change_scores(O.window_q(a, b, 8), 96)
    full = (W * 8) ** 2 * 256.0 ** 2
    assert sc[40 - W] == full + 1.0
    assert int(np.argmax(sc)) + W == 40


# -- selection -----------------------------------------------------------------------------------

def nms_twin(scores, max_segments, tau):
    """Greedy non-maximum suppression in sorted order: walk candidates by (-score, t) and keep one
    if it is far enough from every kept one.  A different algorithm with the same definition."""
    order = sorted(range(len(scores)), key=lambda i: (-scores[i], i))
    kept = []
    for i in order:
        if len(kept) == max_segments - 1:
            break
        if any(abs(i - j) <= W - 1 for j in kept):
            continue
        if kept and not scores[i] >= tau:
            break
        kept.append(i)
    return sorted(W + i for i in kept)


def check_selection_twin(seed=0, trials=300):
    rng = np.random.default_rng(seed)
    for trial in range(trials):
        n = int(rng.integers(1, 200))
        # integer-valued scores give many ties; a few trials use heavy ties
        hi = 3 if trial % 3 == 0 else 50
        scores = rng.integers(1, hi, n).astype(np.float64)
        if trial % 5 == 0:
            scores = rng.uniform(1.0, 4.0, n)
        for max_seg in (1, 2, 3, 5, 8):
            for tau in (1.0, 2.0, 2.5):
                got = O.select_cuts(scores, max_seg, tau)
                ref = nms_twin(list(scores), max_seg, tau)
                assert got == ref, (trial, max_seg, tau, got, ref)


def check_step_change_cut():
    """Constructed data whose only change point is known: the cut lands on it exactly."""
    for t0 in (32, 77, 100, 150):
        x = np.zeros((200, 16), np.float16)
        x[t0:] = 0.25
        x[t0 + 1::2] = -0.25
        starts = O.segment_starts(x, max_segments=2)
        assert starts == [0, t0], (t0, starts)


def check_segment_invariants(cid=2, seqs=2, length=4096):
    cfg = dgq_data.get_config(cid, seq_len=length, batch=seqs)
    counts = set()
    for b in range(seqs):
        for h in range(cfg.hkv):
            k, v = dgq_data.head_kv(cfg, 0, 0, b, h, length)
            starts = O.segment_starts(k)
            assert starts[0] == 0
            cuts = starts[1:]
            assert 1 <= len(cuts) <= O.MAX_SEGMENTS - 1
            assert all(W <= c <= length - W for c in cuts)
            assert all(c2 - c1 >= W for c1, c2 in zip(cuts, cuts[1:]))
            counts.add(len(starts))
    # the number of segments follows the data (DGQ article 2.2: 3.8 vs 2.1 groups on average)
    assert len(counts) >= 2, counts
    # short sequences: one segment; empty: none
    assert O.segment_starts(np.zeros((31, 8), np.float16)) == [0]
    assert O.segment_starts(np.zeros((0, 8), np.float16)) == []


def check_tiny_recovery(seed=0):
    """Tiny config: three sigmas from {0.03, 0.15, 0.47} (every ratio >= 3.1); each true
    boundary is found within W/2 tokens."""
    cfg = dgq_data.get_config(1)
    for h in range(cfg.hkv):
        k, _ = dgq_data.head_kv(cfg, seed, 0, 0, h, cfg.seq_len)
        _, true_cuts, _ = dgq_data.head_profile(cfg, seed, 0, 0, h, cfg.seq_len)
        starts = O.segment_starts(k)
        for c in true_cuts:
            assert min(abs(c - s) for s in starts[1:]) <= W // 2, (h, true_cuts, starts)


# -- parameters, bits, codes ---------------------------------------------------------------------

def _some_heads():
    cfg = dgq_data.get_config(2, seq_len=1024, batch=1)
    for h in range(3):
        k, v = dgq_data.head_kv(cfg, 3, 0, 0, h, 1024)
        yield k, v
    cfg3 = dgq_data.get_config(3, seq_len=2048, batch=1)
    k, v = dgq_data.head_kv(cfg3, 0, 0, 0, 0, 2048)
    yield k, v


def check_minmax_library():
    for k, v in _some_heads():
        hc = O.compress_head(k, v)
        bounds = hc.starts + [hc.length]
        for j, s in enumerate(hc.segs):
            sl = slice(bounds[j], bounds[j + 1])
            assert s.kmin == np.min(k[sl]).astype(np.float32) and s.kmax == np.max(k[sl]).astype(np.float32)
            assert s.vmin == np.min(v[sl]).astype(np.float32) and s.vmax == np.max(v[sl]).astype(np.float32)


def check_bits():
    for k, v in _some_heads():
        hc = O.compress_head(k, v)
        assert hc.bits.shape == (hc.length,)                  # 1 bit per token per head
        assert int(hc.bits.sum()) == len(hc.segs) - 1
        assert list(np.flatnonzero(hc.bits)) == hc.starts[1:]
        assert not hc.bits[0]


def _nearest_code_ok(x16, codes, mn, scale):
    """Brute force over all 256 codes: the chosen one is (up to fp32 rounding) the nearest."""
    x = np.asarray(x16, np.float64).reshape(-1, 1)
    allc = np.arange(-128, 128, dtype=np.float64).reshape(1, -1)
    rec = (allc + 128.0) * np.float64(scale) + np.float64(mn)
    err = np.abs(x - rec)
    chosen = err[np.arange(len(x)), codes.reshape(-1).astype(np.int64) + 128]
    slack = 2.0 ** -20 * max(abs(float(mn)), abs(float(mn) + 255 * float(scale)), float(scale))
    return np.all(chosen <= err.min(axis=1) + slack)


def check_codes():
    for k, v in _some_heads():
        hc = O.compress_head(k, v)
        bounds = hc.starts + [hc.length]
        for j, s in enumerate(hc.segs):
            sl = slice(bounds[j], bounds[j + 1])
            for x16, codes, mn, mx, sc in ((k[sl], hc.kcodes[sl], s.kmin, s.kmax, s.kscale),
                                           (v[sl], hc.vcodes[sl], s.vmin, s.vmax, s.vscale)):
                assert codes.dtype == np.int8 and codes.shape == x16.shape
                if mx > mn:
                    # the range ends land on the end codes
                    assert codes.min() == -128 and codes.max() == 127
                    assert np.all(codes[np.asarray(x16, np.float32) == mn] == -128)
                    assert np.all(codes[np.asarray(x16, np.float32) == mx] == 127)
                    assert _nearest_code_ok(x16, codes, mn, sc)
                    rec = O.dequant(codes, mn, sc)
                    bound = 0.5 * float(sc) * (1 + 2.0 ** -10) + 2.0 ** -22 * max(abs(float(mn)), abs(float(mx)))
                    assert np.max(np.abs(rec - np.asarray(x16, np.float64))) <= bound
                # step = (max - min) / 255 in fp32
                assert abs(float(sc) * 255 - (float(mx) - float(mn))) <= 255 * 2.0 ** -23 * max(float(sc), 1e-30) + 2.0 ** -23 * abs(float(mx) - float(mn))


def check_constant_segment_exact():
    """A constant run inside Gaussian data: its own segment, reconstructed exactly."""
    rng = np.random.default_rng(5)
    k = (rng.standard_normal((160, 16)) * 0.3).astype(np.float16)
    v = (rng.standard_normal((160, 16)) * 0.3).astype(np.float16)
    k[64:128] = np.float16(0.0)
    v[64:128] = np.float16(-0.125)
    hc = O.compress_head(k, v, max_segments=3)
    assert hc.starts == [0, 64, 128], hc.starts
    seg = hc.segs[1]
    assert seg.kmin == seg.kmax == 0.0 and seg.vmin == seg.vmax == np.float32(-0.125)
    assert np.all(hc.kcodes[64:128] == -128) and np.all(hc.vcodes[64:128] == -128)
    assert np.all(hc.khat()[64:128] == 0.0) and np.all(hc.vhat()[64:128] == -0.125)


def check_dequant_closed_form():
    mn, mx = np.float32(-1.5), np.float32(2.25)
    sc = O.quant_scale(mn, mx)
    assert O.dequant(np.array([-128], np.int8), mn, sc)[0] == -1.5
    assert abs(O.dequant(np.array([127], np.int8), mn, sc)[0] - 2.25) <= 255 * 2.0 ** -23 * float(sc) * 2
    x = np.array([mn, mx, (mn + mx) / 2], np.float16)
    c = O.encode(x, mn, mx)
    assert list(c) == [-128, 127, 0] or list(c) == [-128, 127, -1]


# -- attention -----------------------------------------------------------------------------------

def _decimal_attention(q, k, v, scale):
    """Softmax attention in 50-digit decimal arithmetic (brute force, no numpy)."""
    ctx = decimal.Context(prec=50)
    dec = lambda t: ctx.create_decimal(repr(float(t)))  # noqa: E731
    out = []
    for g in range(q.shape[0]):
        s = [ctx.multiply(dec(scale), sum((dec(q[g, d]) * dec(k[t, d]) for d in range(k.shape[1])),
                                          decimal.Decimal(0))) for t in range(k.shape[0])]
        m = max(s)
        e = [ctx.exp(x - m) for x in s]
        z = sum(e, decimal.Decimal(0))
        out.append([float(sum((e[t] * dec(v[t, d]) for t in range(k.shape[0])), decimal.Decimal(0)) / z)
                    for d in range(k.shape[1])])
    return np.asarray(out)


def check_attention():
    rng = np.random.default_rng(11)
    length, d = 24, 8
    k = rng.standard_normal((length, d))
    v = rng.standard_normal((length, d))
    q = rng.standard_normal((3, d)).astype(np.float16)
    ref = _decimal_attention(q.astype(np.float64), k, v, 1 / math.sqrt(d))
    got = O.decode_attention(q, k, v)
    assert np.max(np.abs(got - ref)) <= 1e-12
    # q = 0: uniform weights, output = mean of values
    got0 = O.decode_attention(np.zeros((1, d), np.float16), k, v)
    assert np.allclose(got0[0], v.mean(axis=0), atol=1e-14, rtol=0)
    # one token: output = that value row
    got1 = O.decode_attention(q, k[:1], v[:1])
    assert np.allclose(got1, np.broadcast_to(v[0], got1.shape), atol=1e-15, rtol=0)
    # two tokens, closed form p0 = 1 / (1 + exp(s1 - s0))
    s = (k[:2] @ q[0].astype(np.float64)) / math.sqrt(d)
    p0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    got2 = O.decode_attention(q[:1], k[:2], v[:2])
    assert np.allclose(got2[0], p0 * v[0] + (1 - p0) * v[1], atol=1e-14, rtol=0)
    # order of the cached tokens does not matter
    perm = rng.permutation(length)
    assert np.allclose(O.decode_attention(q, k[perm], v[perm]), got, atol=1e-14, rtol=0)
    # empty cache
    assert np.all(O.decode_attention(q, k[:0], v[:0]) == 0)


# -- append --------------------------------------------------------------------------------------

def _prefix_and_tail(sig_tail, seed=1, length=256, tail=96, d=16):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((length + tail, d)) * 0.3).astype(np.float16)
    v = (rng.standard_normal((length + tail, d)) * 0.3).astype(np.float16)
    k[length:] = (rng.standard_normal((tail, d)) * sig_tail).astype(np.float16)
    v[length:] = (rng.standard_normal((tail, d)) * sig_tail).astype(np.float16)
    return k, v


def check_append_join(block_size=32):
    """Tail tokens with the same spread, kept inside the last segment's range: they join it, and
    their codes equal the direct encoding with that segment's range."""
    k, v = _prefix_and_tail(0.3, length=256, tail=3 * block_size)
    hc = O.compress_head(k[:256], v[:256])
    last = hc.segs[-1]
    k[256:] = np.clip(k[256:].astype(np.float32), 0.6 * last.kmin, 0.6 * last.kmax).astype(np.float16)
    v[256:] = np.clip(v[256:].astype(np.float32), 0.6 * last.vmin, 0.6 * last.vmax).astype(np.float16)
    st = O.AppendState(hc, k[:256], block_size)
    for t in range(256, k.shape[0]):
        before = [c.copy() for c in st.kcodes[:st.r0]]
        st.append(k[t], v[t])
        assert all(np.array_equal(a, b) for a, b in zip(before, st.kcodes[:len(before)]))
    snap = st.snapshot()
    assert len(snap.segs) == len(hc.segs)
    assert np.array_equal(snap.kcodes[256:], O.encode(k[256:], last.kmin, last.kmax))
    assert np.array_equal(snap.vcodes[256:], O.encode(v[256:], last.vmin, last.vmax))
    assert st.clamped == 0


def check_append_cut(block_size=32):
    """Tail tokens with 10x the spread: every tail block opens its own segment, whose range is
    numpy's min/max over that block's tokens, and whose codes are the direct encoding."""
    k, v = _prefix_and_tail(3.0, length=256, tail=3 * block_size)
    hc = O.compress_head(k[:256], v[:256])
    st = O.AppendState(hc, k[:256], block_size)
    for t in range(256, k.shape[0]):
        st.append(k[t], v[t])
    snap = st.snapshot()
    assert [s.start for s in snap.segs[len(hc.segs):]] == [256, 256 + block_size, 256 + 2 * block_size]
    for s in snap.segs[len(hc.segs):]:
        sl = slice(s.start, s.start + block_size)
        assert s.kmin == np.min(k[sl]).astype(np.float32) and s.kmax == np.max(k[sl]).astype(np.float32)
        assert s.vmin == np.min(v[sl]).astype(np.float32) and s.vmax == np.max(v[sl]).astype(np.float32)
        assert np.array_equal(snap.kcodes[sl], O.encode(k[sl], s.kmin, s.kmax))
        assert np.array_equal(snap.vcodes[sl], O.encode(v[sl], s.vmin, s.vmax))
        assert snap.bits[s.start]
    assert int(snap.bits.sum()) == len(snap.segs) - 1


def check_append_capacity():
    """With a full segment table the span joins the base segment, codes saturate at the end codes
    and the clamp counter counts every such append."""
    k, v = _prefix_and_tail(3.0, length=256, tail=64)
    hc = O.compress_head(k[:256], v[:256])
    st = O.AppendState(hc, k[:256], 32, seg_capacity=len(hc.segs))
    for t in range(256, 320):
        st.append(k[t], v[t])
    snap = st.snapshot()
    assert len(snap.segs) == len(hc.segs)
    assert st.clamped > 0
    last = hc.segs[-1]
    assert np.array_equal(snap.kcodes[256:], O.encode(k[256:], last.kmin, last.kmax))
    assert set(np.unique(snap.kcodes[256:])) & {-128, 127}


def check_append_matches_prefix_rule(seed=2):
    """Random streams: the decision never flips back within a span; frozen codes never change;
    bits and starts stay equivalent."""
    cfg = dgq_data.get_config(5, seq_len=256, append_steps=192, batch=1)
    for h in range(3):
        k, v = dgq_data.head_kv(cfg, seed, 0, 0, h, 256)
        hc = O.compress_head(k[:256], v[:256])
        st = O.AppendState(hc, k[:256], 64)
        own_seen = False
        for t in range(256, k.shape[0]):
            r0_before = st.r0
            frozen = [c.copy() for c in st.kcodes[:r0_before]]
            st.append(k[t], v[t])
            if st.r0 == r0_before:
                assert not (own_seen and not st.span_own)
                own_seen = st.span_own
            else:
                own_seen = False
            assert all(np.array_equal(a, b) for a, b in zip(frozen, st.kcodes[:r0_before]))
        snap = st.snapshot()
        assert list(np.flatnonzero(snap.bits)) == snap.starts[1:]
        # every token is encoded with the range of the segment that holds it
        assert np.array_equal(snap.kcodes, O.encode_by_segment(k, snap.segs, "k"))
        assert np.array_equal(snap.vcodes, O.encode_by_segment(v, snap.segs, "v"))


def check_append_from_empty(block_size=16):
    """An empty prefix: the first block is segment 0 (no boundary bit at token 0) with the range
    of its own tokens (numpy min/max); the next blocks are compared with it as usual."""
    rng = np.random.default_rng(8)
    k = (rng.standard_normal((3 * block_size, 8)) * 0.2).astype(np.float16)
    v = (rng.standard_normal((3 * block_size, 8)) * 0.2).astype(np.float16)
    st = O.AppendState(O.compress_head(k[:0], v[:0]), k[:0], block_size)
    for t in range(3 * block_size):
        st.append(k[t], v[t])
        snap = st.snapshot()
        first = snap.segs[0]
        assert first.start == 0 and not snap.bits[0]
        if t < block_size:
            assert len(snap.segs) == 1
            assert first.kmin == np.min(k[:t + 1]).astype(np.float32) and first.kmax == np.max(k[:t + 1]).astype(np.float32)
    assert list(np.flatnonzero(snap.bits)) == snap.starts[1:]
    assert np.array_equal(snap.kcodes, O.encode_by_segment(k, snap.segs, "k"))


# -- group-64 baseline -----------------------------------------------------------------------------

def check_group64():
    """Every (token, 64-channel group) is R8 with its own range: compared with the one-segment
    compression of that group alone (a different route through the oracle) and with numpy's
    min/max; nearest-code property; the reconstruction's closed forms at the two end codes and
    its per-element error bound (half a step plus the fp32 rounding of the range)."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((40, 128)) * 0.2).astype(np.float16)
    x[3, :64] = np.float16(0.5)                 # a constant group
    x[7, 64:] = (rng.standard_normal(64) * 0.2 + 3.0).astype(np.float16)   # a group far from 0
    codes, gmin, gmax = O.group64_compress(x)
    for t in range(40):
        for g in range(2):
            sl = slice(64 * g, 64 * g + 64)
            assert gmin[t, g] == np.min(x[t, sl]) and gmax[t, g] == np.max(x[t, sl])
            assert np.array_equal(codes[t, sl], O.encode(x[t, sl], np.float32(gmin[t, g]), np.float32(gmax[t, g])))
            sc = O.quant_scale(np.float32(gmin[t, g]), np.float32(gmax[t, g]))
            assert _nearest_code_ok(x[t, sl], codes[t, sl], np.float32(gmin[t, g]), sc)
    rec = O.group64_dequant(codes, gmin, gmax)
    assert np.all(rec[3, :64] == 0.5)
    mn = gmin.astype(np.float64)
    mx = gmax.astype(np.float64)
    step = (mx - mn) / 255.0
    for t in range(40):
        for g in range(2):
            sl = slice(64 * g, 64 * g + 64)
            bound = 0.5 * step[t, g] * (1 + 2.0 ** -10) + 2.0 ** -22 * max(abs(mn[t, g]), abs(mx[t, g]))
            assert np.max(np.abs(rec[t, sl] - x[t, sl].astype(np.float64))) <= bound, (t, g)
    # closed forms at the end codes: -128 is the group's minimum exactly, 127 its maximum up to
    # the fp32 rounding of (max - min) / 255; a code c sits c + 128 steps above the minimum
    ends = np.zeros((40, 128), np.int8)
    ends[:, 0::2] = -128
    ends[:, 1::2] = 127
    ends[:, 2] = 0
    rec = O.group64_dequant(ends, gmin, gmax)
    for t in range(40):
        for g in range(2):
            lo, hi = rec[t, 64 * g], rec[t, 64 * g + 1]
            assert lo == mn[t, g], (t, g, lo, mn[t, g])
            assert abs(hi - mx[t, g]) <= 2.0 ** -22 * max(abs(mx[t, g] - mn[t, g]), 2.0 ** -126), (t, g, hi, mx[t, g])
            if g == 0:
                mid = rec[t, 2]
                assert abs(mid - (mn[t, 0] + 128.0 * step[t, 0])) <= 2.0 ** -22 * abs(mx[t, 0] - mn[t, 0]) + 1e-300


def check_negative_zero():
    """R1: -0 is stored as +0, so a range is the same bit pattern whatever the order of the values.
    A segment made only of -0 keys stores +0 (bit pattern 0) as its key min and max; a run of mixed
    -0 and +0 values gives the same bits in any token order; a group-64 range over -0 is +0."""
    rng = np.random.default_rng(6)
    d = 16
    k = (rng.standard_normal((160, d)) * 0.3).astype(np.float16)
    v = (rng.standard_normal((160, d)) * 0.3).astype(np.float16)
    k[64:128] = np.float16(-0.0)
    v[64:128] = np.where(rng.random((64, d)) < 0.5, np.float16(-0.0), np.float16(0.0)).astype(np.float16)
    hc = O.compress_head(k, v, max_segments=3)
    assert hc.starts == [0, 64, 128], hc.starts
    seg = hc.segs[1]
    for val in (seg.kmin, seg.kmax, seg.vmin, seg.vmax):
        assert np.float32(val).view(np.uint32) == 0, (val, hex(int(np.float32(val).view(np.uint32))))
    perm = rng.permutation(64)
    v2 = v.copy()
    v2[64:128] = v[64:128][perm]
    hc2 = O.compress_head(k, v2, max_segments=3)
    for a, b in ((seg.vmin, hc2.segs[1].vmin), (seg.vmax, hc2.segs[1].vmax)):
        assert np.float32(a).view(np.uint32) == np.float32(b).view(np.uint32)
    assert np.all(hc.kcodes[64:128] == -128)
    x = np.zeros((2, 128), np.float16)
    x[:, :64] = np.float16(-0.0)
    _, gmin, gmax = O.group64_compress(x)
    assert np.all(gmin.view(np.uint16) == 0) and np.all(gmax.view(np.uint16) == 0), (gmin, gmax)


# -- segment-count policies (R12) ------------------------------------------------------------------

def check_length_cap():
    """The length-aware cap of the DGQ article, section 3.2, at the edges of its three ranges
    (values worked out by hand from the page's rule: 2 below 2048 tokens, 3 below 16384, else
    floor(log2(L / 1024)) + 2 capped at 5)."""
    for length, want in [(1, 2), (2047, 2), (2048, 3), (16383, 3), (16384, 5), (131072, 5)]:
        assert O.length_aware_cap(length) == want, (length, O.length_aware_cap(length), want)
    # four strong change points: the cap, not the data, limits the segment count
    rng = np.random.default_rng(12)
    for length, cap in [(1500, 2), (3000, 3)]:
        sig = np.repeat([0.02, 0.4, 0.02, 0.4, 0.02], length // 5 + 1)[:length]
        x = (rng.standard_normal((length, 64)) * sig[:, None]).astype(np.float16)
        free = O.segment_starts(x, max_segments=5)
        capped = O.segment_starts(x, max_segments=5, length_aware=True)
        assert len(free) == 5 and len(capped) == cap, (length, free, capped)
        assert capped == O.segment_starts(x, max_segments=cap)


def check_min_var_floor():
    """The variance floor (R12) against numpy's population variance of each window, and the
    low-variance change that the floor suppresses."""
    rng = np.random.default_rng(13)
    d, length = 64, 240
    sig = np.where(np.arange(length) < 120, 0.01, 0.03)
    x = (rng.standard_normal((length, d)) * sig[:, None]).astype(np.float16)
    n = O.fixed_point(x).astype(np.float64) / O.FP_SCALE
    a, b = O.token_moments(x)
    q = O.window_q(a, b, d)
    for min_var in (2e-4, 5e-4, 2e-3):
        sc = O.change_scores(q, length, O.variance_floor_q(min_var, d))
        for i, t in enumerate(range(W, length - W + 1)):
            vmax = max(np.var(n[t - W:t]), np.var(n[t:t + W]))
            assert (sc[i] == -np.inf) == (vmax < min_var), (min_var, t, vmax, sc[i])
    # both sides below the floor: no cut at all; floor between them: the change is still cut
    assert O.segment_starts(x, max_segments=2) == O.segment_starts(x, max_segments=2, min_var=5e-4)
    assert len(O.segment_starts(x, max_segments=2)) == 2
    assert O.segment_starts(x, max_segments=2, min_var=2e-3) == [0]
    # the append window test obeys the floor: a quiet span after a louder ring would be cut
    # without it (variance ratio 100) and joins with it
    pre = np.tile(np.array([[0.02], [-0.02]], np.float16), (32, d))            # 64 tokens, var 4e-4
    for min_var, want_cut in [(0.0, True), (1e-3, False)]:
        st = O.AppendState(O.compress_head(pre, pre, max_segments=1), pre, 64, 8, 2.0, min_var)
        for i in range(W):
            row = np.full(d, 0.002 if i % 2 == 0 else -0.002, np.float16)
            st.append(row, row)
        assert (len(st.segs) == 2) == want_cut, (min_var, len(st.segs))


# -- marker format (R13) -----------------------------------------------------------------------------

def _is_marker(codes):
    return (codes == -128) | (codes == 127)


def _nearest_code_marker_ok(x16, codes, mn, scale):
    """Brute force over the 254 data codes of the marker format: the chosen one is (up to fp32
    rounding) the nearest."""
    x = np.asarray(x16, np.float64).reshape(-1, 1)
    allc = np.arange(-127, 127, dtype=np.float64).reshape(1, -1)
    rec = (allc + 127.0) * np.float64(scale) + np.float64(mn)
    err = np.abs(x - rec)
    chosen = err[np.arange(len(x)), codes.reshape(-1).astype(np.int64) + 127]
    slack = 2.0 ** -20 * max(abs(float(mn)), abs(float(mn) + 253 * float(scale)), float(scale))
    return np.all(chosen <= err.min(axis=1) + slack)


def check_marker_format():
    """Same cuts and ranges as the bitmap format; data codes are the nearest of 254 levels; the only
    -128/127 bytes are the markers at (segment start, key channel 0), the identifier read back from
    them equals the bit tensor of the bitmap format, and each marker names the half of the range
    its element lies in."""
    for k, v in _some_heads():
        hb = O.compress_head(k, v)
        hm = O.compress_head(k, v, fmt="marker")
        assert hm.starts == hb.starts
        for sb, sm in zip(hb.segs, hm.segs):
            assert (sb.kmin, sb.kmax, sb.vmin, sb.vmax) == (sm.kmin, sm.kmax, sm.vmin, sm.vmax)
        assert not _is_marker(hm.vcodes).any()
        assert [tuple(int(i) for i in ix) for ix in zip(*np.nonzero(_is_marker(hm.kcodes)))] == \
            [(s, 0) for s in hm.starts[1:]]
        assert np.array_equal(O.marker_bits(hm.kcodes), hb.bits)
        khat, vhat = hm.khat(), hm.vhat()
        bounds = hm.starts + [hm.length]
        for j, s in enumerate(hm.segs):
            sl = slice(bounds[j], bounds[j + 1])
            for x16, codes, rec, mn, mx, sc, is_k in ((k[sl], hm.kcodes[sl], khat[sl], s.kmin, s.kmax, s.kscale, True),
                                                      (v[sl], hm.vcodes[sl], vhat[sl], s.vmin, s.vmax, s.vscale, False)):
                x = np.asarray(x16, np.float64)
                data = np.ones(codes.shape, bool)
                if is_k and j > 0:
                    data[0, 0] = False
                assert np.all((codes[data] >= -127) & (codes[data] <= 126))
                # step = (max - min) / 253 in fp32
                assert abs(float(sc) * 253 - (float(mx) - float(mn))) <= 253 * 2.0 ** -23 * max(float(sc), 1e-30) + 2.0 ** -23 * abs(float(mx) - float(mn))
                if not mx > mn:
                    assert np.all(rec == float(mn))
                    continue
                xf = np.asarray(x16, np.float32)
                assert np.all(codes[data & (xf == mn)] == -127) and np.all(codes[data & (xf == mx)] == 126)
                assert _nearest_code_marker_ok(x16[data], codes[data], mn, sc)
                bound = 0.5 * float(sc) * (1 + 2.0 ** -10) + 2.0 ** -22 * max(abs(float(mn)), abs(float(mx)))
                assert np.max(np.abs(rec[data] - x[data])) <= bound
                if is_k and j > 0:
                    frac = (x[0, 0] - float(mn)) / (float(mx) - float(mn))
                    marker = int(codes[0, 0])
                    assert (marker == 127 and frac >= 126 / 253) or (marker == -128 and frac <= 127 / 253), (frac, marker)
                    assert rec[0, 0] == (O.dequant(np.array([marker], np.int8), mn, sc, "marker")[0])
                    assert abs(rec[0, 0] - x[0, 0]) <= 0.5 * (float(mx) - float(mn)) + 2 * float(sc)


def check_marker_constant_segment():
    """A constant run in the marker format: its codes are the minimum's code -127 except the
    marker, and every byte, the marker included, reconstructs the constant exactly."""
    rng = np.random.default_rng(5)
    k = (rng.standard_normal((160, 16)) * 0.3).astype(np.float16)
    v = (rng.standard_normal((160, 16)) * 0.3).astype(np.float16)
    k[64:128] = np.float16(0.0)
    v[64:128] = np.float16(-0.125)
    hc = O.compress_head(k, v, max_segments=3, fmt="marker")
    assert hc.starts == [0, 64, 128], hc.starts
    assert hc.kcodes[64, 0] == -128 and np.all(hc.kcodes[64:128].reshape(-1)[1:] == -127)
    assert np.all(hc.vcodes[64:128] == -127)
    assert np.all(hc.khat()[64:128] == 0.0) and np.all(hc.vhat()[64:128] == -0.125)
    assert _is_marker(hc.kcodes[128, 0])


def check_marker_append(block_size=32):
    """Appends in the marker format take the same decisions as in the bitmap format; every span
    that opens a segment carries its marker, a joined span none; the whole sequence equals the
    direct marker-format encoding with the final segments; frozen codes never change."""
    for sig_tail, want_new in ((3.0, True), (0.3, False)):
        k, v = _prefix_and_tail(sig_tail, length=256, tail=3 * block_size)
        if not want_new:
            last = O.compress_head(k[:256], v[:256]).segs[-1]
            k[256:] = np.clip(k[256:].astype(np.float32), 0.6 * last.kmin, 0.6 * last.kmax).astype(np.float16)
            v[256:] = np.clip(v[256:].astype(np.float32), 0.6 * last.vmin, 0.6 * last.vmax).astype(np.float16)
        sb = O.AppendState(O.compress_head(k[:256], v[:256]), k[:256], block_size)
        sm = O.AppendState(O.compress_head(k[:256], v[:256], fmt="marker"), k[:256], block_size)
        for t in range(256, k.shape[0]):
            frozen = [c.copy() for c in sm.kcodes[:sm.r0]]
            sb.append(k[t], v[t])
            sm.append(k[t], v[t])
            assert all(np.array_equal(a, b) for a, b in zip(frozen, sm.kcodes[:len(frozen)]))
            snap = sm.snapshot()
            assert snap.starts == sb.snapshot().starts
            assert np.array_equal(O.marker_bits(snap.kcodes), snap.bits)
        snap = sm.snapshot()
        n_new = len(snap.segs) - len(O.compress_head(k[:256], v[:256]).segs)
        assert (n_new == 3) if want_new else (n_new == 0), n_new
        assert np.array_equal(snap.kcodes, O.encode_by_segment(k, snap.segs, "k", "marker"))
        assert np.array_equal(snap.vcodes, O.encode_by_segment(v, snap.segs, "v", "marker"))
        assert not _is_marker(snap.vcodes).any()


def check_marker_bytes():
    """The marker format stores no bit tensor: the cache is exactly 1 byte per element (plus the
    segment table), 1/8 byte per token per head below the bitmap format."""
    lens, hkv, d = [8192] * 16, 8, 128
    b = O.compressed_bytes(lens, hkv, d)
    m = O.compressed_bytes(lens, hkv, d, fmt="marker")
    assert m["codes"] == b["codes"] == 2 * 8192 * 16 * hkv * d
    assert m["bits"] == 0 and b["bits"] == 8192 * 16 * hkv / 8


ALL_CHECKS = [
    check_fixed_point, check_window_q_against_variance, check_scores_closed_form,
    check_selection_twin, check_step_change_cut, check_segment_invariants, check_tiny_recovery,
    check_minmax_library, check_bits, check_codes, check_constant_segment_exact,
    check_dequant_closed_form, check_attention, check_append_join, check_append_cut,
    check_append_capacity, check_append_matches_prefix_rule, check_append_from_empty, check_group64,
    check_negative_zero,
    check_length_cap, check_min_var_floor, check_marker_format, check_marker_constant_segment,
    check_marker_append, check_marker_bytes,
]
