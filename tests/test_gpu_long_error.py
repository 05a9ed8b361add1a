"""Error headroom of the decode at long context, where zero-mean values make the attention output
shrink like 1/sqrt(L) while the terms it is summed from do not.

Data: one kv head with four query heads (GQA 4), head_dim 128, 64-token blocks, five segments of
small spread (sigma 0.03-0.1) for keys and values, zero-mean values plus 1 % outliers at 8 sigma,
either of both signs (the long-context workload's model: the value range is symmetric and the
segment midpoints are near 0) or positive only with the values shifted to zero mean (each
segment's midpoint sits near 1.6 sigma, so the kernel's separately summed midpoint term is large
against the output).  Codes are the oracle's;
the expected output is the oracle's float64 attention over them.

Beside the measured error the test prints a first-order worst-case bound of the kernel's
arithmetic, computed from the same data (DGQ article 3.3 sizes: 131,072 tokens):
  * 24-bit query bytes: every score is off by at most sm * ks_t * amax(q) * 2^-22 * sum_d |c_td|;
  * 24-bit weights p_t * vs_t: each is off by at most vsmax * 2^-23, times sum_t |c_td|;
  * float32 sums of the exponentials, of the midpoint term and of the folded output, each at most
    n * 2^-24 times the sum of the magnitudes of its terms, n the depth of the summation tree
    (per-lane adds, chunk folds, lane and wave combines, partition merge);
all divided by l * |o|_inf, so the float32 part scales with the condition number
sum_t p_t (|mid_t| + vs_t |c_td|) / (l |o|_inf), which grows like sqrt(L) for zero-mean values."""

import math

import numpy as np
import pytest
import torch

import dgq_data
import gpu_helpers as H
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q

pytestmark = pytest.mark.gpu

TOL = 2e-3
U = 2.0 ** -24


def _head(L, one_sided, seed):
    rng = np.random.default_rng([seed, L, int(one_sided)])
    d = 128
    starts = [0] + sorted(int(x) for x in rng.choice(np.arange(64, L - 64, 64), 4, replace=False))
    bounds = starts + [L]
    sig = np.empty(L, np.float32)
    for j in range(5):
        sig[bounds[j]:bounds[j + 1]] = rng.uniform(0.03, 0.1)
    k = rng.standard_normal((L, d), dtype=np.float32) * sig[:, None]
    v = rng.standard_normal((L, d), dtype=np.float32) * sig[:, None]
    for x, pos in ((k, False), (v, one_sided)):
        mask = rng.random((L, d), dtype=np.float32) < 0.01
        sign = np.ones((L, d), np.float32) if pos else rng.integers(0, 2, (L, d)).astype(np.float32) * 2 - 1
        x[mask] = (sign * 8.0 * sig[:, None])[mask]
    if one_sided:
        # zero-mean in expectation (the outliers' mean, 0.08 sigma, is taken off every value), while
        # the range (about -4.6 to +7.9 sigma) and with it the midpoint stay off-centre
        v -= np.float32(0.08) * sig[:, None]
    k16, v16 = k.astype(np.float16), v.astype(np.float16)
    segs = O.segment_params(k16, v16, starts)
    return O.HeadCompressed(L, segs, O.encode_by_segment(k16, segs, "k"), O.encode_by_segment(v16, segs, "v"),
                            O.boundary_bits(starts, L))


def _bound(hc, q16, out_ref, nparts, per):
    """First-order worst-case relative error of the kernel's arithmetic (see the module text).
    Returns (bound, condition number, the bound's 24-bit split part)."""
    L, d = hc.kcodes.shape
    idx = hc.seg_of()
    ks = np.array([s.kscale for s in hc.segs], np.float64)[idx]
    vs = np.array([s.vscale for s in hc.segs], np.float64)[idx]
    midv = np.array([s.vmin + 128.0 * np.float64(s.vscale) for s in hc.segs], np.float64)[idx]
    khat, vhat = hc.khat(), hc.vhat()
    ck = np.abs(hc.kcodes.astype(np.float64))                  # |c| of the centred codes
    cv = np.abs(hc.vcodes.astype(np.float64))
    sm = 1.0 / math.sqrt(d)
    wave_tokens = per * 64
    n1 = 16 + 3 * per + 8          # per-lane token adds, chunk folds, lane combine, epilogue
    n2 = 8 + 2 * nparts + 8        # wave merge, partition merge (rescale + add each), output
    worst = split = cond_max = 0.0
    for i in range(q16.shape[0]):
        q = q16[i].astype(np.float64)
        s = sm * (khat @ q)
        p = np.exp(s - s.max())
        l = p.sum()
        o = out_ref[i]
        oinf = np.abs(o).max()
        amax = np.abs(q).max()
        dev = np.abs(vhat - o[None, :])
        # 24-bit query bytes: score error per token (natural units), moved into the output
        ds = sm * ks * amax * 2.0 ** -22 * ck.sum(axis=1)
        e_q = (p * ds) @ dev / l
        # 24-bit weights p * vs: at most vsmax * 2^-23 each, times |c|, summed linearly
        e_w = vs.max() * 2.0 ** -23 * cv.sum(axis=0) / l
        # exp2 of a rounded float32 argument: 2^-22 relative plus the argument's rounding
        e_x = (2.0 ** -22 + math.log(2) * 2 * U * (np.abs(s - s.max()).max() + 1)) * (p @ dev) / l
        # float32 sums: within a wave over the token terms, above it over the wave partials
        terms = p @ (np.abs(midv)[:, None] + vs[:, None] * cv)
        pv = p[:, None] * vhat
        wave_parts = np.add.reduceat(pv, np.arange(0, L, wave_tokens), axis=0)
        e_f = (n1 * U * terms + n2 * U * np.abs(wave_parts).sum(axis=0)) / l + (n1 + n2) * U * np.abs(o)
        worst = max(worst, float(((e_q + e_w + e_x + e_f) / oinf).max()))
        split = max(split, float(((e_q + e_w) / oinf).max()))
        cond_max = max(cond_max, float((terms / (l * oinf)).max()))
    return worst, cond_max, split


@pytest.mark.parametrize("L", [8192, 32768, 131072])
@pytest.mark.parametrize("one_sided", [False, True], ids=["symmetric", "one_sided"])
def test_long_context_error_headroom(L, one_sided):
    cfg = dgq_data.get_config(3, batch=1, hkv=1, hq=4, seq_len=L)
    hc = _head(L, one_sided, 31)
    table, nblk = dgq_data.block_tables(cfg, 31, lens_total=np.array([L]))
    params = H.params_for(cfg)
    cache = H.cache_from_oracle(params, {(0, 0): hc}, table, nblk, 1)
    q16 = dgq_data.queries(cfg, 31)
    H.say("long-context error headroom", L, "one-sided" if one_sided else "symmetric")
    out = Q.paged_decode_attn_int8(params, torch.from_numpy(q16).cuda(), cache, torch.from_numpy(table).cuda(),
                                   torch.tensor([L], dtype=torch.int32, device="cuda"), L)
    out = out.cpu().numpy()[0]
    ref = O.decode_attention(q16[0], hc.khat(), hc.vhat())
    err = H.rel_err_rows(out, ref)
    # the launch plan of this shape: 64-token chunks over ~1024 waves in 4-wave workgroups
    chunks = L // 64
    per = max(1, min(64, -(-chunks // 1024)))
    nparts = max(1, -(-chunks // (per * 4)))
    bound, cond, split = _bound(hc, q16[0], ref, nparts, per)
    print(f"[headroom] L={L} {'one-sided' if one_sided else 'symmetric'}: measured {err:.3e}, "
          f"first-order bound {bound:.3e} (24-bit split part {split:.3e}), condition {cond:.1f}, "
          f"partitions {nparts}", flush=True)
    assert err <= TOL
    assert err <= bound
