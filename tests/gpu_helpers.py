"""Helpers for the GPU parity tests: move oracle results into a device cache, read device caches
back as logical codes, and compare.  Expected values always come from the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import dgq_data
import paged_layout as PL
from oracle import dgq_oracle as O
import quantized_paged_kv_dgq_amd as Q


def say(*args):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def seg_row(s: O.SegParams) -> np.ndarray:
    row = np.zeros(8, dtype=np.int32)
    row[0] = s.start
    f = np.array([s.kmin, s.kmax, s.vmin, s.vmax, s.kscale, s.vscale], dtype=np.float32)
    row[1:7] = f.view(np.int32)
    return row


def params_for(cfg, **kw) -> Q.DGQParams:
    return Q.DGQParams(cfg.hkv, cfg.hq, cfg.head_dim, cfg.block_size, **kw)


def cache_from_oracle(params: Q.DGQParams, heads, table: np.ndarray, num_blocks: int, batch: int,
                      fill=None) -> Q.DGQCache:
    """A device cache whose pools, bits and segment tables hold the oracle's compression of
    ``heads`` {(b, h): HeadCompressed}; unused pool bytes hold ``fill`` (random if None)."""
    p = params.c
    cache = Q.DGQCache(params, num_blocks, batch)
    rng = np.random.default_rng(123)
    shape = (num_blocks, p.num_kv_heads, p.block_size * p.head_dim)
    if fill is None:
        kp = rng.integers(-128, 128, shape).astype(np.int8)
        vp = rng.integers(-128, 128, shape).astype(np.int8)
    else:
        kp = np.full(shape, fill, np.int8)
        vp = np.full(shape, fill, np.int8)
    bits = np.zeros((num_blocks, p.num_kv_heads, p.block_size // 8), np.uint8)
    segs = np.zeros((batch, p.num_kv_heads, p.seg_capacity, 8), np.int32)
    nseg = np.zeros((batch, p.num_kv_heads), np.int32)
    koff = PL.k_offsets(p.block_size, p.head_dim)
    voff = PL.v_offsets(p.block_size, p.head_dim)
    for (b, h), hc in heads.items():
        PL.scatter_head(kp, table[b], h, hc.kcodes, koff)
        PL.scatter_head(vp, table[b], h, hc.vcodes, voff)
        for t in np.flatnonzero(hc.bits):
            bits[table[b][t // p.block_size], h, (t % p.block_size) // 8] |= np.uint8(1 << (t % 8))
        for i, s in enumerate(hc.segs):
            segs[b, h, i] = seg_row(s)
        nseg[b, h] = len(hc.segs)
    cache.k_pool.copy_(torch.from_numpy(kp))
    cache.v_pool.copy_(torch.from_numpy(vp))
    cache.bits.copy_(torch.from_numpy(bits))
    cache.segs.copy_(torch.from_numpy(segs))
    cache.nseg.copy_(torch.from_numpy(nseg))
    return cache


def fmt_of(params: Q.DGQParams) -> str:
    return "marker" if params.marker else "bitmap"


def identifier_bits(cache: Q.DGQCache, table: np.ndarray, lens) -> np.ndarray:
    """The boundary bits of a cache in the bit-tensor layout, on the host: the bit tensor itself,
    or (marker format) the bits read back from the marker bytes by dgq_marker_bits."""
    if cache.bits is not None:
        return cache.bits.cpu().numpy()
    lens = np.asarray(lens, np.int32)
    out = Q.dgq_marker_bits(cache.params, cache, torch.from_numpy(np.ascontiguousarray(table, np.int32)).cuda(),
                            torch.from_numpy(lens).cuda(), int(max(lens.max(initial=0), 0)))
    return out.cpu().numpy()


def compare_markers(got_k: np.ndarray, ref_k: np.ndarray, what: str) -> None:
    """Marker bytes (-128 / 127) sit at exactly the same places (no 1-LSB slack for them)."""
    gm = (got_k == -128) | (got_k == 127)
    rm = (ref_k == -128) | (ref_k == 127)
    assert np.array_equal(gm, rm), f"{what}: marker positions differ"
    assert np.array_equal(got_k[gm], ref_k[rm]), f"{what}: marker values differ"


def oracle_decode(q16: np.ndarray, heads, lens, hkv: int, group: int) -> np.ndarray:
    """fp64 attention of q [B][Hq][D] over the oracle's dequantized cache."""
    batch, hq, d = q16.shape
    out = np.zeros((batch, hq, d))
    for b in range(batch):
        for h in range(hkv):
            hc = heads[(b, h)]
            out[b, h * group:(h + 1) * group] = O.decode_attention(q16[b, h * group:(h + 1) * group],
                                                                   hc.khat(), hc.vhat())
    return out


def rel_err_rows(out: np.ndarray, ref: np.ndarray) -> float:
    """max over (b, g) of ||out - ref||_inf / ||ref||_inf; rows with ref == 0 need out == 0."""
    out = out.reshape(-1, out.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    num = np.abs(out - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), "empty rows must be zero"
    return float((num[~zero] / den[~zero]).max()) if (~zero).any() else 0.0


def read_codes(cache: Q.DGQCache, table: np.ndarray, b: int, h: int, length: int):
    p = cache.params.c
    kp = cache.k_pool.cpu().numpy()
    vp = cache.v_pool.cpu().numpy()
    kc = PL.gather_head(kp, table[b], h, length, PL.k_offsets(p.block_size, p.head_dim))
    vc = PL.gather_head(vp, table[b], h, length, PL.v_offsets(p.block_size, p.head_dim))
    return kc, vc


def compare_codes(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    """Codes must match; the acceptance bound allows 1-LSB differences on <= 1e-4 of elements."""
    diff = np.abs(got.astype(np.int16) - ref.astype(np.int16))
    n_bad = int((diff > 0).sum())
    assert diff.max(initial=0) <= 1, f"{what}: code differs by {diff.max()}"
    assert n_bad <= 1e-4 * max(diff.size, 1), f"{what}: {n_bad} of {diff.size} codes differ by 1"


def compare_segments(cache: Q.DGQCache, heads, batch: int, hkv: int) -> None:
    starts, prm, nseg = cache.segment_table()
    for b in range(batch):
        for h in range(hkv):
            hc = heads[(b, h)]
            assert nseg[b, h] == len(hc.segs), (b, h, nseg[b, h], hc.starts)
            for i, s in enumerate(hc.segs):
                assert starts[b, h, i] == s.start, (b, h, i, starts[b, h, i], hc.starts)
                want = np.array([s.kmin, s.kmax, s.vmin, s.vmax, s.kscale, s.vscale], np.float32)
                got = prm[b, h, i]
                assert np.array_equal(got.view(np.int32), want.view(np.int32)), (b, h, i, got, want)


def upload_batch(cfg, seed: int, layer: int = 0, prefix_only: bool = True):
    """Token-major K/V of a config on the device (prefix tokens only by default) + host copies."""
    k, v, cu, lens = dgq_data.batch_kv(cfg, seed, layer)
    if prefix_only and cfg.append_steps:
        parts_k, parts_v = [], []
        for b in range(cfg.batch):
            parts_k.append(k[cu[b]:cu[b] + lens[b]])
            parts_v.append(v[cu[b]:cu[b] + lens[b]])
        k, v = np.concatenate(parts_k), np.concatenate(parts_v)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    dk = torch.from_numpy(k).cuda()
    dv = torch.from_numpy(v).cuda()
    return k, v, cu, lens, dk, dv
