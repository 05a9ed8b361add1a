"""The documented paged layout is a bijection per tile and matches the matrix-operand reading
order the header describes (CPU)."""

import numpy as np
import pytest

import paged_layout as PL


@pytest.mark.parametrize("bs", [16, 32, 64])
@pytest.mark.parametrize("d", [64, 128])
def test_offsets_are_bijections(bs, d):
    PL._check_bijection(PL.k_offsets(bs, d))
    PL._check_bijection(PL.v_offsets(bs, d))


@pytest.mark.parametrize("d", [64, 128])
def test_scatter_gather_roundtrip(d):
    rng = np.random.default_rng(0)
    for bs in (16, 32, 64):
        L = 3 * bs + 5
        table = rng.permutation(8)
        pool = np.zeros((8, 2, bs * d), np.int8)
        codes = rng.integers(-128, 128, (L, d)).astype(np.int8)
        PL.scatter_head(pool, table, 1, codes, PL.k_offsets(bs, d))
        assert np.array_equal(PL.gather_head(pool, table, 1, L, PL.k_offsets(bs, d)), codes)
        assert not pool[:, 0].any()


def test_k_tile_reading_order_bs64():
    """Lane l of the QK load for (T, m) reads 16 contiguous bytes at ((T*M+m)*64 + l)*16, which
    hold token 16T + l%16 and channels 64m + 16(l//16) .. +15."""
    d = 128
    off = PL.k_offsets(64, d)
    M = d // 64
    for T in range(4):
        for m in range(M):
            for lane in range(64):
                tok, d0 = 16 * T + lane % 16, 64 * m + 16 * (lane // 16)
                assert list(off[tok, d0:d0 + 16]) == list(range(((T * M + m) * 64 + lane) * 16, ((T * M + m) * 64 + lane) * 16 + 16))


def test_v_tile_reading_order_bs64():
    """Lane l of the PV load for channel tile n reads bytes ((n*64 + l)*16 + e), which hold channel
    16n + l%16 of token 16(e//4) + 4(l//16) + e%4."""
    d = 128
    off = PL.v_offsets(64, d)
    for n in range(d // 16):
        for lane in range(64):
            for e in range(16):
                tok = 16 * (e // 4) + 4 * (lane // 16) + e % 4
                assert off[tok, 16 * n + lane % 16] == (n * 64 + lane) * 16 + e
