"""The paged pool layout that include/dgq.h documents, written out in NumPy for the tests.

It maps between logical codes [token][channel] of one (sequence, kv head) and the bytes of the
(block, head) tiles, so that oracle codes can be placed into a pool (decode-only tests) and pool
bytes read back as logical codes (compression tests).  Nothing here is shared with the library.
"""

import numpy as np


def k_offsets(block_size: int, head_dim: int) -> np.ndarray:
    """int64 [block_size][head_dim]: byte offset of (tau, d) inside a K tile."""
    m_count = head_dim // 64
    tau = np.arange(block_size)[:, None]
    d = np.arange(head_dim)[None, :]
    m, j, e = d // 64, (d % 64) // 16, d % 16
    if block_size == 64:
        T, r = tau // 16, tau % 16
        return (((T * m_count + m) * 4 + j) * 16 + r) * 16 + e
    if block_size == 16:
        T, i = tau // 4, tau % 4
        return ((((T * m_count + m) * 4 + j) * 4 + i) * 16) + e
    if block_size == 32:   # two 16-token tiles one after the other
        return np.concatenate([k_offsets(16, head_dim), 16 * head_dim + k_offsets(16, head_dim)])
    raise ValueError(block_size)


def v_offsets(block_size: int, head_dim: int) -> np.ndarray:
    """int64 [block_size][head_dim]: byte offset of (tau, d) inside a V tile."""
    tau = np.arange(block_size)[:, None]
    d = np.arange(head_dim)[None, :]
    if block_size == 64:
        n, r = d // 16, d % 16
        j, e = (tau % 16) // 4, 4 * (tau // 16) + tau % 4
        return ((n * 4 + j) * 16 + r) * 16 + e
    if block_size == 16:
        return d * 16 + tau
    if block_size == 32:   # two 16-token tiles one after the other
        return np.concatenate([v_offsets(16, head_dim), 16 * head_dim + v_offsets(16, head_dim)])
    raise ValueError(block_size)


def _check_bijection(off: np.ndarray) -> None:
    assert np.array_equal(np.sort(off.reshape(-1)), np.arange(off.size))


def scatter_head(pool: np.ndarray, table_row: np.ndarray, head: int, codes: np.ndarray,
                 offsets: np.ndarray) -> None:
    """Write logical codes [L][D] of one head into pool [nblk][H][bs*D] through the table row."""
    bs = offsets.shape[0]
    length = codes.shape[0]
    for blk in range((length + bs - 1) // bs):
        n = min(bs, length - blk * bs)
        tile = pool[table_row[blk], head]
        tile[offsets[:n].reshape(-1)] = codes[blk * bs:blk * bs + n].reshape(-1)


def gather_head(pool: np.ndarray, table_row: np.ndarray, head: int, length: int,
                offsets: np.ndarray) -> np.ndarray:
    """Read logical codes [length][D] of one head back from the pool."""
    bs, d = offsets.shape
    out = np.empty((length, d), dtype=pool.dtype)
    for blk in range((length + bs - 1) // bs):
        n = min(bs, length - blk * bs)
        tile = pool[table_row[blk], head]
        out[blk * bs:blk * bs + n] = tile[offsets[:n].reshape(-1)].reshape(n, d)
    return out


def gather_bits(bits: np.ndarray, table_row: np.ndarray, head: int, length: int, block_size: int) -> np.ndarray:
    """bool [length]: the boundary bit of every token."""
    out = np.zeros(length, dtype=bool)
    for t in range(length):
        byte = bits[table_row[t // block_size], head, (t % block_size) // 8]
        out[t] = bool((int(byte) >> (t % 8)) & 1)
    return out
