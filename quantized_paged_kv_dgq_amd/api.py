"""Python binding of libdgq with the C ABI's names (include/dgq.h).

Only argument marshalling lives here: tensors become device pointers, the current torch stream
becomes the HIP stream, and status codes become exceptions.  Every step of compression, append
and decode runs in the library's HIP kernels; there is no fallback path.  torch provides device
memory (the caller-owned buffers of a cache and the scratch workspaces) and streams.
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import (DGQ_COMPRESS_MULTIPASS, DGQ_FORMAT_MARKER, DGQ_POLICY_LENGTH_AWARE, Cache, G64Cache, Params,
                   check)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# torch's current-stream handle of a device as a plain integer, without building a Stream object
# (that costs a few microseconds per call, as much as a small kernel).
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _raw_current_stream is not None:
        return _raw_current_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


class DGQParams:
    """dgq_params_t: shapes and method constants (window 16; segments 2..max_segments; tau), plus
    the segment-count policies: ``length_aware`` (cap by sequence length) and ``min_var``
    (variance floor below which a window pair is not a change point), and the identifier format:
    ``marker`` keeps it in the codes (no bit tensor) instead of the bit tensor.  ``multipass``
    makes dgq_compress use its separate launches also for short sequences (same results)."""

    def __init__(self, num_kv_heads: int, num_q_heads: int, head_dim: int, block_size: int,
                 max_segments: int = 5, seg_capacity: int = 16, tau: float = 2.0, win: int = 16,
                 length_aware: bool = False, min_var: float = 0.0, marker: bool = False,
                 multipass: bool = False):
        flags = ((DGQ_POLICY_LENGTH_AWARE if length_aware else 0) | (DGQ_FORMAT_MARKER if marker else 0)
                 | (DGQ_COMPRESS_MULTIPASS if multipass else 0))
        self.c = Params(num_kv_heads, num_q_heads, head_dim, block_size, win, max_segments,
                        seg_capacity, flags, float(tau), float(min_var))

    def __getattr__(self, name):
        return getattr(self.__dict__["c"], name)

    @property
    def group(self) -> int:
        return self.c.num_q_heads // self.c.num_kv_heads

    @property
    def length_aware(self) -> bool:
        return bool(self.c.flags & DGQ_POLICY_LENGTH_AWARE)

    @property
    def marker(self) -> bool:
        return bool(self.c.flags & DGQ_FORMAT_MARKER)

    @property
    def multipass(self) -> bool:
        return bool(self.c.flags & DGQ_COMPRESS_MULTIPASS)


class DGQCache:
    """The caller-owned device buffers of one layer's compressed cache (dgq_cache_t).  In the
    marker format there is no bit tensor (``bits`` is None)."""

    def __init__(self, params: DGQParams, num_blocks: int, batch: int, device="cuda"):
        p = params.c
        dev = torch.device(device)
        tile = p.block_size * p.head_dim
        self.params = params
        self.num_blocks = num_blocks
        self.batch = batch
        self.k_pool = torch.zeros((num_blocks, p.num_kv_heads, tile), dtype=torch.int8, device=dev)
        self.v_pool = torch.zeros_like(self.k_pool)
        self.bits = None if params.marker else torch.zeros((num_blocks, p.num_kv_heads, p.block_size // 8),
                                                           dtype=torch.uint8, device=dev)
        self.segs = torch.zeros((batch, p.num_kv_heads, p.seg_capacity, 8), dtype=torch.int32, device=dev)
        self.nseg = torch.zeros((batch, p.num_kv_heads), dtype=torch.int32, device=dev)
        self.tail = torch.zeros((batch, p.num_kv_heads, 56), dtype=torch.int32, device=dev)
        self.k_stage = torch.zeros((batch, p.num_kv_heads, p.block_size, p.head_dim), dtype=torch.float16, device=dev)
        self.v_stage = torch.zeros_like(self.k_stage)
        self.status = torch.zeros(4, dtype=torch.int64, device=dev)
        self.c = Cache(_ptr(self.k_pool), _ptr(self.v_pool), _ptr(self.bits), _ptr(self.segs),
                       _ptr(self.nseg), _ptr(self.tail), _ptr(self.k_stage), _ptr(self.v_stage),
                       _ptr(self.status), num_blocks, batch)

    def read_status(self, stream=None) -> dict:
        """The device status words through dgq_read_device_status (waits for the stream): appends
        that wanted a new segment but found the table full, groups of inputs with a non-finite
        value, and device-side inconsistencies that were skipped or clamped (see
        dgq_cache_t.status)."""
        v = (ctypes.c_ulonglong * 4)()
        check(_lib.load().dgq_read_device_status(ctypes.byref(self.c), v, _stream(stream)), "dgq_read_device_status")
        return {"clamped_appends": v[0], "nonfinite_groups": v[1], "inconsistencies": v[2]}

    # host-side views for tests and reports (copies)
    def segment_table(self):
        """(starts int32 [B][H][cap], params float32 [B][H][cap][6], nseg [B][H]) on the host."""
        raw = self.segs.cpu()
        return raw[..., 0].numpy(), raw[..., 1:7].contiguous().view(torch.float32).numpy(), self.nseg.cpu().numpy()


class DGQG64Cache:
    """Device buffers of one layer's fixed 64-channel group cache (dgq_g64_cache_t)."""

    def __init__(self, params: DGQParams, num_blocks: int, device="cuda"):
        p = params.c
        dev = torch.device(device)
        tile = p.block_size * p.head_dim
        self.params = params
        self.num_blocks = num_blocks
        self.k_pool = torch.zeros((num_blocks, p.num_kv_heads, tile), dtype=torch.int8, device=dev)
        self.v_pool = torch.zeros_like(self.k_pool)
        ng = p.head_dim // 64
        self.k_range = torch.zeros((num_blocks, p.num_kv_heads, p.block_size, ng), dtype=torch.int32, device=dev)
        self.v_range = torch.zeros_like(self.k_range)
        self.status = torch.zeros(4, dtype=torch.int64, device=dev)
        self.c = G64Cache(_ptr(self.k_pool), _ptr(self.v_pool), _ptr(self.k_range), _ptr(self.v_range),
                          _ptr(self.status), num_blocks, 0)


class BlockPool:
    """Host block pool (dgq_pool_*): free list with all-or-nothing allocation."""

    def __init__(self, num_blocks: int):
        lib = _lib.load()
        h = ctypes.c_void_p()
        check(lib.dgq_pool_create(num_blocks, ctypes.byref(h)), "dgq_pool_create")
        self._h = h

    def alloc(self, n: int) -> list:
        ids = (ctypes.c_int32 * max(n, 1))()
        check(_lib.load().dgq_block_alloc(self._h, n, ids), "dgq_block_alloc")
        return list(ids[:n])

    def free(self, ids: Sequence[int]) -> None:
        """Drop one reference per listed id (dgq_block_free)."""
        arr = (ctypes.c_int32 * max(len(ids), 1))(*ids)
        check(_lib.load().dgq_block_free(self._h, len(ids), arr), "dgq_block_free")

    def share(self, ids: Sequence[int]) -> None:
        """Add one reference per listed id (dgq_block_share)."""
        arr = (ctypes.c_int32 * max(len(ids), 1))(*ids)
        check(_lib.load().dgq_block_share(self._h, len(ids), arr), "dgq_block_share")

    def refcount(self, block_id: int) -> int:
        return _lib.load().dgq_block_refcount(self._h, block_id)

    def cow(self, ids: Sequence[int]) -> list:
        """Exclusive ids for blocks about to be written (dgq_block_cow): a changed entry names a
        fresh block that must receive a copy of the listed one."""
        arr = (ctypes.c_int32 * max(len(ids), 1))(*ids)
        out = (ctypes.c_int32 * max(len(ids), 1))()
        check(_lib.load().dgq_block_cow(self._h, len(ids), arr, out), "dgq_block_cow")
        return list(out[:len(ids)])

    @property
    def num_free(self) -> int:
        return _lib.load().dgq_pool_num_free(self._h)

    def close(self) -> None:
        if self._h:
            _lib.load().dgq_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def compress_workspace_size(params: DGQParams, batch: int, total_tokens: int, max_seq_len: int) -> int:
    return int(_lib.load().dgq_compress_workspace_size(ctypes.byref(params.c), batch, total_tokens, max_seq_len))


def decode_workspace_size(params: DGQParams, batch: int, max_seq_len: int) -> int:
    return int(_lib.load().dgq_decode_workspace_size(ctypes.byref(params.c), batch, max_seq_len))


def workspace_size(params: DGQParams, op: int, batch: int, total_tokens: int, max_seq_len: int) -> int:
    """dgq_workspace_size: workspace bytes of operation ``op`` (DGQ_OP_*)."""
    return int(_lib.load().dgq_workspace_size(ctypes.byref(params.c), op, batch, total_tokens, max_seq_len))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device scratch buffer (256-byte aligned by the caching allocator), zero-filled: the
    decode workspace's completion counters must start at zero (the library leaves them zero)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def dgq_compress(params: DGQParams, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                 block_table: torch.Tensor, cache: DGQCache, max_seq_len: int, total_tokens: int,
                 ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """Compress token-major fp16 K/V [total][Hkv][D] (see dgq_compress in include/dgq.h)."""
    _need(k.dtype == torch.float16 and v.dtype == torch.float16, "k, v must be float16")
    _need(k.shape == v.shape and k.stride() == v.stride() and k.dim() == 3, "k, v: [tokens][heads][dim], same strides")
    _need(k.stride(2) == 1, "channels must be contiguous")
    _need(cu_seqlens.dtype == torch.int32 and block_table.dtype == torch.int32, "int32 index tensors")
    batch = cu_seqlens.numel() - 1
    if ws is None:
        ws = workspace(compress_workspace_size(params, batch, total_tokens, max_seq_len), k.device)
    st = _lib.load().dgq_compress(
        ctypes.byref(params.c), _ptr(k), _ptr(v), k.stride(0), k.stride(1), _ptr(cu_seqlens), batch,
        max_seq_len, total_tokens, _ptr(block_table), block_table.shape[1], ctypes.byref(cache.c),
        _ptr(ws), ws.numel(), _stream(stream))
    check(st, "dgq_compress")


def dgq_append(params: DGQParams, k_tok: torch.Tensor, v_tok: torch.Tensor, seq_lens: torch.Tensor,
               block_table: torch.Tensor, cache: DGQCache, stream=None) -> None:
    """Append one fp16 token per sequence, k_tok/v_tok [B][Hkv][D] (see dgq_append)."""
    _need(k_tok.dtype == torch.float16 and k_tok.is_contiguous() and v_tok.is_contiguous(), "contiguous float16 tokens")
    _need(seq_lens.dtype == torch.int32 and block_table.dtype == torch.int32, "int32 index tensors")
    st = _lib.load().dgq_append(
        ctypes.byref(params.c), _ptr(k_tok), _ptr(v_tok), _ptr(seq_lens), seq_lens.numel(),
        _ptr(block_table), block_table.shape[1], ctypes.byref(cache.c), _stream(stream))
    check(st, "dgq_append")


def paged_decode_attn_int8(params: DGQParams, q: torch.Tensor, cache: DGQCache,
                           block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                           softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                           ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode attention of q [B][Hq][D] fp16 over the compressed cache; returns fp32 [B][Hq][D]."""
    _need(q.dtype == torch.float16 and q.is_contiguous(), "q: contiguous float16 [B][Hq][D]")
    _need(seq_lens.dtype == torch.int32 and block_table.dtype == torch.int32, "int32 index tensors")
    batch = q.shape[0]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(params.c.head_dim)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(decode_workspace_size(params, batch, max_seq_len), q.device)
    st = _lib.load().paged_decode_attn_int8(
        ctypes.byref(params.c), _ptr(q), ctypes.byref(cache.c), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), batch, max_seq_len, float(softmax_scale), _ptr(out), _ptr(ws), ws.numel(),
        _stream(stream))
    check(st, "paged_decode_attn_int8")
    return out


def paged_decode_attn_int8_noalloc(params: DGQParams, q: torch.Tensor, cache: DGQCache,
                                   block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                                   out: torch.Tensor, softmax_scale: Optional[float] = None,
                                   stream=None) -> torch.Tensor:
    """paged_decode_attn_int8 without a workspace (paged_decode_attn_int8_noalloc): the library's
    fixed per-device scratch array holds the partials.  ``out`` (fp32 [B][Hq][D]) is required, so
    that this call allocates nothing either."""
    _need(q.dtype == torch.float16 and q.is_contiguous(), "q: contiguous float16 [B][Hq][D]")
    _need(out.dtype == torch.float32 and out.is_contiguous() and out.shape == q.shape, "out: contiguous float32 like q")
    _need(seq_lens.dtype == torch.int32 and block_table.dtype == torch.int32, "int32 index tensors")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(params.c.head_dim)
    st = _lib.load().paged_decode_attn_int8_noalloc(
        ctypes.byref(params.c), _ptr(q), ctypes.byref(cache.c), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), q.shape[0], max_seq_len, float(softmax_scale), _ptr(out), _stream(stream))
    check(st, "paged_decode_attn_int8_noalloc")
    return out


def dgq_append_decode(params: DGQParams, k_tok: torch.Tensor, v_tok: torch.Tensor, seq_lens: torch.Tensor,
                      q: torch.Tensor, block_table: torch.Tensor, cache: DGQCache, max_seq_len: int,
                      softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Append one token per sequence (k_tok/v_tok [B][Hkv][D] at positions seq_lens) and decode
    q [B][Hq][D] over seq_lens + 1 tokens, in one launch (see dgq_append_decode); returns fp32."""
    _need(k_tok.dtype == torch.float16 and k_tok.is_contiguous() and v_tok.is_contiguous(), "contiguous float16 tokens")
    _need(q.dtype == torch.float16 and q.is_contiguous(), "q: contiguous float16 [B][Hq][D]")
    _need(seq_lens.dtype == torch.int32 and block_table.dtype == torch.int32, "int32 index tensors")
    batch = q.shape[0]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(params.c.head_dim)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(decode_workspace_size(params, batch, max_seq_len), q.device)
    st = _lib.load().dgq_append_decode(
        ctypes.byref(params.c), _ptr(k_tok), _ptr(v_tok), _ptr(seq_lens), _ptr(q), batch, _ptr(block_table),
        block_table.shape[1], max_seq_len, float(softmax_scale), ctypes.byref(cache.c), _ptr(out), _ptr(ws),
        ws.numel(), _stream(stream))
    check(st, "dgq_append_decode")
    return out


def _ids(t: torch.Tensor, what: str) -> torch.Tensor:
    _need(t.dtype == torch.int32 and t.is_contiguous() and t.dim() == 1, f"{what}: contiguous int32 vector")
    return t


def dgq_copy_blocks(params: DGQParams, cache: DGQCache, src_ids: torch.Tensor, dst_ids: torch.Tensor,
                    stream=None) -> None:
    """Copy whole compressed blocks src_ids[i] -> dst_ids[i] (device int32 vectors)."""
    _need(src_ids.numel() == dst_ids.numel(), "src_ids and dst_ids differ in length")
    _ids(src_ids, "src_ids")
    _ids(dst_ids, "dst_ids")
    st = _lib.load().dgq_copy_blocks(ctypes.byref(params.c), ctypes.byref(cache.c), _ptr(src_ids), _ptr(dst_ids),
                                     src_ids.numel(), _stream(stream))
    check(st, "dgq_copy_blocks")


def dgq_copy_seq_state(params: DGQParams, cache: DGQCache, src_rows: torch.Tensor, dst_rows: torch.Tensor,
                       stream=None) -> None:
    """Copy cache rows src_rows[i] -> dst_rows[i] (segment table, row count, append state, staging)."""
    _need(src_rows.numel() == dst_rows.numel(), "src_rows and dst_rows differ in length")
    _ids(src_rows, "src_rows")
    _ids(dst_rows, "dst_rows")
    st = _lib.load().dgq_copy_seq_state(ctypes.byref(params.c), ctypes.byref(cache.c), _ptr(src_rows),
                                        _ptr(dst_rows), src_rows.numel(), _stream(stream))
    check(st, "dgq_copy_seq_state")


def swap_image_bytes(params: DGQParams, n_blocks: int) -> int:
    return int(_lib.load().dgq_swap_image_bytes(ctypes.byref(params.c), n_blocks))


def dgq_swap_out(params: DGQParams, cache: DGQCache, row: int, ids: torch.Tensor, staging: torch.Tensor,
                 host: Optional[torch.Tensor] = None, stream=None) -> None:
    """Pack cache row `row` and blocks ids (device int32, logical order) into staging (device
    uint8), then copy it to `host` (pinned uint8) when given."""
    _need(staging.dtype == torch.uint8 and staging.is_contiguous(), "staging: contiguous uint8")
    _need(host is None or (host.dtype == torch.uint8 and host.is_contiguous() and host.numel() >= staging.numel()),
          "host: contiguous uint8 at least as large as staging")
    _ids(ids, "ids")
    st = _lib.load().dgq_swap_out(ctypes.byref(params.c), ctypes.byref(cache.c), row, _ptr(ids), ids.numel(),
                                  _ptr(staging), staging.numel(), _ptr(host), _stream(stream))
    check(st, "dgq_swap_out")


def dgq_swap_in(params: DGQParams, cache: DGQCache, row: int, ids: torch.Tensor, staging: torch.Tensor,
                host: Optional[torch.Tensor] = None, stream=None) -> None:
    """The inverse of dgq_swap_out: (host ->) staging -> cache row `row` and blocks ids."""
    _need(staging.dtype == torch.uint8 and staging.is_contiguous(), "staging: contiguous uint8")
    _need(host is None or (host.dtype == torch.uint8 and host.is_contiguous() and host.numel() >= staging.numel()),
          "host: contiguous uint8 at least as large as staging")
    _ids(ids, "ids")
    st = _lib.load().dgq_swap_in(ctypes.byref(params.c), ctypes.byref(cache.c), row, _ptr(ids), ids.numel(),
                                 _ptr(staging), staging.numel(), _ptr(host), _stream(stream))
    check(st, "dgq_swap_in")


def dgq_marker_bits(params: DGQParams, cache: DGQCache, block_table: torch.Tensor, seq_lens: torch.Tensor,
                    max_seq_len: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The boundary bits of a marker-format cache, read back from its marker bytes, in the
    bit-tensor layout uint8 [num_blocks][Hkv][block_size/8] (see dgq_marker_bits)."""
    p = params.c
    _need(seq_lens.dtype == torch.int32 and block_table.dtype == torch.int32, "int32 index tensors")
    if out is None:
        out = torch.zeros((cache.num_blocks, p.num_kv_heads, p.block_size // 8), dtype=torch.uint8,
                          device=cache.k_pool.device)
    st = _lib.load().dgq_marker_bits(ctypes.byref(params.c), ctypes.byref(cache.c), _ptr(block_table),
                                     block_table.shape[1], _ptr(seq_lens), seq_lens.numel(), max_seq_len,
                                     _ptr(out), _stream(stream))
    check(st, "dgq_marker_bits")
    return out


def dgq_g64_quantize(params: DGQParams, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                     block_table: torch.Tensor, cache: DGQG64Cache, max_rows: int, total_rows: int,
                     max_seq_len: int, first_pos: Optional[torch.Tensor] = None, stream=None) -> None:
    """Quantize rows into the group-64 cache (see dgq_g64_quantize in include/dgq.h)."""
    _need(k.dtype == torch.float16 and v.dtype == torch.float16 and k.stride() == v.stride(), "float16 k, v")
    _need(k.stride(-1) == 1, "channels must be contiguous")
    batch = cu_seqlens.numel() - 1
    st = _lib.load().dgq_g64_quantize(
        ctypes.byref(params.c), _ptr(k), _ptr(v), k.stride(0), k.stride(1), _ptr(cu_seqlens), _ptr(first_pos),
        batch, max_rows, total_rows, _ptr(block_table), block_table.shape[1], max_seq_len, ctypes.byref(cache.c),
        _stream(stream))
    check(st, "dgq_g64_quantize")


def paged_decode_attn_g64(params: DGQParams, q: torch.Tensor, cache: DGQG64Cache, block_table: torch.Tensor,
                          seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: Optional[float] = None,
                          out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """Decode attention over a group-64 cache; returns fp32 [B][Hq][D]."""
    _need(q.dtype == torch.float16 and q.is_contiguous(), "q: contiguous float16 [B][Hq][D]")
    batch = q.shape[0]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(params.c.head_dim)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(decode_workspace_size(params, batch, max_seq_len), q.device)
    st = _lib.load().paged_decode_attn_g64(
        ctypes.byref(params.c), _ptr(q), ctypes.byref(cache.c), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), batch, max_seq_len, float(softmax_scale), _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    check(st, "paged_decode_attn_g64")
    return out
