"""ctypes view of libdgq.so (include/dgq.h).  Argument marshalling only."""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdgq.so")

DGQ_OK = 0
DGQ_ERR_INVALID_ARG = -1
DGQ_ERR_UNSUPPORTED = -2
DGQ_ERR_POOL_EXHAUSTED = -3
DGQ_ERR_WORKSPACE_TOO_SMALL = -4
DGQ_ERR_HIP = -5


class Params(ctypes.Structure):
    _fields_ = [
        ("num_kv_heads", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("win", ctypes.c_int32),
        ("max_segments", ctypes.c_int32),
        ("seg_capacity", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("tau", ctypes.c_double),
        ("min_var", ctypes.c_double),
    ]


class Seg(ctypes.Structure):
    _fields_ = [
        ("start", ctypes.c_int32),
        ("kmin", ctypes.c_float), ("kmax", ctypes.c_float),
        ("vmin", ctypes.c_float), ("vmax", ctypes.c_float),
        ("kscale", ctypes.c_float), ("vscale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
    ]


class Tail(ctypes.Structure):
    _fields_ = [
        ("r0", ctypes.c_int32),
        ("ring_len", ctypes.c_int32),
        ("span_own", ctypes.c_int32),
        ("window_done", ctypes.c_int32),
        ("ring_a", ctypes.c_int32 * 16),
        ("ring_b", ctypes.c_int64 * 16),
        ("span_range", ctypes.c_float * 4),
    ]


class G64Cache(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("k_range", ctypes.c_void_p),
        ("v_range", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class Cache(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("bits", ctypes.c_void_p),
        ("segs", ctypes.c_void_p),
        ("nseg", ctypes.c_void_p),
        ("tail", ctypes.c_void_p),
        ("k_stage", ctypes.c_void_p),
        ("v_stage", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("batch", ctypes.c_int32),
    ]


DGQ_POLICY_LENGTH_AWARE = 1
DGQ_FORMAT_MARKER = 2
DGQ_COMPRESS_MULTIPASS = 4
DGQ_NOALLOC_SCRATCH_BYTES = 16 << 20
DGQ_OP_COMPRESS, DGQ_OP_APPEND, DGQ_OP_DECODE, DGQ_OP_APPEND_DECODE, DGQ_OP_G64_DECODE = range(5)

assert ctypes.sizeof(Params) == 48
assert ctypes.sizeof(Seg) == 32
assert ctypes.sizeof(Tail) == 224

# Every symbol include/dgq.h declares.
EXPORTS = [
    "dgq_status_string", "dgq_last_error",
    "dgq_pool_create", "dgq_pool_destroy", "dgq_block_alloc", "dgq_block_free", "dgq_pool_num_free",
    "dgq_block_share", "dgq_block_refcount", "dgq_block_cow",
    "dgq_copy_blocks", "dgq_copy_seq_state", "dgq_swap_image_bytes", "dgq_swap_out", "dgq_swap_in",
    "dgq_marker_bits",
    "dgq_compress_workspace_size", "dgq_decode_workspace_size", "dgq_workspace_size", "dgq_read_device_status",
    "dgq_compress", "dgq_append", "paged_decode_attn_int8", "paged_decode_attn_int8_noalloc",
    "dgq_append_decode",
    "dgq_g64_quantize", "paged_decode_attn_g64",
]

_lib = None


def load() -> ctypes.CDLL:
    """Load libdgq.so; raises if it is not built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libdgq.so is not built at {LIB_PATH}; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.dgq_status_string.argtypes = [i32]
    lib.dgq_status_string.restype = ctypes.c_char_p
    lib.dgq_last_error.argtypes = []
    lib.dgq_last_error.restype = ctypes.c_char_p
    lib.dgq_pool_create.argtypes = [i32, P(vp)]
    lib.dgq_pool_create.restype = i32
    lib.dgq_pool_destroy.argtypes = [vp]
    lib.dgq_pool_destroy.restype = i32
    lib.dgq_block_alloc.argtypes = [vp, i32, P(i32)]
    lib.dgq_block_alloc.restype = i32
    lib.dgq_block_free.argtypes = [vp, i32, P(i32)]
    lib.dgq_block_free.restype = i32
    lib.dgq_pool_num_free.argtypes = [vp]
    lib.dgq_pool_num_free.restype = i32
    lib.dgq_block_share.argtypes = [vp, i32, P(i32)]
    lib.dgq_block_share.restype = i32
    lib.dgq_block_refcount.argtypes = [vp, i32]
    lib.dgq_block_refcount.restype = i32
    lib.dgq_block_cow.argtypes = [vp, i32, P(i32), P(i32)]
    lib.dgq_block_cow.restype = i32
    lib.dgq_copy_blocks.argtypes = [P(Params), P(Cache), vp, vp, i32, vp]
    lib.dgq_copy_blocks.restype = i32
    lib.dgq_copy_seq_state.argtypes = [P(Params), P(Cache), vp, vp, i32, vp]
    lib.dgq_copy_seq_state.restype = i32
    lib.dgq_swap_image_bytes.argtypes = [P(Params), i32]
    lib.dgq_swap_image_bytes.restype = sz
    lib.dgq_swap_out.argtypes = [P(Params), P(Cache), i32, vp, i32, vp, sz, vp, vp]
    lib.dgq_swap_out.restype = i32
    lib.dgq_swap_in.argtypes = [P(Params), P(Cache), i32, vp, i32, vp, sz, vp, vp]
    lib.dgq_swap_in.restype = i32
    lib.dgq_marker_bits.argtypes = [P(Params), P(Cache), vp, i32, vp, i32, i32, vp, vp]
    lib.dgq_marker_bits.restype = i32
    lib.dgq_compress_workspace_size.argtypes = [P(Params), i32, i64, i32]
    lib.dgq_compress_workspace_size.restype = sz
    lib.dgq_decode_workspace_size.argtypes = [P(Params), i32, i32]
    lib.dgq_decode_workspace_size.restype = sz
    lib.dgq_workspace_size.argtypes = [P(Params), i32, i32, i64, i32]
    lib.dgq_workspace_size.restype = sz
    lib.dgq_read_device_status.argtypes = [P(Cache), P(ctypes.c_ulonglong), vp]
    lib.dgq_read_device_status.restype = i32
    lib.dgq_compress.argtypes = [P(Params), vp, vp, i64, i64, vp, i32, i32, i64, vp, i32,
                                 P(Cache), vp, sz, vp]
    lib.dgq_compress.restype = i32
    lib.dgq_append.argtypes = [P(Params), vp, vp, vp, i32, vp, i32, P(Cache), vp]
    lib.dgq_append.restype = i32
    lib.paged_decode_attn_int8.argtypes = [P(Params), vp, P(Cache), vp, i32, vp, i32, i32,
                                           ctypes.c_float, vp, vp, sz, vp]
    lib.paged_decode_attn_int8.restype = i32
    lib.paged_decode_attn_int8_noalloc.argtypes = [P(Params), vp, P(Cache), vp, i32, vp, i32, i32,
                                                   ctypes.c_float, vp, vp]
    lib.paged_decode_attn_int8_noalloc.restype = i32
    lib.dgq_append_decode.argtypes = [P(Params), vp, vp, vp, vp, i32, vp, i32, i32, ctypes.c_float,
                                      P(Cache), vp, vp, sz, vp]
    lib.dgq_append_decode.restype = i32
    lib.dgq_g64_quantize.argtypes = [P(Params), vp, vp, i64, i64, vp, vp, i32, i32, i64, vp, i32, i32,
                                     P(G64Cache), vp]
    lib.dgq_g64_quantize.restype = i32
    lib.paged_decode_attn_g64.argtypes = [P(Params), vp, P(G64Cache), vp, i32, vp, i32, i32,
                                          ctypes.c_float, vp, vp, sz, vp]
    lib.paged_decode_attn_g64.restype = i32
    _lib = lib
    return lib


class DGQError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        text = lib.dgq_status_string(status).decode()
        detail = lib.dgq_last_error().decode() if status == DGQ_ERR_HIP else ""
        super().__init__(f"{where}: {text} ({status}){': ' + detail if detail else ''}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != DGQ_OK:
        raise DGQError(status, where)
