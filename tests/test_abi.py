"""The C ABI on the CPU: the library loads, exports every symbol include/dgq.h declares, the host
block pool behaves, and argument checks reject bad calls before any device work."""

import ctypes
import os
import re

import pytest

from quantized_paged_kv_dgq_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libdgq.so is not built; run __graft_entry__.build()")
    return _lib.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dgq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"sizeof"})


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.dgq_status_string(0) == b"ok"
    assert lib.dgq_status_string(-3) == b"block pool exhausted"
    assert lib.dgq_status_string(42) == b"unknown status"


def test_pool(lib):
    h = ctypes.c_void_p()
    assert lib.dgq_pool_create(8, ctypes.byref(h)) == 0
    assert lib.dgq_pool_num_free(h) == 8
    ids = (ctypes.c_int32 * 8)()
    assert lib.dgq_block_alloc(h, 3, ids) == 0
    assert list(ids[:3]) == [0, 1, 2]
    assert lib.dgq_pool_num_free(h) == 5
    # all or nothing
    assert lib.dgq_block_alloc(h, 6, ids) == _lib.DGQ_ERR_POOL_EXHAUSTED
    assert lib.dgq_pool_num_free(h) == 5
    # double free / out of range / repeated id leave the pool unchanged
    bad = (ctypes.c_int32 * 2)(3, 3)
    assert lib.dgq_block_free(h, 1, (ctypes.c_int32 * 1)(3)) == _lib.DGQ_ERR_INVALID_ARG  # 3 is free
    assert lib.dgq_block_free(h, 2, (ctypes.c_int32 * 2)(1, 1)) == _lib.DGQ_ERR_INVALID_ARG
    assert lib.dgq_block_free(h, 1, (ctypes.c_int32 * 1)(99)) == _lib.DGQ_ERR_INVALID_ARG
    assert lib.dgq_pool_num_free(h) == 5
    del bad
    assert lib.dgq_block_free(h, 2, (ctypes.c_int32 * 2)(2, 0)) == 0
    assert lib.dgq_pool_num_free(h) == 7
    # last freed first
    assert lib.dgq_block_alloc(h, 2, ids) == 0 and list(ids[:2]) == [0, 2]
    assert lib.dgq_pool_destroy(h) == 0
    assert lib.dgq_pool_num_free(None) == -1
    assert lib.dgq_pool_create(-1, ctypes.byref(h)) == _lib.DGQ_ERR_INVALID_ARG


def _params(**kw):
    base = dict(num_kv_heads=8, num_q_heads=32, head_dim=128, block_size=16, win=16,
                max_segments=5, seg_capacity=16, flags=0, tau=2.0, min_var=0.0)
    base.update(kw)
    return _lib.Params(**base)


def test_workspace_sizes(lib):
    p = _params()
    assert lib.dgq_compress_workspace_size(ctypes.byref(p), 16, 16 * 8192, 8192) > 16 * 8192 * 8 * 20
    assert lib.dgq_decode_workspace_size(ctypes.byref(p), 16, 8192) > 0
    for bad in (_params(head_dim=96), _params(block_size=48), _params(win=8), _params(num_q_heads=20),
                _params(max_segments=9), _params(seg_capacity=4), _params(tau=0.5), _params(flags=8),
                _params(min_var=-1.0), _params(min_var=float("nan"))):
        assert lib.dgq_compress_workspace_size(ctypes.byref(bad), 1, 10, 10) == 0
        assert lib.dgq_decode_workspace_size(ctypes.byref(bad), 1, 10) == 0


def test_workspace_size_by_operation(lib):
    """dgq_workspace_size(op) equals the per-operation functions; append takes none; an unknown op
    or invalid parameters give 0."""
    for p in (_params(), _params(head_dim=64, block_size=64, num_q_heads=8), _params(flags=7)):
        for batch, total, L in ((16, 16 * 8192, 8192), (1, 131072, 131072), (100, 234194, 4096), (1, 256, 256)):
            comp = lib.dgq_compress_workspace_size(ctypes.byref(p), batch, total, L)
            dec = lib.dgq_decode_workspace_size(ctypes.byref(p), batch, L)
            assert comp > 0 and dec > 0
            ws = lambda op: lib.dgq_workspace_size(ctypes.byref(p), op, batch, total, L)  # noqa: E731
            assert ws(_lib.DGQ_OP_COMPRESS) == comp
            assert ws(_lib.DGQ_OP_APPEND) == 0
            assert ws(_lib.DGQ_OP_DECODE) == dec
            assert ws(_lib.DGQ_OP_APPEND_DECODE) == dec
            assert ws(_lib.DGQ_OP_G64_DECODE) == dec
            assert ws(5) == 0 and ws(-1) == 0
    bad = _params(head_dim=96)
    assert lib.dgq_workspace_size(ctypes.byref(bad), _lib.DGQ_OP_DECODE, 1, 10, 10) == 0


def test_read_device_status_argument_checks(lib):
    """Null cache, status pointer or output: refused before any HIP call."""
    out = (ctypes.c_ulonglong * 4)()
    assert lib.dgq_read_device_status(None, out, None) == _lib.DGQ_ERR_INVALID_ARG
    cache = _lib.Cache()
    assert lib.dgq_read_device_status(ctypes.byref(cache), out, None) == _lib.DGQ_ERR_INVALID_ARG
    cache.status = 1 << 20                  # never dereferenced: the null output fails first
    assert lib.dgq_read_device_status(ctypes.byref(cache), None, None) == _lib.DGQ_ERR_INVALID_ARG


def test_policy_params_accepted(lib):
    """The length-aware flag, a variance floor, the marker format and the multi-pass compress
    switch are valid parameters."""
    for good in (_params(flags=_lib.DGQ_POLICY_LENGTH_AWARE), _params(min_var=0.01),
                 _params(flags=1, min_var=1e-4), _params(flags=_lib.DGQ_FORMAT_MARKER), _params(flags=3),
                 _params(flags=_lib.DGQ_COMPRESS_MULTIPASS), _params(flags=7)):
        assert lib.dgq_compress_workspace_size(ctypes.byref(good), 1, 10, 10) > 0


def test_argument_checks_queue_nothing(lib):
    """Every bad call fails in the host checks (no device pointer is ever touched)."""
    p = _params()
    fake = ctypes.c_void_p(1 << 20)         # never dereferenced: the checks fail first
    cache = _lib.Cache(fake, fake, fake, fake, fake, fake, fake, fake, fake, 64, 4)
    # unsupported shapes
    for bad, code in ((_params(head_dim=96), _lib.DGQ_ERR_UNSUPPORTED),
                      (_params(num_q_heads=20), _lib.DGQ_ERR_INVALID_ARG),
                      (_params(num_q_heads=24), _lib.DGQ_ERR_UNSUPPORTED),
                      (_params(num_q_heads=64), _lib.DGQ_ERR_UNSUPPORTED)):
        assert lib.paged_decode_attn_int8(ctypes.byref(bad), fake, ctypes.byref(cache), fake, 4, fake,
                                          1, 64, 1.0, fake, fake, 1 << 30, None) == code
    # null query
    assert lib.paged_decode_attn_int8(ctypes.byref(p), None, ctypes.byref(cache), fake, 4, fake, 1, 64,
                                      1.0, fake, fake, 1 << 30, None) == _lib.DGQ_ERR_INVALID_ARG
    # max_seq_len beyond the table
    assert lib.paged_decode_attn_int8(ctypes.byref(p), fake, ctypes.byref(cache), fake, 4, fake, 1, 65,
                                      1.0, fake, fake, 1 << 30, None) == _lib.DGQ_ERR_INVALID_ARG
    # workspace too small
    assert lib.paged_decode_attn_int8(ctypes.byref(p), fake, ctypes.byref(cache), fake, 4, fake, 1, 64,
                                      1.0, fake, fake, 16, None) == _lib.DGQ_ERR_WORKSPACE_TOO_SMALL
    # misaligned input / bad strides / too many tokens for the batch
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert lib.dgq_compress(ctypes.byref(p), odd, fake, 1024, 128, fake, 1, 64, 64, fake, 4,
                            ctypes.byref(cache), fake, 1 << 30, None) == _lib.DGQ_ERR_INVALID_ARG
    assert lib.dgq_compress(ctypes.byref(p), fake, fake, 1020, 128, fake, 1, 64, 64, fake, 4,
                            ctypes.byref(cache), fake, 1 << 30, None) == _lib.DGQ_ERR_INVALID_ARG
    assert lib.dgq_compress(ctypes.byref(p), fake, fake, 1024, 128, fake, 1, 64, 65, fake, 4,
                            ctypes.byref(cache), fake, 1 << 30, None) == _lib.DGQ_ERR_INVALID_ARG
    # cache too small for the batch
    assert lib.dgq_compress(ctypes.byref(p), fake, fake, 1024, 128, fake, 5, 64, 64, fake, 4,
                            ctypes.byref(cache), fake, 1 << 30, None) == _lib.DGQ_ERR_INVALID_ARG
    # append without staging buffers
    nostage = _lib.Cache(fake, fake, fake, fake, fake, fake, None, None, fake, 64, 4)
    assert lib.dgq_append(ctypes.byref(p), fake, fake, fake, 1, fake, 4, ctypes.byref(nostage),
                          None) == _lib.DGQ_ERR_INVALID_ARG
    # an empty batch is a no-op
    assert lib.dgq_append(ctypes.byref(p), None, None, None, 0, None, 0, None, None) == 0
    # a batch beyond the launch grid's 65535 is refused before anything is touched
    big = _lib.Cache(fake, fake, fake, fake, fake, fake, fake, fake, fake, 64, 70000)
    assert lib.dgq_append(ctypes.byref(p), fake, fake, fake, 65536, fake, 4, ctypes.byref(big),
                          None) == _lib.DGQ_ERR_UNSUPPORTED
    assert lib.paged_decode_attn_int8(ctypes.byref(p), fake, ctypes.byref(big), fake, 4, fake, 65536, 64,
                                      1.0, fake, fake, 1 << 30, None) == _lib.DGQ_ERR_UNSUPPORTED


def _arr(*v):
    return (ctypes.c_int32 * max(len(v), 1))(*v)


def test_pool_reference_counts(lib):
    """Shared blocks: a block goes back on the free list when its last reference is dropped."""
    h = ctypes.c_void_p()
    assert lib.dgq_pool_create(6, ctypes.byref(h)) == 0
    ids = (ctypes.c_int32 * 6)()
    assert lib.dgq_block_alloc(h, 3, ids) == 0 and list(ids[:3]) == [0, 1, 2]
    assert [lib.dgq_block_refcount(h, i) for i in range(6)] == [1, 1, 1, 0, 0, 0]
    assert lib.dgq_block_share(h, 3, _arr(0, 1, 1)) == 0
    assert [lib.dgq_block_refcount(h, i) for i in range(3)] == [2, 3, 1]
    # sharing a free or out-of-range block fails and changes nothing
    assert lib.dgq_block_share(h, 2, _arr(0, 4)) == _lib.DGQ_ERR_INVALID_ARG
    assert lib.dgq_block_share(h, 1, _arr(-1)) == _lib.DGQ_ERR_INVALID_ARG
    assert [lib.dgq_block_refcount(h, i) for i in range(3)] == [2, 3, 1]
    # one reference per listed entry; more entries than references is rejected as a whole
    assert lib.dgq_block_free(h, 4, _arr(1, 1, 1, 1)) == _lib.DGQ_ERR_INVALID_ARG
    assert lib.dgq_block_free(h, 2, _arr(1, 1)) == 0
    assert lib.dgq_block_refcount(h, 1) == 1 and lib.dgq_pool_num_free(h) == 3
    assert lib.dgq_block_free(h, 1, _arr(1)) == 0
    assert lib.dgq_block_refcount(h, 1) == 0 and lib.dgq_pool_num_free(h) == 4
    assert lib.dgq_block_refcount(h, 6) == -1 and lib.dgq_block_refcount(None, 0) == -1
    assert lib.dgq_pool_destroy(h) == 0


def test_pool_copy_on_write(lib):
    h = ctypes.c_void_p()
    assert lib.dgq_pool_create(4, ctypes.byref(h)) == 0
    ids = (ctypes.c_int32 * 4)()
    assert lib.dgq_block_alloc(h, 2, ids) == 0             # 0, 1
    assert lib.dgq_block_share(h, 2, _arr(0, 0)) == 0      # block 0: three owners
    out = (ctypes.c_int32 * 4)()
    # entries in order: the first two owners of block 0 get fresh blocks, the last keeps it;
    # block 1 has one owner and is kept
    assert lib.dgq_block_cow(h, 4, _arr(0, 1, 0, 0), out) == 0
    assert list(out) == [2, 1, 3, 0]
    assert [lib.dgq_block_refcount(h, i) for i in range(4)] == [1, 1, 1, 1]
    assert lib.dgq_pool_num_free(h) == 0
    # a copy that needs a block from an empty pool changes nothing
    assert lib.dgq_block_share(h, 1, _arr(3)) == 0
    assert lib.dgq_block_cow(h, 2, _arr(1, 3), out) == _lib.DGQ_ERR_POOL_EXHAUSTED
    assert lib.dgq_block_refcount(h, 3) == 2
    # a free block cannot be written through copy-on-write
    assert lib.dgq_block_free(h, 1, _arr(2)) == 0
    assert lib.dgq_block_cow(h, 1, _arr(2), out) == _lib.DGQ_ERR_INVALID_ARG
    assert lib.dgq_block_cow(h, 1, _arr(3), out) == 0 and out[0] == 2
    assert lib.dgq_block_refcount(h, 3) == 1 and lib.dgq_block_refcount(h, 2) == 1
    # two writers for a block with one owner: refused, nothing changes
    assert lib.dgq_block_cow(h, 2, _arr(3, 3), out) == _lib.DGQ_ERR_INVALID_ARG
    assert lib.dgq_block_refcount(h, 3) == 1 and lib.dgq_pool_num_free(h) == 0
    assert lib.dgq_pool_destroy(h) == 0


def test_swap_image_bytes(lib):
    """State (segment rows, row counts, append states, K and V staging) then per block K codes,
    V codes and bits, each padded to 16 bytes."""
    for hkv, d, bs, cap in ((8, 128, 64, 16), (2, 64, 16, 5), (3, 64, 16, 7)):
        p = _params(num_kv_heads=hkv, num_q_heads=hkv, head_dim=d, block_size=bs, seg_capacity=cap,
                    max_segments=5)
        pad = lambda x: (x + 15) // 16 * 16
        state = pad(hkv * cap * 32) + pad(hkv * 4) + pad(hkv * 224) + 2 * pad(hkv * bs * d * 2)
        block = 2 * pad(hkv * bs * d) + pad(hkv * bs // 8)
        for n in (0, 1, 37):
            assert lib.dgq_swap_image_bytes(ctypes.byref(p), n) == state + n * block
    assert lib.dgq_swap_image_bytes(ctypes.byref(_params()), -1) == 0
    assert lib.dgq_swap_image_bytes(ctypes.byref(_params(head_dim=96)), 1) == 0


def test_lifecycle_argument_checks(lib):
    p = _params()
    fake = ctypes.c_void_p(1 << 20)
    cache = _lib.Cache(fake, fake, fake, fake, fake, fake, fake, fake, fake, 64, 4)
    nostage = _lib.Cache(fake, fake, fake, fake, fake, fake, None, None, fake, 64, 4)
    need = lib.dgq_swap_image_bytes(ctypes.byref(p), 3)
    E = _lib.DGQ_ERR_INVALID_ARG
    assert lib.dgq_copy_blocks(ctypes.byref(p), ctypes.byref(cache), fake, fake, 0, None) == 0
    assert lib.dgq_copy_blocks(ctypes.byref(p), ctypes.byref(cache), None, fake, 2, None) == E
    assert lib.dgq_copy_blocks(ctypes.byref(p), ctypes.byref(cache), fake, fake, -1, None) == E
    assert lib.dgq_copy_seq_state(ctypes.byref(p), ctypes.byref(nostage), fake, fake, 1, None) == E
    assert lib.dgq_copy_seq_state(ctypes.byref(_params(block_size=48)), ctypes.byref(cache), fake, fake, 1,
                                  None) == _lib.DGQ_ERR_UNSUPPORTED
    for row in (-1, 4):
        assert lib.dgq_swap_out(ctypes.byref(p), ctypes.byref(cache), row, fake, 3, fake, need, None, None) == E
        assert lib.dgq_swap_in(ctypes.byref(p), ctypes.byref(cache), row, fake, 3, fake, need, None, None) == E
    assert lib.dgq_swap_out(ctypes.byref(p), ctypes.byref(cache), 0, fake, 3, fake, need - 16, None,
                            None) == _lib.DGQ_ERR_WORKSPACE_TOO_SMALL
    assert lib.dgq_swap_in(ctypes.byref(p), ctypes.byref(cache), 0, None, 3, fake, need, None, None) == E
    assert lib.dgq_swap_in(ctypes.byref(p), ctypes.byref(cache), 0, fake, 3, ctypes.c_void_p((1 << 20) + 8),
                           need, None, None) == E
    assert lib.dgq_swap_out(ctypes.byref(p), ctypes.byref(nostage), 0, fake, 3, fake, need, None, None) == E


def test_block_size_32_accepted_except_group64(lib):
    """32-token blocks are valid for the DGQ calls; the group-64 baseline refuses them before any
    HIP call."""
    p = _params(block_size=32)
    assert lib.dgq_compress_workspace_size(ctypes.byref(p), 1, 100, 100) > 0
    assert lib.dgq_decode_workspace_size(ctypes.byref(p), 1, 100) > 0
    fake = ctypes.c_void_p(1 << 20)
    g = _lib.G64Cache(fake, fake, fake, fake, fake, 64, 0)
    U = _lib.DGQ_ERR_UNSUPPORTED
    assert lib.dgq_g64_quantize(ctypes.byref(p), fake, fake, 1024, 128, fake, None, 1, 64, 64, fake, 4, 128,
                                ctypes.byref(g), None) == U
    assert lib.paged_decode_attn_g64(ctypes.byref(p), fake, ctypes.byref(g), fake, 4, fake, 1, 128, 1.0, fake,
                                     fake, 1 << 20, None) == U
    assert lib.dgq_swap_image_bytes(ctypes.byref(p), 10) > 0


def test_marker_format_checks(lib):
    """The marker format needs no bit tensor; the bitmap format does; the marker read-back is
    refused for a bitmap-format cache."""
    fake = ctypes.c_void_p(1 << 20)
    nobits = _lib.Cache(fake, fake, None, fake, fake, fake, fake, fake, fake, 64, 4)
    E = _lib.DGQ_ERR_INVALID_ARG
    bitmap, marker = _params(), _params(flags=_lib.DGQ_FORMAT_MARKER)
    # bitmap: a missing bit tensor is rejected before anything is queued
    assert lib.dgq_append(ctypes.byref(bitmap), fake, fake, fake, 1, fake, 4, ctypes.byref(nobits), None) == E
    assert lib.dgq_marker_bits(ctypes.byref(bitmap), ctypes.byref(nobits), fake, 4, fake, 1, 64, fake, None) == E
    # marker: the same cache passes the bit-tensor check and fails only on the later ones
    assert lib.dgq_marker_bits(ctypes.byref(marker), ctypes.byref(nobits), fake, 4, None, 1, 64, fake, None) == E
    assert lib.dgq_marker_bits(ctypes.byref(marker), ctypes.byref(nobits), fake, 4, fake, 1, 65, fake, None) == E
    assert lib.dgq_marker_bits(ctypes.byref(marker), ctypes.byref(nobits), fake, 4, fake, 0, 64, None, None) == 0
    assert lib.paged_decode_attn_int8(ctypes.byref(marker), fake, ctypes.byref(nobits), fake, 4, fake, 1, 64,
                                      1.0, fake, fake, 16, None) == _lib.DGQ_ERR_WORKSPACE_TOO_SMALL
    # swap images carry no bits in the marker format
    pb = lib.dgq_swap_image_bytes(ctypes.byref(bitmap), 10)
    pm = lib.dgq_swap_image_bytes(ctypes.byref(marker), 10)
    assert pb - pm == 10 * 16          # 8 heads x 16 tokens / 8 = 16 bytes of bits per block


def test_noalloc_decode_refuses_beyond_scratch(lib):
    """The allocation-free decode refuses, on the host and before any HIP call, a batch whose
    partials exceed its fixed scratch array (DGQ_NOALLOC_SCRATCH_BYTES)."""
    p = _params(num_kv_heads=32, num_q_heads=32)
    fake = ctypes.c_void_p(1 << 20)
    big_batch = 4096                         # 4096 x 32 heads x (128 + 2) x 4 B > 16 MiB
    cache = _lib.Cache(fake, fake, fake, fake, fake, fake, fake, fake, fake, 64, big_batch)
    assert lib.paged_decode_attn_int8_noalloc(ctypes.byref(p), fake, ctypes.byref(cache), fake, 4, fake,
                                              big_batch, 64, 0.1, fake, None) == _lib.DGQ_ERR_WORKSPACE_TOO_SMALL
    # the usual argument checks come first
    assert lib.paged_decode_attn_int8_noalloc(ctypes.byref(p), None, ctypes.byref(cache), fake, 4, fake,
                                              1, 64, 0.1, fake, None) == _lib.DGQ_ERR_INVALID_ARG
    assert lib.paged_decode_attn_int8_noalloc(ctypes.byref(p), fake, ctypes.byref(cache), fake, 4, fake,
                                              1, 65, 0.1, fake, None) == _lib.DGQ_ERR_INVALID_ARG
    assert _lib.DGQ_NOALLOC_SCRATCH_BYTES == 16 << 20
