"""MI355X-native dynamic-group INT8 KV-cache compression (DGQ) with paged INT8 decode attention.

The compute lives in ``libdgq.so`` (hand-written HIP for gfx950, C ABI in ``include/dgq.h``);
this package is its Python binding.  Importing it does not load the library; the first call
does, and fails loudly if it is not built.
"""

from ._lib import (DGQ_OP_APPEND, DGQ_OP_APPEND_DECODE, DGQ_OP_COMPRESS, DGQ_OP_DECODE,  # noqa: F401
                   DGQ_OP_G64_DECODE, DGQError, EXPORTS, LIB_PATH, load)
from .api import (  # noqa: F401
    BlockPool,
    DGQCache,
    DGQG64Cache,
    DGQParams,
    compress_workspace_size,
    decode_workspace_size,
    dgq_append,
    dgq_append_decode,
    dgq_compress,
    dgq_copy_blocks,
    dgq_copy_seq_state,
    dgq_marker_bits,
    dgq_swap_in,
    dgq_swap_out,
    dgq_g64_quantize,
    paged_decode_attn_g64,
    paged_decode_attn_int8,
    paged_decode_attn_int8_noalloc,
    swap_image_bytes,
    workspace,
    workspace_size,
)
