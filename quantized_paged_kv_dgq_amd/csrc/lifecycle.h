// Internal declarations of the block-lifecycle launches (lifecycle.hip) and of the marker
// read-back (markers.hip); not part of the C ABI.
#pragma once

#include "dgq_internal.h"

namespace dgq {

size_t swap_image_bytes(const dgq_params_t *p, int32_t n_blocks);
dgq_status_t launch_copy_blocks(const dgq_params_t *p, const dgq_cache_t *cache, const int32_t *src,
                                const int32_t *dst, int32_t n, hipStream_t stream);
dgq_status_t launch_copy_seq_state(const dgq_params_t *p, const dgq_cache_t *cache, const int32_t *src,
                                   const int32_t *dst, int32_t n, hipStream_t stream);
// out: cache -> staging (-> host if not NULL); else (host ->) staging -> cache.
dgq_status_t launch_swap(const dgq_params_t *p, const dgq_cache_t *cache, int32_t row, const int32_t *ids,
                         int32_t n_blocks, void *staging, void *host, bool out, hipStream_t stream);

dgq_status_t launch_marker_bits(const dgq_params_t *p, const dgq_cache_t *cache, const int32_t *block_table,
                                int32_t max_blocks, const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                uint8_t *bits_out, hipStream_t stream);

}  // namespace dgq
