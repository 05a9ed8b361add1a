// Internal declarations shared by the libdgq translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "dgq.h"

namespace dgq {

constexpr int kWin = 16;          // sliding-window length (DGQ article 2.2)
constexpr int kChunk = 64;        // tokens per decode / encode chunk
constexpr int kMaxSegCap = 64;    // segment-table rows per (sequence, kv head), upper bound
constexpr int kMaxCuts = 7;       // max_segments <= 8

// The variance floor on the window-statistic scale: Q = N^2 * 512^2 * (population variance of the
// window), N = 16 * head_dim, so the floor is min_var * N^2 * 2^18 (an exact power-of-two scaling).
inline double variance_floor_q(double min_var, int head_dim) {
  const double n = 16.0 * head_dim;
  return min_var * (n * n) * 262144.0;
}

// Most segments a sequence of L tokens may get under the length-aware policy (DGQ article 3.2):
// 2 below 2048 tokens, 3 below 16384, else floor(log2(L / 1024)) + 2, at most 5.
__host__ __device__ inline int length_aware_cap(int L) {
  if (L < 2048) return 2;
  if (L < 16384) return 3;
  int lg = 0;
  for (int x = L; x > 1; x >>= 1) ++lg;   // floor(log2 L)
  return lg - 10 + 2 < 5 ? lg - 10 + 2 : 5;
}

// Record a HIP failure for dgq_last_error(); returns DGQ_ERR_HIP.
dgq_status_t hip_fail(hipError_t err, const char *where);

// Check the last launch on this thread.
inline dgq_status_t check_launch(const char *where) {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? DGQ_OK : hip_fail(e, where);
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// How codes are stored.  Bitmap format: 255 steps between min and max, the minimum at code -128,
// the identifier in the bit tensor.  Marker format (DGQ article 3.2): 253 steps, the minimum at
// -127, the two end byte values free for the markers that replace the first key byte of a segment.
struct CodeFormat {
  float levels;    // steps between min and max
  int32_t low;     // code of the minimum
  int32_t marker;  // 1: marker format
};
inline CodeFormat code_format(const dgq_params_t *p) {
  const bool m = (p->flags & DGQ_FORMAT_MARKER) != 0;
  return CodeFormat{m ? 253.0f : 255.0f, m ? -127 : -128, m ? 1 : 0};
}

// ---- decode ----
struct DecodePlan {
  int part_tokens;  // tokens per workgroup, multiple of kChunk
  int nparts;       // partitions per sequence at max_seq_len
};
// Waves a decode launch aims at: the DGQ decode runs one 4-wave workgroup per CU; the group-64
// baseline does more work per chunk and wants two.
constexpr int64_t kDgqDecodeWaves = 1024;
constexpr int64_t kG64DecodeWaves = 2048;
DecodePlan decode_plan(const dgq_params_t *p, int32_t batch, int32_t max_seq_len, int64_t target_waves);
size_t decode_workspace_bytes(const dgq_params_t *p, int32_t batch, int32_t max_seq_len);
// Workspace bytes one decoder's launch plan (target_waves) uses.
size_t decode_workspace_bytes_for(const dgq_params_t *p, int32_t batch, int32_t max_seq_len,
                                  int64_t target_waves);

dgq_status_t launch_decode(const dgq_params_t *p, const uint16_t *q, const dgq_cache_t *cache,
                           const int32_t *block_table, int32_t max_blocks,
                           const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                           float softmax_scale, float *out, void *ws, hipStream_t stream);

// ---- compress ----
struct CompressLayout {
  size_t a_off, b_off, score_off, ext_off, tile_off, text_off, map_off, total;
  int nsub;    // 16-token sub-blocks per sequence at max_seq_len
  int ntile;   // 256-candidate tiles per sequence at max_seq_len
  int64_t map_tiles;   // bound on the batch's real 64-token tiles: total_tokens / 64 + batch
};
CompressLayout compress_layout(const dgq_params_t *p, int32_t batch, int64_t total_tokens,
                               int32_t max_seq_len);

dgq_status_t launch_compress(const dgq_params_t *p, const uint16_t *k, const uint16_t *v,
                             int64_t stride_tok, int64_t stride_head, const int32_t *cu_seqlens,
                             int32_t batch, int32_t max_seq_len, int64_t total_tokens,
                             const int32_t *block_table, int32_t max_blocks,
                             const dgq_cache_t *cache, void *ws, hipStream_t stream);

// ---- append ----
dgq_status_t launch_append_decode(const dgq_params_t *p, const uint16_t *k_tok, const uint16_t *v_tok,
                                  const int32_t *seq_lens, const uint16_t *q, int32_t batch,
                                  const int32_t *block_table, int32_t max_blocks, int32_t max_seq_len,
                                  float softmax_scale, const dgq_cache_t *cache, float *out, void *ws,
                                  hipStream_t stream);
dgq_status_t launch_append(const dgq_params_t *p, const uint16_t *k_tok, const uint16_t *v_tok,
                           const int32_t *seq_lens, int32_t batch, const int32_t *block_table,
                           int32_t max_blocks, const dgq_cache_t *cache, hipStream_t stream);

// ---- fixed 64-channel group baseline ----
dgq_status_t launch_g64_quantize(const dgq_params_t *p, const uint16_t *k, const uint16_t *v,
                                 int64_t stride_tok, int64_t stride_head, const int32_t *cu_seqlens,
                                 const int32_t *first_pos, int32_t batch, int32_t max_rows,
                                 int64_t total_rows, const int32_t *block_table, int32_t max_blocks,
                                 int32_t max_seq_len, const dgq_g64_cache_t *cache, hipStream_t stream);
dgq_status_t launch_g64_decode(const dgq_params_t *p, const uint16_t *q, const dgq_g64_cache_t *cache,
                               const int32_t *block_table, int32_t max_blocks, const int32_t *seq_lens,
                               int32_t batch, int32_t max_seq_len, float softmax_scale, float *out,
                               void *ws, hipStream_t stream);

}  // namespace dgq

// ---- device helpers ----
#if defined(__HIPCC__)
namespace dgq {

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  union { uint16_t u; _Float16 f; } c;
  c.u = (uint16_t)h;
  return (float)c.f;
}

// Byte offset of (token tau of its block, channel d) inside one (block, head) K tile.  A 32-token
// block is two 16-token tiles one after the other.
template <int D, int BS>
__device__ __forceinline__ int k_tile_offset(int tau, int d) {
  constexpr int M = D / 64;
  const int m = d >> 6, j = (d & 63) >> 4, e = d & 15;
  if constexpr (BS == 32) {
    return (tau >> 4) * (16 * D) + k_tile_offset<D, 16>(tau & 15, d);
  } else if constexpr (BS == 64) {
    const int T = tau >> 4, r = tau & 15;
    return (((T * M + m) * 4 + j) * 16 + r) * 16 + e;
  } else {
    const int T = tau >> 2, i = tau & 3;
    return ((((T * M + m) * 4 + j) * 4 + i) * 16) + e;
  }
}

// Byte offset of (token tau, channel d) inside one (block, head) V tile (32-token blocks: two
// 16-token tiles).
template <int D, int BS>
__device__ __forceinline__ int v_tile_offset(int tau, int d) {
  if constexpr (BS == 32) {
    return (tau >> 4) * (16 * D) + v_tile_offset<D, 16>(tau & 15, d);
  } else if constexpr (BS == 64) {
    const int n = d >> 4, r = d & 15, j = (tau & 15) >> 2, e = ((tau >> 4) << 2) | (tau & 3);
    return ((n * 4 + j) * 16 + r) * 16 + e;
  } else {
    return d * 16 + tau;
  }
}

// DGQ code of one value (exact IEEE steps: subtract, multiply, round to nearest even, clamp to
// [0, levels], shift by the code of the minimum).
__device__ __forceinline__ int dgq_encode_value(float x, float mn, float inv, float levels = 255.0f,
                                                int low = -128) {
#pragma clang fp contract(off)
  const float dlt = x - mn;
  const float u = dlt * inv;
  float r = __builtin_rintf(u);
  r = fminf(fmaxf(r, 0.0f), levels);
  return (int)r + low;
}

// fp32(levels / fp32(mx - mn)), or 0 for an empty range.  The float64 quotient rounded to float32
// equals the correctly rounded float32 quotient (53 >= 2*24 + 2 bits).
__device__ __forceinline__ float dgq_inv(float mn, float mx, float levels = 255.0f) {
#pragma clang fp contract(off)
  const float diff = mx - mn;
  return diff > 0.0f ? (float)((double)levels / (double)diff) : 0.0f;
}

// fp32(fp32(mx - mn) / levels), correctly rounded by the same argument.
__device__ __forceinline__ float dgq_scale(float mn, float mx, float levels = 255.0f) {
#pragma clang fp contract(off)
  const float diff = mx - mn;
  return (float)((double)diff / (double)levels);
}

// Marker byte that replaces the code byte c of a segment's first key element (marker format):
// 127 (0x7F) for a code in the upper half of the range, -128 (0x80) for one in the lower half.
__device__ __forceinline__ uint32_t dgq_marker_byte(uint32_t c) {
  return (c & 0x80u) ? 0x80u : 0x7Fu;
}

// Bounds of sequence b in the packed input, clamped so that no kernel reads past max_seq_len or
// the packed token count; an inconsistency is counted in status[2] (by the caller's lane 0).
__device__ __forceinline__ void seq_range(const int32_t *cu, int b, int max_seq_len, int64_t total,
                                          int &c0, int &L, bool &bad) {
  c0 = cu[b];
  const int c1 = cu[b + 1];
  L = c1 - c0;
  bad = false;
  if (c0 < 0 || L < 0 || (int64_t)c1 > total) {
    L = 0;
    c0 = 0;
    bad = true;
  } else if (L > max_seq_len) {
    L = max_seq_len;
    bad = true;
  }
}

// Physical block id, replaced by 0 (and flagged) when it is not a pool block.
__device__ __forceinline__ int checked_block(int id, int num_blocks, bool &bad) {
  if ((unsigned)id >= (unsigned)num_blocks) {
    bad = true;
    return 0;
  }
  return id;
}

// Buffer resource over `bytes` bytes at `base` (raw, untyped, 32-bit data format): loads past the
// end return zero without touching memory, stores past the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;   // a buffer offset past any resource used here

// Fixed-point image for the variance statistics: rint(clamp(x, -32, 32) * 512).
__device__ __forceinline__ int dgq_fixed_point(float x) {
  const float c = fminf(fmaxf(x, -32.0f), 32.0f);
  return (int)__builtin_rintf(c * 512.0f);
}

}  // namespace dgq
#endif
