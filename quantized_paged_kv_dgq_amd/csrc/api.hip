// Exported C entry points of libdgq: argument checks on the host, then the kernel launches.
// Nothing is queued unless every check passes.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "dgq_internal.h"
#include "lifecycle.h"

namespace dgq {

static thread_local char g_last_error[256] = "";

dgq_status_t hip_fail(hipError_t err, const char *where) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", where, hipGetErrorString(err));
  return DGQ_ERR_HIP;
}

// Sequences are the z (or y) dimension of every launch grid, which holds at most 65535.
constexpr int32_t kMaxGridBatch = 65535;

static bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static dgq_status_t check_params(const dgq_params_t *p) {
  if (p == nullptr) return DGQ_ERR_INVALID_ARG;
  if (p->num_kv_heads < 1 || p->num_q_heads < 1 || p->num_q_heads % p->num_kv_heads != 0)
    return DGQ_ERR_INVALID_ARG;
  if (p->num_kv_heads > kMaxGridBatch) return DGQ_ERR_UNSUPPORTED;   // a launch-grid dimension too
  const int g = p->num_q_heads / p->num_kv_heads;
  if (g != 1 && g != 2 && g != 4) return DGQ_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return DGQ_ERR_UNSUPPORTED;
  if (p->block_size != 16 && p->block_size != 32 && p->block_size != 64) return DGQ_ERR_UNSUPPORTED;
  if (p->win != kWin) return DGQ_ERR_UNSUPPORTED;
  if (p->max_segments < 1 || p->max_segments > kMaxCuts + 1) return DGQ_ERR_INVALID_ARG;
  if (p->seg_capacity < p->max_segments || p->seg_capacity > kMaxSegCap) return DGQ_ERR_INVALID_ARG;
  if ((p->flags & ~(uint32_t)(DGQ_POLICY_LENGTH_AWARE | DGQ_FORMAT_MARKER | DGQ_COMPRESS_MULTIPASS)) != 0)
    return DGQ_ERR_INVALID_ARG;
  if (!std::isfinite(p->tau) || p->tau < 1.0) return DGQ_ERR_INVALID_ARG;
  if (!std::isfinite(p->min_var) || p->min_var < 0.0) return DGQ_ERR_INVALID_ARG;
  return DGQ_OK;
}

// The bit tensor is required in the bitmap format only.
static dgq_status_t check_cache(const dgq_params_t *p, const dgq_cache_t *c, int32_t batch, bool need_stage) {
  if (c == nullptr) return DGQ_ERR_INVALID_ARG;
  const bool need_bits = (p->flags & DGQ_FORMAT_MARKER) == 0;
  if (!c->k_pool || !c->v_pool || (need_bits && !c->bits) || !c->segs || !c->nseg || !c->tail || !c->status)
    return DGQ_ERR_INVALID_ARG;
  if (need_stage && (!c->k_stage || !c->v_stage)) return DGQ_ERR_INVALID_ARG;
  if (!aligned(c->k_pool, 16) || !aligned(c->v_pool, 16) || !aligned(c->segs, 16) ||
      !aligned(c->tail, 16) || !aligned(c->status, 8))
    return DGQ_ERR_INVALID_ARG;
  if (need_stage && (!aligned(c->k_stage, 16) || !aligned(c->v_stage, 16))) return DGQ_ERR_INVALID_ARG;
  if (c->num_blocks < 1 || c->batch < batch) return DGQ_ERR_INVALID_ARG;
  return DGQ_OK;
}

static dgq_status_t check_table(const dgq_params_t *p, const int32_t *block_table,
                                int32_t max_blocks, int32_t max_seq_len) {
  if (block_table == nullptr || max_blocks < 1 || max_seq_len < 0) return DGQ_ERR_INVALID_ARG;
  if ((int64_t)max_seq_len > (int64_t)max_blocks * p->block_size) return DGQ_ERR_INVALID_ARG;
  return DGQ_OK;
}

}  // namespace dgq

using namespace dgq;

extern "C" const char *dgq_status_string(int32_t status) {
  switch (status) {
    case DGQ_OK: return "ok";
    case DGQ_ERR_INVALID_ARG: return "invalid argument";
    case DGQ_ERR_UNSUPPORTED: return "unsupported shape";
    case DGQ_ERR_POOL_EXHAUSTED: return "block pool exhausted";
    case DGQ_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DGQ_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

extern "C" const char *dgq_last_error(void) { return g_last_error; }

extern "C" size_t dgq_compress_workspace_size(const dgq_params_t *p, int32_t batch,
                                              int64_t total_tokens, int32_t max_seq_len) {
  if (check_params(p) != DGQ_OK || batch < 0 || total_tokens < 0 || max_seq_len < 0) return 0;
  return compress_layout(p, batch, total_tokens, max_seq_len).total;
}

extern "C" size_t dgq_decode_workspace_size(const dgq_params_t *p, int32_t batch, int32_t max_seq_len) {
  if (check_params(p) != DGQ_OK || batch < 0 || max_seq_len < 0) return 0;
  return decode_workspace_bytes(p, batch, max_seq_len);
}

extern "C" size_t dgq_workspace_size(const dgq_params_t *p, int32_t op, int32_t batch, int64_t total_tokens,
                                     int32_t max_seq_len) {
  switch (op) {
    case DGQ_OP_COMPRESS: return dgq_compress_workspace_size(p, batch, total_tokens, max_seq_len);
    case DGQ_OP_APPEND: return 0;
    case DGQ_OP_DECODE:
    case DGQ_OP_APPEND_DECODE:
    case DGQ_OP_G64_DECODE: return dgq_decode_workspace_size(p, batch, max_seq_len);
    default: return 0;
  }
}

extern "C" dgq_status_t dgq_read_device_status(const dgq_cache_t *cache, unsigned long long *out,
                                               hipStream_t stream) {
  if (cache == nullptr || cache->status == nullptr || out == nullptr) return DGQ_ERR_INVALID_ARG;
  hipError_t e = hipMemcpyAsync(out, cache->status, 4 * sizeof(unsigned long long), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "dgq_read_device_status copy");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "dgq_read_device_status synchronize");
  return DGQ_OK;
}

extern "C" dgq_status_t dgq_compress(const dgq_params_t *p, const uint16_t *k, const uint16_t *v,
                                     int64_t stride_tok, int64_t stride_head,
                                     const int32_t *cu_seqlens, int32_t batch, int32_t max_seq_len,
                                     int64_t total_tokens, const int32_t *block_table,
                                     int32_t max_blocks, const dgq_cache_t *cache, void *ws,
                                     size_t ws_bytes, hipStream_t stream) {
  dgq_status_t st = check_params(p);
  if (st != DGQ_OK) return st;
  if (batch < 0 || max_seq_len < 0 || total_tokens < 0) return DGQ_ERR_INVALID_ARG;
  if (batch == 0) return DGQ_OK;
  if (batch > kMaxGridBatch) return DGQ_ERR_UNSUPPORTED;
  if (total_tokens > (int64_t)batch * max_seq_len || total_tokens >= (int64_t)1 << 31)
    return DGQ_ERR_INVALID_ARG;
  if (!k || !v || !cu_seqlens || !aligned(k, 16) || !aligned(v, 16)) return DGQ_ERR_INVALID_ARG;
  if (stride_tok <= 0 || stride_head < 0 || stride_tok % 8 != 0 || stride_head % 8 != 0)
    return DGQ_ERR_INVALID_ARG;
  if (p->num_kv_heads > 1 && stride_head < p->head_dim && stride_tok < (int64_t)p->num_kv_heads * p->head_dim)
    return DGQ_ERR_INVALID_ARG;
  if ((st = check_table(p, block_table, max_blocks, max_seq_len)) != DGQ_OK) return st;
  if ((st = check_cache(p, cache, batch, false)) != DGQ_OK) return st;
  const size_t need = compress_layout(p, batch, total_tokens, max_seq_len).total;
  if (ws == nullptr || !aligned(ws, 256)) return DGQ_ERR_INVALID_ARG;
  if (ws_bytes < need) return DGQ_ERR_WORKSPACE_TOO_SMALL;
  return launch_compress(p, k, v, stride_tok, stride_head, cu_seqlens, batch, max_seq_len,
                         total_tokens, block_table, max_blocks, cache, ws, stream);
}

extern "C" dgq_status_t dgq_append(const dgq_params_t *p, const uint16_t *k_tok,
                                   const uint16_t *v_tok, const int32_t *seq_lens, int32_t batch,
                                   const int32_t *block_table, int32_t max_blocks,
                                   const dgq_cache_t *cache, hipStream_t stream) {
  dgq_status_t st = check_params(p);
  if (st != DGQ_OK) return st;
  if (batch < 0) return DGQ_ERR_INVALID_ARG;
  if (batch == 0) return DGQ_OK;
  if (batch > kMaxGridBatch) return DGQ_ERR_UNSUPPORTED;
  if (!k_tok || !v_tok || !seq_lens || !aligned(k_tok, 16) || !aligned(v_tok, 16)) return DGQ_ERR_INVALID_ARG;
  if (block_table == nullptr || max_blocks < 1) return DGQ_ERR_INVALID_ARG;
  if ((st = check_cache(p, cache, batch, true)) != DGQ_OK) return st;
  return launch_append(p, k_tok, v_tok, seq_lens, batch, block_table, max_blocks, cache, stream);
}

extern "C" dgq_status_t paged_decode_attn_int8(const dgq_params_t *p, const uint16_t *q,
                                               const dgq_cache_t *cache, const int32_t *block_table,
                                               int32_t max_blocks, const int32_t *seq_lens,
                                               int32_t batch, int32_t max_seq_len,
                                               float softmax_scale, float *out, void *ws,
                                               size_t ws_bytes, hipStream_t stream) {
  dgq_status_t st = check_params(p);
  if (st != DGQ_OK) return st;
  if (batch < 0 || max_seq_len < 0) return DGQ_ERR_INVALID_ARG;
  if (batch == 0) return DGQ_OK;
  if (batch > kMaxGridBatch) return DGQ_ERR_UNSUPPORTED;
  if (!q || !out || !seq_lens || !aligned(q, 16) || !aligned(out, 16)) return DGQ_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return DGQ_ERR_INVALID_ARG;
  if ((st = check_table(p, block_table, max_blocks, max_seq_len)) != DGQ_OK) return st;
  if ((st = check_cache(p, cache, batch, false)) != DGQ_OK) return st;
  const size_t need = decode_workspace_bytes(p, batch, max_seq_len);
  if (ws == nullptr || !aligned(ws, 256)) return DGQ_ERR_INVALID_ARG;
  if (ws_bytes < need) return DGQ_ERR_WORKSPACE_TOO_SMALL;
  return launch_decode(p, q, cache, block_table, max_blocks, seq_lens, batch, max_seq_len,
                       softmax_scale, out, ws, stream);
}

// ---- Allocation-free decode: the split-sequence partials and completion counters live in a
// file-scope device array instead of a caller workspace.  Each device that runs the call holds its
// own copy of the array until the process ends.  In host code `scratch` only names the array's
// host-side stand-in; its device address comes from hipGetSymbolAddress, once per device. ----

constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static_assert(kNoAllocScratchBytes == DGQ_NOALLOC_SCRATCH_BYTES, "header and library disagree");
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, set up on first use

// The device address of `scratch` on device `dev`, looked up with `dev` current (the calling
// thread's current device is restored afterwards).
dgq_status_t scratch_address(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return DGQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (e2 != hipSuccess) return hip_fail(e2, "hipSetDevice");
    if (ptr == nullptr || !aligned(ptr, 256)) return hip_fail(hipErrorInvalidSymbol, "scratch address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DGQ_OK;
}

// Zero n 32-bit words (the merge's completion counters) with a kernel, so that the clearing is
// an ordinary stream-ordered launch (also inside a captured graph).
__global__ void __launch_bounds__(256) zero_words_kernel(unsigned *w, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) w[i] = 0u;
}

}  // namespace

extern "C" dgq_status_t paged_decode_attn_int8_noalloc(const dgq_params_t *p, const uint16_t *q,
                                                       const dgq_cache_t *cache,
                                                       const int32_t *block_table, int32_t max_blocks,
                                                       const int32_t *seq_lens, int32_t batch,
                                                       int32_t max_seq_len, float softmax_scale,
                                                       float *out, hipStream_t stream) {
  dgq_status_t st = check_params(p);
  if (st != DGQ_OK) return st;
  if (batch < 0 || max_seq_len < 0) return DGQ_ERR_INVALID_ARG;
  if (batch == 0) return DGQ_OK;
  if (batch > kMaxGridBatch) return DGQ_ERR_UNSUPPORTED;
  if (!q || !out || !seq_lens || !aligned(q, 16) || !aligned(out, 16)) return DGQ_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return DGQ_ERR_INVALID_ARG;
  if ((st = check_table(p, block_table, max_blocks, max_seq_len)) != DGQ_OK) return st;
  if ((st = check_cache(p, cache, batch, false)) != DGQ_OK) return st;
  if (decode_workspace_bytes_for(p, batch, max_seq_len, kDgqDecodeWaves) > kNoAllocScratchBytes)
    return DGQ_ERR_WORKSPACE_TOO_SMALL;
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  void *ws = nullptr;
  if ((st = scratch_address(dev, &ws)) != DGQ_OK) return st;
  const int nctr = batch * p->num_kv_heads;
  hipLaunchKernelGGL(zero_words_kernel, dim3((nctr + 255) / 256), dim3(256), 0, stream,
                     reinterpret_cast<unsigned *>(ws), nctr);
  if ((st = check_launch("paged_decode_attn_int8_noalloc clear")) != DGQ_OK) return st;
  return launch_decode(p, q, cache, block_table, max_blocks, seq_lens, batch, max_seq_len,
                       softmax_scale, out, ws, stream);
}

extern "C" dgq_status_t dgq_append_decode(const dgq_params_t *p, const uint16_t *k_tok,
                                          const uint16_t *v_tok, const int32_t *seq_lens,
                                          const uint16_t *q, int32_t batch, const int32_t *block_table,
                                          int32_t max_blocks, int32_t max_seq_len, float softmax_scale,
                                          const dgq_cache_t *cache, float *out, void *ws,
                                          size_t ws_bytes, hipStream_t stream) {
  dgq_status_t st = check_params(p);
  if (st != DGQ_OK) return st;
  if (batch < 0 || max_seq_len < 1) return DGQ_ERR_INVALID_ARG;
  if (batch == 0) return DGQ_OK;
  if (batch > kMaxGridBatch) return DGQ_ERR_UNSUPPORTED;
  if (!k_tok || !v_tok || !aligned(k_tok, 16) || !aligned(v_tok, 16)) return DGQ_ERR_INVALID_ARG;
  if (!q || !out || !seq_lens || !aligned(q, 16) || !aligned(out, 16)) return DGQ_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return DGQ_ERR_INVALID_ARG;
  if ((st = check_table(p, block_table, max_blocks, max_seq_len)) != DGQ_OK) return st;
  if ((st = check_cache(p, cache, batch, true)) != DGQ_OK) return st;
  const size_t need = decode_workspace_bytes(p, batch, max_seq_len);
  if (ws == nullptr || !aligned(ws, 256)) return DGQ_ERR_INVALID_ARG;
  if (ws_bytes < need) return DGQ_ERR_WORKSPACE_TOO_SMALL;
  return launch_append_decode(p, k_tok, v_tok, seq_lens, q, batch, block_table, max_blocks, max_seq_len,
                              softmax_scale, cache, out, ws, stream);
}

extern "C" dgq_status_t dgq_copy_blocks(const dgq_params_t *p, const dgq_cache_t *cache,
                                        const int32_t *src_ids, const int32_t *dst_ids, int32_t n,
                                        hipStream_t stream) {
  dgq_status_t st = check_params(p);
  if (st != DGQ_OK) return st;
  if (n < 0) return DGQ_ERR_INVALID_ARG;
  if (n == 0) return DGQ_OK;
  if (!src_ids || !dst_ids) return DGQ_ERR_INVALID_ARG;
  if ((st = check_cache(p, cache, 0, false)) != DGQ_OK) return st;
  return launch_copy_blocks(p, cache, src_ids, dst_ids, n, stream);
}

extern "C" dgq_status_t dgq_copy_seq_state(const dgq_params_t *p, const dgq_cache_t *cache,
                                           const int32_t *src_rows, const int32_t *dst_rows, int32_t n,
                                           hipStream_t stream) {
  dgq_status_t st = check_params(p);
  if (st != DGQ_OK) return st;
  if (n < 0) return DGQ_ERR_INVALID_ARG;
  if (n == 0) return DGQ_OK;
  if (!src_rows || !dst_rows) return DGQ_ERR_INVALID_ARG;
  if ((st = check_cache(p, cache, 0, true)) != DGQ_OK) return st;
  return launch_copy_seq_state(p, cache, src_rows, dst_rows, n, stream);
}

extern "C" size_t dgq_swap_image_bytes(const dgq_params_t *p, int32_t n_blocks) {
  if (check_params(p) != DGQ_OK || n_blocks < 0) return 0;
  return swap_image_bytes(p, n_blocks);
}

static dgq_status_t check_swap(const dgq_params_t *p, const dgq_cache_t *cache, int32_t row,
                               const int32_t *ids, int32_t n_blocks, const void *staging,
                               size_t staging_bytes) {
  dgq_status_t st = check_params(p);
  if (st != DGQ_OK) return st;
  if ((st = check_cache(p, cache, 0, true)) != DGQ_OK) return st;
  if (row < 0 || row >= cache->batch || n_blocks < 0 || (n_blocks > 0 && ids == nullptr))
    return DGQ_ERR_INVALID_ARG;
  if (staging == nullptr || !aligned(staging, 16)) return DGQ_ERR_INVALID_ARG;
  if (staging_bytes < swap_image_bytes(p, n_blocks)) return DGQ_ERR_WORKSPACE_TOO_SMALL;
  return DGQ_OK;
}

extern "C" dgq_status_t dgq_swap_out(const dgq_params_t *p, const dgq_cache_t *cache, int32_t row,
                                     const int32_t *ids, int32_t n_blocks, void *staging,
                                     size_t staging_bytes, void *host_dst, hipStream_t stream) {
  const dgq_status_t st = check_swap(p, cache, row, ids, n_blocks, staging, staging_bytes);
  if (st != DGQ_OK) return st;
  return launch_swap(p, cache, row, ids, n_blocks, staging, host_dst, true, stream);
}

extern "C" dgq_status_t dgq_swap_in(const dgq_params_t *p, const dgq_cache_t *cache, int32_t row,
                                    const int32_t *ids, int32_t n_blocks, void *staging,
                                    size_t staging_bytes, const void *host_src, hipStream_t stream) {
  const dgq_status_t st = check_swap(p, cache, row, ids, n_blocks, staging, staging_bytes);
  if (st != DGQ_OK) return st;
  return launch_swap(p, cache, row, ids, n_blocks, staging, const_cast<void *>(host_src), false, stream);
}

extern "C" dgq_status_t dgq_marker_bits(const dgq_params_t *p, const dgq_cache_t *cache,
                                        const int32_t *block_table, int32_t max_blocks,
                                        const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                        uint8_t *bits_out, hipStream_t stream) {
  dgq_status_t st = check_params(p);
  if (st != DGQ_OK) return st;
  if ((p->flags & DGQ_FORMAT_MARKER) == 0) return DGQ_ERR_INVALID_ARG;
  if (batch < 0 || max_seq_len < 0) return DGQ_ERR_INVALID_ARG;
  if (batch == 0) return DGQ_OK;
  if (batch > kMaxGridBatch) return DGQ_ERR_UNSUPPORTED;
  if (!seq_lens || !bits_out) return DGQ_ERR_INVALID_ARG;
  if ((st = check_table(p, block_table, max_blocks, max_seq_len)) != DGQ_OK) return st;
  if ((st = check_cache(p, cache, batch, false)) != DGQ_OK) return st;
  return launch_marker_bits(p, cache, block_table, max_blocks, seq_lens, batch, max_seq_len, bits_out, stream);
}

static dgq_status_t check_g64_cache(const dgq_g64_cache_t *c) {
  if (c == nullptr || !c->k_pool || !c->v_pool || !c->k_range || !c->v_range || !c->status) return DGQ_ERR_INVALID_ARG;
  if (!aligned(c->k_pool, 16) || !aligned(c->v_pool, 16) || !aligned(c->k_range, 4) ||
      !aligned(c->v_range, 4) || !aligned(c->status, 8) || c->num_blocks < 1)
    return DGQ_ERR_INVALID_ARG;
  return DGQ_OK;
}

extern "C" dgq_status_t dgq_g64_quantize(const dgq_params_t *p, const uint16_t *k, const uint16_t *v,
                                         int64_t stride_tok, int64_t stride_head,
                                         const int32_t *cu_seqlens, const int32_t *first_pos,
                                         int32_t batch, int32_t max_rows, int64_t total_rows,
                                         const int32_t *block_table, int32_t max_blocks,
                                         int32_t max_seq_len, const dgq_g64_cache_t *cache,
                                         hipStream_t stream) {
  dgq_status_t st = check_params(p);
  if (st != DGQ_OK) return st;
  if (p->block_size == 32) return DGQ_ERR_UNSUPPORTED;   // the group-64 baseline keeps 16 and 64
  if (batch < 0 || max_rows < 0 || total_rows < 0 || max_seq_len < 0) return DGQ_ERR_INVALID_ARG;
  if (batch == 0) return DGQ_OK;
  if (batch > kMaxGridBatch) return DGQ_ERR_UNSUPPORTED;
  if (total_rows > (int64_t)batch * max_rows || total_rows >= (int64_t)1 << 31) return DGQ_ERR_INVALID_ARG;
  if (!k || !v || !cu_seqlens || !aligned(k, 16) || !aligned(v, 16)) return DGQ_ERR_INVALID_ARG;
  if (stride_tok <= 0 || stride_head < 0 || stride_tok % 8 != 0 || stride_head % 8 != 0) return DGQ_ERR_INVALID_ARG;
  if ((st = check_table(p, block_table, max_blocks, max_seq_len)) != DGQ_OK) return st;
  if ((st = check_g64_cache(cache)) != DGQ_OK) return st;
  return launch_g64_quantize(p, k, v, stride_tok, stride_head, cu_seqlens, first_pos, batch, max_rows,
                             total_rows, block_table, max_blocks, max_seq_len, cache, stream);
}

extern "C" dgq_status_t paged_decode_attn_g64(const dgq_params_t *p, const uint16_t *q,
                                              const dgq_g64_cache_t *cache, const int32_t *block_table,
                                              int32_t max_blocks, const int32_t *seq_lens, int32_t batch,
                                              int32_t max_seq_len, float softmax_scale, float *out,
                                              void *ws, size_t ws_bytes, hipStream_t stream) {
  dgq_status_t st = check_params(p);
  if (st != DGQ_OK) return st;
  if (p->block_size == 32) return DGQ_ERR_UNSUPPORTED;   // the group-64 baseline keeps 16 and 64
  if (batch < 0 || max_seq_len < 0) return DGQ_ERR_INVALID_ARG;
  if (batch == 0) return DGQ_OK;
  if (batch > kMaxGridBatch) return DGQ_ERR_UNSUPPORTED;
  if (!q || !out || !seq_lens || !aligned(q, 16) || !aligned(out, 16)) return DGQ_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return DGQ_ERR_INVALID_ARG;
  if ((st = check_table(p, block_table, max_blocks, max_seq_len)) != DGQ_OK) return st;
  if ((st = check_g64_cache(cache)) != DGQ_OK) return st;
  const size_t need = decode_workspace_bytes(p, batch, max_seq_len);
  if (ws == nullptr || !aligned(ws, 256)) return DGQ_ERR_INVALID_ARG;
  if (ws_bytes < need) return DGQ_ERR_WORKSPACE_TOO_SMALL;
  return launch_g64_decode(p, q, cache, block_table, max_blocks, seq_lens, batch, max_seq_len,
                           softmax_scale, out, ws, stream);
}
