/*
 * dgq.h -- C ABI of libdgq: dynamic-group INT8 compression of the attention KV cache and paged
 * INT8 decode attention, for AMD Instinct MI355X (gfx950).
 *
 * Sources of the method (titles of the pages; addresses for the reader):
 *   DGQ article           http://www.pptc.cn/news/101026  -- section 2.2 (per-head variance curve,
 *                         16-token sliding window, 3~5 segments cut at variance change points,
 *                         per-segment min/max, INT8 codes, 1-bit segment identifier), section 3.1
 *                         (dequantize inside the paged attention step), section 3.2 (identifier
 *                         storage), section 3.3 (memory formula: 1 byte per element + 1 bit per
 *                         token per head).
 *   PagedAttention article https://deepseek.csdn.net/6a0bbfa610ee7a33f27399ed.html -- logical
 *                         blocks mapped to discrete physical blocks through a block table with a
 *                         free list; block-granular allocation; paged forward pass with
 *                         block_tables; 64-token blocks for long contexts.
 *   Quantization article  http://cnnetsun.cn/a/2561798 -- section 2.1 asymmetric quantization
 *                         template clamp(round(x / scale) + zero_point, lo, hi); section 3.2
 *                         page-table entries with a reference count (shared physical pages).
 *
 * Conventions for every entry point
 *   - Device pointers are caller-owned HIP device memory; the library never allocates or frees
 *     device memory and never synchronizes a stream.  Work is queued on `stream` in order.  (The
 *     one library-owned device buffer is the fixed array of paged_decode_attn_int8_noalloc.)
 *   - The device entry points other than dgq_swap_out / dgq_swap_in (which copy to or from
 *     host memory) queue kernel launches only: no memset, copy or event.  They may be captured in
 *     a HIP graph; a replay reads the buffers' contents at replay time.
 *   - Host pointers are marked (host).  The block pool handle is owned by the library until
 *     dgq_pool_destroy.
 *   - Calls that take a batch of sequences accept at most 65535 of them (DGQ_ERR_UNSUPPORTED
 *     above that: the batch is a launch-grid dimension).
 *   - Every call returns a dgq_status_t.  Arguments are checked on the host before anything is
 *     queued; a failed check queues nothing and writes nothing.  A failed kernel launch returns
 *     DGQ_ERR_HIP; dgq_last_error() gives the HIP error text of the calling thread's last failure.
 *   - Conditions that depend on device data are never turned into errors: they are counted in
 *     the cache's status words (see dgq_cache_t.status), which the caller reads after a sync.
 *   - Device data is not trusted to be consistent: a block id outside the pool, a sequence length
 *     above max_seq_len or a cu_seqlens entry outside the input is never followed out of bounds;
 *     it is skipped or clamped and counted in status[2], and the affected results are unspecified.
 *   - fp16 data is passed as uint16_t (IEEE binary16 bit patterns).
 *
 * Paged layout (per layer; the block table is shared by all layers)
 *   k_pool, v_pool: int8 [num_blocks][num_kv_heads][block_size * head_dim].  One (block, head)
 *   tile holds the codes of block_size tokens.  Inside a tile the codes are stored in the order
 *   the decode kernel's matrix-core instructions consume them, so that every wave-wide 16-byte
 *   load reads 256 contiguous bytes or more.  With M = head_dim / 64, a token tau of the block
 *   (0 <= tau < block_size) and a channel d:
 *     K, block_size 64: T = tau/16, r = tau%16, m = d/64, j = (d%64)/16, e = d%16
 *                       offset = (((T*M + m)*4 + j)*16 + r)*16 + e
 *     K, block_size 16: T = tau/4, i = tau%4 (m, j, e as above)
 *                       offset = ((((T*M + m)*4 + j)*4 + i)*16) + e
 *     V, block_size 64: n = d/16, r = d%16, j = (tau%16)/4, e = 4*(tau/16) + tau%4
 *                       offset = ((n*4 + j)*16 + r)*16 + e
 *     V, block_size 16: offset = d*16 + tau
 *     block_size 32: two 16-token tiles one after the other (tokens 0..15, then 16..31), each in
 *                    the block_size 16 order: offset = (tau/16)*16*head_dim + the 16-token offset
 *                    of (tau%16, d), for K and for V
 *   A code is the signed byte c in [-128, 127]; the value it stands for is (c + 128) * scale + min
 *   with the (scale, min) of the token's segment.
 *   bits: uint8 [num_blocks][num_kv_heads][block_size/8]; bit (tau % 8) of byte tau/8 is 1 iff
 *   the token starts a segment other than the first (the 1-bit identifier, kept in its own
 *   tensor as in the DGQ article's original scheme).
 *
 * Marker format (flag DGQ_FORMAT_MARKER; DGQ article 3.2, the identifier kept inside the INT8
 * data): data codes are c in [-127, 126] standing for (c + 127) * scale + min with
 * scale = fp32((max - min) / 253); the byte values -128 and 127 are markers.  The key byte of
 * channel 0 of the first token of every segment but the first holds 127 if that element's own
 * code is >= 0, else -128, and is dequantized with the same formula (min - scale or
 * max + scale).  There is no bit tensor (dgq_cache_t.bits may be NULL and is never touched);
 * dgq_marker_bits reads the identifier back from the markers.
 */
#ifndef DGQ_H
#define DGQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dgq_status {
  DGQ_OK = 0,
  DGQ_ERR_INVALID_ARG = -1,         /* null pointer, bad size, misaligned buffer, bad stride */
  DGQ_ERR_UNSUPPORTED = -2,         /* valid but unsupported shape (head_dim, block_size, group) */
  DGQ_ERR_POOL_EXHAUSTED = -3,      /* not enough free blocks; nothing was allocated */
  DGQ_ERR_WORKSPACE_TOO_SMALL = -4, /* ws_bytes below the matching *_workspace_size() */
  DGQ_ERR_HIP = -5                  /* a HIP call failed; see dgq_last_error() */
} dgq_status_t;

/* dgq_params_t.flags: segment-count policies (DGQ article 3.2 and 5.3) and the storage format
 * of the segment identifier (DGQ article 3.2). */
enum {
  /* Length-aware cap: a sequence of L tokens gets at most 2 segments below 2048 tokens, 3 below
   * 16384, else min(5, floor(log2(L / 1024)) + 2); the cap only lowers max_segments. */
  DGQ_POLICY_LENGTH_AWARE = 1u,
  /* Marker format (see the layout notes above) instead of the bit tensor.  A cache must be
   * written and read with the same format. */
  DGQ_FORMAT_MARKER = 2u,
  /* dgq_compress only: run the separate stats / selection / encode launches even where the
   * one-launch path for short sequences (at most 256 tokens at head_dim 128, 512 at 64) applies.
   * Both paths write bit-identical results; the flag is for comparing them.  Other calls ignore
   * it. */
  DGQ_COMPRESS_MULTIPASS = 4u
};

/* Shape and method parameters, passed to every call (48 bytes).  Defaults: win 16,
 * max_segments 5, seg_capacity 16, flags 0, tau 2.0, min_var 0. */
typedef struct dgq_params {
  int32_t num_kv_heads;  /* >= 1 */
  int32_t num_q_heads;   /* num_kv_heads * G with G in {1, 2, 4}; query head g uses kv head g / G */
  int32_t head_dim;      /* 64 or 128 */
  int32_t block_size;    /* tokens per physical block: 16, 32 or 64 (the group-64 baseline: 16
                            or 64) */
  int32_t win;           /* sliding-window length of the variance curve; must be 16 (DGQ 2.2) */
  int32_t max_segments;  /* 1..8 segments per (sequence, kv head) from dgq_compress */
  int32_t seg_capacity;  /* segment-table rows per (sequence, kv head): max_segments..64 */
  uint32_t flags;        /* DGQ_POLICY_LENGTH_AWARE | DGQ_FORMAT_MARKER | DGQ_COMPRESS_MULTIPASS;
                            other bits must be 0 */
  double tau;            /* change-point threshold on the window-variance ratio, finite, >= 1 */
  double min_var;        /* variance floor, finite, >= 0 (0 = off): a candidate cut whose two
                            16-token windows both have a population variance below it is not a
                            change point, in dgq_compress and in dgq_append's window test */
} dgq_params_t;

/* One segment-table row (32 bytes).  kscale = fp32((kmax - kmin) / 255), likewise vscale (253 in
 * place of 255 in the marker format). */
typedef struct dgq_seg {
  int32_t start;         /* first token of the segment */
  float kmin, kmax, vmin, vmax;
  float kscale, vscale;
  int32_t reserved;
} dgq_seg_t;

/* Append state of one (sequence, kv head), 224 bytes; written by dgq_compress, advanced by
 * dgq_append.  The open span is [r0, length): tokens appended since the tail block was last
 * sealed.  The ring holds the fixed-point moments of the 16 sealed tokens before r0. */
typedef struct dgq_tail {
  int32_t r0;
  int32_t ring_len;      /* 0..16 */
  int32_t span_own;      /* 1 if the open span has its own segment-table row */
  int32_t window_done;   /* 1 once the span's first-16-token window test came out "no change" */
  int32_t ring_a[16];    /* oldest first */
  int64_t ring_b[16];
  float span_range[4];   /* K min, K max, V min, V max of the open span (valid while it is not empty) */
} dgq_tail_t;

/* The compressed cache of one layer: caller-owned device buffers. */
typedef struct dgq_cache {
  int8_t *k_pool;        /* [num_blocks][num_kv_heads][block_size*head_dim], 16-byte aligned */
  int8_t *v_pool;        /* same */
  uint8_t *bits;         /* [num_blocks][num_kv_heads][block_size/8]; NULL allowed (and unused)
                            in the marker format */
  dgq_seg_t *segs;       /* [batch][num_kv_heads][seg_capacity] */
  int32_t *nseg;         /* [batch][num_kv_heads] rows in use */
  dgq_tail_t *tail;      /* [batch][num_kv_heads] */
  uint16_t *k_stage;     /* [batch][num_kv_heads][block_size][head_dim] fp16 copy of the open span */
  uint16_t *v_stage;     /* same */
  unsigned long long *status; /* [4] counters, only ever incremented (the caller zeroes them):
                                 [0] appends that wanted a new segment but found the table full
                                     (the span joins the segment before it; codes saturate);
                                 [1] groups of inputs that held a non-finite value (their codes
                                     are unspecified);
                                 [2] device-side inconsistencies that were skipped or clamped
                                     instead of read out of bounds: a sequence length above
                                     max_seq_len or outside cu_seqlens, a block id >= num_blocks,
                                     an append state that does not fit the new position;
                                 [3] reserved. */
  int32_t num_blocks;    /* blocks in each pool */
  int32_t batch;         /* rows of segs/nseg/tail/stage */
} dgq_cache_t;

/* Human-readable text for a status code (static storage). */
const char *dgq_status_string(int32_t status);
/* HIP error text of the calling thread's last DGQ_ERR_HIP (static per thread; "" if none). */
const char *dgq_last_error(void);

/* ---- Block pool (PagedAttention article, "PagedAttention implementation": BlockTable with a
 * free list, block-granular allocation and release).  Host-only, no device work. ---- */

/* Create a pool of num_blocks ids 0..num_blocks-1, all free; *pool (host) receives the handle. */
dgq_status_t dgq_pool_create(int32_t num_blocks, void **pool);
/* Destroy a pool (NULL is a no-op). */
dgq_status_t dgq_pool_destroy(void *pool);
/* Take n ids into ids (host, n entries).  All or nothing: DGQ_ERR_POOL_EXHAUSTED leaves the pool
 * unchanged.  Ids come from the free list in last-freed-first order. */
dgq_status_t dgq_block_alloc(void *pool, int32_t n, int32_t *ids);
/* Drop one reference per entry of ids (host, n entries); a block whose count reaches 0 goes back
 * on the free list.  An id may be listed as often as it has references.  DGQ_ERR_INVALID_ARG,
 * with the pool unchanged, if any id is out of range or listed more often than its count. */
dgq_status_t dgq_block_free(void *pool, int32_t n, const int32_t *ids);
/* Number of free ids, or -1 for a NULL pool. */
int32_t dgq_pool_num_free(const void *pool);

/* ---- Block lifecycle: shared blocks, copy-on-write, swap (Quantization article, section 3.2:
 * reference-counted page-table entries; DGQ article, section 3.1: the cache engine's swap in/out
 * works on compressed blocks).  A compressed block carries its INT8 codes and its boundary bits;
 * a sequence's segment table, row count, append state and staging live in its cache row.  Blocks
 * before the tail block are frozen (dgq_append never writes them), so they can be shared by
 * several sequences; the tail block is written by every append and must be owned by one. ---- */

/* Add one reference per entry of ids (host, n entries), e.g. when a forked sequence's block table
 * takes the parent's blocks.  DGQ_ERR_INVALID_ARG, with the pool unchanged, if any id is out of
 * range or free. */
dgq_status_t dgq_block_share(void *pool, int32_t n, const int32_t *ids);
/* References of one block: 0 if free, -1 for a NULL pool or an id out of range. */
int32_t dgq_block_refcount(const void *pool, int32_t id);
/* Copy-on-write for a list of blocks about to be written (host, n entries each).  Entries are
 * served in order: a block with one reference is kept (out_ids[i] = ids[i]); a block with more
 * takes a fresh block (out_ids[i], one reference) and drops one reference of ids[i].  The caller
 * then copies every changed pair with dgq_copy_blocks and writes out_ids into its block table.
 * All or nothing: DGQ_ERR_POOL_EXHAUSTED, or DGQ_ERR_INVALID_ARG (an id out of range or free, or
 * listed more often than it has references), leaves the pool unchanged. */
dgq_status_t dgq_block_cow(void *pool, int32_t n, const int32_t *ids, int32_t *out_ids);

/* Copy whole compressed blocks of one layer: for i < n, the K and V codes of every kv head and the
 * boundary bits (bit-tensor format) of block src_ids[i] are copied to block dst_ids[i].
 *   src_ids, dst_ids (device) int32 [n].  A dst id must not appear twice nor among the src ids
 *   (the copies run in parallel).  A pair with an id outside [0, num_blocks) is skipped and
 *   counted in status[2].  n == 0 queues nothing. */
dgq_status_t dgq_copy_blocks(const dgq_params_t *p, const dgq_cache_t *cache, const int32_t *src_ids,
                             const int32_t *dst_ids, int32_t n, hipStream_t stream);
/* Copy the per-sequence state of one layer from cache row src_rows[i] to row dst_rows[i], i < n:
 * segment-table rows, row count, append state and the fp16 staging of the open span, for every
 * kv head.  With dgq_block_share on the block table and dgq_block_cow + dgq_copy_blocks on the
 * tail block before the next append, this forks a sequence.
 *   src_rows, dst_rows (device) int32 [n]; the same rules as dgq_copy_blocks' ids, against
 *   [0, cache->batch).  The cache must have its staging buffers. */
dgq_status_t dgq_copy_seq_state(const dgq_params_t *p, const dgq_cache_t *cache,
                                const int32_t *src_rows, const int32_t *dst_rows, int32_t n,
                                hipStream_t stream);

/* Bytes of the swap image of one sequence with n_blocks blocks (one layer): the cache row's state
 * (segment-table rows, row counts, append state, staging), then per block its K codes, V codes
 * and bits (none in the marker format), each part padded to 16 bytes.  0 for invalid arguments. */
size_t dgq_swap_image_bytes(const dgq_params_t *p, int32_t n_blocks);
/* Swap out one sequence of one layer: its cache row `row` (host int) and blocks ids[0..n_blocks)
 * (device int32, in logical order) are packed into `staging` (device, >= dgq_swap_image_bytes,
 * 16-byte aligned); then, if host_dst is not NULL, the image is copied to host_dst (host memory
 * of the same size, pinned for the copy to be asynchronous) on the same stream.  The cache is not
 * modified; the caller frees the blocks once the copy has completed.  Block ids outside the pool
 * are skipped (their part of the image is left as is) and counted in status[2]. */
dgq_status_t dgq_swap_out(const dgq_params_t *p, const dgq_cache_t *cache, int32_t row,
                          const int32_t *ids, int32_t n_blocks, void *staging, size_t staging_bytes,
                          void *host_dst, hipStream_t stream);
/* Swap in: the inverse.  If host_src is not NULL the image is first copied from host_src to
 * `staging`; then the state is written to cache row `row` and the blocks to ids[0..n_blocks)
 * (device int32, freshly allocated by the caller; any ids: the codes do not depend on where a
 * block lives).  The sequence then decodes and appends exactly as before it was swapped out. */
dgq_status_t dgq_swap_in(const dgq_params_t *p, const dgq_cache_t *cache, int32_t row,
                         const int32_t *ids, int32_t n_blocks, void *staging, size_t staging_bytes,
                         const void *host_src, hipStream_t stream);

/* ---- Workspace sizes (bytes; 0 for invalid arguments) ---- */

/* dgq_compress scratch for `batch` sequences of at most max_seq_len tokens, total_tokens in all. */
size_t dgq_compress_workspace_size(const dgq_params_t *p, int32_t batch, int64_t total_tokens,
                                   int32_t max_seq_len);
/* paged_decode_attn_int8 scratch (split-sequence partial results). */
size_t dgq_decode_workspace_size(const dgq_params_t *p, int32_t batch, int32_t max_seq_len);

/* The operations of dgq_workspace_size. */
enum {
  DGQ_OP_COMPRESS = 0,       /* dgq_compress */
  DGQ_OP_APPEND = 1,         /* dgq_append: takes no workspace (size 0) */
  DGQ_OP_DECODE = 2,         /* paged_decode_attn_int8 */
  DGQ_OP_APPEND_DECODE = 3,  /* dgq_append_decode */
  DGQ_OP_G64_DECODE = 4      /* paged_decode_attn_g64 */
};
/* Workspace bytes of operation `op` for `batch` sequences of at most max_seq_len tokens
 * (total_tokens in all; read for DGQ_OP_COMPRESS only): one entry for every operation, equal to
 * the per-operation functions above.  0 for invalid arguments or an unknown op. */
size_t dgq_workspace_size(const dgq_params_t *p, int32_t op, int32_t batch, int64_t total_tokens,
                          int32_t max_seq_len);

/* Copy the cache's four device status words (see dgq_cache_t.status) to host memory out[0..3],
 * after everything queued on `stream` before this call: enqueues the copy on `stream` and then
 * synchronizes that stream (the one library call that waits).  out: host, 4 elements.  The words
 * are not reset.  DGQ_ERR_INVALID_ARG for a null cache, status pointer or out. */
dgq_status_t dgq_read_device_status(const dgq_cache_t *cache, unsigned long long *out, hipStream_t stream);

/* ---- DGQ compression (DGQ article 2.2) ----
 * For every (sequence b, kv head h): the variance curve of the keys over a sliding 16-token
 * window, cuts at its change points (2..max_segments segments when the sequence has >= 32
 * tokens), per-segment K and V min/max, INT8 codes of every token written into the blocks the
 * block table names, boundary bits, the segment table, and the append state (open span empty at
 * the compressed length).
 *   k, v        fp16 token-major input; element (token t of sequence b, head h, channel d) is at
 *               [ (cu_seqlens[b] + t) * stride_tok + h * stride_head + d ].  16-byte aligned;
 *               stride_tok and stride_head multiples of 8 elements.
 *   cu_seqlens  (device) int32 [batch+1], nondecreasing, cu_seqlens[0] = 0; sequence b has
 *               cu_seqlens[b+1] - cu_seqlens[b] <= max_seq_len tokens.
 *   total_tokens (host) cu_seqlens[batch].
 *   block_table (device) int32 [batch][max_blocks]; max_seq_len <= max_blocks * block_size.
 *   cache       (host struct, device buffers) with cache->batch >= batch.
 *   ws          device scratch of dgq_compress_workspace_size() bytes, 256-byte aligned.
 * Non-finite inputs increment status[1]; their codes are unspecified. */
dgq_status_t dgq_compress(const dgq_params_t *p, const uint16_t *k, const uint16_t *v,
                          int64_t stride_tok, int64_t stride_head, const int32_t *cu_seqlens,
                          int32_t batch, int32_t max_seq_len, int64_t total_tokens,
                          const int32_t *block_table, int32_t max_blocks,
                          const dgq_cache_t *cache, void *ws, size_t ws_bytes, hipStream_t stream);

/* ---- Append one token per sequence (DGQ article 2.2: the segmentation is revisited as new
 * tokens arrive; only the tail block's open span is re-decided, frozen blocks are never
 * rewritten) ----
 *   k_tok, v_tok (device) fp16 [batch][num_kv_heads][head_dim], 16-byte aligned.
 *   seq_lens     (device) int32 [batch]: tokens already cached; the new token lands at that
 *                position, whose block must already be in block_table.  The caller advances
 *                seq_lens afterwards.
 * Rule: the span joins the segment before it unless a span key or value falls outside that
 * segment's range, or the span's first 16 tokens' window variance differs from the 16 tokens
 * before the span by a ratio >= tau; then the span is a segment of its own (at most one per
 * tail block).  The span's codes are rewritten with the chosen range; when the block fills, the
 * span is sealed.  A full segment table makes the span join instead and increments status[0]. */
dgq_status_t dgq_append(const dgq_params_t *p, const uint16_t *k_tok, const uint16_t *v_tok,
                        const int32_t *seq_lens, int32_t batch, const int32_t *block_table,
                        int32_t max_blocks, const dgq_cache_t *cache, hipStream_t stream);

/* ---- Paged INT8 decode attention (DGQ article 3.1: dequantize while attending; PagedAttention
 * article: paged forward pass through block_tables) ----
 * out[b][g][:] = sum_t softmax_t(softmax_scale * q[b][g] . khat_t) * vhat_t over the seq_lens[b]
 * cached tokens of kv head g / G, where khat, vhat are the dequantized codes.  The dequantization
 * is folded into the dot products; no dequantized copy is written.
 *   q    (device) fp16 [batch][num_q_heads][head_dim], 16-byte aligned.
 *   out  (device) fp32 [batch][num_q_heads][head_dim], 16-byte aligned; an empty sequence gives
 *        zeros.
 *   seq_lens (device) int32 [batch], each <= max_seq_len <= max_blocks * block_size.
 *   ws   device scratch of dgq_decode_workspace_size() bytes, 256-byte aligned.  Its first
 *        bytes are completion counters of the split-sequence merge: they must be zero before the
 *        first call that uses this buffer (zero-fill it once when allocating it), and every call
 *        leaves them zero again.  Calls that share one workspace must not overlap in time. */
dgq_status_t paged_decode_attn_int8(const dgq_params_t *p, const uint16_t *q,
                                    const dgq_cache_t *cache, const int32_t *block_table,
                                    int32_t max_blocks, const int32_t *seq_lens, int32_t batch,
                                    int32_t max_seq_len, float softmax_scale, float *out,
                                    void *ws, size_t ws_bytes, hipStream_t stream);

/* ---- Allocation-free paged INT8 decode, for callers that cannot allocate device memory or
 * hand in a workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as paged_decode_attn_int8, without ws / ws_bytes: the
 * split-sequence partials and completion counters live in a device array of
 * DGQ_NOALLOC_SCRATCH_BYTES (16 MiB) inside the library's code object, one copy per GPU, held
 * until the process ends.  The call allocates nothing (no hipMalloc, no allocating library
 * routine); its first use on a device (the device of `stream`) looks up that device's copy.
 * Each call queues a small kernel that zeroes the counters it uses, then the decode (kernel
 * launches only, so it may be captured).
 *   Limit: DGQ_ERR_WORKSPACE_TOO_SMALL, queuing nothing, when the call's partials need more than
 *   the array: each partition of a (sequence, query head) takes (head_dim + 2) * 4 bytes, and
 *   the launch plan aims at about 256 workgroups.  With head_dim 128 and 32 query heads: 16 x 8192
 *   tokens or one 131072-token sequence need 0.53 MB, 100 sequences of up to 4096 tokens 1.7 MB;
 *   about 1000 sequences fit, larger batches are refused.
 *   Every call on one GPU shares that GPU's array and leaves in it what the last call wrote:
 *   calls that overlap in time on one GPU (two streams, or two threads) race and give unspecified
 *   results; serialize them. */
#define DGQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
dgq_status_t paged_decode_attn_int8_noalloc(const dgq_params_t *p, const uint16_t *q,
                                            const dgq_cache_t *cache, const int32_t *block_table,
                                            int32_t max_blocks, const int32_t *seq_lens, int32_t batch,
                                            int32_t max_seq_len, float softmax_scale, float *out,
                                            hipStream_t stream);

/* ---- Fused decode step: dgq_append followed by paged_decode_attn_int8, in one launch (DGQ
 * article 3.1: the new token's key/value is quantized inside the paged attention step).
 *   seq_lens     (device) int32 [batch]: tokens BEFORE this step; the token is appended at that
 *                position and the query attends to seq_lens[b] + 1 tokens.
 *   max_seq_len  bound on seq_lens[b] + 1; <= max_blocks * block_size.
 *   k_tok, v_tok, block_table, cache: as dgq_append; q, softmax_scale, out: as
 *                paged_decode_attn_int8; ws: dgq_decode_workspace_size(p, batch, max_seq_len) bytes,
 *                zero-filled once (shared with paged_decode_attn_int8 under the same rules).
 * Results equal dgq_append followed by paged_decode_attn_int8 with lengths seq_lens + 1: the
 * workgroup whose partition holds the tail block appends first and decodes with the updated
 * segment rows; the new row count is published after every workgroup of the (sequence, head) is
 * done, so no workgroup sees a half-written row. ---- */
dgq_status_t dgq_append_decode(const dgq_params_t *p, const uint16_t *k_tok, const uint16_t *v_tok,
                               const int32_t *seq_lens, const uint16_t *q, int32_t batch,
                               const int32_t *block_table, int32_t max_blocks, int32_t max_seq_len,
                               float softmax_scale, const dgq_cache_t *cache, float *out, void *ws,
                               size_t ws_bytes, hipStream_t stream);

/* ---- Identifier read-back in the marker format (DGQ article 3.2: the identifier is taken out
 * of the INT8 data with a bit mask) ---- */

/* Write the boundary bits of every sequence, in the bit-tensor layout, from the marker bytes of a
 * marker-format cache: bit tau of block table[b][j] and head h is 1 iff token j*block_size + tau
 * (< seq_lens[b]) has a marker in its channel-0 key byte.
 *   block_table (device) int32 [batch][max_blocks]; seq_lens (device) int32 [batch], each
 *   <= max_seq_len <= max_blocks * block_size; bits_out (device) uint8
 *   [num_blocks][num_kv_heads][block_size/8]: the blocks of the sequences are overwritten (bits of
 *   tokens at or past seq_lens[b] are 0), other blocks are not touched.
 * DGQ_ERR_INVALID_ARG unless p->flags has DGQ_FORMAT_MARKER. */
dgq_status_t dgq_marker_bits(const dgq_params_t *p, const dgq_cache_t *cache, const int32_t *block_table,
                             int32_t max_blocks, const int32_t *seq_lens, int32_t batch,
                             int32_t max_seq_len, uint8_t *bits_out, hipStream_t stream);

/* ---- Fixed 64-channel group INT8 baseline (DGQ article 2.2: the LLM.int8()-style grouping the
 * DGQ design is compared against -- every 64-channel chunk of every token has its own min/max).
 * Same pool layout, code formula and dequantization as DGQ; the ranges are kept per (token,
 * group) instead of per segment.  Provided to compare error and throughput on the same data. ---- */
typedef struct dgq_g64_cache {
  int8_t *k_pool;        /* [num_blocks][num_kv_heads][block_size*head_dim], layout as dgq_cache_t */
  int8_t *v_pool;
  uint32_t *k_range;     /* [num_blocks][num_kv_heads][block_size][head_dim/64]: fp16 min in bits
                            0..15, fp16 max in bits 16..31 */
  uint32_t *v_range;
  unsigned long long *status;  /* [4], as dgq_cache_t.status ([2] used) */
  int32_t num_blocks;
  int32_t reserved;
} dgq_g64_cache_t;

/* Quantize rows into the group-64 cache.  Rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of k/v (token-
 * major, strides as dgq_compress) go to cache positions first_pos[b] + r (first_pos may be NULL:
 * all zero); max_rows bounds the rows per sequence, total_rows = cu_seqlens[batch], and every
 * position must be < max_seq_len <= max_blocks * block_size.  Used both for a whole prefix and
 * for one appended token per sequence (cu_seqlens = 0, 1, ..., batch; first_pos = lengths). */
dgq_status_t dgq_g64_quantize(const dgq_params_t *p, const uint16_t *k, const uint16_t *v,
                              int64_t stride_tok, int64_t stride_head, const int32_t *cu_seqlens,
                              const int32_t *first_pos, int32_t batch, int32_t max_rows,
                              int64_t total_rows, const int32_t *block_table, int32_t max_blocks,
                              int32_t max_seq_len, const dgq_g64_cache_t *cache, hipStream_t stream);

/* Paged decode attention over a group-64 cache; arguments and workspace (including its zeroed
 * counters, dgq_decode_workspace_size) as paged_decode_attn_int8.  The group-64 calls take block
 * sizes 16 and 64 (DGQ_ERR_UNSUPPORTED for 32). */
dgq_status_t paged_decode_attn_g64(const dgq_params_t *p, const uint16_t *q,
                                   const dgq_g64_cache_t *cache, const int32_t *block_table,
                                   int32_t max_blocks, const int32_t *seq_lens, int32_t batch,
                                   int32_t max_seq_len, float softmax_scale, float *out, void *ws,
                                   size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DGQ_H */
