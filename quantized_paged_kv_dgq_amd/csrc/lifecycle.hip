// Block lifecycle on the device: copying compressed blocks (copy-on-write of a shared tail block),
// copying a sequence's state row (fork), and packing / unpacking a sequence into a swap image
// (Quantization article 3.2: reference-counted pages; DGQ article 3.1: swap in/out works on the
// compressed blocks).  All of it is data movement at HBM speed: 16-byte vector loads and stores,
// four in flight per lane.
#include "lifecycle.h"

namespace dgq {

constexpr int kThreads = 256;
constexpr int kParts = 5;

// Sizes of the pieces a state row and a block are made of (bytes, host-computed).
struct Geometry {
  int64_t tile;       // codes of one block for all kv heads: hkv * block_size * head_dim
  int64_t bits;       // boundary bits of one block for all kv heads: hkv * block_size / 8 (or 0)
  int64_t segs;       // segment-table rows of one sequence: hkv * seg_capacity * 32
  int64_t nseg;       // row counts of one sequence: hkv * 4
  int64_t tail;       // append states of one sequence: hkv * 224
  int64_t stage;      // fp16 staging of one sequence (K or V): hkv * block_size * head_dim * 2
  int64_t state_img;  // image bytes of the state (parts padded to 16)
  int64_t block_img;  // image bytes of one block
};

static Geometry geometry(const dgq_params_t *p) {
  Geometry g;
  const int64_t h = p->num_kv_heads;
  g.tile = h * p->block_size * p->head_dim;
  g.bits = (p->flags & DGQ_FORMAT_MARKER) ? 0 : h * p->block_size / 8;   // no bit tensor in the marker format
  g.segs = h * p->seg_capacity * (int64_t)sizeof(dgq_seg_t);
  g.nseg = h * 4;
  g.tail = h * (int64_t)sizeof(dgq_tail_t);
  g.stage = h * p->block_size * p->head_dim * 2;
  g.state_img = (int64_t)align_up(g.segs, 16) + (int64_t)align_up(g.nseg, 16) +
                (int64_t)align_up(g.tail, 16) + 2 * (int64_t)align_up(g.stage, 16);
  g.block_img = 2 * (int64_t)align_up(g.tile, 16) + (int64_t)align_up(g.bits, 16);
  return g;
}

// A list of byte ranges; two lists with the same sizes describe a copy.
struct Parts {
  uint8_t *ptr[kParts];
  int64_t bytes[kParts];
  int n;
};

__device__ Parts state_parts(const dgq_cache_t &c, const Geometry &g, int row) {
  Parts s;
  s.ptr[0] = reinterpret_cast<uint8_t *>(c.segs) + row * g.segs;
  s.ptr[1] = reinterpret_cast<uint8_t *>(c.nseg) + row * g.nseg;
  s.ptr[2] = reinterpret_cast<uint8_t *>(c.tail) + row * g.tail;
  s.ptr[3] = reinterpret_cast<uint8_t *>(c.k_stage) + row * g.stage;
  s.ptr[4] = reinterpret_cast<uint8_t *>(c.v_stage) + row * g.stage;
  s.bytes[0] = g.segs;
  s.bytes[1] = g.nseg;
  s.bytes[2] = g.tail;
  s.bytes[3] = g.stage;
  s.bytes[4] = g.stage;
  s.n = 5;
  return s;
}

__device__ Parts block_parts(const dgq_cache_t &c, const Geometry &g, int blk) {
  Parts s;
  s.ptr[0] = reinterpret_cast<uint8_t *>(c.k_pool) + blk * g.tile;
  s.ptr[1] = reinterpret_cast<uint8_t *>(c.v_pool) + blk * g.tile;
  s.ptr[2] = c.bits + blk * g.bits;
  s.bytes[0] = g.tile;
  s.bytes[1] = g.tile;
  s.bytes[2] = g.bits;
  s.n = 3;
  return s;
}

// The same pieces laid out back to back in an image, each padded to 16 bytes.
__device__ Parts image_parts(uint8_t *img, const Parts &like) {
  Parts s = like;
  int64_t off = 0;
  for (int i = 0; i < like.n; ++i) {
    s.ptr[i] = img + off;
    off += (like.bytes[i] + 15) & ~int64_t(15);
  }
  return s;
}

// Copy every piece of src to the matching piece of dst with the whole workgroup.
__device__ void move(const Parts &dst, const Parts &src) {
  for (int i = 0; i < src.n; ++i) {
    uint8_t *d = dst.ptr[i];
    const uint8_t *s = src.ptr[i];
    const int64_t nb = src.bytes[i];
    const bool vec = ((reinterpret_cast<uintptr_t>(d) | reinterpret_cast<uintptr_t>(s) | (uintptr_t)nb) & 15) == 0;
    if (vec) {
      const int64_t n16 = nb >> 4;
      uint4 *d4 = reinterpret_cast<uint4 *>(d);
      const uint4 *s4 = reinterpret_cast<const uint4 *>(s);
      for (int64_t j = threadIdx.x; j < n16; j += 4 * kThreads) {
        uint4 r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (j + u * kThreads < n16) r[u] = s4[j + u * kThreads];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (j + u * kThreads < n16) d4[j + u * kThreads] = r[u];
      }
    } else {
      for (int64_t j = threadIdx.x; j < nb; j += kThreads) d[j] = s[j];
    }
  }
}

__device__ void count_bad(const dgq_cache_t &c) {
  if (threadIdx.x == 0) atomicAdd(&c.status[2], 1ull);
}

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(dgq_cache_t c, Geometry g, const int32_t *src,
                                                               const int32_t *dst) {
  const int s = src[blockIdx.x], d = dst[blockIdx.x];
  if ((unsigned)s >= (unsigned)c.num_blocks || (unsigned)d >= (unsigned)c.num_blocks) {
    count_bad(c);
    return;
  }
  if (s != d) move(block_parts(c, g, d), block_parts(c, g, s));
}

__global__ __launch_bounds__(kThreads) void copy_state_kernel(dgq_cache_t c, Geometry g, const int32_t *src,
                                                              const int32_t *dst) {
  const int s = src[blockIdx.x], d = dst[blockIdx.x];
  if ((unsigned)s >= (unsigned)c.batch || (unsigned)d >= (unsigned)c.batch) {
    count_bad(c);
    return;
  }
  if (s != d) move(state_parts(c, g, d), state_parts(c, g, s));
}

// Workgroup 0 moves the state row, workgroup 1 + i block ids[i].  PACK: cache -> image.
template <bool PACK>
__global__ __launch_bounds__(kThreads) void swap_kernel(dgq_cache_t c, Geometry g, int row, const int32_t *ids,
                                                        uint8_t *img) {
  Parts cache_side, img_side;
  if (blockIdx.x == 0) {
    cache_side = state_parts(c, g, row);
    img_side = image_parts(img, cache_side);
  } else {
    const int i = blockIdx.x - 1;
    const int blk = ids[i];
    if ((unsigned)blk >= (unsigned)c.num_blocks) {
      count_bad(c);
      return;
    }
    cache_side = block_parts(c, g, blk);
    img_side = image_parts(img + g.state_img + (int64_t)i * g.block_img, cache_side);
  }
  if (PACK) move(img_side, cache_side);
  else move(cache_side, img_side);
}

size_t swap_image_bytes(const dgq_params_t *p, int32_t n_blocks) {
  const Geometry g = geometry(p);
  return (size_t)(g.state_img + (int64_t)n_blocks * g.block_img);
}

dgq_status_t launch_copy_blocks(const dgq_params_t *p, const dgq_cache_t *cache, const int32_t *src,
                                const int32_t *dst, int32_t n, hipStream_t stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n), dim3(kThreads), 0, stream, *cache, geometry(p), src, dst);
  return check_launch("dgq_copy_blocks kernel");
}

dgq_status_t launch_copy_seq_state(const dgq_params_t *p, const dgq_cache_t *cache, const int32_t *src,
                                   const int32_t *dst, int32_t n, hipStream_t stream) {
  hipLaunchKernelGGL(copy_state_kernel, dim3(n), dim3(kThreads), 0, stream, *cache, geometry(p), src, dst);
  return check_launch("dgq_copy_seq_state kernel");
}

dgq_status_t launch_swap(const dgq_params_t *p, const dgq_cache_t *cache, int32_t row, const int32_t *ids,
                         int32_t n_blocks, void *staging, void *host, bool out, hipStream_t stream) {
  const size_t bytes = swap_image_bytes(p, n_blocks);
  uint8_t *img = static_cast<uint8_t *>(staging);
  if (out) {
    hipLaunchKernelGGL((swap_kernel<true>), dim3(1 + n_blocks), dim3(kThreads), 0, stream, *cache,
                       geometry(p), row, ids, img);
    dgq_status_t st = check_launch("dgq_swap_out kernel");
    if (st != DGQ_OK || host == nullptr) return st;
    const hipError_t e = hipMemcpyAsync(host, img, bytes, hipMemcpyDeviceToHost, stream);
    return e == hipSuccess ? DGQ_OK : hip_fail(e, "dgq_swap_out copy to host");
  }
  if (host != nullptr) {
    const hipError_t e = hipMemcpyAsync(img, host, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "dgq_swap_in copy from host");
  }
  hipLaunchKernelGGL((swap_kernel<false>), dim3(1 + n_blocks), dim3(kThreads), 0, stream, *cache,
                     geometry(p), row, ids, img);
  return check_launch("dgq_swap_in kernel");
}

}  // namespace dgq
