// Read the segment identifier back from a marker-format cache (DGQ article 3.2: the identifier
// lives in the INT8 data and is taken out with a bit mask).  One 256-thread workgroup per 256
// tokens of a (sequence, kv head): lane t tests the channel-0 key byte of its token, a wave-wide
// ballot packs 64 bits, and eight lanes write them as bytes in the bit-tensor layout.
#include "lifecycle.h"

namespace dgq {

struct MarkerArgs {
  const int8_t *k_pool;
  const int32_t *block_table;
  const int32_t *seq_lens;
  uint8_t *bits_out;
  unsigned long long *status;
  int32_t max_blocks, hkv, num_blocks, max_seq_len;
};

template <int D, int BS>
__global__ __launch_bounds__(256) void marker_bits_kernel(MarkerArgs a) {
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, lane = tid & 63;
  const int L_raw = a.seq_lens[b];
  const int L = L_raw < 0 ? 0 : (L_raw > a.max_seq_len ? a.max_seq_len : L_raw);
  if (blockIdx.x == 0 && h == 0 && tid == 0 && L != L_raw) atomicAdd(a.status + 2, 1ull);
  const int t0 = blockIdx.x * 256 + (tid & ~63);           // first token of this wave
  if (t0 >= L) return;
  const int32_t *bt = a.block_table + (size_t)b * a.max_blocks;
  const int t = t0 + lane;
  bool mark = false;
  if (t < L) {
    bool bad = false;
    const int blk = checked_block(bt[t / BS], a.num_blocks, bad);
    if (bad) {
      if (t % BS == 0) atomicAdd(a.status + 2, 1ull);
    } else {
      const uint32_t c = (uint8_t)a.k_pool[((size_t)blk * a.hkv + h) * (size_t)BS * D + k_tile_offset<D, BS>(t % BS, 0)];
      mark = c == 0x80u || c == 0x7Fu;
    }
  }
  const unsigned long long m = __ballot(mark);
  // lane i < 8 writes the byte of tokens t0 + 8i .. t0 + 8i + 7 (within one block: BS % 8 == 0)
  const int g = t0 + 8 * lane;
  if (lane < 8 && g < (L + BS - 1) / BS * BS) {
    bool bad = false;
    const int blk = checked_block(bt[g / BS], a.num_blocks, bad);
    if (!bad) a.bits_out[((size_t)blk * a.hkv + h) * (BS / 8) + (g % BS) / 8] = (uint8_t)(m >> (8 * lane));
  }
}

namespace {

template <int D>
void launch_bs(const MarkerArgs &a, int bs, int batch, hipStream_t s) {
  const int nx = (a.max_seq_len + 255) / 256;
  const dim3 grid(nx > 0 ? nx : 1, a.hkv, batch);
  if (bs == 64) hipLaunchKernelGGL((marker_bits_kernel<D, 64>), grid, dim3(256), 0, s, a);
  else if (bs == 32) hipLaunchKernelGGL((marker_bits_kernel<D, 32>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((marker_bits_kernel<D, 16>), grid, dim3(256), 0, s, a);
}

}  // namespace

dgq_status_t launch_marker_bits(const dgq_params_t *p, const dgq_cache_t *cache, const int32_t *block_table,
                                int32_t max_blocks, const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                uint8_t *bits_out, hipStream_t stream) {
  MarkerArgs a;
  a.k_pool = cache->k_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.bits_out = bits_out;
  a.status = cache->status;
  a.max_blocks = max_blocks;
  a.hkv = p->num_kv_heads;
  a.num_blocks = cache->num_blocks;
  a.max_seq_len = max_seq_len;
  if (p->head_dim == 128) launch_bs<128>(a, p->block_size, batch, stream);
  else launch_bs<64>(a, p->block_size, batch, stream);
  return check_launch("dgq_marker_bits kernel");
}

}  // namespace dgq
