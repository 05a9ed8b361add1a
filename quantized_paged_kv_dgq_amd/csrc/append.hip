// dgq_append: one workgroup per (sequence, kv head) runs append_one (append_common.h).
#include "append_common.h"

namespace dgq {

template <int D, int BS>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  AppendOut out;
  append_one<D, BS>(a, blockIdx.y, blockIdx.x, true, out);
}

template <int D>
static void launch_bs(const AppendArgs &a, int bs, int batch, hipStream_t s) {
  dim3 grid(a.hkv, batch);
  if (bs == 64) hipLaunchKernelGGL((append_kernel<D, 64>), grid, dim3(256), 0, s, a);
  else if (bs == 32) hipLaunchKernelGGL((append_kernel<D, 32>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((append_kernel<D, 16>), grid, dim3(256), 0, s, a);
}

AppendArgs make_append_args(const dgq_params_t *p, const uint16_t *k_tok, const uint16_t *v_tok,
                            const int32_t *seq_lens, const int32_t *block_table, int32_t max_blocks,
                            const dgq_cache_t *cache) {
  AppendArgs a;
  a.k_tok = k_tok;
  a.v_tok = v_tok;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.hkv = p->num_kv_heads;
  a.seg_cap = p->seg_capacity;
  a.num_blocks = cache->num_blocks;
  a.tau = p->tau;
  a.qfloor = variance_floor_q(p->min_var, p->head_dim);
  a.fmt = code_format(p);
  a.cache = *cache;
  return a;
}

dgq_status_t launch_append(const dgq_params_t *p, const uint16_t *k_tok, const uint16_t *v_tok,
                           const int32_t *seq_lens, int32_t batch, const int32_t *block_table,
                           int32_t max_blocks, const dgq_cache_t *cache, hipStream_t stream) {
  const AppendArgs a = make_append_args(p, k_tok, v_tok, seq_lens, block_table, max_blocks, cache);
  if (p->head_dim == 128) launch_bs<128>(a, p->block_size, batch, stream);
  else launch_bs<64>(a, p->block_size, batch, stream);
  return check_launch("dgq_append kernel");
}

}  // namespace dgq
