// Paged INT8 decode attention over DGQ-compressed KV blocks.
//
// What it computes: for every sequence b and query head g, softmax(scale * q . khat_t) . vhat_t
// over the cached tokens, where khat/vhat are the dequantized DGQ codes (DGQ article 3.1:
// dequantize inside the paged attention step; PagedAttention article: gather blocks through the
// block table).
//
// How (gfx950):
//  * One wave per (partition, kv head, sequence).  A partition is a run of 64-token chunks.
//  * The dequantization is folded into integer dot products: q . khat_t = ks_t * (q . c_t) +
//    midK_t * sum(q) and sum_t p_t vhat_t = sum_t (p_t vs_t) c_t + sum_t p_t midV_t, where
//    (ks, midK, vs, midV) belong to the segment of token t and mid = min + 128 * scale.
//  * q . c and (p vs) . c run on the int8 matrix cores (v_mfma_i32_16x16x64_i8) with exact int32
//    sums.  The float operand is split into three signed bytes (24-bit fixed point with a
//    power-of-two scale), one byte per matrix column: the 16 columns are (query head of the
//    group, byte) pairs.  Keys are the A operand (16 tokens x 64 channels), values the A operand
//    of the second product (16 channels x 64 tokens); both come straight from the pool, whose
//    tile order matches the operand layouts, so every load is a 16-byte lane load of contiguous
//    memory and no code is ever converted to float.
//  * Online softmax in base 2 per chunk; partial (max, sum, output) per partition; a second
//    kernel merges partitions by log-sum-exp.
#include <climits>
#include <cmath>

#include "dgq_internal.h"

namespace dgq {

typedef int v4i __attribute__((ext_vector_type(4)));

struct DecodeArgs {
  const uint16_t *q;
  const int8_t *k_pool;
  const int8_t *v_pool;
  const dgq_seg_t *segs;
  const int32_t *nseg;
  const int32_t *block_table;
  const int32_t *seq_lens;
  float *part_ml;   // [batch][hq][nparts][2]
  float *part_o;    // [batch][hq][nparts][D]
  float *out;       // [batch][hq][D]
  unsigned long long *status;
  int32_t hkv, hq, max_blocks, seg_cap, part_tokens, nparts, max_seq_len, num_blocks;
  float sm_log2;    // softmax_scale * log2(e)
};

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// The signed byte `piece` (0: bits 16.., 1: bits 8.., 2: bits 0..) of the balanced base-256
// digits of X, as an unsigned byte pattern; piece 3 is always 0.
__device__ __forceinline__ uint32_t piece_byte(int x, int piece) {
  const int v = piece == 0 ? ((x + 0x8080) >> 16) : piece == 1 ? ((x + 0x80) >> 8) : x;
  return piece < 3 ? (uint32_t)(v & 0xFF) : 0u;
}

template <int D, int G, int BS>
__global__ __launch_bounds__(64) void decode_partition_kernel(DecodeArgs a) {
  constexpr int M = D / 64;    // 64-channel slices of a key row
  constexpr int NT = D / 16;   // 16-channel tiles of the output
  const int p = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L_raw = a.seq_lens[b];
  const int L = L_raw < 0 ? 0 : (L_raw > a.max_seq_len ? a.max_seq_len : L_raw);
  if (p == 0 && threadIdx.x == 0 && h == 0 && L != L_raw) atomicAdd(a.status + 2, 1ull);
  const int t_begin = p * a.part_tokens;
  if (t_begin >= L) return;
  const int t_end = min(L, t_begin + a.part_tokens);

  const int lane = threadIdx.x;
  const int j = lane >> 4, col = lane & 15, g = col >> 2, piece = col & 3;
  const bool live = (g < G) && (piece < 3);

  // ---- segment table: lane k holds row k ----
  const int bh = b * a.hkv + h;
  const int ns = min(a.nseg[bh], a.seg_cap);
  int s_start = INT_MAX;
  float s_ks = 0.f, s_midk = 0.f, s_vs = 0.f, s_midv = 0.f;
  if (lane < ns) {
    const dgq_seg_t sg = a.segs[(size_t)bh * a.seg_cap + lane];
    s_start = sg.start;
    s_ks = sg.kscale;
    s_midk = sg.kmin + 128.0f * sg.kscale;
    s_vs = sg.vscale;
    s_midv = sg.vmin + 128.0f * sg.vscale;
  }
  float vsmax = s_vs;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) vsmax = fmaxf(vsmax, __shfl_xor(vsmax, o));
  const float wfac_unit = vsmax > 0.f ? 4194304.0f / vsmax : 0.f;   // 2^22 / vsmax
  const float s_wf = s_vs * wfac_unit;

  // ---- query: three signed bytes per channel, one per column of the B operand ----
  const int qh = h * G + (g < G ? g : 0);
  const uint16_t *qrow = a.q + ((size_t)b * a.hq + qh) * D;
  float qv[M][16];
  float amax = 0.f, qsum = 0.f;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint4 *src = reinterpret_cast<const uint4 *>(qrow + 64 * m + 16 * j);
    const uint4 w0 = src[0], w1 = src[1];
    const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[m][2 * e] = half_bits_to_float(ws[e] & 0xFFFFu);
      qv[m][2 * e + 1] = half_bits_to_float(ws[e] >> 16);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      amax = fmaxf(amax, fabsf(qv[m][e]));
      qsum += qv[m][e];
    }
  }
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  qsum += __shfl_xor(qsum, 16);
  qsum += __shfl_xor(qsum, 32);
  int qexp = 0;
  if (amax > 0.f) {
    int ex;
    frexpf(amax, &ex);
    qexp = 22 - ex;   // amax * 2^qexp in [2^21, 2^22)
  }
  v4i qfrag[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int x = (int)__builtin_rintf(ldexpf(qv[m][e], qexp));
      const uint32_t by = live ? piece_byte(x, piece) : 0u;
      wv[e >> 2] |= by << (8 * (e & 3));
    }
    qfrag[m] = v4i{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
  }
  // per-lane weight of this byte's partial dot product, in log2 units of the softmax
  const float wq = live ? ldexpf(a.sm_log2, 16 - 8 * piece - qexp) : 0.f;
  const float qsum_s = qsum * a.sm_log2;

  // ---- main loop over 64-token chunks ----
  float m_run = -INFINITY, l_run = 0.f, mv_run = 0.f;
  float O[NT][4];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) O[n][i] = 0.f;

  const int nblk_seq = (L + BS - 1) / BS;
  const int32_t *bt = a.block_table + (size_t)b * a.max_blocks;
  const size_t tile_bytes = (size_t)BS * D;

  for (int t0 = t_begin; t0 < t_end; t0 += kChunk) {
    v4i kf[4][M];
    v4i vf[NT];
    bool bad_blk = false;
    if constexpr (BS == 64) {
      const size_t blk = (size_t)checked_block(bt[t0 / 64], a.num_blocks, bad_blk);
      const int8_t *kb = a.k_pool + (blk * a.hkv + h) * tile_bytes;
      const int8_t *vb = a.v_pool + (blk * a.hkv + h) * tile_bytes;
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int m = 0; m < M; ++m)
          kf[T][m] = *reinterpret_cast<const v4i *>(kb + (((T * M + m) * 64) + lane) * 16);
#pragma unroll
      for (int n = 0; n < NT; ++n) vf[n] = *reinterpret_cast<const v4i *>(vb + (n * 64 + lane) * 16);
    } else {
      const int lb = t0 / 16;
      int bk = lb + ((lane & 15) >> 2);
      bk = bk < nblk_seq ? bk : lb;
      int bv = lb + j;
      bv = bv < nblk_seq ? bv : lb;
      const int8_t *kb = a.k_pool + ((size_t)checked_block(bt[bk], a.num_blocks, bad_blk) * a.hkv + h) * tile_bytes;
      const int8_t *vb = a.v_pool + ((size_t)checked_block(bt[bv], a.num_blocks, bad_blk) * a.hkv + h) * tile_bytes;
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int m = 0; m < M; ++m)
          kf[T][m] = *reinterpret_cast<const v4i *>(kb + ((((T * M + m) * 4 + j) * 4 + (lane & 3)) * 16));
#pragma unroll
      for (int n = 0; n < NT; ++n) vf[n] = *reinterpret_cast<const v4i *>(vb + (16 * n + (lane & 15)) * 16);
    }

    if (__ballot(bad_blk) != 0ull && lane == 0) atomicAdd(a.status + 2, 1ull);

    // S^T = K . Q^T : rows = tokens of tile T, columns = (query head, byte)
    float S[4][4];
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < M; ++m) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf[T][m], qfrag[m], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[T][i] = (float)acc[i] * wq;
    }
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = S[T][i];
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        S[T][i] = s;
      }

    // token of (T, i) for this lane
    auto tok_of = [&](int T, int i) -> int {
      return BS == 64 ? t0 + 16 * T + 4 * j + i : t0 + 16 * j + 4 * T + i;
    };

    const int t_last = min(t0 + kChunk, t_end) - 1;
    const int sf = max(__popcll(__ballot(s_start <= t0)) - 1, 0);
    const int sl = max(__popcll(__ballot(s_start <= t_last)) - 1, 0);
    float s2[4][4], wf[4][4], mvv[4][4];
    if (sf == sl) {
      const float ks = readlane_f(s_ks, sf), mk = readlane_f(s_midk, sf) * qsum_s;
      const float wfs = readlane_f(s_wf, sf), mvs = readlane_f(s_midv, sf);
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tok_of(T, i);
          s2[T][i] = t < t_end ? fmaf(ks, S[T][i], mk) : -INFINITY;
          wf[T][i] = wfs;
          mvv[T][i] = mvs;
        }
    } else {
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tok_of(T, i);
          int idx = 0;
          for (int k = 1; k < ns; ++k) idx += (t >= __builtin_amdgcn_readlane(s_start, k)) ? 1 : 0;
          const float ks = __shfl(s_ks, idx), mk = __shfl(s_midk, idx) * qsum_s;
          wf[T][i] = __shfl(s_wf, idx);
          mvv[T][i] = __shfl(s_midv, idx);
          s2[T][i] = t < t_end ? fmaf(ks, S[T][i], mk) : -INFINITY;
        }
    }

    // online softmax (base 2)
    float cmax = -INFINITY;
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, s2[T][i]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f, pmv = 0.f;
    uint32_t pw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = __builtin_amdgcn_exp2f(s2[T][i] - m_new);
        psum += pr;
        pmv = fmaf(pr, mvv[T][i], pmv);
        const int x = (int)__builtin_rintf(pr * wf[T][i]);
        const uint32_t by = live ? piece_byte(x, piece) : 0u;
        pw[T] |= by << (8 * i);
      }
    l_run = fmaf(l_run, alpha, psum);
    mv_run = fmaf(mv_run, alpha, pmv);
    const v4i pfrag = v4i{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};

    // O^T += V^T . P^T : rows = channels of tile n, columns = (query head, byte)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      v4i c = {0, 0, 0, 0};
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(vf[n], pfrag, c, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) O[n][i] = fmaf(O[n][i], alpha, (float)c[i]);
    }
  }

  // ---- epilogue: combine the byte columns, add the mid term, write the partial ----
  const float wv = live ? ldexpf(vsmax, -6 - 8 * piece) : 0.f;   // 2^(16-8*piece) * vsmax / 2^22
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  mv_run += __shfl_xor(mv_run, 16);
  mv_run += __shfl_xor(mv_run, 32);
  const size_t prow = ((size_t)b * a.hq + qh) * a.nparts + p;
  float *po = a.part_o + prow * D;
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = O[n][i] * wv;
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      if (piece == 0 && g < G) po[16 * n + 4 * j + i] = v + mv_run;
    }
  if (j == 0 && piece == 0 && g < G) {
    a.part_ml[prow * 2 + 0] = m_run;
    a.part_ml[prow * 2 + 1] = l_run;
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeArgs a) {
  const int qh = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L_raw = a.seq_lens[b];
  const int L = L_raw < 0 ? 0 : (L_raw > a.max_seq_len ? a.max_seq_len : L_raw);
  const int P = (L + a.part_tokens - 1) / a.part_tokens;
  const size_t row = (size_t)b * a.hq + qh;
  float res = 0.f;
  if (P > 0) {
    const float *ml = a.part_ml + row * a.nparts * 2;
    const float *po = a.part_o + row * a.nparts * D;
    float mx = -INFINITY;
    for (int p = 0; p < P; ++p) mx = fmaxf(mx, ml[2 * p]);
    float num = 0.f, den = 0.f;
    for (int p = 0; p < P; ++p) {
      const float w = __builtin_amdgcn_exp2f(ml[2 * p] - mx);
      num = fmaf(w, po[(size_t)p * D + d], num);
      den = fmaf(w, ml[2 * p + 1], den);
    }
    res = num / den;
  }
  a.out[row * D + d] = res;
}

DecodePlan decode_plan(const dgq_params_t *p, int32_t batch, int32_t max_seq_len) {
  DecodePlan plan;
  const int64_t chunks_seq = (max_seq_len + kChunk - 1) / kChunk;
  const int64_t total = (int64_t)batch * p->num_kv_heads * chunks_seq;
  const int64_t target = 2048;   // about one wave of residency on 256 CUs
  int64_t per = total > 0 ? (total + target - 1) / target : 1;
  if (per < 1) per = 1;
  if (per > 16) per = 16;
  plan.part_tokens = (int)(per * kChunk);
  plan.nparts = (int)((max_seq_len + plan.part_tokens - 1) / plan.part_tokens);
  if (plan.nparts < 1) plan.nparts = 1;
  return plan;
}

template <int D, int G, int BS>
static void launch_part(const DecodeArgs &a, int batch, hipStream_t s) {
  dim3 grid(a.nparts, a.hkv, batch);
  hipLaunchKernelGGL((decode_partition_kernel<D, G, BS>), grid, dim3(64), 0, s, a);
}

template <int D, int G>
static void launch_part_bs(const DecodeArgs &a, int bs, int batch, hipStream_t s) {
  if (bs == 64) launch_part<D, G, 64>(a, batch, s);
  else launch_part<D, G, 16>(a, batch, s);
}

template <int D>
static void launch_part_g(const DecodeArgs &a, int G, int bs, int batch, hipStream_t s) {
  if (G == 1) launch_part_bs<D, 1>(a, bs, batch, s);
  else if (G == 2) launch_part_bs<D, 2>(a, bs, batch, s);
  else launch_part_bs<D, 4>(a, bs, batch, s);
}

dgq_status_t launch_decode(const dgq_params_t *p, const uint16_t *q, const dgq_cache_t *cache,
                           const int32_t *block_table, int32_t max_blocks,
                           const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                           float softmax_scale, float *out, void *ws, hipStream_t stream) {
  const DecodePlan plan = decode_plan(p, batch, max_seq_len);
  const int D = p->head_dim, G = p->num_q_heads / p->num_kv_heads;
  DecodeArgs a;
  a.q = q;
  a.k_pool = cache->k_pool;
  a.v_pool = cache->v_pool;
  a.segs = cache->segs;
  a.nseg = cache->nseg;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.part_ml = reinterpret_cast<float *>(ws);
  a.part_o = a.part_ml + align_up((size_t)batch * p->num_q_heads * plan.nparts * 2, 64);
  a.out = out;
  a.hkv = p->num_kv_heads;
  a.hq = p->num_q_heads;
  a.max_blocks = max_blocks;
  a.seg_cap = p->seg_capacity;
  a.part_tokens = plan.part_tokens;
  a.nparts = plan.nparts;
  a.max_seq_len = max_seq_len;
  a.num_blocks = cache->num_blocks;
  a.status = cache->status;
  a.sm_log2 = softmax_scale * 1.4426950408889634f;
  if (D == 128) launch_part_g<128>(a, G, p->block_size, batch, stream);
  else launch_part_g<64>(a, G, p->block_size, batch, stream);
  dgq_status_t st = check_launch("paged_decode_attn_int8 partition kernel");
  if (st != DGQ_OK) return st;
  dim3 grid(p->num_q_heads, batch);
  if (D == 128) hipLaunchKernelGGL(decode_reduce_kernel<128>, grid, dim3(128), 0, stream, a);
  else hipLaunchKernelGGL(decode_reduce_kernel<64>, grid, dim3(64), 0, stream, a);
  return check_launch("paged_decode_attn_int8 reduce kernel");
}

size_t decode_workspace_bytes(const dgq_params_t *p, int32_t batch, int32_t max_seq_len) {
  const DecodePlan plan = decode_plan(p, batch, max_seq_len);
  const size_t rows = (size_t)batch * p->num_q_heads * plan.nparts;
  return (align_up(rows * 2, 64) + rows * p->head_dim) * sizeof(float) + 256;
}

}  // namespace dgq
