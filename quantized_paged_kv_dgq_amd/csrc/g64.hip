// Fixed 64-channel group INT8 baseline (DGQ article 2.2: the LLM.int8()-style scheme the DGQ
// design is compared against -- every 64-channel chunk of every token has its own min/max).
//
// Same pool layout and code formula as DGQ; the per-(token, group) ranges are stored as fp16
// (min, max) pairs beside the pools.  The decode kernel is the DGQ decode with per-token-group
// scales: the two 64-channel slices of the QK product keep separate accumulators, and the PV
// weights carry the value scale of each channel group (rescaled per chunk).
#include "decode_common.h"

namespace dgq {

struct G64QArgs {
  const uint16_t *k;
  const uint16_t *v;
  int64_t stride_tok, stride_head;
  const int32_t *cu;
  const int32_t *first_pos;   // nullable: cache position of each sequence's first row
  const int32_t *block_table;
  int32_t max_blocks, hkv, max_rows, max_seq_len, num_blocks;
  int64_t total;
  int8_t *k_pool;
  int8_t *v_pool;
  uint32_t *k_range;
  uint32_t *v_range;
  unsigned long long *status;
};

typedef unsigned int u32x4_g __attribute__((ext_vector_type(4)));

// The quantizer reads its fp16 input once: non-temporal 16-byte loads (the lines are not kept).
__device__ __forceinline__ uint4 load_once(const uint16_t *p) {
  const u32x4_g v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_g *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t pack_range(float mn, float mx) {
  union { _Float16 f; uint16_t u; } a, b;
  a.f = (_Float16)mn;   // exact: both are fp16 values
  b.f = (_Float16)mx;
  return (uint32_t)a.u | ((uint32_t)b.u << 16);
}

template <int D, int BS>
__global__ __launch_bounds__(256) void g64_quantize_kernel(G64QArgs a) {
  constexpr int M = D / 64;
  constexpr int ROW = D + 8;   // padded LDS row (halves)
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  int c0, n;
  bool bad_seq;
  seq_range(a.cu, b, a.max_rows, a.total, c0, n, bad_seq);
  const int r0 = chunk * kChunk;
  if (r0 >= n) {
    if (chunk == 0 && tid == 0 && h == 0 && bad_seq) atomicAdd(a.status + 2, 1ull);
    return;
  }
  const int pos0 = a.first_pos ? a.first_pos[b] : 0;
  if (pos0 < 0 || pos0 + n > a.max_seq_len || pos0 + n > a.max_blocks * BS) {
    if (tid == 0 && h == 0 && chunk == 0) atomicAdd(a.status + 2, 1ull);
    return;
  }
  __shared__ uint16_t kt[kChunk * ROW];
  __shared__ uint16_t vt[kChunk * ROW];
  __shared__ float2 srange[2][kChunk][M];
  constexpr int VPR = D / 8;
  for (int x = tid; x < kChunk * VPR; x += 256) {
    const int tau = x / VPR, cc = x % VPR;
    uint4 wk = make_uint4(0u, 0u, 0u, 0u), wv = wk;
    if (r0 + tau < n) {
      const size_t off = (size_t)(c0 + r0 + tau) * a.stride_tok + (size_t)h * a.stride_head + 8 * cc;
      wk = load_once(a.k + off);
      wv = load_once(a.v + off);
    }
    uint32_t *dk = reinterpret_cast<uint32_t *>(kt + tau * ROW + 8 * cc);
    uint32_t *dv = reinterpret_cast<uint32_t *>(vt + tau * ROW + 8 * cc);
    dk[0] = wk.x; dk[1] = wk.y; dk[2] = wk.z; dk[3] = wk.w;
    dv[0] = wv.x; dv[1] = wv.y; dv[2] = wv.z; dv[3] = wv.w;
  }
  __syncthreads();
  const int32_t *bt = a.block_table + (size_t)b * a.max_blocks;
  // ranges: one (row, group, K|V) per thread
  for (int task = tid; task < kChunk * M * 2; task += 256) {
    const int which = task / (kChunk * M), rest = task % (kChunk * M);
    const int tau = rest / M, g = rest % M;
    const uint16_t *row = (which ? vt : kt) + tau * ROW + 64 * g;
    float mn = INFINITY, mx = -INFINITY;
    for (int e = 0; e < 64; ++e) {
      const float x = half_bits_to_float(row[e]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    mn += 0.0f;
    mx += 0.0f;
    srange[which][tau][g] = make_float2(mn, mx);
    if (r0 + tau < n) {
      const int pos = pos0 + r0 + tau;
      bool bad = false;
      const int blk = checked_block(bt[pos / BS], a.num_blocks, bad);
      if (!bad) {
        uint32_t *dst = (which ? a.v_range : a.k_range) + (((size_t)blk * a.hkv + h) * BS + pos % BS) * M + g;
        *dst = pack_range(mn, mx);
      } else {
        atomicAdd(a.status + 2, 1ull);
      }
    }
  }
  __syncthreads();
  const size_t tile_bytes = (size_t)BS * D;
  // keys: one unit = 16 channels of one row
  for (int u = tid; u < kChunk * D / 16; u += 256) {
    const int tau = u / (D / 16), d0 = 16 * (u % (D / 16));
    if (r0 + tau >= n) continue;
    const float2 rg = srange[0][tau][d0 / 64];
    const float inv = dgq_inv(rg.x, rg.y);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e)
      w[e >> 2] |= (uint32_t)(dgq_encode_value(half_bits_to_float(kt[tau * ROW + d0 + e]), rg.x, inv) & 0xFF) << (8 * (e & 3));
    const int pos = pos0 + r0 + tau;
    bool bad = false;
    const int blk = checked_block(bt[pos / BS], a.num_blocks, bad);
    if (bad) continue;
    int8_t *dst = a.k_pool + ((size_t)blk * a.hkv + h) * tile_bytes + k_tile_offset<D, BS>(pos % BS, d0);
    __builtin_nontemporal_store(u32x4_g{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4_g *>(dst));
  }
  // values: whole 16-token units when the chunk starts a block, single bytes otherwise
  if (pos0 % kChunk == 0) {
    for (int u = tid; u < kChunk * D / 16; u += 256) {
      int d, lb, taus[16];
      if constexpr (BS == 64) {
        const int nn = u / 64, jj = (u / 16) % 4, r = u % 16;
        d = 16 * nn + r;
        lb = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) taus[e] = 16 * (e >> 2) + 4 * jj + (e & 3);
      } else {
        lb = u / D;
        d = u % D;
#pragma unroll
        for (int e = 0; e < 16; ++e) taus[e] = 16 * lb + e;
      }
      const int pos_blk = pos0 + r0 + (BS == 64 ? 0 : 16 * lb);
      if (pos_blk >= pos0 + n) continue;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tau = taus[e];
        uint32_t c = 0u;
        if (r0 + tau < n) {
          const float2 rg = srange[1][tau][d / 64];
          c = (uint32_t)(dgq_encode_value(half_bits_to_float(vt[tau * ROW + d]), rg.x, dgq_inv(rg.x, rg.y)) & 0xFF);
        }
        w[e >> 2] |= c << (8 * (e & 3));
      }
      bool bad = false;
      const int blk = checked_block(bt[pos_blk / BS], a.num_blocks, bad);
      if (bad) continue;
      int8_t *tilep = a.v_pool + ((size_t)blk * a.hkv + h) * tile_bytes;
      int off;
      if constexpr (BS == 64) {
        const int nn = u / 64, jj = (u / 16) % 4, r = u % 16;
        off = ((nn * 4 + jj) * 16 + r) * 16;
      } else {
        off = d * 16;
      }
      __builtin_nontemporal_store(u32x4_g{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4_g *>(tilep + off));
    }
  } else {
    for (int x = tid; x < kChunk * D; x += 256) {
      const int tau = x / D, d = x % D;
      if (r0 + tau >= n) continue;
      const float2 rg = srange[1][tau][d / 64];
      const int pos = pos0 + r0 + tau;
      bool bad = false;
      const int blk = checked_block(bt[pos / BS], a.num_blocks, bad);
      if (bad) continue;
      a.v_pool[((size_t)blk * a.hkv + h) * tile_bytes + v_tile_offset<D, BS>(pos % BS, d)] =
          (int8_t)dgq_encode_value(half_bits_to_float(vt[tau * ROW + d]), rg.x, dgq_inv(rg.x, rg.y));
    }
  }
}

// ------------------------------------------------------------------------------------------------
// decode
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ float2 unpack_range(uint32_t w) {
  return make_float2(half_bits_to_float(w & 0xFFFFu), half_bits_to_float(w >> 16));
}

template <int D, int G, int BS>
__global__ __launch_bounds__(64 * kWaves, 2) void g64_decode_kernel(DecodeArgs a) {
  constexpr int M = D / 64;    // channel groups = 64-channel slices
  constexpr int NT = D / 16;
  // the kv head is rotated by the sequence index, as in the DGQ decode, so that every XCD serves
  // every head
  const int p = blockIdx.x, b = blockIdx.z, h = (int)((blockIdx.y + blockIdx.z) % (unsigned)a.hkv);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4, col = lane & 15, g = col >> 2, piece = col & 3;
  const bool live = (g < G) && (piece < 3);
  const ByteSel bsel = byte_sel(piece, live);
  const int L_raw = a.seq_lens[b];
  const int L = L_raw < 0 ? 0 : (L_raw > a.max_seq_len ? a.max_seq_len : L_raw);
  if (p == 0 && threadIdx.x == 0 && h == 0 && L != L_raw) atomicAdd(a.status + 2, 1ull);
  if (L == 0 && p == 0) {
    for (int e = threadIdx.x; e < G * D; e += 64 * kWaves) a.out[((size_t)b * a.hq + h * G) * D + e] = 0.f;
    return;
  }
  const int wg_begin = p * a.part_tokens * kWaves;
  if (p >= parts_of(L, a.part_tokens * kWaves)) return;
  const WaveRange wr = wave_range(wg_begin, a.part_tokens * kWaves, L, wave);
  const int t_begin = wr.t_begin, t_end = wr.t_end;
  const bool active = t_begin < t_end;
  const int wblk0 = wg_begin / BS;
  __shared__ int sh_blk[SpanBlocks<BS>::kBlocks];
  {
    SpanBlocks<BS> span_blk;
    span_blk.load(a.block_table + (size_t)b * a.max_blocks, a.max_blocks, wblk0);
    span_blk.publish(wblk0, (L + BS - 1) / BS, a.num_blocks, sh_blk, a.status);
  }
  __syncthreads();
  __shared__ float sh_o[kWaves][G][D];
  __shared__ float sh_m[kWaves][G], sh_l[kWaves][G];
  __shared__ uint32_t sh_rng[kWaves][2][kChunk][M];   // this chunk's K and V ranges

  float m_run = -INFINITY, l_run = 0.f, mv_run[M];
  float O[NT][4];
#pragma unroll
  for (int m = 0; m < M; ++m) mv_run[m] = 0.f;
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) O[n][i] = 0.f;

  if (active) {
    // query: three signed bytes per channel; per-group sums for the mid term
    const int qh = h * G + (g < G ? g : 0);
    const uint16_t *qrow = a.q + ((size_t)b * a.hq + qh) * D;
    float qv[M][16], qsum[M];
    float amax = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4 *src = reinterpret_cast<const uint4 *>(qrow + 64 * m + 16 * j);
      const uint4 w0 = src[0], w1 = src[1];
      const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      qsum[m] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[m][2 * e] = half_bits_to_float(ws[e] & 0xFFFFu);
        qv[m][2 * e + 1] = half_bits_to_float(ws[e] >> 16);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        amax = fmaxf(amax, fabsf(qv[m][e]));
        qsum[m] += qv[m][e];
      }
      qsum[m] += __shfl_xor(qsum[m], 16);
      qsum[m] += __shfl_xor(qsum[m], 32);
      qsum[m] *= a.sm_log2;
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    int qexp = 0;
    if (amax > 0.f) {
      int ex;
      frexpf(amax, &ex);
      qexp = 22 - ex;
    }
    const float qmul = ldexpf(1.0f, qexp);
    v4i qfrag[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      uint32_t wq4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) wq4[e >> 2] |= sel_byte(fmaf(qv[m][e], qmul, kMagic), bsel) << (8 * (e & 3));
      qfrag[m] = v4i{(int)wq4[0], (int)wq4[1], (int)wq4[2], (int)wq4[3]};
    }
    const float wq = live ? ldexpf(a.sm_log2, 16 - 8 * piece - qexp) : 0.f;
    const float wpiece = live ? ldexpf(1.0f, -6 - 8 * piece) : 0.f;   // 2^(16 - 8 piece) / 2^22

    // block ids come from sh_blk: chunk c of the wave is local chunk lc0 + c of the workgroup
    const int lc0 = (t_begin - wg_begin) / kChunk;
    const size_t tile_bytes = (size_t)BS * D;
    const size_t blk_stride = (size_t)a.hkv * tile_bytes;
    const int8_t *kpool = a.k_pool + (size_t)h * tile_bytes;
    const int8_t *vpool = a.v_pool + (size_t)h * tile_bytes;

    const int nchunks = (t_end - t_begin + kChunk - 1) / kChunk;
    for (int c = 0; c < nchunks; ++c) {
      const int t0 = t_begin + c * kChunk;
      v4i kf[4][M], vf[NT];
      // ranges of the chunk: lane = token of the chunk
      {
        const int blk_l = BS == 64 ? sh_blk[lc0 + c] : sh_blk[4 * (lc0 + c) + (lane >> 4)];
        const size_t ridx = (((size_t)blk_l * a.hkv + h) * BS + (t0 + lane) % BS) * M;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          // read once per call, like the codes: non-temporal
          sh_rng[wave][0][lane][m] = t0 + lane < t_end ? __builtin_nontemporal_load(a.k_range + ridx + m) : 0u;
          sh_rng[wave][1][lane][m] = t0 + lane < t_end ? __builtin_nontemporal_load(a.v_range + ridx + m) : 0u;
        }
      }
      if constexpr (BS == 64) {
        const int blk = __builtin_amdgcn_readfirstlane(sh_blk[lc0 + c]);
        const int8_t *kb = kpool + (size_t)blk * blk_stride;
        const int8_t *vb = vpool + (size_t)blk * blk_stride;
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int m = 0; m < M; ++m) kf[T][m] = load_codes(kb + (((T * M + m) * 64) + lane) * 16);
#pragma unroll
        for (int n = 0; n < NT; ++n) vf[n] = load_codes(vb + (n * 64 + lane) * 16);
      } else {
        const int8_t *kb = kpool + (size_t)sh_blk[4 * (lc0 + c) + ((lane & 15) >> 2)] * blk_stride;
        const int8_t *vb = vpool + (size_t)sh_blk[4 * (lc0 + c) + j] * blk_stride;
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int m = 0; m < M; ++m)
            kf[T][m] = load_codes(kb + ((((T * M + m) * 4 + j) * 4 + (lane & 3)) * 16));
#pragma unroll
        for (int n = 0; n < NT; ++n) vf[n] = load_codes(vb + (16 * n + (lane & 15)) * 16);
      }
      auto tau_of = [&](int T, int i) -> int { return BS == 64 ? 16 * T + 4 * j + i : 16 * j + 4 * T + i; };

      // scores: per token, sum over groups of scale_g * (q_g . c_g) + mid_g * sum(q_g)
      float S[4][4];
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        v4i acc[M];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf[T][m], qfrag[m], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tau = tau_of(T, i);
          float s = 0.f, mid = 0.f;
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const float2 rg = unpack_range(sh_rng[wave][0][tau][m]);
            const float ks = (rg.y - rg.x) * (1.0f / 255.0f);
            s = fmaf((float)acc[m][i], ks, s);
            mid = fmaf(fmaf(128.0f, ks, rg.x), qsum[m], mid);
          }
          s *= wq;
          s += quad_xor1(s);
          s += quad_xor2(s);
          S[T][i] = t0 + tau < t_end ? s + mid : -INFINITY;
        }
      }
      float cmax = -INFINITY;
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, S[T][i]);
      cmax = max_xor32(max_xor16(cmax));
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      // value weights per group: p * vs_g, scaled by this chunk's largest vs_g
      float P[4][4], vsg[4][4][M], wmax[M];
#pragma unroll
      for (int m = 0; m < M; ++m) wmax[m] = 0.f;
      float psum = 0.f, pmv[M];
#pragma unroll
      for (int m = 0; m < M; ++m) pmv[m] = 0.f;
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tau = tau_of(T, i);
          P[T][i] = __builtin_amdgcn_exp2f(S[T][i] - m_new);
          psum += P[T][i];
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const float2 rg = unpack_range(sh_rng[wave][1][tau][m]);
            const float vs = (rg.y - rg.x) * (1.0f / 255.0f);
            vsg[T][i][m] = vs;
            wmax[m] = fmaxf(wmax[m], vs);
            pmv[m] = fmaf(P[T][i], fmaf(128.0f, vs, rg.x), pmv[m]);
          }
        }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        wmax[m] = wave_max(wmax[m]);
        mv_run[m] = fmaf(mv_run[m], alpha, pmv[m]);
      }
      l_run = fmaf(l_run, alpha, psum);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float wf = wmax[m] > 0.f ? 4194304.0f / wmax[m] : 0.f;
        uint32_t pw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int i = 0; i < 4; ++i) pw[T] |= sel_byte(fmaf(P[T][i] * vsg[T][i][m], wf, kMagic), bsel) << (8 * i);
        const v4i pfrag = v4i{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};
        const float fold = wmax[m] * wpiece;
#pragma unroll
        for (int n = m * (NT / M); n < (m + 1) * (NT / M); ++n) {
          const v4i cacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(vf[n], pfrag, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) O[n][i] = fmaf(O[n][i], alpha, (float)cacc[i] * fold);
        }
      }
    }
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    mv_run[m] += __shfl_xor(mv_run[m], 16);
    mv_run[m] += __shfl_xor(mv_run[m], 32);
  }
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = O[n][i];
      v += quad_xor1(v);
      v += quad_xor2(v);
      if (piece == 0 && g < G) sh_o[wave][g][16 * n + 4 * j + i] = active ? v + mv_run[n / (NT / M)] : 0.f;
    }
  if (j == 0 && piece == 0 && g < G) {
    sh_m[wave][g] = active ? m_run : -INFINITY;
    sh_l[wave][g] = active ? l_run : 0.f;
  }
  finish_partition<D, G>(a, b, h, p, L, sh_o, sh_m, sh_l);
}

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------
dgq_status_t launch_g64_quantize(const dgq_params_t *p, const uint16_t *k, const uint16_t *v,
                                 int64_t stride_tok, int64_t stride_head, const int32_t *cu_seqlens,
                                 const int32_t *first_pos, int32_t batch, int32_t max_rows,
                                 int64_t total_rows, const int32_t *block_table, int32_t max_blocks,
                                 int32_t max_seq_len, const dgq_g64_cache_t *cache, hipStream_t stream) {
  if (max_rows == 0) return DGQ_OK;
  G64QArgs a;
  a.k = k;
  a.v = v;
  a.stride_tok = stride_tok;
  a.stride_head = stride_head;
  a.cu = cu_seqlens;
  a.first_pos = first_pos;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.hkv = p->num_kv_heads;
  a.max_rows = max_rows;
  a.max_seq_len = max_seq_len;
  a.num_blocks = cache->num_blocks;
  a.total = total_rows;
  a.k_pool = cache->k_pool;
  a.v_pool = cache->v_pool;
  a.k_range = cache->k_range;
  a.v_range = cache->v_range;
  a.status = cache->status;
  dim3 grid((max_rows + kChunk - 1) / kChunk, p->num_kv_heads, batch);
  if (p->head_dim == 128) {
    if (p->block_size == 64) hipLaunchKernelGGL((g64_quantize_kernel<128, 64>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((g64_quantize_kernel<128, 16>), grid, dim3(256), 0, stream, a);
  } else {
    if (p->block_size == 64) hipLaunchKernelGGL((g64_quantize_kernel<64, 64>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((g64_quantize_kernel<64, 16>), grid, dim3(256), 0, stream, a);
  }
  return check_launch("dgq_g64_quantize kernel");
}

template <int D, int G>
static void launch_g64_dec(const DecodeArgs &a, int bs, int batch, hipStream_t s) {
  dim3 grid(a.nparts, a.hkv, batch);
  if (bs == 64) hipLaunchKernelGGL((g64_decode_kernel<D, G, 64>), grid, dim3(64 * kWaves), 0, s, a);
  else hipLaunchKernelGGL((g64_decode_kernel<D, G, 16>), grid, dim3(64 * kWaves), 0, s, a);
}

template <int D>
static void launch_g64_dec_g(const DecodeArgs &a, int G, int bs, int batch, hipStream_t s) {
  if (G == 1) launch_g64_dec<D, 1>(a, bs, batch, s);
  else if (G == 2) launch_g64_dec<D, 2>(a, bs, batch, s);
  else launch_g64_dec<D, 4>(a, bs, batch, s);
}

dgq_status_t launch_g64_decode(const dgq_params_t *p, const uint16_t *q, const dgq_g64_cache_t *cache,
                               const int32_t *block_table, int32_t max_blocks, const int32_t *seq_lens,
                               int32_t batch, int32_t max_seq_len, float softmax_scale, float *out,
                               void *ws, hipStream_t stream) {
  DecodeArgs a = make_decode_args(p, q, cache->k_pool, cache->v_pool, cache->num_blocks, cache->status,
                                  block_table, max_blocks, seq_lens, batch, max_seq_len, softmax_scale, out, ws,
                                  kG64DecodeWaves);
  a.k_range = cache->k_range;
  a.v_range = cache->v_range;
  const int G = p->num_q_heads / p->num_kv_heads;
  if (p->head_dim == 128) launch_g64_dec_g<128>(a, G, p->block_size, batch, stream);
  else launch_g64_dec_g<64>(a, G, p->block_size, batch, stream);
  return check_launch("paged_decode_attn_g64 kernel");
}

}  // namespace dgq
