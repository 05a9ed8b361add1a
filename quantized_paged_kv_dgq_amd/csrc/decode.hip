// Paged INT8 decode attention over DGQ-compressed KV blocks.
//
// What it computes: for every sequence b and query head g, softmax(scale * q . khat_t) . vhat_t
// over the cached tokens, where khat/vhat are the dequantized DGQ codes (DGQ article 3.1:
// dequantize inside the paged attention step; PagedAttention article: gather blocks through the
// block table).
//
// How (gfx950):
//  * A workgroup of four waves per (partition, kv head, sequence); the partition's 64-token
//    chunks are split evenly over the waves, the waves are merged in LDS, and the last workgroup
//    of each (sequence, kv head) to finish merges the partitions by log-sum-exp.
//  * The dequantization is folded into integer dot products: q . khat_t = ks_t * (q . c_t) +
//    midK_t * sum(q) and sum_t p_t vhat_t = sum_t (p_t vs_t) c_t + sum_t p_t midV_t, where
//    (ks, midK, vs, midV) belong to the segment of token t and mid = min + 128 * scale (127 in
//    the marker format, whose codes start at -127).
//  * q . c and (p vs) . c run on the int8 matrix cores (v_mfma_i32_16x16x64_i8) with exact int32
//    sums.  The float operand is split into three signed bytes (24-bit fixed point with a
//    power-of-two scale), one byte per matrix column: the 16 columns are (query head of the
//    group, byte) pairs.  Keys are the A operand (16 tokens x 64 channels), values the A operand
//    of the second product (16 channels x 64 tokens); both come straight from the pool, whose
//    tile order matches the operand layouts, so every load is a 16-byte lane load of contiguous
//    memory and no code is ever converted to float.
//  * The PV products accumulate in the int32 matrix accumulators across chunks and are folded
//    into the float output only when the running maximum of some query head moves.
//  * Loads are software-pipelined: the next chunk's keys are requested as soon as the QK product
//    has consumed the key registers, its values as soon as the PV product has consumed the value
//    registers; the partition's block ids are read once, one per lane.
#include <algorithm>
#include <climits>
#include <cmath>

#include "append_common.h"
#include "decode_common.h"

namespace dgq {

// The decode of one workgroup; APPEND = true is the fused append + decode step, in which
// seq_lens holds the lengths before this step's token: the workgroup of the last partition of
// (b, h), the one whose tokens include the tail block, first appends the token and decodes with
// the updated segment rows; the new row count is published once every workgroup of (b, h) is
// done.
template <int D, int G, int BS, bool APPEND>
__device__ __forceinline__ void decode_body(const DecodeArgs &a, const AppendArgs *ap) {
  constexpr int M = D / 64;    // 64-channel slices of a key row
  constexpr int NT = D / 16;   // 16-channel tiles of the output
  // Consecutive workgroup ids go to consecutive XCDs.  With one partition per (sequence, head)
  // and 8 kv heads, XCD k would serve kv head k of every sequence; rotating the head by the
  // sequence index gives every XCD every head (measured 0.5 us off the 64 x 2048-token step).
  const int p = blockIdx.x, b = blockIdx.z, h = (int)((blockIdx.y + blockIdx.z) % (unsigned)a.hkv);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4, col = lane & 15, g = col >> 2, piece = col & 3;
  const bool live = (g < G) && (piece < 3);
  const ByteSel bsel = byte_sel(piece, live);
  const int bh = b * a.hkv + h;
  const int span = a.part_tokens * kWaves;
  const int wg_begin = p * span;

  // The sequence length goes out first, then (fused step) the append's loads that depend only on
  // (b, h), so that they land before the first chunks of all workgroups crowd the memory system;
  // a workgroup that turns out not to append has spent about a kilobyte on them.  Then the loads
  // that do not depend on the length: the block ids of the workgroup's span, the segment-table
  // row of this lane and the query slice of this lane.
  const int len_raw = a.seq_lens[b];
  AppendLoads ald;
  if constexpr (APPEND) ald = append_loads_state<D>(*ap, b, h);
  const int32_t *bt = a.block_table + (size_t)b * a.max_blocks;
  const int wblk0 = wg_begin / BS;
  SpanBlocks<BS> span_blk;
  span_blk.load(bt, a.max_blocks, wblk0);
  // the segment-table row of this lane and the row count (the append's loads already hold them)
  int ns_raw;
  dgq_seg_t seg_raw = {};
  if constexpr (APPEND) {
    ns_raw = ald.nseg;
    seg_raw = __builtin_bit_cast(dgq_seg_t, ald.seg);
  } else {
    ns_raw = a.nseg[bh];
    if (lane < a.seg_cap) seg_raw = a.segs[(size_t)bh * a.seg_cap + lane];
  }
  const int qh = h * G + (g < G ? g : 0);
  const uint16_t *qrow = a.q + ((size_t)b * a.hq + qh) * D;
  uint4 qraw[M][2];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint4 *src = reinterpret_cast<const uint4 *>(qrow + 64 * m + 16 * j);
    qraw[m][0] = src[0];
    qraw[m][1] = src[1];
  }

  const int L_raw = len_raw + (APPEND ? 1 : 0);
  const int L = L_raw < 0 ? 0 : (L_raw > a.max_seq_len ? a.max_seq_len : L_raw);
  if (p == 0 && threadIdx.x == 0 && h == 0 && L != L_raw) atomicAdd(a.status + 2, 1ull);
  if (L == 0 && p == 0) {                          // an empty sequence attends to nothing: zeros
    for (int e = threadIdx.x; e < G * D; e += 64 * kWaves) a.out[((size_t)b * a.hq + h * G) * D + e] = 0.f;
    return;
  }
  const int P = parts_of(L, span);
  if (p >= P) return;                              // the whole workgroup has nothing to do
  AppendOut aout;
  AppendDecision adec;
  const WaveRange wr = wave_range(wg_begin, span, L, wave);
  const int t_begin = wr.t_begin, t_end = wr.t_end;
  const bool active = t_begin < t_end;
  const bool appending = APPEND && p == P - 1;
  // the appended token's block id is one of the span's (a length clamped to max_seq_len aside)
  __shared__ int sh_blk[SpanBlocks<BS>::kBlocks];
  __shared__ int sh_tail_raw;
  int tail_slot = -1;
  if constexpr (APPEND) {
    ald.t = len_raw;
    ald.t_ok = len_raw >= 0 && len_raw / BS < ap->max_blocks;
    ald.blk = 0;
    const int rs = len_raw / BS - wblk0;
    if (appending && ald.t_ok && rs >= 0 && rs < SpanBlocks<BS>::kBlocks) tail_slot = rs;
  }
  span_blk.publish(wblk0, (L + BS - 1) / BS, a.num_blocks, sh_blk, a.status, tail_slot, &sh_tail_raw);
  __syncthreads();
  if constexpr (APPEND) {
    // (a length clamped to max_seq_len puts the tail block outside the span: one load, no branch)
    const int fb = (int)__builtin_amdgcn_raw_buffer_load_b32(
        raw_rsrc(ap->block_table + (size_t)b * ap->max_blocks, (uint32_t)ap->max_blocks * 4u),
        appending && ald.t_ok && tail_slot < 0 ? (uint32_t)(len_raw / BS) * 4u : kOutOfRange, 0, 0);
    ald.blk = tail_slot >= 0 ? sh_tail_raw : fb;
  }

  // block ids come from sh_blk: chunk c of the wave is local chunk lc0 + c of the workgroup
  const int lc0 = (t_begin - wg_begin) / kChunk;
  const size_t tile_bytes = (size_t)BS * D;
  const int8_t *kpool = a.k_pool + (size_t)h * tile_bytes;
  const int8_t *vpool = a.v_pool + (size_t)h * tile_bytes;
  const size_t blk_stride = (size_t)a.hkv * tile_bytes;

  // Fragment loads of chunk c (64 tokens) of the partition.  Keys: tile T (16 tokens) x slice m
  // (64 channels) per A operand; values: channel tile n (16 channels) x 64 tokens per A operand.
  auto load_k = [&](int c, v4i (&kf)[4][M]) {
    if constexpr (BS == 64) {
      const int blk = __builtin_amdgcn_readfirstlane(sh_blk[lc0 + c]);
      const int8_t *kb = kpool + (size_t)blk * blk_stride;
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int m = 0; m < M; ++m)
          kf[T][m] = load_codes(kb + (((T * M + m) * 64) + lane) * 16);
    } else {
      // 16-token blocks, or 32-token blocks made of two 16-token tiles
      const int g4 = (lane & 15) >> 2;
      const int8_t *kb = BS == 16 ? kpool + (size_t)sh_blk[4 * (lc0 + c) + g4] * blk_stride
                                   : kpool + (size_t)sh_blk[2 * (lc0 + c) + (g4 >> 1)] * blk_stride + (g4 & 1) * 16 * D;
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int m = 0; m < M; ++m)
          kf[T][m] = load_codes(kb + ((((T * M + m) * 4 + j) * 4 + (lane & 3)) * 16));
    }
  };
  auto load_v = [&](int c, v4i (&vf)[NT]) {
    if constexpr (BS == 64) {
      const int blk = __builtin_amdgcn_readfirstlane(sh_blk[lc0 + c]);
      const int8_t *vb = vpool + (size_t)blk * blk_stride;
#pragma unroll
      for (int n = 0; n < NT; ++n) vf[n] = load_codes(vb + (n * 64 + lane) * 16);
    } else {
      const int8_t *vb = BS == 16 ? vpool + (size_t)sh_blk[4 * (lc0 + c) + j] * blk_stride
                                   : vpool + (size_t)sh_blk[2 * (lc0 + c) + (j >> 1)] * blk_stride + (j & 1) * 16 * D;
#pragma unroll
      for (int n = 0; n < NT; ++n) vf[n] = load_codes(vb + (16 * n + (lane & 15)) * 16);
    }
  };
  // Every workgroup requests each wave's first chunk as soon as it has the block ids, the one that
  // appends too: its common steps need no load after the append's own (issued at the start), and
  // a step that re-encodes the span waits for its staging copy behind the chunk (loads return in
  // issue order), which costs those few workgroups less than a later first chunk costs all of
  // them (58.0 against 59.7 us per streaming step).  The chunk is kept when none of its tokens is
  // in the tail block (the only block the append writes); otherwise (or for a wave with no
  // tokens) it is requested again after the append.
  v4i kf[4][M];
  v4i vf[NT];
  const int tail_start = (L - 1) / BS * BS;
  const bool early = appending && active && t_begin + kChunk <= tail_start;
  load_k(0, kf);   // every wave (a wave with no tokens reads a valid block it does not use): a
  load_v(0, vf);   // branch here would make the waits below count only the loads before it
  // ---- query: three signed bytes per channel, one per column of the B operand (its fp16 values
  // were requested at the start, ahead of the chunk) ----
  float qv[M][16];
  float amax = 0.f, qsum = 0.f;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint4 w0 = qraw[m][0], w1 = qraw[m][1];
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
  AppendStage<D, BS> st;
  if constexpr (APPEND) {
    if (appending) append_begin<D, BS>(*ap, b, h, aout, adec, ald, st);
  }
  int qexp = 0;
  if (amax > 0.f) {
    int ex;
    frexpf(amax, &ex);
    qexp = 22 - ex;   // amax * 2^qexp in [2^21, 2^22)
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
  // per-lane weight of this byte's partial dot product, in log2 units of the softmax
  const float wq = live ? ldexpf(a.sm_log2, 16 - 8 * piece - qexp) : 0.f;
  const float qsum_s = qsum * a.sm_log2;

  if constexpr (APPEND) {
    // a step that re-encodes the span, tests its window or seals the block takes the whole
    // workgroup (with barriers); any other step writes only the new token's codes, which the wave
    // that decodes the tail block does itself before it reads that block (its own stores precede
    // its own loads), so the other waves start their chunks at once
    // (a length clamped to max_seq_len leaves the new token outside every wave's tokens: then a
    // fixed wave writes it, as the append kernel does)
    if (appending) {
      const bool writes_token = ald.t == L - 1 ? active && t_begin <= L - 1 && L - 1 < t_end : wave == kNewTokenWave;
      if (append_needs_span(adec, st)) append_span<D, BS>(*ap, b, h, aout, adec, ald, st);
      else if (st.go && writes_token) append_new_token<D, BS>(*ap, b, h, adec, ald, st);
      append_stash<D, BS>(adec, st);
    }
  }
  __shared__ float sh_o[kWaves][G][D];
  __shared__ float sh_m[kWaves][G], sh_l[kWaves][G];

  float m_run = -INFINITY, l_run = 0.f, mv_run = 0.f;
  float oacc[NT * 4];   // float output of each lane (C layout), folded from the int32 sums when a maximum moves
#pragma unroll
  for (int r = 0; r < NT * 4; ++r) oacc[r] = 0.f;
  float wv = 0.f;

  if (active) {
    const int nchunks = (t_end - t_begin + kChunk - 1) / kChunk;
    if (appending && !early) {   // the chunk holds the tail block: read it after the append
      load_k(0, kf);
      load_v(0, vf);
    }
    // ---- segment table: lane k holds row k (after this step's append, for its workgroup) ----
    const bool appended = appending;
    const int ns = min(appended ? aout.ns : ns_raw, a.seg_cap);
    int s_start = INT_MAX;
    float s_ks = 0.f, s_midk = 0.f, s_vs = 0.f, s_midv = 0.f;
    if (lane < ns) {
      const dgq_seg_t sg = appended && lane == aout.use_row ? aout.chosen : seg_raw;
      s_start = sg.start;
      s_ks = sg.kscale;
      s_midk = sg.kmin + a.code_mid * sg.kscale;
      s_vs = sg.vscale;
      s_midv = sg.vmin + a.code_mid * sg.vscale;
    }
    // the largest value scale among the segments this wave's tokens can use (rows starting after
    // its last token are left out: they cannot apply, and in the fused step the open span's row
    // may be rewritten while other workgroups run)
    float vsmax = s_start <= t_end - 1 ? s_vs : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) vsmax = fmaxf(vsmax, __shfl_xor(vsmax, o));
    const float wfac_unit = vsmax > 0.f ? 4194304.0f / vsmax : 0.f;   // 2^22 / vsmax
    const float s_wf = s_vs * wfac_unit;
    wv = live ? ldexpf(vsmax, -6 - 8 * piece) : 0.f;                // 2^(16-8*piece) * vsmax / 2^22

    // segment index of token t (rows are sorted by start; row 0 starts at 0)
    auto seg_of = [&](int t) -> int {
      int idx = 0;
      for (int k = 1; k < ns; ++k) idx += (t >= __builtin_amdgcn_readlane(s_start, k)) ? 1 : 0;
      return idx;
    };

    v4i cacc[NT];   // int32 PV sums since the last fold into O
#pragma unroll
    for (int n = 0; n < NT; ++n) cacc[n] = v4i{0, 0, 0, 0};

    for (int c = 0; c < nchunks; ++c) {
      const int t0 = t_begin + c * kChunk;

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
      if (c + 1 < nchunks) load_k(c + 1, kf);
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = S[T][i];
          s += quad_xor1(s);
          s += quad_xor2(s);
          S[T][i] = s;
        }

      // token of (T, i) for this lane
      auto tok_of = [&](int T, int i) -> int {
        return BS == 64 ? t0 + 16 * T + 4 * j + i : t0 + 16 * j + 4 * T + i;
      };

      // scores in log2 units, with the segment's (ks, midK) of every token
      const int t_last = min(t0 + kChunk, t_end) - 1;
      const int sf = max(__popcll(__ballot(s_start <= t0)) - 1, 0);
      const int sl = max(__popcll(__ballot(s_start <= t_last)) - 1, 0);
      const bool uni = sf == sl;
      if (uni) {
        const float ks = readlane_f(s_ks, sf), mk = readlane_f(s_midk, sf) * qsum_s;
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[T][i] = fmaf(ks, S[T][i], mk);
      } else {
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int idx = seg_of(tok_of(T, i));
            S[T][i] = fmaf(__shfl(s_ks, idx), S[T][i], __shfl(s_midk, idx) * qsum_s);
          }
      }
      if (t0 + kChunk > t_end) {   // partial last chunk: tokens past the end weigh nothing
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[T][i] = tok_of(T, i) < t_end ? S[T][i] : -INFINITY;
      }

      // online softmax (base 2)
      float cmax = -INFINITY;
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, S[T][i]);
      cmax = max_xor32(max_xor16(cmax));
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      if (__ballot(m_new > m_run) != 0ull) {
        // some head's maximum moved: fold the int32 sums (relative to the old maximum) into O
#pragma unroll
        for (int n = 0; n < NT; ++n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[4 * n + i] = (oacc[4 * n + i] + (float)cacc[n][i]) * alpha;
          cacc[n] = v4i{0, 0, 0, 0};
        }
      }
      m_run = m_new;
      float psum = 0.f, pmv = 0.f;
      uint32_t pw[4] = {0u, 0u, 0u, 0u};
      if (uni) {
        const float wfs = readlane_f(s_wf, sf), mvs = readlane_f(s_midv, sf);
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pr = __builtin_amdgcn_exp2f(S[T][i] - m_new);
            psum += pr;
            pw[T] |= sel_byte(fmaf(pr, wfs, kMagic), bsel) << (8 * i);
          }
        pmv = psum * mvs;
      } else {
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int idx = seg_of(tok_of(T, i));
            const float pr = __builtin_amdgcn_exp2f(S[T][i] - m_new);
            psum += pr;
            pmv = fmaf(pr, __shfl(s_midv, idx), pmv);
            pw[T] |= sel_byte(fmaf(pr, __shfl(s_wf, idx), kMagic), bsel) << (8 * i);
          }
      }
      l_run = fmaf(l_run, alpha, psum);
      mv_run = fmaf(mv_run, alpha, pmv);
      const v4i pfrag = v4i{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};

      // O^T += V^T . P^T : rows = channels of tile n, columns = (query head, byte)
#pragma unroll
      for (int n = 0; n < NT; ++n) cacc[n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(vf[n], pfrag, cacc[n], 0, 0, 0);
      if (c + 1 < nchunks) load_v(c + 1, vf);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[4 * n + i] += (float)cacc[n][i];
  }

  // ---- epilogue: combine the byte columns and the mid term per wave, then merge the waves of
  // the workgroup in LDS and write one partial (m, l, o) per query head ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  mv_run += __shfl_xor(mv_run, 16);
  mv_run += __shfl_xor(mv_run, 32);
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = oacc[4 * n + i] * wv;
      v += quad_xor1(v);
      v += quad_xor2(v);
      if (piece == 0 && g < G) sh_o[wave][g][16 * n + 4 * j + i] = active ? v + mv_run : 0.f;
    }
  if (j == 0 && piece == 0 && g < G) {
    sh_m[wave][g] = active ? m_run : -INFINITY;
    sh_l[wave][g] = active ? l_run : 0.f;
  }
  const int done = finish_partition<D, G>(a, b, h, p, L, sh_o, sh_m, sh_l, APPEND && p == P - 1 ? aout.ns : -1);
  if constexpr (APPEND) {
    // the append's state stores: every wave has passed the merge's first barrier, so none is
    // still reading the state; nothing in this launch reads what they write
    if (appending) append_store_state<D, BS>(*ap, b, h, false);
  }
  // an append whose state did not fit the new position (nothing was appended) is counted once
  if (appending && threadIdx.x == 0 && !aout.ok) atomicAdd(ap->cache.status + 2, 1ull);
  if (APPEND && done != kPartialOnly && threadIdx.x == 0) {
    // every workgroup of (b, h) has read the old row count: publish the new one
    const size_t bhs = (size_t)b * a.hkv + h;
    ap->cache.nseg[bhs] = done == kWroteOutput ? aout.ns
                                               : __hip_atomic_load(a.pend_nseg + bhs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}


template <int D, int G, int BS>
__global__ __launch_bounds__(64 * kWaves, 2) void decode_partition_kernel(DecodeArgs a) {
  decode_body<D, G, BS, false>(a, nullptr);
}

template <int D, int G, int BS>
__global__ __launch_bounds__(64 * kWaves, 2) void append_decode_kernel(DecodeArgs a, AppendArgs ap) {
  decode_body<D, G, BS, true>(a, &ap);
}

DecodePlan decode_plan(const dgq_params_t *p, int32_t batch, int32_t max_seq_len, int64_t target_waves) {
  // Each workgroup takes up to kWaves * per consecutive 64-token chunks of one (sequence, kv
  // head) and writes one partial; its waves split them evenly.  Aim at target_waves in all (1024 =
  // one workgroup per compute unit for the DGQ decode: fewer, longer workgroups leave fewer
  // partials to merge, and one wave per SIMD already keeps enough loads in flight).  Then even out
  // the partitions of the longest sequence, so that no workgroup is left with a small remainder.
  DecodePlan plan;
  // a partial last chunk rides along with the last partition (parts_of), so count full chunks
  const int64_t chunks_seq = std::max<int64_t>(max_seq_len / kChunk, 1);
  const int64_t total = (int64_t)batch * p->num_kv_heads * chunks_seq;
  const int64_t target = target_waves;
  int64_t per = total > 0 ? (total + target - 1) / target : 1;
  if (per < 1) per = 1;
  if (per > kMaxRun) per = kMaxRun;
  int64_t nparts = (chunks_seq + per * kWaves - 1) / (per * kWaves);
  if (nparts < 1) nparts = 1;
  per = (chunks_seq + nparts * kWaves - 1) / (nparts * kWaves);
  if (per < 1) per = 1;
  plan.part_tokens = (int)(per * kChunk);
  plan.nparts = (int)nparts;
  return plan;
}

template <int D, int G, int BS>
static void launch_part(const DecodeArgs &a, int batch, hipStream_t s) {
  dim3 grid(a.nparts, a.hkv, batch);
  hipLaunchKernelGGL((decode_partition_kernel<D, G, BS>), grid, dim3(64 * kWaves), 0, s, a);
}

template <int D, int G>
static void launch_part_bs(const DecodeArgs &a, int bs, int batch, hipStream_t s) {
  if (bs == 64) launch_part<D, G, 64>(a, batch, s);
  else if (bs == 32) launch_part<D, G, 32>(a, batch, s);
  else launch_part<D, G, 16>(a, batch, s);
}

template <int D>
static void launch_part_g(const DecodeArgs &a, int G, int bs, int batch, hipStream_t s) {
  if (G == 1) launch_part_bs<D, 1>(a, bs, batch, s);
  else if (G == 2) launch_part_bs<D, 2>(a, bs, batch, s);
  else launch_part_bs<D, 4>(a, bs, batch, s);
}

DecodeArgs make_decode_args(const dgq_params_t *p, const uint16_t *q, const int8_t *k_pool,
                            const int8_t *v_pool, int32_t num_blocks, unsigned long long *status,
                            const int32_t *block_table, int32_t max_blocks, const int32_t *seq_lens,
                            int32_t batch, int32_t max_seq_len, float softmax_scale, float *out,
                            void *ws, int64_t target_waves) {
  const DecodePlan plan = decode_plan(p, batch, max_seq_len, target_waves);
  DecodeArgs a = {};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  char *w = reinterpret_cast<char *>(ws);
  const size_t ctr_bytes = align_up((size_t)batch * p->num_kv_heads * sizeof(unsigned), 256);
  a.counters = reinterpret_cast<unsigned *>(w);
  a.pend_nseg = reinterpret_cast<int32_t *>(w + ctr_bytes);
  a.part_ml = reinterpret_cast<float *>(w + 2 * ctr_bytes);
  a.part_o = a.part_ml + align_up((size_t)batch * p->num_q_heads * plan.nparts * 2, 64);
  a.out = out;
  a.status = status;
  a.hkv = p->num_kv_heads;
  a.hq = p->num_q_heads;
  a.max_blocks = max_blocks;
  a.seg_cap = p->seg_capacity;
  a.part_tokens = plan.part_tokens;
  a.nparts = plan.nparts;
  a.max_seq_len = max_seq_len;
  a.num_blocks = num_blocks;
  a.sm_log2 = softmax_scale * 1.4426950408889634f;
  a.code_mid = (float)-code_format(p).low;
  return a;
}

dgq_status_t launch_decode(const dgq_params_t *p, const uint16_t *q, const dgq_cache_t *cache,
                           const int32_t *block_table, int32_t max_blocks,
                           const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                           float softmax_scale, float *out, void *ws, hipStream_t stream) {
  DecodeArgs a = make_decode_args(p, q, cache->k_pool, cache->v_pool, cache->num_blocks, cache->status,
                                  block_table, max_blocks, seq_lens, batch, max_seq_len, softmax_scale, out, ws,
                                  kDgqDecodeWaves);
  a.segs = cache->segs;
  a.nseg = cache->nseg;
  const int D = p->head_dim, G = p->num_q_heads / p->num_kv_heads;
  if (D == 128) launch_part_g<128>(a, G, p->block_size, batch, stream);
  else launch_part_g<64>(a, G, p->block_size, batch, stream);
  return check_launch("paged_decode_attn_int8 kernel");
}

template <int D, int G>
static void launch_fused_bs(const DecodeArgs &a, const AppendArgs &ap, int bs, int batch, hipStream_t s) {
  dim3 grid(a.nparts, a.hkv, batch);
  if (bs == 64) hipLaunchKernelGGL((append_decode_kernel<D, G, 64>), grid, dim3(64 * kWaves), 0, s, a, ap);
  else if (bs == 32) hipLaunchKernelGGL((append_decode_kernel<D, G, 32>), grid, dim3(64 * kWaves), 0, s, a, ap);
  else hipLaunchKernelGGL((append_decode_kernel<D, G, 16>), grid, dim3(64 * kWaves), 0, s, a, ap);
}

template <int D>
static void launch_fused_g(const DecodeArgs &a, const AppendArgs &ap, int G, int bs, int batch, hipStream_t s) {
  if (G == 1) launch_fused_bs<D, 1>(a, ap, bs, batch, s);
  else if (G == 2) launch_fused_bs<D, 2>(a, ap, bs, batch, s);
  else launch_fused_bs<D, 4>(a, ap, bs, batch, s);
}

dgq_status_t launch_append_decode(const dgq_params_t *p, const uint16_t *k_tok, const uint16_t *v_tok,
                                  const int32_t *seq_lens, const uint16_t *q, int32_t batch,
                                  const int32_t *block_table, int32_t max_blocks, int32_t max_seq_len,
                                  float softmax_scale, const dgq_cache_t *cache, float *out, void *ws,
                                  hipStream_t stream) {
  DecodeArgs a = make_decode_args(p, q, cache->k_pool, cache->v_pool, cache->num_blocks, cache->status,
                                  block_table, max_blocks, seq_lens, batch, max_seq_len, softmax_scale, out, ws,
                                  kDgqDecodeWaves);
  a.segs = cache->segs;
  a.nseg = cache->nseg;
  AppendArgs ap = make_append_args(p, k_tok, v_tok, seq_lens, block_table, max_blocks, cache);
  const int D = p->head_dim, G = p->num_q_heads / p->num_kv_heads;
  if (D == 128) launch_fused_g<128>(a, ap, G, p->block_size, batch, stream);
  else launch_fused_g<64>(a, ap, G, p->block_size, batch, stream);
  return check_launch("dgq_append_decode kernel");
}

static size_t workspace_bytes_for_parts(const dgq_params_t *p, int32_t batch, int32_t nparts) {
  // completion counters, handed-over row counts, then (m, l) and the output of every partial
  const size_t rows = (size_t)batch * p->num_q_heads * nparts;
  return 2 * align_up((size_t)batch * p->num_kv_heads * sizeof(unsigned), 256) +
         (align_up(rows * 2, 64) + rows * p->head_dim) * sizeof(float) + 256;
}

size_t decode_workspace_bytes(const dgq_params_t *p, int32_t batch, int32_t max_seq_len) {
  // one size for both decoders: the larger partial count of their two plans
  const int32_t nparts = std::max(decode_plan(p, batch, max_seq_len, kDgqDecodeWaves).nparts,
                                  decode_plan(p, batch, max_seq_len, kG64DecodeWaves).nparts);
  return workspace_bytes_for_parts(p, batch, nparts);
}

size_t decode_workspace_bytes_for(const dgq_params_t *p, int32_t batch, int32_t max_seq_len,
                                  int64_t target_waves) {
  return workspace_bytes_for_parts(p, batch, decode_plan(p, batch, max_seq_len, target_waves).nparts);
}

}  // namespace dgq
