// Append one token to a DGQ-compressed (sequence, kv head), re-deciding only the open span of the
// tail block (DGQ article 2.2: the grouping is re-examined as tokens are generated).  Shared by the
// append kernel and the fused append + decode kernel.
//
// The span [r0, L] (L = tokens before this call) lives in an fp16 staging copy; the decision
// "join the segment before the span" versus "own segment" is re-taken from the span's K/V ranges
// and, once the span has 16 tokens, from the ratio of its first 16-token window variance to the 16
// sealed tokens before it (the same fixed-point window statistic and score as the compressor).
// The span's codes are rewritten with the chosen range; frozen tokens are never touched.  When the
// block fills, the span is sealed.
#pragma once

#include <climits>
#include <cmath>

#include "dgq_internal.h"

namespace dgq {

struct AppendArgs {
  const uint16_t *k_tok;
  const uint16_t *v_tok;
  const int32_t *seq_lens;
  const int32_t *block_table;
  int32_t max_blocks, hkv, seg_cap, num_blocks;
  double tau;
  double qfloor;   // variance floor on the Q scale (0 = off)
  CodeFormat fmt;
  dgq_cache_t cache;
};

// What one append left for a decode that follows it in the same workgroup.
struct AppendOut {
  int ok;            // 0: the state was inconsistent and nothing was appended (status[2] counted)
  int ns;            // segment-table rows after the append
  int use_row;       // row the open span is encoded with
  dgq_seg_t chosen;  // that row after the append
};

// The loads an append needs, all independent of one another: the new token (thread d < D holds
// channel d), the segment-table rows (thread k < seg_cap holds row k), the append state (thread i
// holds its 16-byte word i), and the row count and the new token's block id (thread 0).  A fused
// decode issues them before its first chunk: loads return in the order they were issued, so an
// append queued behind a chunk would wait for the whole chunk.  Every value stays with the
// thread that loaded it until the append passes it through LDS, so no wait is forced before the
// chunk's loads go out.
struct AppendLoads {
  uint16_t kb, vb;
  uint4 seg[2];
  uint4 tail;
  int nseg;
  int blk;      // the new token's block id (when t_ok)
  int t;        // position of the new token
  bool t_ok;
};
constexpr int kTailWords = (int)(sizeof(dgq_tail_t) / 16);
static_assert(sizeof(dgq_tail_t) % 16 == 0 && sizeof(dgq_seg_t) == 32, "16-byte words");

// The loads that depend only on (b, h).
template <int D>
__device__ __forceinline__ AppendLoads append_loads_state(const AppendArgs &a, int b, int h) {
  static_assert(D <= 256, "one channel per thread");
  const int tid = threadIdx.x;
  const size_t bh = (size_t)b * a.hkv + h;
  AppendLoads l;
  l.kb = 0;
  l.vb = 0;
  if (tid < D) {
    l.kb = a.k_tok[bh * D + tid];
    l.vb = a.v_tok[bh * D + tid];
  }
  if (tid < a.seg_cap) {
    const uint4 *row = reinterpret_cast<const uint4 *>(a.cache.segs + bh * a.seg_cap + tid);
    l.seg[0] = row[0];
    l.seg[1] = row[1];
  }
  if (tid < kTailWords) l.tail = reinterpret_cast<const uint4 *>(a.cache.tail + bh)[tid];
  l.nseg = tid == 0 ? a.cache.nseg[bh] : 0;
  return l;
}

// The new token's position t and block: a consistent state has the open span in that same block.
template <int BS>
__device__ __forceinline__ void append_load_block(const AppendArgs &a, int b, int t, AppendLoads &l) {
  l.t = t;
  l.t_ok = t >= 0 && t / BS < a.max_blocks;
  l.blk = 0;
  if (threadIdx.x == 0 && l.t_ok) l.blk = a.block_table[(size_t)b * a.max_blocks + t / BS];
}

// The append of one token to (sequence b, kv head h), by all 256 threads of a workgroup, from the
// loads of append_loads_state and append_load_block.  With publish_nseg false the new row count
// is left to the caller (out.ns): a fused decode publishes it only after every workgroup of the
// same (sequence, head) has read the old count.
template <int D, int BS>
__device__ __forceinline__ void append_one(const AppendArgs &a, int b, int h, bool publish_nseg, AppendOut &out,
                                           const AppendLoads &ld) {
  const int tid = threadIdx.x;
  const size_t bh = (size_t)b * a.hkv + h;
  const int t = ld.t;
  __shared__ __align__(16) dgq_tail_t tl;
  __shared__ int ns_sh, blk_sh, use_row, own_now, clamp_now;
  __shared__ float rk[4];                      // span ranges: kmin kmax vmin vmax
  __shared__ float4 red4[4];
  __shared__ long long span_a[kWin];
  __shared__ long long span_b[kWin];
  __shared__ long long tail_a[kWin];
  __shared__ long long tail_b[kWin];
  __shared__ dgq_seg_t chosen;
  __shared__ int reenc_all;                    // 1: every span token's codes change, 0: only the new one
  __shared__ __align__(16) dgq_seg_t srow[kMaxSegCap];   // the segment table as it was before this append
  const uint16_t kb = ld.kb, vb = ld.vb;
  if (tid < a.seg_cap) {
    uint4 *row = reinterpret_cast<uint4 *>(&srow[tid]);
    row[0] = ld.seg[0];
    row[1] = ld.seg[1];
  }
  if (tid < kTailWords) reinterpret_cast<uint4 *>(&tl)[tid] = ld.tail;
  if (tid == 0) {
    ns_sh = ld.nseg;
    blk_sh = ld.blk;
  }
  const bool t_ok = ld.t_ok;
  __syncthreads();
  const int blk_t = t_ok ? blk_sh : -1;
  const int r0 = tl.r0;
  const int slot0 = r0 < 0 ? 0 : r0 % BS;
  const int span_len = t + 1 - r0;             // including the new token
  {
    // the state must place the new token inside the open span's block, and the block must exist
    // (r0 <= t and slot0 + span_len <= BS put r0 and t in the same block)
    bool bad = !t_ok || r0 < 0 || r0 > t || slot0 + span_len > BS || ns_sh < 0 || ns_sh > a.seg_cap ||
               tl.ring_len < 0 || tl.ring_len > kWin;
    if (!bad) checked_block(blk_t, a.cache.num_blocks, bad);
    if (bad) {
      if (tid == 0) {
        atomicAdd(a.cache.status + 2, 1ull);
        out.ok = 0;
        out.ns = ns_sh;
        out.use_row = -1;
      }
      __syncthreads();
      return;
    }
  }
  uint16_t *ks = a.cache.k_stage + bh * (size_t)BS * D;
  uint16_t *vs = a.cache.v_stage + bh * (size_t)BS * D;

  // 1. stage the new token, and take its ranges (and a non-finite check) on the way
  const int slot = t % BS;
  float4 r = make_float4(INFINITY, -INFINITY, INFINITY, -INFINITY);
  float bad = 0.f;
  if (tid < D) {
    ks[slot * D + tid] = kb;
    vs[slot * D + tid] = vb;
    const float kx = half_bits_to_float(kb), vx = half_bits_to_float(vb);
    r.x = fminf(r.x, kx);
    r.y = fmaxf(r.y, kx);
    r.z = fminf(r.z, vx);
    r.w = fmaxf(r.w, vx);
    bad = fmaf(kx, 0.f, bad);
    bad = fmaf(vx, 0.f, bad);
  }

  // 2. span ranges: the stored range of the earlier span tokens, widened by the new token
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    r.x = fminf(r.x, __shfl_xor(r.x, o));
    r.y = fmaxf(r.y, __shfl_xor(r.y, o));
    r.z = fminf(r.z, __shfl_xor(r.z, o));
    r.w = fmaxf(r.w, __shfl_xor(r.w, o));
  }
  const bool wave_bad = __ballot(!(bad == 0.f)) != 0ull;
  if ((tid & 63) == 0) {
    red4[tid >> 6] = r;
    if (wave_bad) atomicAdd(a.cache.status + 1, 1ull);
  }
  __syncthreads();
  if (tid == 0) {
    float4 q = red4[0];
    for (int w = 1; w < 4; ++w) {
      q.x = fminf(q.x, red4[w].x);
      q.y = fmaxf(q.y, red4[w].y);
      q.z = fminf(q.z, red4[w].z);
      q.w = fmaxf(q.w, red4[w].w);
    }
    if (span_len > 1) {
      q.x = fminf(q.x, tl.span_range[0]);
      q.y = fmaxf(q.y, tl.span_range[1]);
      q.z = fminf(q.z, tl.span_range[2]);
      q.w = fmaxf(q.w, tl.span_range[3]);
    }
    rk[0] = q.x + 0.0f;
    rk[1] = q.y + 0.0f;
    rk[2] = q.z + 0.0f;
    rk[3] = q.w + 0.0f;
  }

  // 3. window statistics of the span's first 16 tokens: needed once the span has 16 tokens, and
  // only until the test has said "no change" (the window and the ring stay fixed for the span)
  const bool window_test = span_len >= kWin && tl.ring_len == kWin && !tl.span_own && !tl.window_done;
  if (window_test) {
    // moments of span token i (i < 16): wave w handles tokens 4w..4w+3, 16 lanes each
    const int w = tid >> 6, lane = tid & 63;
    for (int i = 4 * w + (lane >> 4); i < 4 * w + 4; i += 4) {
      int as = 0;
      long long bs2 = 0;
      for (int d = lane & 15; d < D; d += 16) {
        const int n = dgq_fixed_point(half_bits_to_float(ks[(slot0 + i) * D + d]));
        as += n;
        bs2 += (long long)(n * n);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        as += __shfl_xor(as, o);
        bs2 += __shfl_xor(bs2, o);
      }
      if ((lane & 15) == 0) {
        span_a[i] = as;
        span_b[i] = bs2;
      }
    }
  }
  __syncthreads();

  // 4. decision (one thread)
  if (tid == 0) {
    int ns = ns_sh;
    const int base = tl.span_own ? ns - 2 : ns - 1;
    bool want = tl.span_own != 0 || base < 0;
    if (!want) {
      const dgq_seg_t S = srow[base];
      want = rk[0] < S.kmin || rk[1] > S.kmax || rk[2] < S.vmin || rk[3] > S.vmax;
      if (!want && window_test) {
        long long la = 0, lb = 0, ra = 0, rb = 0;
        for (int i = 0; i < kWin; ++i) {
          la += tl.ring_a[i];
          lb += tl.ring_b[i];
          ra += span_a[i];
          rb += span_b[i];
        }
        const long long nel = (long long)kWin * D;
        const long long ql = nel * lb - la * la, qr = nel * rb - ra * ra;
        const long long hi = ql > qr ? ql : qr, lo = ql > qr ? qr : ql;
        want = !((double)hi < a.qfloor) && (double)(hi + 1) / (double)(lo + 1) >= a.tau;
        if (!want) tl.window_done = 1;
      }
    }
    int clampv = 0;
    int all = 0;
    if (want && !tl.span_own) {
      if (ns >= a.seg_cap) {
        clampv = 1;
        want = false;
      } else {
        dgq_seg_t row;
        row.start = r0;
        row.kmin = rk[0];
        row.kmax = rk[1];
        row.vmin = rk[2];
        row.vmax = rk[3];
        row.kscale = dgq_scale(row.kmin, row.kmax, a.fmt.levels);
        row.vscale = dgq_scale(row.vmin, row.vmax, a.fmt.levels);
        row.reserved = 0;
        a.cache.segs[bh * a.seg_cap + ns] = row;
        srow[ns] = row;
        ns += 1;
        tl.span_own = 1;
        all = 1;                                 // the span moves to its own range
        if (r0 > 0 && !a.fmt.marker) {
          uint8_t *byte = a.cache.bits + ((size_t)blk_t * a.hkv + h) * (BS / 8) + (r0 % BS) / 8;
          *byte = (uint8_t)(*byte | (1u << (r0 % 8)));
        }
      }
    } else if (want && tl.span_own) {
      dgq_seg_t row = srow[ns - 1];
      all = row.kmin != rk[0] || row.kmax != rk[1] || row.vmin != rk[2] || row.vmax != rk[3];
      row.kmin = rk[0];
      row.kmax = rk[1];
      row.vmin = rk[2];
      row.vmax = rk[3];
      row.kscale = dgq_scale(row.kmin, row.kmax, a.fmt.levels);
      row.vscale = dgq_scale(row.vmin, row.vmax, a.fmt.levels);
      a.cache.segs[bh * a.seg_cap + ns - 1] = row;
      srow[ns - 1] = row;
    }
    ns_sh = ns;
    use_row = tl.span_own ? ns - 1 : base;
    chosen = srow[use_row];
    out.ok = 1;
    out.ns = ns;
    out.use_row = use_row;
    out.chosen = chosen;
    own_now = tl.span_own;
    clamp_now = clampv;
    reenc_all = all;
    if (clampv) atomicAdd(a.cache.status + 0, 1ull);
  }
  __syncthreads();

  // 5. encode with the chosen segment's range: the whole span when that range changed (a new row,
  // or the span's own row widened), else only the new token (every other span code is unchanged)
  const dgq_seg_t row = chosen;
  const float lv = a.fmt.levels;
  const int low = a.fmt.low;
  const float kinv = dgq_inv(row.kmin, row.kmax, lv), vinv = dgq_inv(row.vmin, row.vmax, lv);
  // marker format: the span's own segment starts at r0, whose first key byte is the marker
  const bool mark = a.fmt.marker && own_now && r0 > 0;
  const int blk = blk_t;                       // the block of r0 and t (checked above)
  int8_t *kt = a.cache.k_pool + ((size_t)blk * a.hkv + h) * (size_t)BS * D;
  int8_t *vt = a.cache.v_pool + ((size_t)blk * a.hkv + h) * (size_t)BS * D;
  if (!reenc_all) {
    // only the new token changes: thread d < D still holds its channel d
    if (tid < D) {
      uint32_t kc = (uint32_t)(dgq_encode_value(half_bits_to_float(kb), row.kmin, kinv, lv, low) & 0xFF);
      if (mark && slot == slot0 && tid == 0) kc = dgq_marker_byte(kc);
      kt[k_tile_offset<D, BS>(slot, tid)] = (int8_t)kc;
      vt[v_tile_offset<D, BS>(slot, tid)] = (int8_t)dgq_encode_value(half_bits_to_float(vb), row.vmin, vinv, lv, low);
    }
  } else {
    // the whole span: one unit = 8 channels of one span token, a 16-byte load from the staging
    // copy and 8 key codes stored as 8 contiguous bytes of the tile; a thread's loads all go out
    // before any use
    constexpr int CPU = D / 8;                              // units per token
    constexpr int UPT = (BS * CPU + 255) / 256;             // units per thread, at most
    const int nunits = span_len * CPU;
    uint4 kw[UPT], vw[UPT];
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 256 * i;
      if (u < nunits) {
        const int s = slot0 + u / CPU, d0 = 8 * (u % CPU);
        kw[i] = *reinterpret_cast<const uint4 *>(ks + s * D + d0);
        vw[i] = *reinterpret_cast<const uint4 *>(vs + s * D + d0);
      }
    }
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 256 * i;
      if (u < nunits) {
        const int s = slot0 + u / CPU, d0 = 8 * (u % CPU);
        const uint32_t kh[4] = {kw[i].x, kw[i].y, kw[i].z, kw[i].w};
        const uint32_t vh[4] = {vw[i].x, vw[i].y, vw[i].z, vw[i].w};
        uint32_t kc[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kx = half_bits_to_float(e & 1 ? kh[e >> 1] >> 16 : kh[e >> 1] & 0xFFFFu);
          const float vx = half_bits_to_float(e & 1 ? vh[e >> 1] >> 16 : vh[e >> 1] & 0xFFFFu);
          kc[e >> 2] |= (uint32_t)(dgq_encode_value(kx, row.kmin, kinv, lv, low) & 0xFF) << (8 * (e & 3));
          vt[v_tile_offset<D, BS>(s, d0 + e)] = (int8_t)dgq_encode_value(vx, row.vmin, vinv, lv, low);
        }
        if (mark && s == slot0 && d0 == 0) kc[0] = (kc[0] & ~0xFFu) | dgq_marker_byte(kc[0] & 0xFFu);
        *reinterpret_cast<uint2 *>(kt + k_tile_offset<D, BS>(s, d0)) = make_uint2(kc[0], kc[1]);
      }
    }
  }

  // 6. seal a full block: the ring keeps the moments of the last 16 sealed tokens
  const bool seal = (t + 1) % BS == 0;
  const int m_tail = span_len < kWin ? span_len : kWin;   // span tokens that enter the ring
  if (seal) {
    const int w = tid >> 6, lane = tid & 63;
    for (int i = 4 * w + (lane >> 4); i < kWin; i += 16) {
      int as = 0;
      long long bs2 = 0;
      if (i < m_tail) {
        const int s = slot0 + span_len - m_tail + i;
        for (int d = lane & 15; d < D; d += 16) {
          const int n = dgq_fixed_point(half_bits_to_float(ks[s * D + d]));
          as += n;
          bs2 += (long long)(n * n);
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        as += __shfl_xor(as, o);
        bs2 += __shfl_xor(bs2, o);
      }
      if ((lane & 15) == 0) {
        tail_a[i] = as;
        tail_b[i] = bs2;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (publish_nseg) a.cache.nseg[bh] = ns_sh;
    if (seal) {
      // new ring = last 16 of (old ring, span tokens)
      const int old_keep = m_tail < kWin ? (tl.ring_len < kWin - m_tail ? tl.ring_len : kWin - m_tail) : 0;
      int32_t na[kWin];
      long long nb[kWin];
      int n = 0;
      for (int i = tl.ring_len - old_keep; i < tl.ring_len; ++i) {
        na[n] = tl.ring_a[i];
        nb[n] = tl.ring_b[i];
        ++n;
      }
      for (int i = 0; i < m_tail; ++i) {
        na[n] = (int32_t)tail_a[i];
        nb[n] = tail_b[i];
        ++n;
      }
      for (int i = 0; i < kWin; ++i) {
        tl.ring_a[i] = i < n ? na[i] : 0;
        tl.ring_b[i] = i < n ? nb[i] : 0;
      }
      tl.ring_len = n;
      tl.r0 = t + 1;
      tl.span_own = 0;
      tl.window_done = 0;
    } else {
      tl.span_own = own_now;
      for (int i = 0; i < 4; ++i) tl.span_range[i] = rk[i];
    }
    (void)clamp_now;
    a.cache.tail[bh] = tl;
  }
  // the span's codes must have landed before a fused decode in this workgroup loads the block
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// The append kernel's form: the loads, then the append.
template <int D, int BS>
__device__ __forceinline__ void append_one(const AppendArgs &a, int b, int h, bool publish_nseg, AppendOut &out) {
  const int t = a.seq_lens[b];
  AppendLoads l = append_loads_state<D>(a, b, h);
  append_load_block<BS>(a, b, t, l);
  append_one<D, BS>(a, b, h, publish_nseg, out, l);
}

AppendArgs make_append_args(const dgq_params_t *p, const uint16_t *k_tok, const uint16_t *v_tok,
                            const int32_t *seq_lens, const int32_t *block_table, int32_t max_blocks,
                            const dgq_cache_t *cache);

}  // namespace dgq
