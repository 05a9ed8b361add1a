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
#include <type_traits>

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
// chunk's loads go out.  (The fused decode takes the block id from the block ids it reads for its
// own span, which go out with these loads, instead of a second dependent load.)
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

// (min, max, min, max) of r over the wave, in every lane, without an LDS round trip: neighbour and
// pair exchanges within quads, the 8- and 16-lane mirrors of a row (DPP), then the permlane swaps
// of 16-lane rows and 32-lane halves.  (Minima and maxima do not depend on the order.)
template <int C>
__device__ __forceinline__ float append_dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), C, 0xF, 0xF, false));
}
__device__ __forceinline__ float4 span_wave_minmax(float4 r) {
  auto step = [&](auto tag) {
    constexpr int C = decltype(tag)::value;
    r.x = fminf(r.x, append_dpp<C>(r.x));
    r.y = fmaxf(r.y, append_dpp<C>(r.y));
    r.z = fminf(r.z, append_dpp<C>(r.z));
    r.w = fmaxf(r.w, append_dpp<C>(r.w));
  };
  step(std::integral_constant<int, 0xB1>{});    // quad_perm [1, 0, 3, 2]
  step(std::integral_constant<int, 0x4E>{});    // quad_perm [2, 3, 0, 1]
  step(std::integral_constant<int, 0x141>{});   // row_half_mirror
  step(std::integral_constant<int, 0x140>{});   // row_mirror: every lane holds its row's values
  auto swap16 = [](float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return make_float2(__uint_as_float(p[0]), __uint_as_float(p[1]));
  };
  auto swap32 = [](float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return make_float2(__uint_as_float(p[0]), __uint_as_float(p[1]));
  };
  float2 t;
  t = swap16(r.x); r.x = fminf(t.x, t.y);
  t = swap16(r.y); r.y = fmaxf(t.x, t.y);
  t = swap16(r.z); r.z = fminf(t.x, t.y);
  t = swap16(r.w); r.w = fmaxf(t.x, t.y);
  t = swap32(r.x); r.x = fminf(t.x, t.y);
  t = swap32(r.y); r.y = fmaxf(t.x, t.y);
  t = swap32(r.z); r.z = fminf(t.x, t.y);
  t = swap32(r.w); r.w = fmaxf(t.x, t.y);
  return r;
}

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

// The append of one token to (sequence b, kv head h), by all 256 threads of a workgroup, in two
// halves so that a fused decode can put its first chunk's loads between them:
//
//  * append_begin: from the loads above (one memory round trip), the span's new ranges and every
//    part of the decision that needs no more data; then, only when the span's codes may be
//    rewritten, its first-16-token window is tested or the block seals, the requests for the
//    span's fp16 staging copy (one 16-byte unit per thread and pass), and the bitmap byte a new
//    row would mark.  It stores nothing to global memory: every store of the append comes in
//    append_end, after the decision.
//  * append_end: the window and ring moments from the staged keys, the decision, the encode and
//    all the stores (the new token's staging copy included).  Nothing waits for a store: the
//    closing barrier orders the code stores before any later load by the same workgroup (a
//    decode of the tail block), and other workgroups or kernels only read them after this launch.
//
// With publish_nseg false the new row count is left to the caller (out.ns): a fused decode
// publishes it only after every workgroup of the same (sequence, head) has read the old count.
template <int D, int BS>
struct AppendShared {
  dgq_tail_t tl;
  uint16_t newk[D], newv[D];     // the new token
  int wbad[4];                   // per wave: the new token held a non-finite value
  dgq_seg_t srow[kMaxSegCap];   // the segment table as it was before this append
  dgq_seg_t chosen;
  int ns, blk, use_row, own_now, reenc_all;
  float4 red4[4];
  int mom_a[BS];                 // fixed-point moments of the span's tokens (span-relative index)
  long long mom_b[BS];
};

template <int D, int BS>
__device__ __forceinline__ AppendShared<D, BS> &append_shared() {
  __shared__ __align__(16) AppendShared<D, BS> sm;
  return sm;
}

// What append_begin hands to append_end (uniform across the workgroup, except the staged units
// and the bitmap byte, which stay with the thread that loaded them).
template <int D, int BS>
struct AppendStage {
  static constexpr int CPU = D / 8;                   // 16-byte units per token
  static constexpr int UPT = (BS * CPU + 255) / 256;  // units per thread, at most
  uint4 kw[UPT], vw[UPT];   // staged unit tid + 256 i: 8 channels of span token u / CPU
  uint32_t bits_old;        // thread 0: the bitmap byte holding r0's bit
  float4 rk;                // the span's K min, K max, V min, V max with the new token
  int t, r0, slot0, span_len, nunits, blk;
  bool go;                  // false: the state did not fit, nothing was appended
  bool window_test, seal, staged;
};

template <int D, int BS>
__device__ __forceinline__ void append_begin(const AppendArgs &a, int b, int h, AppendOut &out, const AppendLoads &ld,
                                             AppendStage<D, BS> &st) {
  const int tid = threadIdx.x;
  const size_t bh = (size_t)b * a.hkv + h;
  const int t = ld.t;
  AppendShared<D, BS> &sm = append_shared<D, BS>();
  if (tid < a.seg_cap) {
    uint4 *row = reinterpret_cast<uint4 *>(&sm.srow[tid]);
    row[0] = ld.seg[0];
    row[1] = ld.seg[1];
  }
  if (tid < kTailWords) reinterpret_cast<uint4 *>(&sm.tl)[tid] = ld.tail;
  if (tid < D) {
    sm.newk[tid] = ld.kb;
    sm.newv[tid] = ld.vb;
  }
  if (tid == 0) {
    sm.ns = ld.nseg;
    sm.blk = ld.blk;
  }
  const bool t_ok = ld.t_ok;
  __syncthreads();
  const int blk_t = t_ok ? sm.blk : -1;
  const int r0 = sm.tl.r0;
  const int ns = sm.ns;
  const int slot0 = r0 < 0 ? 0 : r0 % BS;
  const int span_len = t + 1 - r0;             // including the new token
  st.go = true;
  {
    // the state must place the new token inside the open span's block, and the block must exist
    // (r0 <= t and slot0 + span_len <= BS put r0 and t in the same block)
    bool bad = !t_ok || r0 < 0 || r0 > t || slot0 + span_len > BS || ns < 0 || ns > a.seg_cap ||
               (sm.tl.span_own != 0 && ns < 1) || sm.tl.ring_len < 0 || sm.tl.ring_len > kWin;
    if (!bad) checked_block(blk_t, a.cache.num_blocks, bad);
    if (bad) {
      if (tid == 0) {
        out.ok = 0;
        out.ns = ns;
        out.use_row = -1;
      }
      st.go = false;           // the caller counts it (out.ok == 0)
      return;
    }
  }
  const uint16_t *ks = a.cache.k_stage + bh * (size_t)BS * D;
  const uint16_t *vs = a.cache.v_stage + bh * (size_t)BS * D;

  // 1. the new token's ranges (and a non-finite check)
  float4 r = make_float4(INFINITY, -INFINITY, INFINITY, -INFINITY);
  float bad = 0.f;
  if (tid < D) {
    const float kx = half_bits_to_float(ld.kb), vx = half_bits_to_float(ld.vb);
    r.x = fminf(r.x, kx);
    r.y = fmaxf(r.y, kx);
    r.z = fminf(r.z, vx);
    r.w = fmaxf(r.w, vx);
    bad = fmaf(kx, 0.f, bad);
    bad = fmaf(vx, 0.f, bad);
  }
  r = span_wave_minmax(r);
  const bool wave_bad = __ballot(!(bad == 0.f)) != 0ull;
  if ((tid & 63) == 0) {
    sm.red4[tid >> 6] = r;
    sm.wbad[tid >> 6] = wave_bad ? 1 : 0;
  }
  __syncthreads();

  // 2. the span's ranges: the stored range of the earlier span tokens, widened by the new token
  // (every thread computes the same values in the same order)
  float4 q = sm.red4[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    q.x = fminf(q.x, sm.red4[w].x);
    q.y = fmaxf(q.y, sm.red4[w].y);
    q.z = fminf(q.z, sm.red4[w].z);
    q.w = fmaxf(q.w, sm.red4[w].w);
  }
  if (span_len > 1) {
    q.x = fminf(q.x, sm.tl.span_range[0]);
    q.y = fmaxf(q.y, sm.tl.span_range[1]);
    q.z = fminf(q.z, sm.tl.span_range[2]);
    q.w = fmaxf(q.w, sm.tl.span_range[3]);
  }
  const float4 rk = make_float4(q.x + 0.0f, q.y + 0.0f, q.z + 0.0f, q.w + 0.0f);

  // 3. what the decision can still need: the window test runs once the span has 16 tokens (until
  // it has said "no change": window and ring stay fixed for the span); the span's codes are
  // rewritten when it gets its own row (its range leaves the row before it, or the window test
  // says so) or its own row widens; a full block seals
  const bool own = sm.tl.span_own != 0;
  const int base = own ? ns - 2 : ns - 1;
  bool may_reenc;
  if (own) {
    const dgq_seg_t &R = sm.srow[ns - 1];
    may_reenc = R.kmin != rk.x || R.kmax != rk.y || R.vmin != rk.z || R.vmax != rk.w;
  } else {
    may_reenc = base < 0 || rk.x < sm.srow[base].kmin || rk.y > sm.srow[base].kmax || rk.z < sm.srow[base].vmin ||
                rk.w > sm.srow[base].vmax;
  }
  const bool window_test = !own && !may_reenc && span_len >= kWin && sm.tl.ring_len == kWin && !sm.tl.window_done;
  const bool seal = (t + 1) % BS == 0;
  const bool staged = may_reenc || window_test || seal;
  constexpr int CPU = AppendStage<D, BS>::CPU;
  const int nunits = span_len * CPU;
  // buffer loads of the earlier span tokens (the new one comes from LDS in append_end), every one
  // issued: a unit that is not needed gets an offset past the resource (zero, no memory access),
  // so no branch separates these loads from the caller's next ones
  const __amdgpu_buffer_rsrc_t rks = raw_rsrc(ks, BS * D * 2), rvs = raw_rsrc(vs, BS * D * 2);
#pragma unroll
  for (int i = 0; i < AppendStage<D, BS>::UPT; ++i) {
    const int u = tid + 256 * i;
    const uint32_t off = staged && u < nunits - CPU ? (uint32_t)(((slot0 + u / CPU) * D + 8 * (u % CPU)) * 2) : kOutOfRange;
    st.kw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rks, off, 0, 0));
    st.vw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rvs, off, 0, 0));
  }
  // the bitmap byte holding r0's bit, for a new row (thread 0)
  const bool want_bits = tid == 0 && !own && r0 > 0 && !a.fmt.marker && (may_reenc || window_test);
  const uint8_t *bits_blk = a.fmt.marker ? nullptr : a.cache.bits + ((size_t)blk_t * a.hkv + h) * (BS / 8);
  st.bits_old = __builtin_amdgcn_raw_buffer_load_b8(raw_rsrc(bits_blk, BS / 8), want_bits ? (uint32_t)((r0 % BS) / 8) : kOutOfRange,
                                                     0, 0);
  st.rk = rk;
  st.t = t;
  st.r0 = r0;
  st.slot0 = slot0;
  st.span_len = span_len;
  st.nunits = nunits;
  st.blk = blk_t;
  st.window_test = window_test;
  st.seal = seal;
  st.staged = staged;
}

template <int D, int BS>
__device__ __forceinline__ void append_end(const AppendArgs &a, int b, int h, bool publish_nseg, AppendOut &out,
                                           const AppendLoads &ld, const AppendStage<D, BS> &st) {
  if (!st.go) {
    __syncthreads();
    return;
  }
  constexpr int CPU = AppendStage<D, BS>::CPU;
  constexpr int UPT = AppendStage<D, BS>::UPT;
  const int tid = threadIdx.x;
  const size_t bh = (size_t)b * a.hkv + h;
  AppendShared<D, BS> &sm = append_shared<D, BS>();
  const int t = st.t, r0 = st.r0, slot0 = st.slot0, span_len = st.span_len;
  const int slot = t % BS;
  // the new token's units come from LDS (a select, so that the staged loads are waited for here,
  // before any store: see append_begin)
  uint4 kw[UPT], vw[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + 256 * i;
    const bool mine = u >= st.nunits - CPU && u < st.nunits;
    const uint4 nk = *reinterpret_cast<const uint4 *>(&sm.newk[8 * (u % CPU)]);
    const uint4 nv = *reinterpret_cast<const uint4 *>(&sm.newv[8 * (u % CPU)]);
    kw[i] = mine ? nk : st.kw[i];
    vw[i] = mine ? nv : st.vw[i];
  }

  // 4. fixed-point moments of the staged span tokens, for the window test and the ring: the CPU
  // units of a token sit in CPU consecutive lanes of one pass
  if (st.window_test || st.seal) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 256 * i;
      const uint32_t kh[4] = {kw[i].x, kw[i].y, kw[i].z, kw[i].w};
      int as = 0;
      long long bs2 = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int n = dgq_fixed_point(half_bits_to_float(e & 1 ? kh[e >> 1] >> 16 : kh[e >> 1] & 0xFFFFu));
        as += n;
        bs2 += (long long)(n * n);
      }
      if (u >= st.nunits) {
        as = 0;
        bs2 = 0;
      }
#pragma unroll
      for (int o = 1; o < CPU; o <<= 1) {
        as += __shfl_xor(as, o);
        bs2 += __shfl_xor(bs2, o);
      }
      if (u < st.nunits && u % CPU == 0) {
        sm.mom_a[u / CPU] = as;
        sm.mom_b[u / CPU] = bs2;
      }
    }
  }
  __syncthreads();

  // 5. decision (one thread)
  if (tid == 0) {
    const int nbad = sm.wbad[0] + sm.wbad[1] + sm.wbad[2] + sm.wbad[3];
    if (nbad > 0) atomicAdd(a.cache.status + 1, (unsigned long long)nbad);
    dgq_tail_t &tl = sm.tl;
    int ns = sm.ns;
    const int base = tl.span_own ? ns - 2 : ns - 1;
    const float4 rk = st.rk;
    bool want = tl.span_own != 0 || base < 0;
    if (!want) {
      const dgq_seg_t S = sm.srow[base];
      want = rk.x < S.kmin || rk.y > S.kmax || rk.z < S.vmin || rk.w > S.vmax;
      if (!want && st.window_test) {
        long long la = 0, lb = 0, ra = 0, rb = 0;
        for (int i = 0; i < kWin; ++i) {
          la += tl.ring_a[i];
          lb += tl.ring_b[i];
          ra += sm.mom_a[i];
          rb += sm.mom_b[i];
        }
        const long long nel = (long long)kWin * D;
        const long long ql = nel * lb - la * la, qr = nel * rb - ra * ra;
        const long long hi = ql > qr ? ql : qr, lo = ql > qr ? qr : ql;
        want = !((double)hi < a.qfloor) && (double)(hi + 1) / (double)(lo + 1) >= a.tau;
        if (!want) tl.window_done = 1;
      }
    }
    int all = 0;
    if (want && !tl.span_own) {
      if (ns >= a.seg_cap) {
        atomicAdd(a.cache.status + 0, 1ull);   // the table is full: the span joins the row before it
      } else {
        dgq_seg_t row;
        row.start = r0;
        row.kmin = rk.x;
        row.kmax = rk.y;
        row.vmin = rk.z;
        row.vmax = rk.w;
        row.kscale = dgq_scale(row.kmin, row.kmax, a.fmt.levels);
        row.vscale = dgq_scale(row.vmin, row.vmax, a.fmt.levels);
        row.reserved = 0;
        a.cache.segs[bh * a.seg_cap + ns] = row;
        sm.srow[ns] = row;
        ns += 1;
        tl.span_own = 1;
        all = 1;                                 // the span moves to its own range
        if (r0 > 0 && !a.fmt.marker)
          a.cache.bits[((size_t)st.blk * a.hkv + h) * (BS / 8) + (r0 % BS) / 8] =
              (uint8_t)((st.bits_old & 0xFFu) | (1u << (r0 % 8)));
      }
    } else if (want && tl.span_own) {
      dgq_seg_t row = sm.srow[ns - 1];
      all = row.kmin != rk.x || row.kmax != rk.y || row.vmin != rk.z || row.vmax != rk.w;
      row.kmin = rk.x;
      row.kmax = rk.y;
      row.vmin = rk.z;
      row.vmax = rk.w;
      row.kscale = dgq_scale(row.kmin, row.kmax, a.fmt.levels);
      row.vscale = dgq_scale(row.vmin, row.vmax, a.fmt.levels);
      a.cache.segs[bh * a.seg_cap + ns - 1] = row;
      sm.srow[ns - 1] = row;
    }
    sm.ns = ns;
    sm.use_row = tl.span_own ? ns - 1 : base;
    sm.chosen = sm.srow[sm.use_row];
    sm.own_now = tl.span_own;
    sm.reenc_all = all;
    out.ok = 1;
    out.ns = ns;
    out.use_row = sm.use_row;
    out.chosen = sm.chosen;
  }
  __syncthreads();

  // 6. encode with the chosen segment's range: the whole span when that range changed (a new row,
  // or the span's own row widened), else only the new token (every other span code is unchanged)
  const dgq_seg_t row = sm.chosen;
  const float lv = a.fmt.levels;
  const int low = a.fmt.low;
  const float kinv = dgq_inv(row.kmin, row.kmax, lv), vinv = dgq_inv(row.vmin, row.vmax, lv);
  // marker format: the span's own segment starts at r0, whose first key byte is the marker
  const bool mark = a.fmt.marker && sm.own_now && r0 > 0;
  int8_t *kt = a.cache.k_pool + ((size_t)st.blk * a.hkv + h) * (size_t)BS * D;
  int8_t *vt = a.cache.v_pool + ((size_t)st.blk * a.hkv + h) * (size_t)BS * D;
  if (tid < D) {
    // the new token's staging copy
    a.cache.k_stage[(bh * BS + slot) * D + tid] = ld.kb;
    a.cache.v_stage[(bh * BS + slot) * D + tid] = ld.vb;
  }
  if (!sm.reenc_all) {
    // only the new token changes: thread d < D still holds its channel d
    if (tid < D) {
      uint32_t kc = (uint32_t)(dgq_encode_value(half_bits_to_float(ld.kb), row.kmin, kinv, lv, low) & 0xFF);
      if (mark && slot == slot0 && tid == 0) kc = dgq_marker_byte(kc);
      kt[k_tile_offset<D, BS>(slot, tid)] = (int8_t)kc;
      vt[v_tile_offset<D, BS>(slot, tid)] = (int8_t)dgq_encode_value(half_bits_to_float(ld.vb), row.vmin, vinv, lv, low);
    }
  } else {
    // the whole span, from the staged units: 8 key codes stored as 8 contiguous bytes of the tile
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 256 * i;
      if (u < st.nunits) {
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

  // 7. the state: seal a full block (the ring keeps the moments of the last 16 sealed tokens), or
  // keep the span's ranges
  if (tid == 0) {
    dgq_tail_t &tl = sm.tl;
    if (publish_nseg) a.cache.nseg[bh] = sm.ns;
    if (st.seal) {
      // new ring = last 16 of (old ring, span tokens)
      const int m_tail = span_len < kWin ? span_len : kWin;   // span tokens that enter the ring
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
        na[n] = sm.mom_a[span_len - m_tail + i];
        nb[n] = sm.mom_b[span_len - m_tail + i];
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
      tl.span_range[0] = st.rk.x;
      tl.span_range[1] = st.rk.y;
      tl.span_range[2] = st.rk.z;
      tl.span_range[3] = st.rk.w;
    }
    a.cache.tail[bh] = tl;
  }
  // the code stores above come before any load of the tail block by this workgroup after this
  // barrier (workgroup scope: one compute unit, in-order vector memory)
  __syncthreads();
}

// The append kernel's form: the loads, then the append.
template <int D, int BS>
__device__ __forceinline__ void append_one(const AppendArgs &a, int b, int h, bool publish_nseg, AppendOut &out) {
  const int t = a.seq_lens[b];
  AppendLoads l = append_loads_state<D>(a, b, h);
  append_load_block<BS>(a, b, t, l);
  AppendStage<D, BS> st;
  append_begin<D, BS>(a, b, h, out, l, st);
  append_end<D, BS>(a, b, h, publish_nseg, out, l, st);
  if (threadIdx.x == 0 && !out.ok) atomicAdd(a.cache.status + 2, 1ull);   // the state did not fit
}

AppendArgs make_append_args(const dgq_params_t *p, const uint16_t *k_tok, const uint16_t *v_tok,
                            const int32_t *seq_lens, const int32_t *block_table, int32_t max_blocks,
                            const dgq_cache_t *cache);

}  // namespace dgq
