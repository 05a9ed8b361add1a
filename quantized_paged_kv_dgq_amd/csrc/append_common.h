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

// What one append left for a decode that follows it in the same workgroup (every thread holds
// the same values).
struct AppendOut {
  int ok;            // 0: the state was inconsistent and nothing was appended (status[2] counted)
  int ns;            // segment-table rows after the append
  int use_row;       // row the open span is encoded with
  dgq_seg_t chosen;  // that row after the append
};

// The loads an append needs, all independent of one another and all made by every wave: the new
// token (lane l < D/2 holds channels 2l and 2l+1), the segment-table rows (lane k < seg_cap holds
// row k), the append state (lane i holds its 16-byte word i) and the row count.  Every wave can
// then take the whole decision from its own registers.  A fused decode issues them before its
// first chunk: loads return in the order they were issued, so an append queued behind a chunk
// would wait for the whole chunk.  (The fused decode takes the new token's block id from the
// block ids it reads for its own span instead of a second dependent load.)
struct AppendLoads {
  uint32_t kp, vp;
  uint4 seg[2];
  uint4 tail;
  int nseg;
  int blk;      // the new token's block id (when t_ok), the same in every thread
  int t;        // position of the new token
  bool t_ok;
};
constexpr int kTailWords = (int)(sizeof(dgq_tail_t) / 16);
static_assert(sizeof(dgq_tail_t) % 16 == 0 && sizeof(dgq_seg_t) == 32, "16-byte words");
// word 0: r0, ring_len, span_own, window_done; words 1-4: ring_a; words 5-12: ring_b; word 13: span_range
static_assert(offsetof(dgq_tail_t, ring_a) == 16 && offsetof(dgq_tail_t, ring_b) == 80 &&
              offsetof(dgq_tail_t, span_range) == 208 && kTailWords == 14, "append state words");

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

// The loads that depend only on (b, h).  Buffer loads: a lane past the end of its resource reads
// zeros without touching memory, so no branch separates these loads from the caller's next ones.
template <int D>
__device__ __forceinline__ AppendLoads append_loads_state(const AppendArgs &a, int b, int h) {
  static_assert(D % 2 == 0 && D / 2 <= 64, "two channels per lane");
  const uint32_t lane = threadIdx.x & 63;
  const size_t bh = (size_t)b * a.hkv + h;
  AppendLoads l;
  l.kp = __builtin_amdgcn_raw_buffer_load_b32(raw_rsrc(a.k_tok + bh * D, D * 2), lane * 4, 0, 0);
  l.vp = __builtin_amdgcn_raw_buffer_load_b32(raw_rsrc(a.v_tok + bh * D, D * 2), lane * 4, 0, 0);
  const __amdgpu_buffer_rsrc_t rs = raw_rsrc(a.cache.segs + bh * a.seg_cap, (uint32_t)a.seg_cap * 32u);
  l.seg[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 32, 0, 0));
  l.seg[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 32 + 16, 0, 0));
  l.tail = __builtin_bit_cast(
      uint4, __builtin_amdgcn_raw_buffer_load_b128(raw_rsrc(a.cache.tail + bh, sizeof(dgq_tail_t)), lane * 16, 0, 0));
  l.nseg = a.cache.nseg[bh];
  l.blk = 0;
  l.t = 0;
  l.t_ok = false;
  return l;
}

// The new token's position t and block: a consistent state has the open span in that same block.
template <int BS>
__device__ __forceinline__ void append_load_block(const AppendArgs &a, int b, int t, AppendLoads &l) {
  l.t = t;
  l.t_ok = t >= 0 && t / BS < a.max_blocks;
  l.blk = (int)__builtin_amdgcn_raw_buffer_load_b32(raw_rsrc(a.block_table + (size_t)b * a.max_blocks, (uint32_t)a.max_blocks * 4u),
                                                    l.t_ok ? (uint32_t)(t / BS) * 4u : kOutOfRange, 0, 0);
}

// The outcome of the join-or-own decision.
struct AppendDecision {
  dgq_seg_t chosen;   // the row the span is encoded with, after the append
  int ns;             // rows after the append
  int use_row;        // index of that row
  int write_row;      // row this append stores (-1: none)
  bool new_row;       // the span gets a row of its own now
  bool own_now;       // the span has its own row after the append
  bool all;           // the span's range changed: every span code is rewritten
  bool full;          // a row of its own was wanted but the table is full (the span joins)
  bool wdone;         // the window test has said "no change" for this span
};

// want: the span should have its own row (it has one, its range left the row before it, or the
// window test says so).  R is row ns - 1: the span's own row, or the row it would join.
__device__ __forceinline__ AppendDecision append_decide(bool want, bool own, int ns, int seg_cap, int r0,
                                                        const dgq_seg_t &R, float4 rk, float levels) {
  AppendDecision d;
  d.chosen = R;
  d.ns = ns;
  d.use_row = ns - 1;
  d.write_row = -1;
  d.new_row = false;
  d.own_now = own;
  d.all = false;
  d.full = false;
  d.wdone = false;
  if (want && !own) {
    if (ns >= seg_cap) {
      d.full = true;
    } else {
      d.chosen.start = r0;
      d.chosen.kmin = rk.x;
      d.chosen.kmax = rk.y;
      d.chosen.vmin = rk.z;
      d.chosen.vmax = rk.w;
      d.chosen.kscale = dgq_scale(rk.x, rk.y, levels);
      d.chosen.vscale = dgq_scale(rk.z, rk.w, levels);
      d.chosen.reserved = 0;
      d.ns = ns + 1;
      d.use_row = ns;
      d.write_row = ns;
      d.new_row = true;
      d.own_now = true;
      d.all = true;   // the span moves to its own range
    }
  } else if (want) {
    // its own row, widened (or rewritten unchanged)
    d.all = (R.kmin != rk.x) | (R.kmax != rk.y) | (R.vmin != rk.z) | (R.vmax != rk.w);
    d.chosen.kmin = rk.x;
    d.chosen.kmax = rk.y;
    d.chosen.vmin = rk.z;
    d.chosen.vmax = rk.w;
    d.chosen.kscale = dgq_scale(rk.x, rk.y, levels);
    d.chosen.vscale = dgq_scale(rk.z, rk.w, levels);
    d.write_row = ns - 1;
  }
  return d;
}

// The append of one token to (sequence b, kv head h), by the four waves of a workgroup:
//
//  * append_begin: every wave, from its own registers (no barrier): the state, the span's new
//    ranges (DPP and permlane reductions), and the decision unless the window test is due; then,
//    only when the span's codes may be rewritten, its first-16-token window is tested or the block
//    seals, the requests for the span's fp16 staging copy (one 16-byte unit per thread and pass),
//    the value-tile words that hold frozen tokens of the same block, and the bitmap byte a new row
//    would mark.  It stores nothing.
//  * append_span (the window test, a seal or a re-encoded span; the whole workgroup): the window
//    and ring moments (one barrier), the encode and the code stores, then a barrier, which orders
//    the code stores before any later load of the tail block by the same workgroup (a decode of
//    the tail block); other workgroups or kernels only read them after this launch.
//  * append_new_token (any other step; one wave, no barrier): the new token's codes and staging
//    copy.  In a fused decode the wave that decodes the tail block writes them before it reads
//    that block, so its own stores come first.
//  * append_stash, then after a barrier append_store_state (wave 0): the status counts, the
//    segment row, the bitmap byte, the row count and the state, stored only once every wave has
//    read the state they replace.
//
// A re-encoded span's value codes go through an LDS image of the value tile and out as whole
// 16-byte words: a value tile interleaves the tokens of a block inside each word, so the codes of
// one token are single bytes 16 bytes apart, and storing them one by one costs a memory
// transaction per byte.
//
// With publish_nseg false the new row count is left to the caller (out.ns): a fused decode
// publishes it only after every workgroup of the same (sequence, head) has read the old count.
constexpr int kNewTokenWave = 3;   // the last of the workgroup's four waves

// What the state stores need, kept in LDS from the decision to the stores (a fused decode makes
// them after its chunks, and registers held that long would crowd the decode loop).
struct AppendPending {
  dgq_seg_t chosen;
  float4 rk;
  int t, r0, span_len, ring_len, blk, ns, write_row, nbad;
  uint32_t bits_old;
  int go, full, new_row, own_now, wdone, seal;
};

template <int D, int BS>
struct AppendShared {
  AppendPending pend;
  uint8_t vimg[BS * D];          // value codes of the tail block (re-encoded spans), words swizzled
  uint4 tw[kTailWords];          // the state words (window test and seal)
  int mom_a[BS];                 // fixed-point moments of the span's tokens (span-relative index)
  long long mom_b[BS];
};

template <int D, int BS>
__device__ __forceinline__ AppendShared<D, BS> &append_shared() {
  __shared__ __align__(16) AppendShared<D, BS> sm;
  return sm;
}

// Word W of a value tile sits at LDS word vimg_word(W): the low three bits of W are XORed with
// the channel-tile bits above them, so the bytes that one pass of units writes (16 channels of 4
// tokens) fall into different banks.  A bijection within each group of 8 words.
template <int BS>
__device__ __forceinline__ int vimg_word(int W) {
  if constexpr (BS == 64) return W ^ ((W >> 6) & 7);
  else return W ^ ((W >> 4) & 7);
}
template <int D, int BS>
__device__ __forceinline__ int vimg_byte(int tau, int d) {
  const int off = v_tile_offset<D, BS>(tau, d);
  return (vimg_word<BS>(off >> 4) << 4) | (off & 15);
}
// The token (of its block) whose code is byte e of value-tile word W.
template <int D, int BS>
__device__ __forceinline__ int vword_token(int W, int e) {
  if constexpr (BS == 64) return 16 * (e >> 2) + 4 * ((W >> 4) & 3) + (e & 3);
  else if constexpr (BS == 32) return 16 * (W / D) + e;
  else return e;
}

// Codes of up to four values packed into the bytes of one word (byte e = value e), the same steps
// as dgq_encode_value: the difference and the product in float32, the clamp to [0, levels], then
// the packing conversion, which rounds to nearest even (and clamps to [0, 255]); a NaN gives 0, as
// there.  code_bytes then adds the code of the minimum to every byte, modulo 256, without carries.
template <int N>
__device__ __forceinline__ uint32_t encode_packed(const float (&x)[N], float mn, float inv, float levels) {
#pragma clang fp contract(off)
  static_assert(N >= 1 && N <= 4, "one word");
  uint32_t w = 0u;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float dlt = x[e] - mn;
    const float u = fminf(fmaxf(dlt * inv, 0.0f), levels);
    w = __builtin_amdgcn_cvt_pk_u8_f32(u, (uint32_t)e, w);
  }
  return w;
}
__device__ __forceinline__ uint32_t code_bytes(uint32_t w, int low) {
  const uint32_t c = ((uint32_t)low & 0xFFu) * 0x01010101u;
  return ((w & 0x7F7F7F7Fu) + (c & 0x7F7F7F7Fu)) ^ ((w ^ c) & 0x80808080u);
}

// What append_begin hands to the later parts (uniform across the workgroup, except the staged
// units, the old value words and the bitmap byte, which stay with the thread that loaded them).
template <int D, int BS>
struct AppendStage {
  static constexpr int CPU = D / 8;                   // 16-byte units per token
  static constexpr int UPT = (BS * CPU + 255) / 256;  // units per thread, at most
  static constexpr int VWORDS = BS * D / 16;          // 16-byte words of a value tile
  static constexpr int VW = (VWORDS + 255) / 256;     // value-tile words per thread, at most
  uint4 kw[UPT], vw[UPT];   // staged unit tid + 256 i: 8 channels of span token u / CPU
  uint4 vold[VW];           // value-tile word tid + 256 k as it was (only after frozen tokens)
  uint32_t bits_old;        // thread 0: the bitmap byte holding r0's bit
  float4 rk;                // the span's K min, K max, V min, V max with the new token
  dgq_seg_t R;              // row ns - 1 before the append
  int t, r0, slot0, span_len, nunits, blk, ns, ring_len, nbad;
  bool go;                  // false: the state did not fit, nothing was appended
  bool window_test, seal;
};

template <int D, int BS>
__device__ __forceinline__ void append_begin(const AppendArgs &a, int b, int h, AppendOut &out, AppendDecision &dec,
                                             const AppendLoads &ld, AppendStage<D, BS> &st) {
  constexpr int CPU = AppendStage<D, BS>::CPU;
  const int tid = threadIdx.x, lane = tid & 63;
  const size_t bh = (size_t)b * a.hkv + h;
  const int t = ld.t;
  auto lane_i = [](uint32_t v, int l) { return __builtin_amdgcn_readlane((int)v, l); };
  auto lane_f = [](uint32_t v, int l) { return __int_as_float(__builtin_amdgcn_readlane((int)v, l)); };
  // the state: words 0 and 13 of the append state, from the lanes that loaded them
  const int r0 = lane_i(ld.tail.x, 0), ring_len = lane_i(ld.tail.y, 0);
  const bool own = lane_i(ld.tail.z, 0) != 0;
  const bool wdone = lane_i(ld.tail.w, 0) != 0;
  const float4 srange = make_float4(lane_f(ld.tail.x, 13), lane_f(ld.tail.y, 13), lane_f(ld.tail.z, 13), lane_f(ld.tail.w, 13));
  const int ns = __builtin_amdgcn_readfirstlane(ld.nseg);
  const int blk_raw = __builtin_amdgcn_readfirstlane(ld.blk);
  const int slot0 = r0 < 0 ? 0 : r0 % BS;
  const int span_len = t + 1 - r0;             // including the new token
  // the state must place the new token inside the open span's block, and the block must exist
  // (r0 <= t and slot0 + span_len <= BS put r0 and t in the same block)
  bool bad = !ld.t_ok || r0 < 0 || r0 > t || slot0 + span_len > BS || ns < 0 || ns > a.seg_cap ||
             (own && ns < 1) || ring_len < 0 || ring_len > kWin;
  const int blk_t = checked_block(blk_raw, a.cache.num_blocks, bad);
  const bool go = !bad;
  st.go = go;
  out.ok = go ? 1 : 0;
  out.ns = ns;
  out.use_row = -1;

  // 1. the new token's ranges over all its channels (every wave), and the 64-channel groups that
  // hold a non-finite value
  float4 r = make_float4(INFINITY, -INFINITY, INFINITY, -INFINITY);
  float badv = 0.f;
  if (lane < D / 2) {
    const float k0 = half_bits_to_float(ld.kp & 0xFFFFu), k1 = half_bits_to_float(ld.kp >> 16);
    const float v0 = half_bits_to_float(ld.vp & 0xFFFFu), v1 = half_bits_to_float(ld.vp >> 16);
    r.x = fminf(fminf(r.x, k0), k1);
    r.y = fmaxf(fmaxf(r.y, k0), k1);
    r.z = fminf(fminf(r.z, v0), v1);
    r.w = fmaxf(fmaxf(r.w, v0), v1);
    badv = fmaf(k0, 0.f, badv);
    badv = fmaf(k1, 0.f, badv);
    badv = fmaf(v0, 0.f, badv);
    badv = fmaf(v1, 0.f, badv);
  }
  r = span_wave_minmax(r);
  const unsigned long long badm = __ballot(!(badv == 0.f));
  st.nbad = ((badm & 0xFFFFFFFFull) != 0ull ? 1 : 0) + ((badm >> 32) != 0ull ? 1 : 0);

  // 2. the span's ranges: the stored range of the earlier span tokens, widened by the new token
  if (span_len > 1) {
    r.x = fminf(r.x, srange.x);
    r.y = fmaxf(r.y, srange.y);
    r.z = fminf(r.z, srange.z);
    r.w = fmaxf(r.w, srange.w);
  }
  // (every lane holds the same ranges; taking them from the first lane tells the compiler so, and
  // keeps the decision and the row count that the decode loops on in scalar registers)
  auto uni = [](float x) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x))); };
  const float4 rk = make_float4(uni(r.x + 0.0f), uni(r.y + 0.0f), uni(r.z + 0.0f), uni(r.w + 0.0f));

  // 3. row ns - 1, the one row the decision can need (its own row, or the row the span would
  // join), from the lane that loaded it; then the decision, unless the window test is due (once
  // the span has 16 tokens and until it has said "no change": window and ring stay fixed for the
  // span).  The span's codes are rewritten when it gets its own row or its own row widens; a
  // full block seals.
  const int rr = ns >= 1 && ns <= a.seg_cap ? ns - 1 : 0;
  dgq_seg_t R;
  R.start = lane_i(ld.seg[0].x, rr);
  R.kmin = lane_f(ld.seg[0].y, rr);
  R.kmax = lane_f(ld.seg[0].z, rr);
  R.vmin = lane_f(ld.seg[0].w, rr);
  R.vmax = lane_f(ld.seg[1].x, rr);
  R.kscale = lane_f(ld.seg[1].y, rr);
  R.vscale = lane_f(ld.seg[1].z, rr);
  R.reserved = lane_i(ld.seg[1].w, rr);
  bool may_reenc;
  if (own) may_reenc = (R.kmin != rk.x) | (R.kmax != rk.y) | (R.vmin != rk.z) | (R.vmax != rk.w);
  else may_reenc = (ns < 1) | (rk.x < R.kmin) | (rk.y > R.kmax) | (rk.z < R.vmin) | (rk.w > R.vmax);
  const bool window_test = go && !own && !may_reenc && span_len >= kWin && ring_len == kWin && !wdone;
  const bool seal = go && (t + 1) % BS == 0;
  const bool staged = go && (may_reenc || window_test || seal);
  dec = append_decide(own || may_reenc, own, ns, a.seg_cap, r0, R, rk, a.fmt.levels);
  dec.wdone = wdone;
  if (go) {
    out.ns = dec.ns;
    out.use_row = dec.use_row;
    out.chosen = dec.chosen;
  }

  // 4. buffer loads of the earlier span tokens (the new one comes from its channel pairs),
  // every one issued: a unit that is not needed gets an offset past the resource (zero, no memory
  // access), so no branch separates these loads from the caller's next ones
  const int nunits = span_len * CPU;
  const uint16_t *ks = a.cache.k_stage + bh * (size_t)BS * D;
  const uint16_t *vs = a.cache.v_stage + bh * (size_t)BS * D;
  const __amdgpu_buffer_rsrc_t rks = raw_rsrc(ks, BS * D * 2), rvs = raw_rsrc(vs, BS * D * 2);
#pragma unroll
  for (int i = 0; i < AppendStage<D, BS>::UPT; ++i) {
    const int u = tid + 256 * i;
    const uint32_t off = staged && u < nunits - CPU ? (uint32_t)(((slot0 + u / CPU) * D + 8 * (u % CPU)) * 2) : kOutOfRange;
    st.kw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rks, off, 0, 0));
    st.vw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rvs, off, 0, 0));
  }
  // the value-tile words as they are, where frozen tokens of the block precede the span (they
  // keep their bytes when a re-encoded span's words are written)
  const int8_t *vt = a.cache.v_pool + ((size_t)blk_t * a.hkv + h) * (size_t)BS * D;
  const __amdgpu_buffer_rsrc_t rvt = raw_rsrc(vt, BS * D);
#pragma unroll
  for (int k = 0; k < AppendStage<D, BS>::VW; ++k) {
    const int W = tid + 256 * k;
    const uint32_t off = staged && slot0 > 0 && W < AppendStage<D, BS>::VWORDS ? (uint32_t)W * 16u : kOutOfRange;
    st.vold[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rvt, off, 0, 0));
  }
  // the bitmap byte holding r0's bit, for a new row (thread 0)
  const bool want_bits = tid == 0 && go && !own && r0 > 0 && !a.fmt.marker && (may_reenc || window_test);
  const uint8_t *bits_blk = a.fmt.marker ? nullptr : a.cache.bits + ((size_t)blk_t * a.hkv + h) * (BS / 8);
  st.bits_old = __builtin_amdgcn_raw_buffer_load_b8(raw_rsrc(bits_blk, BS / 8), want_bits ? (uint32_t)((r0 % BS) / 8) : kOutOfRange,
                                                     0, 0);
  st.rk = rk;
  st.R = R;
  st.t = t;
  st.r0 = r0;
  st.slot0 = slot0;
  st.span_len = span_len;
  st.nunits = nunits;
  st.blk = blk_t;
  st.ns = ns;
  st.ring_len = ring_len;
  st.window_test = window_test;
  st.seal = seal;
}

// The row the span is encoded with, and where its codes go.
template <int D, int BS>
struct AppendCoder {
  dgq_seg_t row;
  float kinv, vinv, lv;
  int low;
  bool mark;   // marker format: the span's own segment starts at r0, whose first key byte is the marker
  int8_t *kt, *vt;
  __device__ __forceinline__ AppendCoder(const AppendArgs &a, int h, const AppendDecision &dec, const AppendStage<D, BS> &st)
      : row(dec.chosen), lv(a.fmt.levels), low(a.fmt.low) {
    kinv = dgq_inv(row.kmin, row.kmax, lv);
    vinv = dgq_inv(row.vmin, row.vmax, lv);
    mark = a.fmt.marker && dec.own_now && st.r0 > 0;
    kt = a.cache.k_pool + ((size_t)st.blk * a.hkv + h) * (size_t)BS * D;
    vt = a.cache.v_pool + ((size_t)st.blk * a.hkv + h) * (size_t)BS * D;
  }
};

// The new token's codes and staging copy, by one wave (lane l < D/2: channels 2l and 2l + 1); its
// value codes go into the value image when the whole span is re-encoded.
template <int D, int BS>
__device__ __forceinline__ void append_new_token(const AppendArgs &a, int b, int h, const AppendDecision &dec,
                                                 const AppendLoads &ld, const AppendStage<D, BS> &st) {
  const int lane = threadIdx.x & 63;
  if (lane >= D / 2) return;
  const size_t bh = (size_t)b * a.hkv + h;
  const int slot = st.t % BS;
  const AppendCoder<D, BS> cd(a, h, dec, st);
  *reinterpret_cast<uint32_t *>(a.cache.k_stage + (bh * BS + slot) * D + 2 * lane) = ld.kp;
  *reinterpret_cast<uint32_t *>(a.cache.v_stage + (bh * BS + slot) * D + 2 * lane) = ld.vp;
  const float kx[2] = {half_bits_to_float(ld.kp & 0xFFFFu), half_bits_to_float(ld.kp >> 16)};
  const float vx[2] = {half_bits_to_float(ld.vp & 0xFFFFu), half_bits_to_float(ld.vp >> 16)};
  uint32_t kc = code_bytes(encode_packed(kx, cd.row.kmin, cd.kinv, cd.lv), cd.low);
  if (cd.mark && slot == st.slot0 && lane == 0) kc = (kc & ~0xFFu) | dgq_marker_byte(kc & 0xFFu);
  *reinterpret_cast<uint16_t *>(cd.kt + k_tile_offset<D, BS>(slot, 2 * lane)) = (uint16_t)kc;
  const uint32_t vc = code_bytes(encode_packed(vx, cd.row.vmin, cd.vinv, cd.lv), cd.low);
  if (dec.all) {
    AppendShared<D, BS> &sm = append_shared<D, BS>();
    sm.vimg[vimg_byte<D, BS>(slot, 2 * lane)] = (uint8_t)vc;
    sm.vimg[vimg_byte<D, BS>(slot, 2 * lane + 1)] = (uint8_t)(vc >> 8);
  } else {
    cd.vt[v_tile_offset<D, BS>(slot, 2 * lane)] = (int8_t)vc;
    cd.vt[v_tile_offset<D, BS>(slot, 2 * lane + 1)] = (int8_t)(vc >> 8);
  }
}

// Whether the step needs the whole workgroup (the window test, a seal or a re-encoded span); the
// other steps write only the new token's codes, which one wave does without a barrier.
template <int D, int BS>
__device__ __forceinline__ bool append_needs_span(const AppendDecision &dec, const AppendStage<D, BS> &st) {
  return st.go && (dec.all || st.window_test || st.seal);
}

// The whole-workgroup part of a step: the window test and the ring moments, the span's encode and
// the new token's codes, then a barrier, which orders the code stores before any later load of
// the tail block by the same workgroup (workgroup scope: one compute unit, in-order vector memory).
template <int D, int BS>
__device__ __forceinline__ void append_span(const AppendArgs &a, int b, int h, AppendOut &out, AppendDecision &dec,
                                            const AppendLoads &ld, const AppendStage<D, BS> &st) {
  constexpr int CPU = AppendStage<D, BS>::CPU;
  constexpr int UPT = AppendStage<D, BS>::UPT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  AppendShared<D, BS> &sm = append_shared<D, BS>();
  const int t = st.t, r0 = st.r0, slot0 = st.slot0, span_len = st.span_len;
  const int slot = t % BS;
  const int nold = st.nunits - CPU;   // staged units (the span tokens before the new one)
  const float k0 = half_bits_to_float(ld.kp & 0xFFFFu), k1 = half_bits_to_float(ld.kp >> 16);

  // 1. window test and seal: the fixed-point moments of the span's tokens (the CPU units of a
  // token sit in CPU consecutive lanes of one pass; the new token's from wave 0's channel pairs)
  if (st.window_test || st.seal) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 256 * i;
      const uint32_t kh[4] = {st.kw[i].x, st.kw[i].y, st.kw[i].z, st.kw[i].w};
      int as = 0;
      long long bs2 = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int n = dgq_fixed_point(half_bits_to_float(e & 1 ? kh[e >> 1] >> 16 : kh[e >> 1] & 0xFFFFu));
        as += n;
        bs2 += (long long)(n * n);
      }
#pragma unroll
      for (int o = 1; o < CPU; o <<= 1) {
        as += __shfl_xor(as, o);
        bs2 += __shfl_xor(bs2, o);
      }
      if (u < nold && u % CPU == 0) {
        sm.mom_a[u / CPU] = as;
        sm.mom_b[u / CPU] = bs2;
      }
    }
    if (wave == 0) {
      int as = 0;
      long long bs2 = 0;
      if (lane < D / 2) {
        const int n0 = dgq_fixed_point(k0), n1 = dgq_fixed_point(k1);
        as = n0 + n1;
        bs2 = (long long)(n0 * n0) + (long long)(n1 * n1);
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        as += __shfl_xor(as, o);
        bs2 += __shfl_xor(bs2, o);
      }
      if (lane == 0) {
        sm.mom_a[span_len - 1] = as;
        sm.mom_b[span_len - 1] = bs2;
      }
      if (lane < kTailWords) sm.tw[lane] = ld.tail;
    }
    __syncthreads();
    if (st.window_test) {
      // every lane sums the ring and the span's first 16 tokens over lanes (l & 15) of its row,
      // so every lane holds the same totals
      const dgq_tail_t &tl = *reinterpret_cast<const dgq_tail_t *>(sm.tw);
      const int i = lane & 15;
      long long la = tl.ring_a[i], lb = tl.ring_b[i], ra = sm.mom_a[i], rb = sm.mom_b[i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        la += __shfl_xor(la, o);
        lb += __shfl_xor(lb, o);
        ra += __shfl_xor(ra, o);
        rb += __shfl_xor(rb, o);
      }
      const long long nel = (long long)kWin * D;
      const long long ql = nel * lb - la * la, qr = nel * rb - ra * ra;
      const long long hi = ql > qr ? ql : qr, lo = ql > qr ? qr : ql;
      const bool want = __builtin_amdgcn_readfirstlane(
                            (!((double)hi < a.qfloor) && (double)(hi + 1) / (double)(lo + 1) >= a.tau) ? 1 : 0) != 0;
      dec = append_decide(want, false, st.ns, a.seg_cap, r0, st.R, st.rk, a.fmt.levels);
      dec.wdone = !want;
      out.ns = dec.ns;
      out.use_row = dec.use_row;
      out.chosen = dec.chosen;
    }
  }

  // 2. encode with the chosen row: the whole span when that range changed (a new row, or the
  // span's own row widened), else only the new token (every other span code is unchanged); the
  // new token by the last wave, which has the fewest span units (units go to threads in order)
  if (wave == kNewTokenWave) append_new_token<D, BS>(a, b, h, dec, ld, st);
  if (dec.all) {
    const AppendCoder<D, BS> cd(a, h, dec, st);
    const dgq_seg_t &row = cd.row;
    const float kinv = cd.kinv, vinv = cd.vinv, lv = cd.lv;
    const int low = cd.low;
    const bool mark = cd.mark;
    int8_t *kt = cd.kt, *vt = cd.vt;
    // the earlier span tokens, from the staged units: 8 key codes stored as 8 contiguous bytes of
    // the tile, 8 value codes into the image
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 256 * i;
      if (u < nold) {
        const int s = slot0 + u / CPU, d0 = 8 * (u % CPU);
        const uint32_t kh[4] = {st.kw[i].x, st.kw[i].y, st.kw[i].z, st.kw[i].w};
        const uint32_t vh[4] = {st.vw[i].x, st.vw[i].y, st.vw[i].z, st.vw[i].w};
        uint32_t kc[2], vc[2];
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
          const float kx[4] = {half_bits_to_float(kh[2 * hw] & 0xFFFFu), half_bits_to_float(kh[2 * hw] >> 16),
                               half_bits_to_float(kh[2 * hw + 1] & 0xFFFFu), half_bits_to_float(kh[2 * hw + 1] >> 16)};
          const float vx[4] = {half_bits_to_float(vh[2 * hw] & 0xFFFFu), half_bits_to_float(vh[2 * hw] >> 16),
                               half_bits_to_float(vh[2 * hw + 1] & 0xFFFFu), half_bits_to_float(vh[2 * hw + 1] >> 16)};
          kc[hw] = code_bytes(encode_packed(kx, row.kmin, kinv, lv), low);
          vc[hw] = code_bytes(encode_packed(vx, row.vmin, vinv, lv), low);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.vimg[vimg_byte<D, BS>(s, d0 + e)] = (uint8_t)(vc[e >> 2] >> (8 * (e & 3)));
        if (mark && s == slot0 && d0 == 0) kc[0] = (kc[0] & ~0xFFu) | dgq_marker_byte(kc[0] & 0xFFu);
        *reinterpret_cast<uint2 *>(kt + k_tile_offset<D, BS>(s, d0)) = make_uint2(kc[0], kc[1]);
      }
    }
    __syncthreads();
    // the value-tile words that hold a span token, whole from the image: bytes of frozen tokens
    // (before the span) from the word as it was, bytes of tokens after the new one are never read
    // before their own append writes them
#pragma unroll
    for (int k = 0; k < AppendStage<D, BS>::VW; ++k) {
      const int W = tid + 256 * k;
      if (W < AppendStage<D, BS>::VWORDS && slot0 == 0) {
        // the span starts the block: a word holds a span token iff its first byte's token does
        if (vword_token<D, BS>(W, 0) <= slot)
          *reinterpret_cast<uint4 *>(vt + W * 16) = *reinterpret_cast<const uint4 *>(&sm.vimg[vimg_word<BS>(W) << 4]);
      } else if (W < AppendStage<D, BS>::VWORDS) {
        uint32_t span_m = 0u, frozen_m = 0u;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tau = vword_token<D, BS>(W, e);
          span_m |= (uint32_t)(tau >= slot0 && tau <= slot) << e;
          frozen_m |= (uint32_t)(tau < slot0) << e;
        }
        if (span_m != 0u) {
          uint4 w = *reinterpret_cast<const uint4 *>(&sm.vimg[vimg_word<BS>(W) << 4]);
          if (frozen_m != 0u) {
            uint32_t wv[4] = {w.x, w.y, w.z, w.w};
            const uint32_t ov[4] = {st.vold[k].x, st.vold[k].y, st.vold[k].z, st.vold[k].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint32_t m = 0u;
#pragma unroll
              for (int e = 0; e < 4; ++e) m |= ((frozen_m >> (4 * q + e)) & 1u) * (0xFFu << (8 * e));
              wv[q] = (wv[q] & ~m) | (ov[q] & m);
            }
            w = make_uint4(wv[0], wv[1], wv[2], wv[3]);
          }
          *reinterpret_cast<uint4 *>(vt + W * 16) = w;
        }
      }
    }
  }

  __syncthreads();
}

// The decision as the state stores need it, into LDS (thread 0).
template <int D, int BS>
__device__ __forceinline__ void append_stash(const AppendDecision &dec, const AppendStage<D, BS> &st) {
  if (threadIdx.x != 0) return;
  AppendPending &pd = append_shared<D, BS>().pend;
  pd.chosen = dec.chosen;
  pd.rk = st.rk;
  pd.t = st.t;
  pd.r0 = st.r0;
  pd.span_len = st.span_len;
  pd.ring_len = st.ring_len;
  pd.blk = st.blk;
  pd.ns = dec.ns;
  pd.write_row = dec.write_row;
  pd.nbad = st.nbad;
  pd.bits_old = st.bits_old;
  pd.go = st.go;
  pd.full = dec.full;
  pd.new_row = dec.new_row;
  pd.own_now = dec.own_now;
  pd.wdone = dec.wdone;
  pd.seal = st.seal;
}

// The state an append leaves (by wave 0, from what append_stash kept; every wave must have read
// the state first): the status counts, the segment row, the bitmap byte, the row count
// (publish_nseg) and the append state.
template <int D, int BS>
__device__ __forceinline__ void append_store_state(const AppendArgs &a, int b, int h, bool publish_nseg) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) != 0) return;
  AppendShared<D, BS> &sm = append_shared<D, BS>();
  const AppendPending &pd = sm.pend;
  if (!pd.go) return;
  const size_t bh = (size_t)b * a.hkv + h;
  const int t = pd.t, r0 = pd.r0, span_len = pd.span_len, ring_len = pd.ring_len;
  if (lane == 0) {
    if (pd.nbad > 0) atomicAdd(a.cache.status + 1, (unsigned long long)pd.nbad);
    if (pd.full) atomicAdd(a.cache.status + 0, 1ull);   // the table is full: the span joins the row before it
    if (pd.new_row && r0 > 0 && !a.fmt.marker)
      a.cache.bits[((size_t)pd.blk * a.hkv + h) * (BS / 8) + (r0 % BS) / 8] =
          (uint8_t)((pd.bits_old & 0xFFu) | (1u << (r0 % 8)));
    if (publish_nseg) a.cache.nseg[bh] = pd.ns;
  }
  if (pd.write_row >= 0) {
    const dgq_seg_t &c = pd.chosen;
    uint4 *dst = reinterpret_cast<uint4 *>(a.cache.segs + bh * a.seg_cap + pd.write_row);
    if (lane == 0) dst[0] = make_uint4((uint32_t)c.start, __float_as_uint(c.kmin), __float_as_uint(c.kmax), __float_as_uint(c.vmin));
    if (lane == 1) dst[1] = make_uint4(__float_as_uint(c.vmax), __float_as_uint(c.kscale), __float_as_uint(c.vscale), (uint32_t)c.reserved);
  }
  // the state: seal a full block (the ring keeps the moments of the last 16 sealed tokens), or
  // keep the span's ranges
  dgq_tail_t *tp = a.cache.tail + bh;
  if (pd.seal) {
    // new ring = last 16 of (old ring, span tokens): lane i < 16 writes element i
    const dgq_tail_t &tl = *reinterpret_cast<const dgq_tail_t *>(sm.tw);
    const int m_tail = span_len < kWin ? span_len : kWin;   // span tokens that enter the ring
    const int old_keep = m_tail < kWin ? (ring_len < kWin - m_tail ? ring_len : kWin - m_tail) : 0;
    const int n = old_keep + m_tail;
    if (lane < kWin) {
      int32_t ea = 0;
      long long eb = 0;
      if (lane < old_keep) {
        ea = tl.ring_a[ring_len - old_keep + lane];
        eb = tl.ring_b[ring_len - old_keep + lane];
      } else if (lane < n) {
        ea = sm.mom_a[span_len - m_tail + (lane - old_keep)];
        eb = sm.mom_b[span_len - m_tail + (lane - old_keep)];
      }
      tp->ring_a[lane] = ea;
      tp->ring_b[lane] = eb;
    }
    if (lane == 0) *reinterpret_cast<int4 *>(tp) = make_int4(t + 1, n, 0, 0);
  } else {
    if (lane == 0) *reinterpret_cast<int4 *>(tp) = make_int4(r0, ring_len, pd.own_now, pd.wdone);
    if (lane == 13) *reinterpret_cast<float4 *>(tp->span_range) = pd.rk;
  }
}

// The append kernel's form: the loads, then the append.
template <int D, int BS>
__device__ __forceinline__ void append_one(const AppendArgs &a, int b, int h, bool publish_nseg, AppendOut &out) {
  const int t = a.seq_lens[b];
  AppendLoads l = append_loads_state<D>(a, b, h);
  append_load_block<BS>(a, b, t, l);
  AppendStage<D, BS> st;
  AppendDecision dec;
  append_begin<D, BS>(a, b, h, out, dec, l, st);
  if (append_needs_span(dec, st)) append_span<D, BS>(a, b, h, out, dec, l, st);
  else if (st.go && (threadIdx.x >> 6) == kNewTokenWave) append_new_token<D, BS>(a, b, h, dec, l, st);
  append_stash<D, BS>(dec, st);
  __syncthreads();   // every wave has read the state
  append_store_state<D, BS>(a, b, h, publish_nseg);
  if (threadIdx.x == 0 && !out.ok) atomicAdd(a.cache.status + 2, 1ull);   // the state did not fit
}

AppendArgs make_append_args(const dgq_params_t *p, const uint16_t *k_tok, const uint16_t *v_tok,
                            const int32_t *seq_lens, const int32_t *block_table, int32_t max_blocks,
                            const dgq_cache_t *cache);

}  // namespace dgq
