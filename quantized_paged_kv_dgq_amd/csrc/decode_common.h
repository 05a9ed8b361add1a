// Shared pieces of the paged decode kernels (DGQ segments and the fixed 64-channel group
// baseline): byte-column operands of the int8 matrix cores, DPP quad sums, the argument block and
// the split-sequence merge.
#pragma once

#include <climits>
#include <cmath>

#include "dgq_internal.h"

namespace dgq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;   // waves per decode workgroup
constexpr int kMaxRun = 64; // 64-token chunks per wave at most (a workgroup spans <= 16384 tokens)

struct DecodeArgs {
  const uint16_t *q;
  const int8_t *k_pool;
  const int8_t *v_pool;
  const dgq_seg_t *segs;      // DGQ: segment table and row counts
  const int32_t *nseg;
  const uint32_t *k_range;    // group-64 baseline: fp16 (min, max) per (block, head, token, group)
  const uint32_t *v_range;
  const int32_t *block_table;
  const int32_t *seq_lens;
  unsigned *counters;  // [batch][hkv]: workgroups done; zero between calls
  int32_t *pend_nseg;  // [batch][hkv]: fused append + decode: row count to publish after the merge
  float *part_ml;   // [batch][hq][nparts][2]
  float *part_o;    // [batch][hq][nparts][D]
  float *out;       // [batch][hq][D]
  unsigned long long *status;
  int32_t hkv, hq, max_blocks, seg_cap, part_tokens, nparts, max_seq_len, num_blocks;
  float sm_log2;    // softmax_scale * log2(e)
  float code_mid;   // DGQ: -(code of a segment's minimum): 128, or 127 in the marker format
};

// x from the lane whose index differs in bit 0 (XOR1) or bit 1 (XOR2), within quads (DPP).
__device__ __forceinline__ float quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// Maximum of x over lanes l and l ^ 16, and over lanes l and l ^ 32.  The gfx950 permlane swaps
// exchange 16-lane rows (or 32-lane halves) of two registers in the VALU, with no LDS round trip;
// swapping a register with itself leaves {x[l], x[l ^ 16]} (or {x[l], x[l ^ 32]}) in the pair.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum of x over the whole wave with no LDS round trip: the quad exchanges, then the 8-lane and
// 16-lane mirrors of a row (DPP row_half_mirror, row_mirror) leave every lane of a row with the row's
// maximum; the two permlane swaps combine the four rows.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, quad_xor1(x));
  x = fmaxf(x, quad_xor2(x));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false)));
  return max_xor32(max_xor16(x));
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// A 16-byte load of codes, which one call reads exactly once: non-temporal, so the lines are not
// kept in the L2 or the Infinity Cache.  (Ordinary loads left the paged decode about 9 % slower:
// 57.3 against 52.5 us for 16 x 8192 tokens, 54.7 against 49.2 us for 131,072.)
__device__ __forceinline__ v4i load_codes(const int8_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
}

// Rounding to an integer by adding 1.5 * 2^23: for |v| <= 2^22 the float sum's bit pattern is
// 0x4B400000 + rint(v) (round to nearest even).
constexpr float kMagic = 12582912.0f;
constexpr int kMagicBits = 0x4B400000;

// A lane's byte of the balanced base-256 digits (d0, d1, d2) of an integer X, |X| <= 2^22,
// X = d0 * 65536 + d1 * 256 + d2 with d1, d2 in [-128, 127]: byte k = ((X + add_k) >> shift_k)
// & 0xFF with (add, shift) = (0x8080, 16), (0x80, 8), (0, 0).  Column byte 3 (and columns of
// absent heads) read width 0, i.e. always 0.
struct ByteSel {
  int add;          // add_k - kMagicBits: applied to the magic-rounded float's bit pattern
  unsigned shift;
  unsigned width;   // 8, or 0 for an unused column
};

__device__ __forceinline__ ByteSel byte_sel(int piece, bool live) {
  ByteSel s;
  s.add = (piece == 0 ? 0x8080 : piece == 1 ? 0x80 : 0) - kMagicBits;
  s.shift = piece < 3 ? 16u - 8u * (unsigned)piece : 0u;
  s.width = live ? 8u : 0u;
  return s;
}

// byte of rint(v) (v given as a float, |v| <= 2^22), rounding by fma(v, 1, magic)
__device__ __forceinline__ uint32_t sel_byte(float rounded_magic, const ByteSel &s) {
  return __builtin_amdgcn_ubfe((uint32_t)(__float_as_int(rounded_magic) + s.add), s.shift, s.width);
}

DecodeArgs make_decode_args(const dgq_params_t *p, const uint16_t *q, const int8_t *k_pool,
                            const int8_t *v_pool, int32_t num_blocks, unsigned long long *status,
                            const int32_t *block_table, int32_t max_blocks, const int32_t *seq_lens,
                            int32_t batch, int32_t max_seq_len, float softmax_scale, float *out,
                            void *ws, int64_t target_waves);

// Workgroups (partitions) of a sequence of L tokens with `span` tokens each: a partial 64-token
// chunk at the end joins the last partition instead of opening one of its own.
__host__ __device__ __forceinline__ int parts_of(int L, int span) {
  const int full = (L / kChunk) * kChunk;
  const int P = (full + span - 1) / span;
  return P > 1 ? P : 1;
}

// Token range [t_begin, t_end) of one wave: the workgroup's tokens [wg_begin, wg_end) (wg_end =
// wg_begin + span, or L for the last partition) are dealt to the kWaves waves as nearly equal runs
// of whole 64-token chunks, so a short sequence or a sequence's last partition still keeps every
// wave busy.
struct WaveRange {
  int t_begin, t_end;
};
__device__ __forceinline__ WaveRange wave_range(int wg_begin, int span, int L, int wave) {
  const int wg_end = wg_begin / span + 1 == parts_of(L, span) ? L : min(L, wg_begin + span);
  const int nch = (wg_end - wg_begin + kChunk - 1) / kChunk;
  const int c0 = wave * nch / kWaves, c1 = (wave + 1) * nch / kWaves;
  return {wg_begin + c0 * kChunk, min(wg_end, wg_begin + c1 * kChunk)};
}

// The block ids of a workgroup's span, kept in LDS: read from the table before the sequence
// length is known (NB per thread, coalesced), then published once it is: the sequence's blocks
// validated (a bad id is counted and replaced by 0), slots past its last block set to 0, a valid
// block that is only ever read for masked tokens of a partial last chunk.
template <int BS>
struct SpanBlocks {
  // a span of kWaves * kMaxRun chunks plus the partial chunk a last partition may absorb
  static constexpr int kBlocks = (kWaves * kMaxRun + 1) * kChunk / BS;
  static constexpr int NB = (kBlocks + 64 * kWaves - 1) / (64 * kWaves);
  int raw[NB];

  __device__ __forceinline__ void load(const int32_t *bt, int max_blocks, int wblk0) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int slot = (int)threadIdx.x + 64 * kWaves * i;
      raw[i] = slot < kBlocks && wblk0 + slot < max_blocks ? bt[wblk0 + slot] : 0;
    }
  }
  // (raw_slot >= 0: the unchecked id of that slot is also left in *sh_raw, for the append of a
  // fused decode, which checks it itself)
  __device__ __forceinline__ void publish(int wblk0, int nblk_seq, int num_blocks, int *sh_blk,
                                          unsigned long long *status, int raw_slot = -1,
                                          int *sh_raw = nullptr) const {
    bool bad = false;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int slot = (int)threadIdx.x + 64 * kWaves * i;
      if (slot < kBlocks) sh_blk[slot] = wblk0 + slot < nblk_seq ? checked_block(raw[i], num_blocks, bad) : 0;
      if (slot == raw_slot) *sh_raw = raw[i];
    }
    if (__ballot(bad) != 0ull && (threadIdx.x & 63) == 0) atomicAdd(status + 2, 1ull);
  }
};

// Cache policy of the partials: agent (device) scope, i.e. coherent across the XCDs' L2 caches,
// the same policy as relaxed device-scope atomic loads and stores.
constexpr int kAgentScope = 16;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Merge the kWaves per-wave results of a workgroup (already in sh_o / sh_m / sh_l) into one
// partial; with one workgroup per (sequence, kv head) write the output directly, otherwise publish
// the partial and let the last workgroup of (b, h) merge all partials by log-sum-exp.  A
// workgroup may also hand over one integer (pend >= 0) that the merging workgroup reads back.
// Returns kWroteOutput (single workgroup), kMerged (this workgroup merged) or kPartialOnly.
enum { kPartialOnly = 0, kWroteOutput = 1, kMerged = 2 };
template <int D, int G>
__device__ __forceinline__ int finish_partition(const DecodeArgs &a, int b, int h, int p, int L,
                                                float (&sh_o)[kWaves][G][D], float (&sh_m)[kWaves][G],
                                                float (&sh_l)[kWaves][G], int pend = -1) {
  constexpr int NTH = 64 * kWaves;
  constexpr int NQ = D / 4;                          // float4 columns of a head's output
  static_assert(G * NQ <= NTH, "one float4 column per thread");
  __syncthreads();
  const int tid = threadIdx.x;
  const int P = parts_of(L, a.part_tokens * kWaves);   // workgroups of (b, h)
  const size_t row0 = (size_t)b * a.hq + h * G;      // first query head row of this kv head
  if (tid < G * NQ) {
    const int gg = tid / NQ, d = 4 * (tid % NQ);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sh_m[w][gg]);
    v4f o = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = __builtin_amdgcn_exp2f(sh_m[w][gg] - mx);
      o.x = fmaf(sc, sh_o[w][gg][d + 0], o.x);
      o.y = fmaf(sc, sh_o[w][gg][d + 1], o.y);
      o.z = fmaf(sc, sh_o[w][gg][d + 2], o.z);
      o.w = fmaf(sc, sh_o[w][gg][d + 3], o.w);
      l = fmaf(sc, sh_l[w][gg], l);
    }
    if (P == 1) {                                    // the only workgroup of (b, h)
      const float inv = 1.0f / l;
      *reinterpret_cast<float4 *>(a.out + (row0 + gg) * D + d) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    } else {
      // partial p of head row0 + gg, stored at device scope (to the level all XCDs see); the
      // buffer resource covers the G heads of this kv head, so it is the same for every lane
      const int prow = gg * a.nparts + p;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, o), raw_rsrc(a.part_o + row0 * a.nparts * D, G * a.nparts * D * 4),
                                             (prow * D + d) * 4, 0, kAgentScope);
      if (d == 0) {
        const v2f ml = {mx, l};
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2i_t, ml), raw_rsrc(a.part_ml + row0 * a.nparts * 2, G * a.nparts * 8),
                                              prow * 8, 0, kAgentScope);
      }
    }
  }
  if (P == 1) return kWroteOutput;
  if (pend >= 0 && tid == 0)
    __hip_atomic_store(a.pend_nseg + (size_t)b * a.hkv + h, pend, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- the last workgroup of (b, h) to finish merges all partials by log-sum-exp ----
  // Publish: wait until this workgroup's device-scope stores have completed, then count it.
  __shared__ int sh_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.counters + (size_t)b * a.hkv + h, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sh_last = prev == (unsigned)(P - 1);
  }
  __syncthreads();
  if (!sh_last) return kPartialOnly;

  // Merge.  Thread (column, part) takes partitions part, part + SPLIT, ... of its head and
  // column; each round issues the (m, l) and output loads of KB partitions at once (device-scope
  // loads, so no stale cached copy of an earlier call is read), then folds them with a running
  // maximum.  The SPLIT threads of a column are combined in LDS at the end.
  constexpr int SPLIT = NTH / (G * NQ);
  constexpr int KB = 16;
  const int ocol = tid % (G * NQ), part = tid / (G * NQ);
  const int cg = ocol / NQ, d = 4 * (ocol % NQ);
  const int prow = cg * a.nparts;                    // this head's first partial in the resource
  const __amdgpu_buffer_rsrc_t r_o = raw_rsrc(a.part_o + row0 * a.nparts * D, G * a.nparts * D * 4);
  const __amdgpu_buffer_rsrc_t r_ml = raw_rsrc(a.part_ml + row0 * a.nparts * 2, G * a.nparts * 8);
  float mt = -INFINITY, den = 0.f;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = part; k0 < P; k0 += SPLIT * KB) {
    v2f ml[KB];
    v4f o[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int k = min(k0 + u * SPLIT, P - 1);
      ml[u] = __builtin_bit_cast(v2f, __builtin_amdgcn_raw_buffer_load_b64(r_ml, (prow + k) * 8, 0, kAgentScope));
      o[u] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r_o, ((prow + k) * D + d) * 4, 0, kAgentScope));
    }
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (k0 + u * SPLIT >= P) ml[u].x = -INFINITY;  // past the last partition: weight 0
      bm = fmaxf(bm, ml[u].x);
    }
    if (bm > mt) {                                   // bm is finite: partition k0 is real
      const float sc = __builtin_amdgcn_exp2f(mt - bm);
      acc *= sc;
      den *= sc;
      mt = bm;
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const float w = __builtin_amdgcn_exp2f(ml[u].x - mt);
      acc += w * o[u];
      den = fmaf(w, ml[u].y, den);
    }
  }
  __shared__ float4 sh_part[NTH];
  __shared__ float sh_pm[NTH], sh_pd[NTH];
  sh_part[tid] = make_float4(acc.x, acc.y, acc.z, acc.w);
  sh_pm[tid] = mt;
  sh_pd[tid] = den;
  __syncthreads();
  if (tid < G * NQ) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < SPLIT; ++k) M = fmaxf(M, sh_pm[tid + k * G * NQ]);
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    float dn = 0.f;
#pragma unroll
    for (int k = 0; k < SPLIT; ++k) {
      const int src = tid + k * G * NQ;
      const float sc = __builtin_amdgcn_exp2f(sh_pm[src] - M);   // 0 for a thread with no partitions
      const float4 x = sh_part[src];
      r.x = fmaf(sc, x.x, r.x);
      r.y = fmaf(sc, x.y, r.y);
      r.z = fmaf(sc, x.z, r.z);
      r.w = fmaf(sc, x.w, r.w);
      dn = fmaf(sc, sh_pd[src], dn);
    }
    const float inv = 1.0f / dn;
    *reinterpret_cast<float4 *>(a.out + (row0 + cg) * D + d) = make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
  }
  if (tid == 0)   // ready for the next call
    __hip_atomic_store(a.counters + (size_t)b * a.hkv + h, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return kMerged;
}

}  // namespace dgq
