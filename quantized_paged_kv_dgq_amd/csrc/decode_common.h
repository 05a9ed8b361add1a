// Shared pieces of the paged decode kernels (DGQ segments and the fixed 64-channel group
// baseline): byte-column operands of the int8 matrix cores, DPP quad sums, the argument block and
// the split-sequence merge.
#pragma once

#include <climits>
#include <cmath>

#include "dgq_internal.h"

namespace dgq {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;   // waves per decode workgroup

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
  float *part_ml;   // [batch][hq][nparts][2]
  float *part_o;    // [batch][hq][nparts][D]
  float *out;       // [batch][hq][D]
  unsigned long long *status;
  int32_t hkv, hq, max_blocks, seg_cap, part_tokens, nparts, max_seq_len, num_blocks;
  float sm_log2;    // softmax_scale * log2(e)
};

// x from the lane whose index differs in bit 0 (XOR1) or bit 1 (XOR2), within quads (DPP).
__device__ __forceinline__ float quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
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
                            void *ws);

// Merge the kWaves per-wave results of a workgroup (already in sh_o / sh_m / sh_l) into one
// partial; with one workgroup per (sequence, kv head) write the output directly, otherwise publish
// the partial and let the last workgroup of (b, h) merge all partials by log-sum-exp.
template <int D, int G>
__device__ __forceinline__ void finish_partition(const DecodeArgs &a, int b, int h, int p, int L,
                                                 float (&sh_o)[kWaves][G][D], float (&sh_m)[kWaves][G],
                                                 float (&sh_l)[kWaves][G]) {
  __syncthreads();
  const int P = (L + a.part_tokens * kWaves - 1) / (a.part_tokens * kWaves);   // workgroups of (b, h)
  for (int e = threadIdx.x; e < G * D; e += 64 * kWaves) {
    const int gg = e / D, d = e % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sh_m[w][gg]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = __builtin_amdgcn_exp2f(sh_m[w][gg] - mx);
      o = fmaf(sc, sh_o[w][gg][d], o);
      l = fmaf(sc, sh_l[w][gg], l);
    }
    const size_t row = (size_t)b * a.hq + h * G + gg;
    if (P == 1) {
      a.out[row * D + d] = o / l;                    // the only workgroup of (b, h)
    } else {
      // device-scope stores: written through to the level all XCDs see
      const size_t prow = row * a.nparts + p;
      __hip_atomic_store(a.part_o + prow * D + d, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) {
        __hip_atomic_store(a.part_ml + prow * 2 + 0, mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.part_ml + prow * 2 + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (P == 1) return;

  // ---- the last workgroup of (b, h) to finish merges all partials by log-sum-exp ----
  // Publish: wait until this workgroup's device-scope stores have completed, then count it.
  // (A device-scope fence would also write back the whole L2, which is not needed here: the
  // partials themselves were stored at device scope and are read back at device scope.)
  __shared__ int sh_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.counters + (size_t)b * a.hkv + h, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sh_last = prev == (unsigned)(P - 1);
  }
  __syncthreads();
  if (!sh_last) return;

  // Merge: weights 2^(m_p - M) per (head, partition) in LDS, then independent loads of the
  // partial outputs.  A partial must not be read from a stale cached copy of an earlier call:
  // with many partials the merging workgroup drops this XCD's cached lines once (device-scope
  // acquire) and reads float4s through the caches; with few it reads each value at device scope
  // and leaves the caches alone.  Partitions are taken in tiles of TP so that one thread holds
  // one (head, partition) pair per tile.
  const bool via_cache = P >= 16;
  if (via_cache) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  constexpr int NTH = 64 * kWaves;
  constexpr int TP = NTH / G;                        // partitions per tile
  constexpr int NQ = D / 4;                          // float4 columns of a head's output
  constexpr int SPLIT = NTH / (G * NQ);              // threads per output column
  __shared__ float sh_pm[NTH], sh_pw[NTH], sh_scale[G], sh_M[G], sh_den[G];
  __shared__ float4 sh_part[NTH];
  const int tid = threadIdx.x;
  if (tid < G) {
    sh_M[tid] = -INFINITY;
    sh_den[tid] = 0.f;
  }
  const int ocol = tid % (G * NQ), part = tid / (G * NQ);
  const int cg = ocol / NQ, cq = ocol % NQ;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = 0; p0 < P; p0 += TP) {
    const int np = min(TP, P - p0);
    const int tg = tid / TP, tp = tid % TP;
    float mv = -INFINITY, lv = 0.f;
    if (tp < np) {
      float *ml2 = a.part_ml + (((size_t)b * a.hq + h * G + tg) * a.nparts + p0 + tp) * 2;
      if (via_cache) {
        const float2 v2 = *reinterpret_cast<const float2 *>(ml2);
        mv = v2.x;
        lv = v2.y;
      } else {
        mv = __hip_atomic_load(ml2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lv = __hip_atomic_load(ml2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    sh_pm[tid] = mv;
    __syncthreads();
    if (tid < G) {   // new running maximum of head tid over this tile
      float mt = sh_M[tid];
      for (int k = 0; k < np; ++k) mt = fmaxf(mt, sh_pm[tid * TP + k]);
      sh_scale[tid] = __builtin_amdgcn_exp2f(sh_M[tid] - mt);
      sh_M[tid] = mt;
    }
    __syncthreads();
    const float w = tp < np ? __builtin_amdgcn_exp2f(mv - sh_M[tg]) : 0.f;
    sh_pw[tid] = w;
    sh_pm[tid] = w * lv;
    __syncthreads();
    if (tid < G) {
      float dsum = 0.f;
      for (int k = 0; k < np; ++k) dsum += sh_pm[tid * TP + k];
      sh_den[tid] = sh_den[tid] * sh_scale[tid] + dsum;
    }
    // output columns: thread (column, part) sums partitions part, part + SPLIT, ...
    const float sc = sh_scale[cg];
    acc = make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
    float *po = a.part_o + (((size_t)b * a.hq + h * G + cg) * a.nparts + p0) * D + 4 * cq;
    if (via_cache) {
#pragma unroll 8
      for (int k = part; k < np; k += SPLIT) {
        const float wk = sh_pw[cg * TP + k];
        const float4 o4 = *reinterpret_cast<const float4 *>(po + (size_t)k * D);
        acc.x = fmaf(wk, o4.x, acc.x);
        acc.y = fmaf(wk, o4.y, acc.y);
        acc.z = fmaf(wk, o4.z, acc.z);
        acc.w = fmaf(wk, o4.w, acc.w);
      }
    } else {
#pragma unroll 4
      for (int k = part; k < np; k += SPLIT) {
        const float wk = sh_pw[cg * TP + k];
        float *src = po + (size_t)k * D;
        acc.x = fmaf(wk, __hip_atomic_load(src + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), acc.x);
        acc.y = fmaf(wk, __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), acc.y);
        acc.z = fmaf(wk, __hip_atomic_load(src + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), acc.z);
        acc.w = fmaf(wk, __hip_atomic_load(src + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), acc.w);
      }
    }
  }
  sh_part[tid] = acc;
  __syncthreads();
  if (tid < G * NQ) {
    float4 r = sh_part[tid];
    for (int k = 1; k < SPLIT; ++k) {
      const float4 x = sh_part[tid + k * G * NQ];
      r.x += x.x;
      r.y += x.y;
      r.z += x.z;
      r.w += x.w;
    }
    const float inv = 1.0f / sh_den[cg];
    reinterpret_cast<float4 *>(a.out + ((size_t)b * a.hq + h * G + cg) * D)[cq] =
        make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
  }
  if (tid == 0)   // ready for the next call
    __hip_atomic_store(a.counters + (size_t)b * a.hkv + h, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dgq
