// DGQ compression of a batch of sequences (DGQ article 2.2), in four passes on one stream:
//
//  1. stats   -- one read of fp16 K/V.  Per token: exact fixed-point key moments a_t = sum n,
//                b_t = sum n^2 (n = rint(clamp(x, -32, 32) * 512)); per 16-token sub-block:
//                K and V min/max.  Four lanes per token, 64 contiguous bytes per lane group.
//  2. scores  -- per candidate cut t in [16, L-16]: the 16-token window statistics
//                Q = N * sum b - (sum a)^2 left and right of t (integers, exact), and
//                score = (max + 1) / (min + 1) in float64; the best (score, t) of every
//                256-candidate tile.
//  3. select  -- one workgroup per (sequence, kv head): greedy cut selection from the tile
//                maxima (re-scanning only tiles next to a taken cut), then each segment's K/V
//                min/max from the sub-block extrema plus a raw re-read of the at most two
//                sub-blocks a cut splits; writes the segment table, nseg and the append state.
//  4. encode  -- second read of fp16 K/V; writes INT8 codes into the paged pool in the tile order
//                of the decode kernel (values through LDS, since their tiles are channel-major),
//                and the boundary bits.
//
// Sequences of at most 256 tokens (head_dim 128) or 512 (head_dim 64) take one launch instead,
// one workgroup per (sequence, kv head) doing all four steps on one read of the input.
#include <climits>
#include <type_traits>
#include <cmath>

#include "dgq_internal.h"

namespace dgq {

struct CompressArgs {
  const uint16_t *k;
  const uint16_t *v;
  int64_t stride_tok, stride_head;
  const int32_t *cu;
  const int32_t *block_table;
  int32_t max_blocks;
  int32_t hkv, batch, max_segments, seg_cap, nsub, ntile, max_seq_len;
  int64_t total;
  double tau;
  double qfloor;        // variance floor on the Q scale (0 = off)
  int32_t length_aware; // DGQ_POLICY_LENGTH_AWARE: per-sequence segment cap
  int32_t multipass;    // DGQ_COMPRESS_MULTIPASS: no one-launch path for short sequences
  CodeFormat fmt;
  // workspace
  int32_t *ws_a;        // [hkv][total]
  int64_t *ws_b;        // [hkv][total]
  double *ws_score;     // [hkv][total]
  float4 *ws_ext;       // [batch][hkv][nsub]: kmin, kmax, vmin, vmax
  double2 *ws_tile;     // [batch][hkv][ntile]: (score, t as double)
  float4 *ws_text;      // [batch][hkv][ntile]: K min, K max, V min, V max of each 256-token tile
  int4 *tile_map;       // ragged batches: [map_tiles] {sequence, tile, first token, length}; else null
  dgq_cache_t cache;
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// The encode pass is the last reader of the fp16 input: its 16-byte loads are non-temporal, so the
// lines it brings in are not kept (4-5 % off the compress at 16 x 8192 tokens).  The stats pass
// keeps ordinary loads: part of the encode pass's second read of the input is served from the
// caches they fill (non-temporal loads in both passes made the compress 5-6 % slower).
__device__ __forceinline__ uint4 load_last_use(const uint16_t *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Codes are not read again until a later decode: store them non-temporally so they go to HBM
// instead of settling as dirty lines in the Infinity Cache, whose write-back would otherwise be
// paid by whichever kernel runs next.
__device__ __forceinline__ void store_stream(int8_t *dst, const uint32_t (&w)[4]) {
  __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4 *>(dst));
}

// Workgroup order of the two passes over fp16 K/V (grid: chunks x kv heads x sequences): runs of
// kRun consecutive 64-token chunks for every kv head in turn, so that the workgroups in flight read
// whole token rows (all heads' 256-byte pieces of a 2 KB row) of a bounded token range instead of
// one head's pieces of the whole sequence.  A bijection of (chunk, head); a partial last run keeps
// the plain order.
constexpr int kRun = 32;
__device__ __forceinline__ void run_order(int &chunk, int &h) {
  const int tiles = gridDim.x, hkv = gridDim.y;
  const int id = blockIdx.x + tiles * blockIdx.y;
  const int full = tiles / kRun * kRun;
  if (id < full * hkv) {
    const int w = id % (kRun * hkv);
    h = w / kRun;
    chunk = id / (kRun * hkv) * kRun + w % kRun;
  } else {
    const int r = id - full * hkv, rem = tiles - full;
    h = r / rem;
    chunk = full + r % rem;
  }
}

// -------------------------------------------------------------------------------------------
// 0. tile map (ragged batches)
// -------------------------------------------------------------------------------------------
// A grid of max_seq_len / 64 tiles for every sequence leaves most workgroups of a ragged batch
// with nothing to do, and each still waits on a load of cu_seqlens before it can exit.  For such
// batches one workgroup first lists the real 64-token tiles, sequence by sequence: entry i is
// {sequence, tile of the sequence, its first token, its length (clamped as seq_range does)};
// entries past the last real tile are {-1, 0, 0, 0}.  The two passes over the fp16 input then run
// on a grid of map_tiles tiles.  One thread per sequence, so batches of up to kMapThreads.
constexpr int kMapThreads = 1024;

__global__ __launch_bounds__(kMapThreads) void tile_map_kernel(CompressArgs a, int map_tiles) {
  __shared__ int s_scan[kMapThreads];
  __shared__ int s_off[kMapThreads], s_c0[kMapThreads], s_len[kMapThreads];
  const int tid = threadIdx.x;
  int n = 0;
  if (tid < a.batch) {
    int c0, L;
    bool bad;
    seq_range(a.cu, tid, a.max_seq_len, a.total, c0, L, bad);
    s_c0[tid] = c0;
    s_len[tid] = L;
    n = (L + kChunk - 1) / kChunk;
  }
  s_scan[tid] = n;
  __syncthreads();
  for (int o = 1; o < kMapThreads; o <<= 1) {   // inclusive prefix sum of the tile counts
    const int x = tid >= o ? s_scan[tid - o] : 0;
    __syncthreads();
    s_scan[tid] += x;
    __syncthreads();
  }
  if (tid < a.batch) s_off[tid] = s_scan[tid] - n;
  const int real = min(s_scan[kMapThreads - 1], map_tiles);
  __syncthreads();
  for (int i = tid; i < map_tiles; i += kMapThreads) {
    int4 e = make_int4(-1, 0, 0, 0);
    if (i < real) {
      // the last sequence whose first tile is at or before i (empty sequences share their
      // successor's offset, so the last such sequence is the one that owns tile i)
      int lo = 0, hi = a.batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      e = make_int4(lo, i - s_off[lo], s_c0[lo], s_len[lo]);
    }
    a.tile_map[i] = e;
  }
}

// The sequence and 64-token tile of this workgroup, with the sequence's first token and length:
// from the tile map (grid over the real tiles of a ragged batch), else grid z is the sequence.
// False when the tile holds no token.
__device__ __forceinline__ bool compress_tile(const CompressArgs &a, int &tile, int &b, int &c0, int &L) {
  if (a.tile_map != nullptr) {
    const int4 e = a.tile_map[tile];
    if (e.x < 0) return false;
    b = e.x;
    tile = e.y;
    c0 = e.z;
    L = e.w;
    return true;
  }
  b = blockIdx.z;
  bool bad;
  seq_range(a.cu, b, a.max_seq_len, a.total, c0, L, bad);
  return tile * kChunk < L;
}

// -------------------------------------------------------------------------------------------
// wave reductions with DPP row operations and lane reads (no LDS)
// -------------------------------------------------------------------------------------------
template <int C>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, C, 0xF, 0xF, false);
}
template <int C>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<C>(__float_as_int(x)));
}
template <int C>
__device__ __forceinline__ double dpp_d(double x) {
  const long long v = __double_as_longlong(x);
  const int lo = dpp_i<C>((int)v), hi = dpp_i<C>((int)(v >> 32));
  return __longlong_as_double((long long)(unsigned)lo | ((long long)hi << 32));
}
__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ double readlane_d(double x, int l) {
  const long long v = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)v, l), hi = __builtin_amdgcn_readlane((int)(v >> 32), l);
  return __longlong_as_double((long long)(unsigned)lo | ((long long)hi << 32));
}
// DPP controls: swap neighbours, swap pairs (within quads), rotate a 16-lane row by 4 and by 8
constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kRowRor4 = 0x124, kRowRor8 = 0x128;
// mirror each half row of 8 lanes (lane i <-> 7 - i): after the quad swaps, the other quad's value
constexpr int kHalfMirror = 0x141;
// mirror a 16-lane row (lane i <-> 15 - i): after the quad swaps and the half mirror, the row's value
constexpr int kRowMirror = 0x140;

// (score desc, t asc): true if (s2, t2) comes first
__device__ __forceinline__ bool better(double s2, int t2, double s, int t) {
  return s2 > s || (s2 == s && t2 < t);
}
template <int C>
__device__ __forceinline__ void best_step(double &s, int &t) {
  const double s2 = dpp_d<C>(s);
  const int t2 = dpp_i<C>(t);
  if (better(s2, t2, s, t)) {
    s = s2;
    t = t2;
  }
}
// best over the wave, returned uniform
__device__ __forceinline__ void wave_best(double &s, int &t) {
  best_step<kQuadSwap1>(s, t);
  best_step<kQuadSwap2>(s, t);
  best_step<kRowRor4>(s, t);
  best_step<kRowRor8>(s, t);   // every lane holds its row's best
  double bs = readlane_d(s, 0);
  int bt = __builtin_amdgcn_readlane(t, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const double s2 = readlane_d(s, 16 * r);
    const int t2 = __builtin_amdgcn_readlane(t, 16 * r);
    if (better(s2, t2, bs, bt)) {
      bs = s2;
      bt = t2;
    }
  }
  s = bs;
  t = bt;
}
// maximum of an unsigned 64-bit value over the wave, returned uniform
template <int C>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long x) {
  const int lo = dpp_i<C>((int)x), hi = dpp_i<C>((int)(x >> 32));
  return (unsigned long long)(unsigned)lo | ((unsigned long long)(unsigned)hi << 32);
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
  auto step = [&](auto tag) {
    constexpr int C = decltype(tag)::value;
    const unsigned long long y = dpp_u64<C>(x);
    x = y > x ? y : x;
  };
  step(std::integral_constant<int, kQuadSwap1>{});
  step(std::integral_constant<int, kQuadSwap2>{});
  step(std::integral_constant<int, kRowRor4>{});
  step(std::integral_constant<int, kRowRor8>{});   // every lane holds its row's maximum
  unsigned long long m = 0ull;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)x, 16 * r);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(x >> 32), 16 * r);
    const unsigned long long y = (unsigned long long)lo | ((unsigned long long)hi << 32);
    m = y > m ? y : m;
  }
  return m;
}
// (min, max, min, max) over the wave, returned uniform
__device__ __forceinline__ float4 wave_minmax(float4 r) {
  auto step = [&](auto tag) {
    constexpr int C = decltype(tag)::value;
    r.x = fminf(r.x, dpp_f<C>(r.x));
    r.y = fmaxf(r.y, dpp_f<C>(r.y));
    r.z = fminf(r.z, dpp_f<C>(r.z));
    r.w = fmaxf(r.w, dpp_f<C>(r.w));
  };
  step(std::integral_constant<int, kQuadSwap1>{});
  step(std::integral_constant<int, kQuadSwap2>{});
  step(std::integral_constant<int, kRowRor4>{});
  step(std::integral_constant<int, kRowRor8>{});
  float4 o = make_float4(readlane_f(r.x, 0), readlane_f(r.y, 0), readlane_f(r.z, 0), readlane_f(r.w, 0));
#pragma unroll
  for (int q = 1; q < 4; ++q) {
    o.x = fminf(o.x, readlane_f(r.x, 16 * q));
    o.y = fmaxf(o.y, readlane_f(r.y, 16 * q));
    o.z = fminf(o.z, readlane_f(r.z, 16 * q));
    o.w = fmaxf(o.w, readlane_f(r.w, 16 * q));
  }
  return o;
}

// -------------------------------------------------------------------------------------------
// exact per-element arithmetic shared by the passes over the fp16 input
// -------------------------------------------------------------------------------------------
// A pass over the input spends most of its instructions on each element, so each step is kept to
// a few instructions while staying exact: packed fp16 min/max and non-finite tests, the
// fixed-point image by one fused multiply-add into float32's round-to-integer range, sums of n and
// n^2 by 16-bit dot products, and the codes by the float-to-byte conversion.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef short short2_t __attribute__((ext_vector_type(2)));
constexpr short2_t kOnes2 = {1, 1};
__device__ __forceinline__ half2_t as_half2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }

// dgq_fixed_point(x) for every x: the clamped value times 512 is exact, and adding 1.5 * 2^23
// rounds it to the nearest integer (ties to even) in one step, that integer then being the low
// bits of the sum (|x * 512| <= 2^14 < 2^22).
__device__ __forceinline__ int fixed_point_fma(float x) {
  const float c = fminf(fmaxf(x, -32.0f), 32.0f);
  return __float_as_int(fmaf(c, 512.0f, 12582912.0f)) - 0x4B400000;
}

// The code bytes of four values (byte e from x[e], with its segment's min and 1 / scale), equal to
// dgq_encode_value's for every input of dgq_compress: subtract and multiply as there, then the
// float-to-byte conversion, which rounds to nearest even, saturates to [0, 255] and takes NaN to 0.
// The clamp to [0, levels] never binds here: a segment's min and max are those of its own values,
// so 0 <= x - mn <= mx - mn and u <= levels * (1 + 2^-22) < levels + 1/2, and a NaN gives 0 in both.
// The byte is then shifted by the code of the minimum: -128 flips its top bit, -127 adds 129
// modulo 256.
__device__ __forceinline__ uint32_t encode4(const float (&x)[4], const float (&mn)[4], const float (&inv)[4],
                                            bool marker) {
#pragma clang fp contract(off)
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float dlt = x[e] - mn[e];
    const float u = dlt * inv[e];
    w = __builtin_amdgcn_cvt_pk_u8_f32(u, e, w);
  }
  return marker ? (((w & 0x7F7F7F7Fu) + 0x01010101u) ^ ((w ^ 0x81818181u) & 0x80808080u)) : (w ^ 0x80808080u);
}

// -------------------------------------------------------------------------------------------
// 1. stats
// -------------------------------------------------------------------------------------------
// Each load instruction of a wave reads whole 2 D-byte rows: LPR = D / 8 lanes per token row (16 B
// each), TPI = 64 / LPR tokens per instruction, NI = 16 / TPI instructions for the wave's 16
// tokens (one 16-token sub-block).  A lane keeps per-token moment sums for its NI tokens; the LPR
// lanes of a row are combined by DPP, and the extrema and the non-finite test cover the wave.
template <int D>
__global__ __launch_bounds__(256) void stats_kernel(CompressArgs a) {
  constexpr int LPR = D / 8, TPI = 64 / LPR, NI = kWin / TPI;
  int tile, h;
  run_order(tile, h);
  int b, c0, L;
  if (!compress_tile(a, tile, b, c0, L)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane / LPR, col = lane % LPR;
  float kmn = INFINITY, kmx = -INFINITY;
  int asum[NI];
  long long bsum[NI];
  const half2_t zero2 = {(_Float16)0.0f, (_Float16)0.0f};
  half2_t vmn2 = {(_Float16)INFINITY, (_Float16)INFINITY}, vmx2 = -vmn2, bad2 = zero2;
  {
    uint4 kr[NI], vr[NI];
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      const int t = tile * 64 + kWin * w + TPI * c + r;
      kr[c] = vr[c] = make_uint4(0u, 0u, 0u, 0u);
      if (t < L) {
        const size_t off = (size_t)(c0 + t) * a.stride_tok + (size_t)h * a.stride_head + 8 * col;
        kr[c] = *reinterpret_cast<const uint4 *>(a.k + off);
        vr[c] = *reinterpret_cast<const uint4 *>(a.v + off);
      }
    }
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      const int t = tile * 64 + kWin * w + TPI * c + r;
      const uint32_t ks[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
      const uint32_t vs[4] = {vr[c].x, vr[c].y, vr[c].z, vr[c].w};
      int as = 0, bpart = 0;   // sum of 8 squares <= 2^31: wraps as int32, exact read as uint32
      if (t < L) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const half2_t kx = as_half2(ks[e]), vx = as_half2(vs[e]);
          vmn2 = __builtin_elementwise_min(vmn2, vx);
          vmx2 = __builtin_elementwise_max(vmx2, vx);
          bad2 = __builtin_elementwise_fma(kx, zero2, bad2);   // NaN once any value is not finite
          bad2 = __builtin_elementwise_fma(vx, zero2, bad2);
          const float x0 = (float)kx[0], x1 = (float)kx[1];
          kmn = fminf(kmn, fminf(x0, x1));
          kmx = fmaxf(kmx, fmaxf(x0, x1));
          const uint32_t n01 = __builtin_amdgcn_perm((uint32_t)fixed_point_fma(x1), (uint32_t)fixed_point_fma(x0),
                                                     0x05040100u);
          const short2_t n2 = __builtin_bit_cast(short2_t, n01);
          as = __builtin_amdgcn_sdot2(n2, kOnes2, as, false);
          bpart = __builtin_amdgcn_sdot2(n2, n2, bpart, false);
        }
      }
      asum[c] = as;
      bsum[c] = (long long)(unsigned int)bpart;
    }
  }
  // the LPR lanes of a row: quads, then half rows, then (LPR 16) whole rows
#pragma unroll
  for (int c = 0; c < NI; ++c) {
    asum[c] += dpp_i<kQuadSwap1>(asum[c]);
    bsum[c] += (long long)dpp_u64<kQuadSwap1>((unsigned long long)bsum[c]);
    asum[c] += dpp_i<kQuadSwap2>(asum[c]);
    bsum[c] += (long long)dpp_u64<kQuadSwap2>((unsigned long long)bsum[c]);
    asum[c] += dpp_i<kHalfMirror>(asum[c]);
    bsum[c] += (long long)dpp_u64<kHalfMirror>((unsigned long long)bsum[c]);
    if constexpr (LPR == 16) {
      asum[c] += dpp_i<kRowRor8>(asum[c]);
      bsum[c] += (long long)dpp_u64<kRowRor8>((unsigned long long)bsum[c]);
    }
    const int t = tile * 64 + kWin * w + TPI * c + r;
    if (col == 0 && t < L) {
      const size_t idx = (size_t)h * a.total + c0 + t;
      a.ws_a[idx] = asum[c];
      a.ws_b[idx] = bsum[c];
    }
  }
  // sub-block extrema: wave w covers tokens tile*64 + 16w .. +15
  const float vmn = fminf((float)vmn2[0], (float)vmn2[1]);
  const float vmx = fmaxf((float)vmx2[0], (float)vmx2[1]);
  const float4 ext = wave_minmax(make_float4(kmn, kmx, vmn, vmx));
  const int sb = tile * 4 + w;
  if (lane == 0 && sb * 16 < L) a.ws_ext[((size_t)b * a.hkv + h) * a.nsub + sb] = ext;
  const bool bad = !(bad2[0] == (_Float16)0.0f && bad2[1] == (_Float16)0.0f);
  if (__ballot(bad) != 0ull && lane == 0) atomicAdd(a.cache.status + 1, 1ull);
}

// -------------------------------------------------------------------------------------------
// 2. scores
// -------------------------------------------------------------------------------------------
// Two 256-token tiles per workgroup: the launch then fits the compute units in one round of
// workgroups (each is short and mostly waits for its loads).
constexpr int kScoreTiles = 2;

template <int D>
__global__ __launch_bounds__(256) void scores_kernel(CompressArgs a) {
  constexpr int TW = kScoreTiles;
  const int tile0 = TW * blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int c0, L;
  bool bad_seq;
  seq_range(a.cu, b, a.max_seq_len, a.total, c0, L, bad_seq);
  if (tile0 * 256 >= L) return;
  const int tid = threadIdx.x;
  const size_t bh = (size_t)b * a.hkv + h;
  // the key moments of the tiles and the 16 tokens on either side, requested first (into
  // registers) so that their round trip overlaps the extrema's
  constexpr int NM = TW * 256 + 2 * kWin;
  constexpr int NL = (NM + 255) / 256;
  const int base = tile0 * 256 - kWin;
  int ra[NL];
  long long rb[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int i = tid + 256 * u, tok = base + i;
    ra[u] = 0;
    rb[u] = 0;
    if (i < NM && tok >= 0 && tok < L) {
      const size_t idx = (size_t)h * a.total + c0 + tok;
      ra[u] = a.ws_a[idx];
      rb[u] = a.ws_b[idx];
    }
  }
  // each tile's K/V extrema from its sub-blocks (for the segment ranges of the selection): wave q
  // takes tile tile0 + q
  if (tid < 64 * TW) {
    const int tile = tile0 + (tid >> 6), k = tid & 63;
    const int sb = 16 * tile + (k & 15);
    const float4 ident = make_float4(INFINITY, -INFINITY, INFINITY, -INFINITY);
    float4 x = ident;
    if (k < 16 && kWin * sb < L) x = a.ws_ext[bh * a.nsub + sb];
    const float4 r = wave_minmax(x);
    if (k == 0 && tile * 256 < L) a.ws_text[bh * a.ntile + tile] = r;
  }
  if (L < 2 * kWin || tile0 * 256 > L - kWin) return;
  __shared__ int sa[NM];
  __shared__ long long sbm[NM];
  __shared__ int wa[TW * 256 + kWin];           // window sums: wa[i] = sa[i] + ... + sa[i + 15]
  __shared__ long long wbm[TW * 256 + kWin];
  __shared__ double best_s[TW][4];
  __shared__ int best_t[TW][4];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int i = tid + 256 * u;
    if (i < NM) {
      sa[i] = ra[u];
      sbm[i] = rb[u];
    }
  }
  __syncthreads();
  for (int i = tid; i < TW * 256 + kWin; i += 256) {
    int A = 0;
    long long B = 0;
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      A += sa[i + u];
      B += sbm[i + u];
    }
    wa[i] = A;
    wbm[i] = B;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < TW; ++q) {
    const int li = 256 * q + tid, t = tile0 * 256 + li;
    double score = -INFINITY;
    int tb = INT_MAX;
    if (t >= kWin && t <= L - kWin) {
      // Q = N * sum b - (sum a)^2 of the windows [t - 16, t) and [t, t + 16), exact in double
      // (|sum a| <= 2^25, N * sum b <= 2^51, the fused result is an integer below 2^51)
      const double nel = (double)(kWin * D);
      const double Al = (double)wa[li], Ar = (double)wa[li + kWin];
      const double ql = fma(-Al, Al, nel * (double)wbm[li]);
      const double qr = fma(-Ar, Ar, nel * (double)wbm[li + kWin]);
      const double hi = fmax(ql, qr), lo = fmin(ql, qr);
      score = hi < a.qfloor ? -INFINITY : (hi + 1.0) / (lo + 1.0);
      a.ws_score[(size_t)h * a.total + c0 + t] = score;
      tb = t;
    }
    // best (score, smallest t) of the tile
    wave_best(score, tb);
    if ((tid & 63) == 0) {
      best_s[q][tid >> 6] = score;
      best_t[q][tid >> 6] = tb;
    }
  }
  __syncthreads();
  if (tid < TW) {
    const int tile = tile0 + tid;
    if (tile * 256 <= L - kWin) {   // the tiles the selection scans
      double s = best_s[tid][0];
      int tt = best_t[tid][0];
      for (int w = 1; w < 4; ++w)
        if (better(best_s[tid][w], best_t[tid][w], s, tt)) {
          s = best_s[tid][w];
          tt = best_t[tid][w];
        }
      a.ws_tile[bh * a.ntile + tile] = make_double2(s, (double)tt);
    }
  }
}

// -------------------------------------------------------------------------------------------
// 3. select
// -------------------------------------------------------------------------------------------
// One 1024-thread workgroup per (sequence, kv head).  The tile maxima are kept in LDS (sequences
// of up to kSelTiles * 256 tokens; longer ones read them from the workspace), so a greedy round
// costs one scan of LDS plus one re-read of the (at most two) tiles the new cut's suppression
// window touches, both re-scanned at once.
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelTiles = 4096;

template <int D>
__global__ __launch_bounds__(kSelThreads) void select_kernel(CompressArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  int c0, L;
  bool bad_seq;
  seq_range(a.cu, b, a.max_seq_len, a.total, c0, L, bad_seq);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t bh = (size_t)b * a.hkv + h;
  constexpr int MS = kMaxCuts + 1;
  __shared__ double2 stile[kSelTiles];
  __shared__ double wbs[2][kSelWaves];   // per wave: best of the scan (0) and of the re-scan (1)
  __shared__ int wbt[2][kSelWaves];
  __shared__ int cuts[kMaxCuts];
  __shared__ int starts[kMaxCuts + 2];
  if (tid == 0 && bad_seq && h == 0) atomicAdd(a.cache.status + 2, 1ull);
  // the moments of the last min(16, L) tokens, for the append state written at the end
  const int rl = min(kWin, L);
  int ring_a = 0;
  long long ring_b = 0;
  if (tid < rl) {
    const size_t idx = (size_t)h * a.total + c0 + (L - rl + tid);
    ring_a = a.ws_a[idx];
    ring_b = a.ws_b[idx];
  }

  // ---- greedy selection over the tile maxima ----
  double2 *gtiles = a.ws_tile + bh * a.ntile;
  const int ntiles = L >= 2 * kWin ? (L - kWin) / 256 + 1 : 0;
  const bool in_lds = ntiles <= kSelTiles;
  if (in_lds && ntiles > 0) {
    // all loads in flight at once (clamped indices, so every load is in bounds and unconditional)
    constexpr int U = kSelTiles / kSelThreads;
    double2 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = gtiles[min(tid + kSelThreads * u, ntiles - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = tid + kSelThreads * u;
      if (c < ntiles) stile[c] = x[u];
    }
  }
  // tile c: LDS when the tiles fit, else the workspace through a buffer resource (two kinds of
  // access, so that the compiler does not merge them into one generic-pointer access, which would
  // make every wait cover both the LDS and the memory counters)
  const __amdgpu_buffer_rsrc_t rtiles = raw_rsrc(gtiles, (uint32_t)(ntiles * sizeof(double2)));
  auto tile_get = [&](int c) -> double2 {
    if (in_lds) return stile[c];
    return __builtin_bit_cast(double2, __builtin_amdgcn_raw_buffer_load_b128(rtiles, (uint32_t)c * 16u, 0, 0));
  };
  auto tile_put = [&](int c, double2 v) {
    if (in_lds) stile[c] = v;
    else __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rtiles, (uint32_t)c * 16u, 0, 0);
  };
  __syncthreads();
  const int max_seg = a.length_aware ? min(a.max_segments, length_aware_cap(L)) : a.max_segments;
  int nc = 0;
  if (ntiles > 0 && max_seg > 1) {
    for (int r = 0; r < max_seg - 1; ++r) {
      double s = -INFINITY;
      int t = INT_MAX;
      for (int c = tid; c < ntiles; c += kSelThreads) {
        const double2 e = tile_get(c);
        if (better(e.x, (int)e.y, s, t)) {
          s = e.x;
          t = (int)e.y;
        }
      }
      wave_best(s, t);
      if (lane == 0) {
        wbs[0][wave] = s;
        wbt[0][wave] = t;
      }
      __syncthreads();
      s = wbs[0][0];
      t = wbt[0][0];
      for (int w = 1; w < kSelWaves; ++w)
        if (better(wbs[0][w], wbt[0][w], s, t)) {
          s = wbs[0][w];
          t = wbt[0][w];
        }
      if (s == -INFINITY) break;
      if (r > 0 && !(s >= a.tau)) break;
      if (tid == 0) cuts[nc] = t;
      ++nc;
      // re-scan the tiles the suppressed window [t - 15, t + 15] touches (at most two): threads
      // 0..255 the first, 256..511 the second
      const int lo_tile = max(0, (t - (kWin - 1)) / 256), hi_tile = min(ntiles - 1, (t + kWin - 1) / 256);
      const int c = lo_tile + (tid >> 8);
      double sc = -INFINITY;
      int tt = INT_MAX;
      if (c <= hi_tile) {
        const int tc = c * 256 + (tid & 255);
        if (tc >= kWin && tc <= L - kWin) {
          bool alive = abs(tc - t) > kWin - 1;
          for (int k = 0; k + 1 < nc; ++k) alive = alive && abs(tc - cuts[k]) > kWin - 1;
          if (alive) {
            sc = a.ws_score[(size_t)h * a.total + c0 + tc];
            tt = tc;
          }
        }
      }
      wave_best(sc, tt);
      if (lane == 0) {
        wbs[1][wave] = sc;
        wbt[1][wave] = tt;
      }
      __syncthreads();
      // the thread that scans a re-scanned tile folds the four waves of its group and stores the
      // tile's new best itself, so its next scan reads it without another barrier (the scan's
      // results sit in the other half of wbs, so no barrier is needed between reading them and the
      // re-scan either)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int cq = lo_tile + q;
        if (cq <= hi_tile && cq % kSelThreads == tid) {
          double bs = wbs[1][4 * q];
          int bt = wbt[1][4 * q];
          for (int w = 1; w < 4; ++w)
            if (better(wbs[1][4 * q + w], wbt[1][4 * q + w], bs, bt)) {
              bs = wbs[1][4 * q + w];
              bt = wbt[1][4 * q + w];
            }
          tile_put(cq, make_double2(bs, (double)bt));
        }
      }
    }
  }
  // starts = [0] + sorted cuts, then L
  if (tid == 0) {
    starts[0] = 0;
    for (int i = 0; i < nc; ++i) {
      const int x = cuts[i];
      int k = i;
      while (k > 0 && starts[k] > x) {
        starts[k + 1] = starts[k];
        --k;
      }
      starts[k + 1] = x;
    }
    starts[nc + 1] = L;
  }
  __syncthreads();
  const int nseg = L > 0 ? nc + 1 : 0;

  // ---- every segment's K/V min/max ----
  // (1) tiles inside one segment: the tile extrema of the scores pass, one tile per thread and
  //     pass, folded per segment by one wave reduction each (segments in a plain loop, partial
  //     results in the wave's LDS slot);
  // (2) a tile that holds a cut: its 16 sub-blocks, one per lane of a 16-lane group (group c takes
  //     the tile of cut c, unless cut c - 1 took it), folded per segment by a row reduction;
  // (3) a sub-block that a cut splits (cuts are >= 16 apart, so one cut per sub-block; a cut at a
  //     multiple of 16 splits none) is re-read raw by wave c - 1.
  // (Short loops and no per-segment register arrays: this part runs once per head, mostly in
  // one or two waves, so the length of its code is what it costs.)
  const float4 ident = make_float4(INFINITY, -INFINITY, INFINITY, -INFINITY);
  auto fold = [](float4 &r, const float4 x) {
    r.x = fminf(r.x, x.x);
    r.y = fmaxf(r.y, x.y);
    r.z = fminf(r.z, x.z);
    r.w = fmaxf(r.w, x.w);
  };
  auto seg_of = [&](int t) {
    int j = 0;
    for (int k = 1; k < nseg; ++k) j += t >= starts[k] ? 1 : 0;
    return j;
  };
  __shared__ float4 sred[kSelWaves][MS];
  __shared__ float4 scut[kMaxCuts][MS];
  __shared__ float4 sraw[kMaxCuts][2];   // cut c: (left part, right part)
  if (lane == 0)
    for (int j = 0; j < MS; ++j) sred[wave][j] = ident;
  if (tid < kMaxCuts * MS) scut[tid / MS][tid % MS] = ident;
  __syncthreads();
  // Every load of the three parts is requested before any reduction (one round trip, not three).
  const float4 *text = a.ws_text + bh * a.ntile;
  const int ntl = (L + 255) / 256;
  auto tile_ext = [&](int i, float4 &x, int &j0) {   // (1): tile i, if one segment holds it
    x = ident;
    j0 = -1;
    if (i < ntl) {
      const int t0 = 256 * i, t1 = min(t0 + 256, L);
      j0 = seg_of(t0);
      if (seg_of(t1 - 1) == j0) x = text[i];
      else j0 = -1;                                  // (2)
    }
  };
  float4 tx;
  int tj;
  tile_ext(tid, tx, tj);
  const int g = tid >> 4, k = tid & 15;              // (2): 16-lane group g takes cut g's tile
  const bool on = wave < (kMaxCuts + 3) / 4 && g < nc && !(g > 0 && starts[g] / 256 == starts[g + 1] / 256);
  float4 ex = ident;
  int ej = -1;
  if (on) {
    const int sb = 16 * (starts[g + 1] / 256) + k;
    const int s0 = kWin * sb, s1 = min(s0 + kWin, L);
    if (s0 < L) {
      ej = seg_of(s0);
      if (s1 <= starts[ej + 1]) ex = a.ws_ext[bh * a.nsub + sb];
      else ej = -1;                                  // (3)
    }
  }
  const bool raw_on = wave + 1 < nseg;               // (3): wave c - 1 re-reads cut c's sub-block
  const int cut = raw_on ? starts[min(wave + 1, kMaxCuts + 1)] : 0;
  const int t0r = cut - cut % kWin;
  constexpr int PER_LANE = kWin * D / 64;            // halves of the sub-block per lane
  uint4 kw[PER_LANE / 8], vw[PER_LANE / 8];
#pragma unroll
  for (int e = 0; e < PER_LANE / 8; ++e) {
    kw[e] = make_uint4(0u, 0u, 0u, 0u);
    vw[e] = make_uint4(0u, 0u, 0u, 0u);
    const int x = lane * PER_LANE + 8 * e;
    const int tok = t0r + x / D, d = x % D;
    if (raw_on && cut % kWin != 0 && tok < L) {
      const size_t off = (size_t)(c0 + tok) * a.stride_tok + (size_t)h * a.stride_head + d;
      kw[e] = *reinterpret_cast<const uint4 *>(a.k + off);
      vw[e] = *reinterpret_cast<const uint4 *>(a.v + off);
    }
  }

  for (int i0 = 0; i0 < ntl; i0 += kSelThreads) {
    float4 x = tx;
    int j0 = tj;
    if (i0 > 0) tile_ext(i0 + tid, x, j0);
    for (int j = 0; j < nseg; ++j) {
      const float4 r = wave_minmax(j0 == j ? x : ident);
      if (lane == 0) fold(sred[wave][j], r);
    }
  }
  if (wave < (kMaxCuts + 3) / 4) {
    for (int jj = 0; jj < nseg; ++jj) {
      float4 r = ej == jj ? ex : ident;
      auto step = [&](auto tag) {
        constexpr int C = decltype(tag)::value;
        r.x = fminf(r.x, dpp_f<C>(r.x));
        r.y = fmaxf(r.y, dpp_f<C>(r.y));
        r.z = fminf(r.z, dpp_f<C>(r.z));
        r.w = fmaxf(r.w, dpp_f<C>(r.w));
      };
      step(std::integral_constant<int, kQuadSwap1>{});
      step(std::integral_constant<int, kQuadSwap2>{});
      step(std::integral_constant<int, kHalfMirror>{});
      step(std::integral_constant<int, kRowMirror>{});   // every lane of the row holds its result
      if (on && k == 0) scut[g][jj] = r;
    }
  }
  if (raw_on) {
    float4 left = ident, right = ident;
    if (cut % kWin != 0) {
#pragma unroll
      for (int e = 0; e < PER_LANE / 8; ++e) {
        const int x = lane * PER_LANE + 8 * e;
        const int tok = t0r + x / D;
        if (tok < L) {
          const uint32_t kk[4] = {kw[e].x, kw[e].y, kw[e].z, kw[e].w}, vv[4] = {vw[e].x, vw[e].y, vw[e].z, vw[e].w};
          float4 r = ident;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float k0 = half_bits_to_float(kk[q] & 0xFFFFu), k1 = half_bits_to_float(kk[q] >> 16);
            const float v0 = half_bits_to_float(vv[q] & 0xFFFFu), v1 = half_bits_to_float(vv[q] >> 16);
            fold(r, make_float4(fminf(k0, k1), fmaxf(k0, k1), fminf(v0, v1), fmaxf(v0, v1)));
          }
          fold(tok < cut ? left : right, r);
        }
      }
    }
    left = wave_minmax(left);
    right = wave_minmax(right);
    if (lane == 0) {
      sraw[wave][0] = left;
      sraw[wave][1] = right;
    }
  }
  __syncthreads();
  if (tid < nseg) {
    float4 r = sred[0][tid];
    for (int w = 1; w < kSelWaves; ++w) fold(r, sred[w][tid]);
    for (int c = 0; c < nc; ++c) fold(r, scut[c][tid]);
    if (tid > 0) fold(r, sraw[tid - 1][1]);        // right of the cut that starts segment tid
    if (tid + 1 < nseg) fold(r, sraw[tid][0]);      // left of the cut that ends it
    dgq_seg_t row;
    row.start = starts[tid];
    row.kmin = r.x + 0.0f;
    row.kmax = r.y + 0.0f;
    row.vmin = r.z + 0.0f;
    row.vmax = r.w + 0.0f;
    row.kscale = dgq_scale(row.kmin, row.kmax, a.fmt.levels);
    row.vscale = dgq_scale(row.vmin, row.vmax, a.fmt.levels);
    row.reserved = 0;
    a.cache.segs[bh * a.seg_cap + tid] = row;
  }
  // append state: open span starts at L, ring = the last min(16, L) tokens' moments
  dgq_tail_t *tl = a.cache.tail + bh;
  if (tid < kWin) {
    tl->ring_a[tid] = ring_a;
    tl->ring_b[tid] = ring_b;
  }
  if (tid < 4) tl->span_range[tid] = 0.f;
  if (tid == 0) {
    a.cache.nseg[bh] = nseg;
    tl->r0 = L;
    tl->ring_len = rl;
    tl->span_own = 0;
    tl->window_done = 0;
  }
}

// -------------------------------------------------------------------------------------------
// 2+3 fused, for sequences of at most kSmallSeq tokens: one workgroup of 512 (or 256) threads per
// (sequence, kv head) holds the key moments in LDS, keeps the scores of its 16 candidates per
// thread in registers, runs the greedy rounds with no memory traffic, and reduces all segments'
// min/max in one pass over the sub-block extrema (plus the raw tokens of sub-blocks a cut splits).
// Wave reductions use DPP row operations and lane reads, not LDS permutes.
// -------------------------------------------------------------------------------------------
constexpr int kSmallSeq = 8192;     // longest sequence of the fused path
constexpr int kPerThread = kWin;    // 16 candidates (one 16-token sub-block) per thread

// LDS slot of token t, t in [-16, S + 16) for sequences of up to S tokens: one pad slot after every 16 tokens, so that
// thread i reading token 16 i + u (all i of a wave at once) hits distinct banks; the 16 slots on
// either side of the sequence hold zeros, so window sums need no bounds tests
__device__ __forceinline__ int skew(int t) { return (t + kWin) + ((t + kWin) >> 4); }
template <int S>
constexpr int skewed_slots() { return (S + 2 * kWin) + (S + 2 * kWin) / 16; }


// S: the longest sequence the instance handles (8192, or 4096 with half the threads and LDS,
// so that two workgroups share a compute unit when a batch has many short sequences).  One wave
// per cut re-reads the sub-block that cut splits, so an instance takes at most NW cuts:
// small_cuts_ok() is the launch condition.
template <int S>
constexpr int small_waves() { return S / kPerThread / 64; }
constexpr bool small_cuts_ok(int S_waves, int max_segments) { return max_segments - 1 <= S_waves; }
static_assert(small_waves<kSmallSeq>() >= kMaxCuts, "the 8192-token instance takes every cut count");

// What the rounds and the range pass keep in LDS: it takes the place of the key moments b_t,
// which nothing reads once the scores are in registers (so that the 4096-token instance fits three
// workgroups in a compute unit's LDS).
template <int S>
struct SmallSelTail {
  static constexpr int NW = small_waves<S>();
  static constexpr int MS = kMaxCuts + 1;
  float4 ext[S / kWin];          // sub-block extrema
  float4 red[NW][MS];            // per-wave extrema of each segment's whole sub-blocks
  float4 raw[kMaxCuts][2];       // cut c: (left part, right part) of the sub-block it splits
  double gbs[2 * NW];            // wave bests (score, t) of a round, double-buffered
  int gbt[2 * NW];
  int cut[kMaxCuts];
  int start[MS + 1];
};
template <int S>
union SmallSelLds {
  double bd[skewed_slots<S>()];  // key moments b_t (< 2^36, exact in double), until the scores
  SmallSelTail<S> tail;
};
static_assert(sizeof(SmallSelTail<kSmallSeq / 2>) <= sizeof(double) * skewed_slots<kSmallSeq / 2>(), "fits");

// Three 256-thread workgroups per compute unit for the 4096-token instance (LDS and registers
// sized for it), one 512-thread workgroup for the 8192-token one.
template <int S>
constexpr int small_waves_per_simd() { return S == kSmallSeq / 2 ? 3 : 1; }

template <int D, int S>
__global__ __launch_bounds__(S / kPerThread, small_waves_per_simd<S>()) void select_small_kernel(CompressArgs a) {
  constexpr int NT = S / kPerThread;   // threads
  constexpr int NW = small_waves<S>();
  const int h = blockIdx.x, b = blockIdx.y;
  int c0, L;
  bool bad_seq;
  seq_range(a.cu, b, a.max_seq_len, a.total, c0, L, bad_seq);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t bh = (size_t)b * a.hkv + h;
  __shared__ int sa[skewed_slots<S>()];
  __shared__ SmallSelLds<S> su;
  __shared__ long long sring_b[kWin];
  double *sbd = su.bd;
  SmallSelTail<S> &ov = su.tail;
  float4 *sext = ov.ext;
  double *gbs = ov.gbs;
  int *gbt = ov.gbt;
  auto &sred = ov.red;
  int *scut = ov.cut;
  int *sstart = ov.start;
  auto &sraw = ov.raw;
  if (tid == 0 && bad_seq && h == 0) atomicAdd(a.cache.status + 2, 1ull);

  // ---- key moments and sub-block extrema of the sequence into LDS (all loads issued at once) ----
  const size_t mrow = (size_t)h * a.total + c0;
  {
    int ra[kPerThread];
    long long rb[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int t = tid + NT * i;
      ra[i] = t < L ? a.ws_a[mrow + t] : 0;
      rb[i] = t < L ? a.ws_b[mrow + t] : 0;
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int t = tid + NT * i;
      sa[skew(t)] = ra[i];
      sbd[skew(t)] = (double)rb[i];
      if (t < L && t >= L - kWin) sring_b[t - (L - kWin)] = rb[i];   // kept for the append state
    }
  }
  if (tid < 2 * kWin) {   // the zero pads
    const int t = tid < kWin ? tid - kWin : S + tid - kWin;
    sa[skew(t)] = 0;
    sbd[skew(t)] = 0.0;
  }
  // the sub-block extrema wait in registers until the key moments' LDS is free
  const int nsub = (L + kWin - 1) / kWin;
  const float4 ext_in = tid < nsub ? a.ws_ext[bh * a.nsub + tid] : make_float4(0.f, 0.f, 0.f, 0.f);
  __syncthreads();

  // ---- scores of this thread's candidates t = 16 * tid + i (window sums slide over LDS) ----
  // Q = N * sum b - (sum a)^2 is exact in double: |sum a| <= 2^25, N * sum b <= 2^51, N = 2^k.
  const int tb = kPerThread * tid;
  double sc[kPerThread];
  {
    const double nel = (double)(kWin * D);
    int A = 0;
    double Bm = 0.0;
    const int s0 = tb - kWin;
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      A += sa[skew(s0 + u)];
      Bm += sbd[skew(s0 + u)];
    }
    double q[2 * kWin];
#pragma unroll
    for (int k = 0; k < 2 * kWin; ++k) {
      const double Ad = (double)A;
      q[k] = fma(-Ad, Ad, nel * Bm);
      if (k + 1 < 2 * kWin) {
        A += sa[skew(s0 + k + kWin)] - sa[skew(s0 + k)];
        Bm += sbd[skew(s0 + k + kWin)] - sbd[skew(s0 + k)];
      }
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int t = tb + i;
      sc[i] = -INFINITY;
      if (t >= kWin && t <= L - kWin) {
        const double ql = q[i], qr = q[i + kWin];
        sc[i] = fmax(ql, qr) < a.qfloor ? -INFINITY : (fmax(ql, qr) + 1.0) / (fmin(ql, qr) + 1.0);
      }
    }
  }
  __syncthreads();   // every thread has read the key moments: their LDS now takes the rest
  if (tid < nsub) sext[tid] = ext_in;

  // ---- greedy selection: every thread keeps its 16 scores in registers; per round one wave
  // reduction (DPP), one exchange of the 8 wave bests through LDS, and the suppression of the
  // taken cut's neighbours in registers ----
  int nc = 0;
  const int max_seg = a.length_aware ? min(a.max_segments, length_aware_cap(L)) : a.max_segments;
  if (L >= 2 * kWin) {
    for (int r = 0; r < max_seg - 1; ++r) {
      double s = -INFINITY;
      int t = INT_MAX;
#pragma unroll
      for (int i = 0; i < kPerThread; ++i)
        if (sc[i] > s) {   // ascending t: the first maximum is the smallest t
          s = sc[i];
          t = tb + i;
        }
      wave_best(s, t);
      const int buf = r & 1;
      if (lane == 0) {
        gbs[NW * buf + wave] = s;
        gbt[NW * buf + wave] = t;
      }
      __syncthreads();
      s = gbs[NW * buf];
      t = gbt[NW * buf];
#pragma unroll
      for (int w = 1; w < NW; ++w)
        if (better(gbs[NW * buf + w], gbt[NW * buf + w], s, t)) {
          s = gbs[NW * buf + w];
          t = gbt[NW * buf + w];
        }
      if (s == -INFINITY) break;
      if (r > 0 && !(s >= a.tau)) break;
      if (tid == 0) scut[nc] = t;
      ++nc;
#pragma unroll
      for (int i = 0; i < kPerThread; ++i)
        if (abs(tb + i - t) <= kWin - 1) sc[i] = -INFINITY;
    }
  }
  const int nseg = L > 0 ? nc + 1 : 0;
  // starts = [0] + sorted cuts, then L
  if (tid == 0) {
    sstart[0] = 0;
    for (int i = 0; i < nc; ++i) {
      const int x = scut[i];
      int k = i;
      while (k > 0 && sstart[k] > x) {
        sstart[k + 1] = sstart[k];
        --k;
      }
      sstart[k + 1] = x;
    }
    sstart[max(nseg, 1)] = L;
  }
  __syncthreads();
  const int *starts = sstart;

  // ---- all segments' K/V min/max ----
  // (1) whole sub-blocks: thread tid holds sub-block tid; for each segment j (a rolled loop) the
  //     waves reduce the extrema of the sub-blocks that lie inside j.
  // (2) a sub-block that a cut splits (cuts are >= 16 apart, so one cut per sub-block; a cut at a
  //     multiple of 16 splits none) is re-read raw by one wave per cut: wave c - 1 takes cut c and
  //     reduces the parts left and right of it.
  const float4 ident = make_float4(INFINITY, -INFINITY, INFINITY, -INFINITY);
  auto fold = [&](float4 &r, const float4 x) {
    r.x = fminf(r.x, x.x);
    r.y = fmaxf(r.y, x.y);
    r.z = fminf(r.z, x.z);
    r.w = fmaxf(r.w, x.w);
  };
  int my_seg = -1;   // segment holding all of sub-block tid, or -1
  if (tid < nsub) {
    const int t0 = kWin * tid, t1 = min(t0 + kWin, L) - 1;
    int j0 = 0, j1 = 0;
    for (int k = 1; k < nseg; ++k) {
      j0 += t0 >= starts[k] ? 1 : 0;
      j1 += t1 >= starts[k] ? 1 : 0;
    }
    if (j0 == j1) my_seg = j0;
  }
  const float4 my_ext = my_seg >= 0 ? sext[tid] : ident;
#pragma unroll 1
  for (int j = 0; j < nseg; ++j) {
    const float4 r = wave_minmax(my_seg == j ? my_ext : ident);
    if (lane == 0) sred[wave][j] = r;
  }
  if (wave + 1 < nseg) {
    const int cut = starts[wave + 1];
    float4 left = ident, right = ident;
    if (cut % kWin != 0) {
      const int t0 = cut - cut % kWin;
      constexpr int PER_LANE = kWin * D / 64;   // halves of the sub-block per lane
#pragma unroll
      for (int e0 = 0; e0 < PER_LANE; e0 += 8) {
        const int x = lane * PER_LANE + e0;
        const int tok = t0 + x / D, d = x % D;
        if (tok < L) {
          const size_t off = (size_t)(c0 + tok) * a.stride_tok + (size_t)h * a.stride_head + d;
          const uint4 kw = *reinterpret_cast<const uint4 *>(a.k + off);
          const uint4 vw = *reinterpret_cast<const uint4 *>(a.v + off);
          const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w}, vv[4] = {vw.x, vw.y, vw.z, vw.w};
          float4 r = ident;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float k0 = half_bits_to_float(kk[e] & 0xFFFFu), k1 = half_bits_to_float(kk[e] >> 16);
            const float v0 = half_bits_to_float(vv[e] & 0xFFFFu), v1 = half_bits_to_float(vv[e] >> 16);
            fold(r, make_float4(fminf(k0, k1), fmaxf(k0, k1), fminf(v0, v1), fmaxf(v0, v1)));
          }
          fold(tok < cut ? left : right, r);
        }
      }
    }
    left = wave_minmax(left);
    right = wave_minmax(right);
    if (lane == 0) {
      sraw[wave][0] = left;
      sraw[wave][1] = right;
    }
  }
  __syncthreads();
  if (tid < nseg) {
    float4 r = sred[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) fold(r, sred[w][tid]);
    if (tid > 0) fold(r, sraw[tid - 1][1]);        // right of the cut that starts segment tid
    if (tid + 1 < nseg) fold(r, sraw[tid][0]);      // left of the cut that ends it
    dgq_seg_t row;
    row.start = starts[tid];
    row.kmin = r.x + 0.0f;
    row.kmax = r.y + 0.0f;
    row.vmin = r.z + 0.0f;
    row.vmax = r.w + 0.0f;
    row.kscale = dgq_scale(row.kmin, row.kmax, a.fmt.levels);
    row.vscale = dgq_scale(row.vmin, row.vmax, a.fmt.levels);
    row.reserved = 0;
    a.cache.segs[bh * a.seg_cap + tid] = row;
  }
  // append state: open span starts at L, ring = the last min(16, L) tokens' moments
  const int rl = min(kWin, L);
  dgq_tail_t *tl = a.cache.tail + bh;
  if (tid < kWin) {
    tl->ring_a[tid] = tid < rl ? sa[skew(L - rl + tid)] : 0;
    tl->ring_b[tid] = tid < rl ? sring_b[kWin - rl + tid] : 0;
  }
  if (tid == 0) {
    a.cache.nseg[bh] = nseg;
    tl->r0 = L;
    tl->ring_len = rl;
    tl->span_own = 0;
    tl->window_done = 0;
  }
}

// -------------------------------------------------------------------------------------------
// 4. encode
// -------------------------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(256) void encode_kernel(CompressArgs a) {
  constexpr int VROW = D + 8;   // padded LDS row (halves)
  int chunk, h;
  run_order(chunk, h);
  int b, c0, L;
  if (!compress_tile(a, chunk, b, c0, L)) return;
  const int t0 = chunk * kChunk;
  const int tid = threadIdx.x;
  const size_t bh = (size_t)b * a.hkv + h;
  __shared__ int s_start[kMaxSegCap];
  __shared__ float s_kmin[kMaxSegCap], s_kinv[kMaxSegCap], s_vmin[kMaxSegCap], s_vinv[kMaxSegCap];
  __shared__ int segidx[kChunk];
  __shared__ float2 kprm[kChunk], vprm[kChunk];   // per-token segment (min, 1 / scale) of K and V
  __shared__ uint16_t vt[kChunk * VROW];
  const int ns = a.cache.nseg[bh];
  if (tid < ns) {
    const dgq_seg_t row = a.cache.segs[bh * a.seg_cap + tid];
    s_start[tid] = row.start;
    s_kmin[tid] = row.kmin;
    s_kinv[tid] = dgq_inv(row.kmin, row.kmax, a.fmt.levels);
    s_vmin[tid] = row.vmin;
    s_vinv[tid] = dgq_inv(row.vmin, row.vmax, a.fmt.levels);
  }
  __syncthreads();
  if (tid < kChunk) {
    const int tok = t0 + tid;
    int idx = 0;
    for (int k = 1; k < ns; ++k) idx += tok >= s_start[k] ? 1 : 0;
    segidx[tid] = idx;
    kprm[tid] = make_float2(s_kmin[idx], s_kinv[idx]);
    vprm[tid] = make_float2(s_vmin[idx], s_vinv[idx]);
  }
  // stage the value rows of the chunk
  constexpr int VPR = D / 8;   // uint4 per row
  for (int x = tid; x < kChunk * VPR; x += 256) {
    const int tau = x / VPR, cc = x % VPR;
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (t0 + tau < L)
      w = load_last_use(a.v + (size_t)(c0 + t0 + tau) * a.stride_tok + (size_t)h * a.stride_head + 8 * cc);
    uint32_t *dst = reinterpret_cast<uint32_t *>(vt + tau * VROW + 8 * cc);
    dst[0] = w.x;
    dst[1] = w.y;
    dst[2] = w.z;
    dst[3] = w.w;
  }
  __syncthreads();

  const int32_t *bt = a.block_table + (size_t)b * a.max_blocks;
  const int nblk_seq = (L + BS - 1) / BS;
  const size_t tile_bytes = (size_t)BS * D;
  const bool marker = a.fmt.marker != 0;

  // keys: one unit = 16 channels of one token = 16 contiguous bytes of the tile
  constexpr int KU = kChunk * D / 16;
  for (int u = tid; u < KU; u += 256) {
    const int tau = u / (D / 16), d0 = 16 * (u % (D / 16));
    const int tok = t0 + tau;
    if (tok >= L) continue;
    const float2 kp = kprm[tau];
    const float mn[4] = {kp.x, kp.x, kp.x, kp.x};
    const float inv[4] = {kp.y, kp.y, kp.y, kp.y};
    const uint16_t *src = a.k + (size_t)(c0 + tok) * a.stride_tok + (size_t)h * a.stride_head + d0;
    const uint4 w0 = load_last_use(src), w1 = load_last_use(src + 8);
    const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    uint32_t outw[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const half2_t x01 = as_half2(ws[2 * g]), x23 = as_half2(ws[2 * g + 1]);
      const float x[4] = {(float)x01[0], (float)x01[1], (float)x23[0], (float)x23[1]};
      outw[g] = encode4(x, mn, inv, marker);
    }
    // marker format: the first key byte of every segment but the first is its marker
    if (marker && d0 == 0) {
      const int sg = segidx[tau];
      if (sg > 0 && s_start[sg] == tok) outw[0] = (outw[0] & ~0xFFu) | dgq_marker_byte(outw[0] & 0xFFu);
    }
    bool bad_blk = false;
    const int blk = checked_block(bt[tok / BS], a.cache.num_blocks, bad_blk);
    if (bad_blk) {
      atomicAdd(a.cache.status + 2, 1ull);
      continue;
    }
    int8_t *dst = a.cache.k_pool + ((size_t)blk * a.hkv + h) * tile_bytes + k_tile_offset<D, BS>(tok % BS, d0);
    store_stream(dst, outw);
  }

  // values: one unit = 16 tokens of one channel = 16 contiguous bytes of the tile; the code of a
  // token past L is 0
  const int last = L - 1 - t0;   // last token of the sequence in this chunk (>= 0)
  for (int u = tid; u < KU; u += 256) {
    int d, blk_local, taus[16];
    if constexpr (BS == 64) {
      const int n = u / 64, jj = (u / 16) % 4, r = u % 16;
      d = 16 * n + r;
      blk_local = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) taus[e] = 16 * (e >> 2) + 4 * jj + (e & 3);
    } else {
      blk_local = u / D;
      d = u % D;
#pragma unroll
      for (int e = 0; e < 16; ++e) taus[e] = 16 * blk_local + e;
    }
    const int lblk = (t0 + (BS == 64 ? 0 : 16 * blk_local)) / BS;
    if (lblk >= nblk_seq) continue;
    uint32_t outw[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float x[4], mn[4], inv[4];
      uint32_t past = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tau = taus[4 * g + e];
        const int tc = min(tau, last);
        const float2 pr = vprm[tc];
        x[e] = half_bits_to_float(vt[tc * VROW + d]);
        mn[e] = pr.x;
        inv[e] = pr.y;
        past |= tau <= last ? 0u : 0xFFu << (8 * e);
      }
      outw[g] = encode4(x, mn, inv, marker) & ~past;
    }
    bool bad_blk = false;
    const int blk = checked_block(bt[lblk], a.cache.num_blocks, bad_blk);
    if (bad_blk) continue;   // counted once per unit by the key loop above
    int8_t *tilep = a.cache.v_pool + ((size_t)blk * a.hkv + h) * tile_bytes;
    int off;
    if constexpr (BS == 64) {
      const int n = u / 64, jj = (u / 16) % 4, r = u % 16;
      off = ((n * 4 + jj) * 16 + r) * 16;
    } else {
      off = v_tile_offset<D, BS>((t0 + 16 * blk_local) % BS, d);   // the unit's 16-token tile
    }
    store_stream(tilep + off, outw);
  }

  // boundary bits: 8 bytes per chunk (one 64-token block, or four 16-token blocks); none in the
  // marker format
  if (!marker && tid < kChunk / 8) {
    const int tok0 = t0 + 8 * tid;
    const int lblk = tok0 / BS;
    if (lblk < nblk_seq) {
      uint32_t byte = 0;
      for (int i = 0; i < 8; ++i) {
        const int tok = tok0 + i;
        bool start = false;
        for (int k = 1; k < ns; ++k) start = start || (s_start[k] == tok);
        if (tok < L && start) byte |= 1u << i;
      }
      bool bad_blk = false;
      const int blk = checked_block(bt[lblk], a.cache.num_blocks, bad_blk);
      if (!bad_blk) a.cache.bits[((size_t)blk * a.hkv + h) * (BS / 8) + (tok0 % BS) / 8] = (uint8_t)byte;
    }
  }
}

// -------------------------------------------------------------------------------------------
// one launch for short sequences: stats, scores, selection and encode of one (sequence, kv head)
// in one workgroup, for sequences whose fp16 values fit in LDS (L * head_dim <= kShortElems)
// -------------------------------------------------------------------------------------------
// The four passes above cost four launches and a round trip of the moments through the
// workspace; for a short sequence that is most of the time.  Here 1024 threads read the
// sequence's fp16 K and V once (lanes_per_token lanes per token, 32 channels per lane), keep the
// keys in registers and the values in LDS, and compute the same quantities in the same
// precision: exact integer moments, the window statistic as an exact double, the greedy cuts
// with the same tie rule, min/max folds (order-free once -0 is stored as +0), the same encoding
// steps and the same tile layout.  The results are bit-identical to the four-pass path.
constexpr int kShortThreads = 1024;
constexpr int kShortElems = 32768;   // longest sequence * head_dim: 256 tokens at 128, 512 at 64
template <int D>
constexpr int short_tokens() { return kShortElems / D; }

template <int D, int BS>
__global__ __launch_bounds__(kShortThreads) void compress_short_kernel(CompressArgs a) {
  constexpr int S = short_tokens<D>();
  constexpr int LPT = kShortThreads / S;   // lanes per token: 4 at head_dim 128, 2 at 64
  constexpr int PER = D / LPT;             // channels per lane
  static_assert(PER == 32, "each lane holds 32 channels of K and of V");
  constexpr int P = S / 64;                // candidates per lane of the selecting wave
  constexpr int MS = kMaxCuts + 1;
  static_assert(MS <= kShortThreads / 64 - 1, "one wave per segment plus one for the append state");
  const int h = blockIdx.x, b = blockIdx.y;
  int c0, L;
  bool bad_seq;
  seq_range(a.cu, b, a.max_seq_len, a.total, c0, L, bad_seq);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t bh = (size_t)b * a.hkv + h;
  dgq_tail_t *tl = a.cache.tail + bh;
  if (tid == 0 && bad_seq && h == 0) atomicAdd(a.cache.status + 2, 1ull);
  if (L == 0) {   // empty: no segments, empty append state
    if (tid < kWin) {
      tl->ring_a[tid] = 0;
      tl->ring_b[tid] = 0;
    }
    if (tid == 0) {
      a.cache.nseg[bh] = 0;
      tl->r0 = 0;
      tl->ring_len = 0;
      tl->span_own = 0;
      tl->window_done = 0;
    }
    return;
  }
  __shared__ __align__(16) uint32_t ct[S * D / 4];   // value codes, token-major (4 channels a word)
  __shared__ int ta[S];
  __shared__ long long tb[S];
  __shared__ float4 text[S];             // per-token K min, K max, V min, V max
  __shared__ int wa[S];                  // window sums over tokens [t, t + 16)
  __shared__ long long wb[S];
  __shared__ double scs[S];              // score of candidate cut t
  __shared__ float2 kprm[S], vprm[S];    // per-token segment (min, 1 / scale) of K and V
  __shared__ int segid[S];               // per-token segment index
  __shared__ int sstart[MS + 1];
  __shared__ int s_nseg;

  // ---- one read of the sequence: token t, channels [32 q, 32 q + 32) ----
  const int t = tid / LPT, q = tid % LPT;
  const bool valid = t < L;
  uint32_t kw[16], vw[16];
  float kmn = INFINITY, kmx = -INFINITY, vmn, vmx;
  bool bad;
  int asum = 0;
  long long bsum = 0;
  {
    uint4 kr[4], vr[4];
    const size_t row = (size_t)(c0 + (valid ? t : 0)) * a.stride_tok + (size_t)h * a.stride_head + PER * q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[i] = valid ? *reinterpret_cast<const uint4 *>(a.k + row + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
      vr[i] = valid ? *reinterpret_cast<const uint4 *>(a.v + row + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
    }
    const half2_t zero2 = {(_Float16)0.0f, (_Float16)0.0f};
    half2_t vmn2 = {(_Float16)INFINITY, (_Float16)INFINITY}, vmx2 = -vmn2, bad2 = zero2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ks[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
      const uint32_t vs[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
      int bpart = 0;   // sum of 8 squares <= 2^31: wraps as int32, exact read as uint32
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half2_t kx = as_half2(ks[e]), vx = as_half2(vs[e]);
        vmn2 = __builtin_elementwise_min(vmn2, vx);
        vmx2 = __builtin_elementwise_max(vmx2, vx);
        bad2 = __builtin_elementwise_fma(kx, zero2, bad2);   // NaN once any value is not finite
        bad2 = __builtin_elementwise_fma(vx, zero2, bad2);
        const float x0 = (float)kx[0], x1 = (float)kx[1];
        kmn = fminf(kmn, fminf(x0, x1));
        kmx = fmaxf(kmx, fmaxf(x0, x1));
        // the two fixed-point images as int16 halves of one word (|n| <= 2^14), then the sums of
        // n and n^2 by 16-bit dot products
        const uint32_t n01 = __builtin_amdgcn_perm((uint32_t)fixed_point_fma(x1), (uint32_t)fixed_point_fma(x0),
                                                   0x05040100u);
        const short2_t n2 = __builtin_bit_cast(short2_t, n01);
        asum = __builtin_amdgcn_sdot2(n2, kOnes2, asum, false);
        bpart = __builtin_amdgcn_sdot2(n2, n2, bpart, false);
      }
      bsum += (unsigned int)bpart;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kw[4 * i + e] = ks[e];
        vw[4 * i + e] = vs[e];
      }
    }
    vmn = fminf((float)vmn2[0], (float)vmn2[1]);
    vmx = fmaxf((float)vmx2[0], (float)vmx2[1]);
    bad = !(bad2[0] == (_Float16)0.0f && bad2[1] == (_Float16)0.0f);
  }
  // combine the LPT lanes of a token (adjacent lanes of one quad) with DPP quad swaps
  auto quad_combine = [&](auto tag) {
    constexpr int C = decltype(tag)::value;
    asum += dpp_i<C>(asum);
    bsum += (long long)(unsigned)dpp_i<C>((int)bsum) | ((long long)dpp_i<C>((int)(bsum >> 32)) << 32);
    kmn = fminf(kmn, dpp_f<C>(kmn));
    kmx = fmaxf(kmx, dpp_f<C>(kmx));
    vmn = fminf(vmn, dpp_f<C>(vmn));
    vmx = fmaxf(vmx, dpp_f<C>(vmx));
  };
  quad_combine(std::integral_constant<int, kQuadSwap1>{});
  if constexpr (LPT == 4) quad_combine(std::integral_constant<int, kQuadSwap2>{});
  if (q == 0) {
    ta[t] = valid ? asum : 0;
    tb[t] = valid ? bsum : 0;
    text[t] = make_float4(kmn, kmx, vmn, vmx);
  }
  {
    // one count per 16-token group that holds a non-finite value (a group is 16 * LPT lanes)
    const unsigned long long m = __ballot(bad);
    constexpr int GL = kWin * LPT;
    if (lane == 0) {
      unsigned int n = 0;
#pragma unroll
      for (int g = 0; g < 64 / GL; ++g) n += ((m >> (GL * g)) & ((GL == 64) ? ~0ull : ((1ull << GL) - 1))) != 0ull;
      if (n) atomicAdd(a.cache.status + 1, (unsigned long long)n);
    }
  }
  __syncthreads();

  // ---- window sums, then the score of every candidate cut (both windows inside the sequence) ----
  if (tid < S && tid + kWin <= L) {
    int A = 0;
    long long B = 0;
#pragma unroll
    for (int u = 0; u < kWin; ++u) {
      A += ta[tid + u];
      B += tb[tid + u];
    }
    wa[tid] = A;
    wb[tid] = B;
  }
  __syncthreads();
  if (tid < S) {
    double sc = -INFINITY;
    if (tid >= kWin && tid <= L - kWin) {
      // Q = N * sum b - (sum a)^2, exact in double (|sum a| <= 2^25, N * sum b <= 2^51)
      const double nel = (double)(kWin * D);
      const double Al = (double)wa[tid - kWin], Ar = (double)wa[tid];
      const double ql = fma(-Al, Al, nel * (double)wb[tid - kWin]);
      const double qr = fma(-Ar, Ar, nel * (double)wb[tid]);
      sc = fmax(ql, qr) < a.qfloor ? -INFINITY : (fmax(ql, qr) + 1.0) / (fmin(ql, qr) + 1.0);
    }
    scs[tid] = sc;
  }
  __syncthreads();

  // ---- greedy selection in wave 0 alone: lane l holds candidates P l .. P l + P - 1.  A score is
  // compared through its bit pattern as a 64-bit integer (scores are finite and >= 1, and positive
  // doubles order like their bit patterns; 0 = no candidate), so the wave maximum is an integer
  // reduction; among equal maxima the smallest t is the first lane's first one ----
  if (wave == 0) {
    unsigned long long key[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const double v = scs[P * lane + i];
      key[i] = v > -INFINITY ? (unsigned long long)__double_as_longlong(v) : 0ull;
    }
    int cut[kMaxCuts];
    int nc = 0;
    const int max_seg = a.length_aware ? min(a.max_segments, length_aware_cap(L)) : a.max_segments;
    if (L >= 2 * kWin) {
      for (int r = 0; r < max_seg - 1; ++r) {
        unsigned long long kb = 0ull;
        int ib = 0;
#pragma unroll
        for (int i = 0; i < P; ++i)
          if (key[i] > kb) {   // ascending t: the first maximum is the smallest t
            kb = key[i];
            ib = i;
          }
        const unsigned long long wm = wave_max_u64(kb);
        if (wm == 0ull) break;
        if (r > 0 && !(__longlong_as_double((long long)wm) >= a.tau)) break;
        const int wl = __builtin_ctzll(__ballot(kb == wm));
        const int tt = P * wl + __builtin_amdgcn_readlane(ib, wl);
        cut[nc++] = tt;
#pragma unroll
        for (int i = 0; i < P; ++i)
          if (abs(P * lane + i - tt) <= kWin - 1) key[i] = 0ull;
      }
    }
    // starts = [0] + sorted cuts, then L (the cuts are wave-uniform)
    for (int i = 1; i < nc; ++i) {
      const int x = cut[i];
      int k = i;
      while (k > 0 && cut[k - 1] > x) {
        cut[k] = cut[k - 1];
        --k;
      }
      cut[k] = x;
    }
    if (lane == 0) {
      sstart[0] = 0;
      for (int i = 0; i < nc; ++i) sstart[i + 1] = cut[i];
      sstart[nc + 1] = L;
      s_nseg = nc + 1;
    }
  }
  __syncthreads();
  const int nseg = s_nseg;

  // ---- segment j's K/V min/max in wave j, the segment row, and its tokens' parameters; the
  // append state in the last wave ----
  if (wave < nseg) {
    const int s0 = sstart[wave], s1 = sstart[wave + 1];
    float4 r = make_float4(INFINITY, -INFINITY, INFINITY, -INFINITY);
    for (int tok = s0 + lane; tok < s1; tok += 64) {
      const float4 x = text[tok];
      r.x = fminf(r.x, x.x);
      r.y = fmaxf(r.y, x.y);
      r.z = fminf(r.z, x.z);
      r.w = fmaxf(r.w, x.w);
    }
    r = wave_minmax(r);
    dgq_seg_t row;
    row.start = s0;
    row.kmin = r.x + 0.0f;
    row.kmax = r.y + 0.0f;
    row.vmin = r.z + 0.0f;
    row.vmax = r.w + 0.0f;
    row.kscale = dgq_scale(row.kmin, row.kmax, a.fmt.levels);
    row.vscale = dgq_scale(row.vmin, row.vmax, a.fmt.levels);
    row.reserved = 0;
    if (lane == 0) a.cache.segs[bh * a.seg_cap + wave] = row;
    const float2 kp = make_float2(row.kmin, dgq_inv(row.kmin, row.kmax, a.fmt.levels));
    const float2 vp = make_float2(row.vmin, dgq_inv(row.vmin, row.vmax, a.fmt.levels));
    for (int tok = s0 + lane; tok < s1; tok += 64) {
      kprm[tok] = kp;
      vprm[tok] = vp;
      segid[tok] = wave;
    }
  } else if (wave == kShortThreads / 64 - 1) {
    // append state: open span starts at L, ring = the last min(16, L) tokens' moments
    const int rl = min(kWin, L);
    if (lane < kWin) {
      tl->ring_a[lane] = lane < rl ? ta[L - rl + lane] : 0;
      tl->ring_b[lane] = lane < rl ? tb[L - rl + lane] : 0;
    }
    if (lane == 0) {
      a.cache.nseg[bh] = nseg;
      tl->r0 = L;
      tl->ring_len = rl;
      tl->span_own = 0;
      tl->window_done = 0;
    }
  }
  __syncthreads();

  const int32_t *bt = a.block_table + (size_t)b * a.max_blocks;
  const int nblk_seq = (L + BS - 1) / BS;
  const size_t tile_bytes = (size_t)BS * D;
  const bool marker = a.fmt.marker != 0;

  // ---- keys, from the registers: two 16-channel units of token t per lane; values, from the
  // registers into the token-major code array (zeros past L) ----
  {
    uint4 *dst = reinterpret_cast<uint4 *>(ct + (t * D + PER * q) / 4);
    if (valid) {
      const float2 vp = vprm[t];
      const float mn[4] = {vp.x, vp.x, vp.x, vp.x};
      const float inv[4] = {vp.y, vp.y, vp.y, vp.y};
      uint32_t cw[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const half2_t x01 = as_half2(vw[2 * g]), x23 = as_half2(vw[2 * g + 1]);
        const float x[4] = {(float)x01[0], (float)x01[1], (float)x23[0], (float)x23[1]};
        cw[g] = encode4(x, mn, inv, marker);
      }
      dst[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
      dst[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
    } else {
      dst[0] = make_uint4(0u, 0u, 0u, 0u);
      dst[1] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if (valid) {
    const float2 kp = kprm[t];
    const float mn[4] = {kp.x, kp.x, kp.x, kp.x};
    const float inv[4] = {kp.y, kp.y, kp.y, kp.y};
    const bool first = t > 0 && segid[t] != segid[t - 1];   // first token of a segment but the first
    bool bad_blk = false;
    const int blk = checked_block(bt[t / BS], a.cache.num_blocks, bad_blk);
#pragma unroll
    for (int hu = 0; hu < 2; ++hu) {
      const int d0 = PER * q + 16 * hu;
      uint32_t outw[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const half2_t x01 = as_half2(kw[8 * hu + 2 * g]), x23 = as_half2(kw[8 * hu + 2 * g + 1]);
        const float x[4] = {(float)x01[0], (float)x01[1], (float)x23[0], (float)x23[1]};
        outw[g] = encode4(x, mn, inv, marker);
      }
      if (marker && d0 == 0 && first) outw[0] = (outw[0] & ~0xFFu) | dgq_marker_byte(outw[0] & 0xFFu);
      if (bad_blk) {
        atomicAdd(a.cache.status + 2, 1ull);
        continue;
      }
      int8_t *dst = a.cache.k_pool + ((size_t)blk * a.hkv + h) * tile_bytes + k_tile_offset<D, BS>(t % BS, d0);
      store_stream(dst, outw);
    }
  }

  __syncthreads();

  // ---- values: one quad = 4 channels x the 16 tokens of a value unit; its four units are 64
  // contiguous bytes of a tile.  Word g of a unit holds 4 consecutive tokens (byte e = token
  // base_g + e), so each 4 x 4 byte block of the token-major codes is transposed with byte
  // permutes ----
  {
    constexpr int QD = D / 4;                          // channel quads per token row
    const int sets = nblk_seq * (BS / 16);             // 16-token sets of the sequence's blocks
    for (int qi = tid; qi < sets * QD; qi += kShortThreads) {
      const int set = qi / QD, c = qi % QD;
      const int lblk = set / (BS / 16);
      uint32_t out[4][4];                              // [channel j][word g]
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // BS 16 and 32: the set is the 16 tokens 16 set ..; word g = tokens 4 g ..; BS 64: the set
        // is (lblk, jj), word g = tokens 16 g + 4 jj ..
        const int base = BS == 64 ? 64 * lblk + 16 * g + 4 * (set % 4) : 16 * set + 4 * g;
        const uint32_t w0 = ct[(base + 0) * QD + c], w1 = ct[(base + 1) * QD + c];
        const uint32_t w2 = ct[(base + 2) * QD + c], w3 = ct[(base + 3) * QD + c];
        const uint32_t lo01 = __builtin_amdgcn_perm(w1, w0, 0x05010400u), hi01 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
        const uint32_t lo23 = __builtin_amdgcn_perm(w3, w2, 0x05010400u), hi23 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
        out[0][g] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
        out[1][g] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
        out[2][g] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
        out[3][g] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
      }
      bool bad_blk = false;
      const int blk = checked_block(bt[lblk], a.cache.num_blocks, bad_blk);
      if (bad_blk) continue;   // counted by the key loop
      int8_t *tilep = a.cache.v_pool + ((size_t)blk * a.hkv + h) * tile_bytes;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 4 * c + j;
        const int off = BS == 64 ? v_tile_offset<D, BS>(4 * (set % 4), d) : v_tile_offset<D, BS>((16 * set) % BS, d);
        store_stream(tilep + off, out[j]);
      }
    }
  }

  // ---- boundary bits: one byte per 8 tokens of every block of the sequence (bitmap format) ----
  if (!marker && tid < nblk_seq * (BS / 8)) {
    const int tok0 = 8 * tid;
    uint32_t byte = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = tok0 + i;
      if (tok > 0 && tok < L && segid[tok] != segid[tok - 1]) byte |= 1u << i;
    }
    bool bad_blk = false;
    const int blk = checked_block(bt[tok0 / BS], a.cache.num_blocks, bad_blk);
    if (!bad_blk) a.cache.bits[((size_t)blk * a.hkv + h) * (BS / 8) + (tok0 % BS) / 8] = (uint8_t)byte;
  }
}

CompressLayout compress_layout(const dgq_params_t *p, int32_t batch, int64_t total_tokens,
                               int32_t max_seq_len) {
  CompressLayout l;
  const size_t hkv = (size_t)p->num_kv_heads, tot = (size_t)(total_tokens > 0 ? total_tokens : 0);
  l.nsub = (max_seq_len + 15) / 16;
  if (l.nsub < 1) l.nsub = 1;
  l.ntile = (max_seq_len + 255) / 256;
  if (l.ntile < 1) l.ntile = 1;
  size_t off = 0;
  l.a_off = off;
  off = align_up(off + hkv * tot * sizeof(int32_t), 256);
  l.b_off = off;
  off = align_up(off + hkv * tot * sizeof(int64_t), 256);
  l.score_off = off;
  off = align_up(off + hkv * tot * sizeof(double), 256);
  l.ext_off = off;
  off = align_up(off + (size_t)batch * hkv * l.nsub * sizeof(float4), 256);
  l.tile_off = off;
  off = align_up(off + (size_t)batch * hkv * l.ntile * sizeof(double2), 256);
  l.text_off = off;
  off = align_up(off + (size_t)batch * hkv * l.ntile * sizeof(float4), 256);
  l.map_tiles = (int64_t)(tot + kChunk - 1) / kChunk + (batch > 0 ? batch : 0);
  l.map_off = off;
  off = align_up(off + (size_t)l.map_tiles * sizeof(int4), 256);
  l.total = off;
  return l;
}

template <int D>
static dgq_status_t launch_all(const CompressArgs &a, int bs, int max_seq_len, int64_t map_tiles, hipStream_t s) {
  const int batch = a.batch, hkv = a.hkv;
  // the passes over the fp16 input: one workgroup per (64-token tile, kv head) of the padded
  // batch, or of the real tiles (tile map) for a ragged batch
  const bool ragged = a.tile_map != nullptr;
  dim3 g64 = ragged ? dim3((unsigned)map_tiles, hkv, 1) : dim3((max_seq_len + 63) / 64, hkv, batch);
  dgq_status_t st;
  if (!a.multipass && max_seq_len <= short_tokens<D>()) {
    if (bs == 64) hipLaunchKernelGGL((compress_short_kernel<D, 64>), dim3(hkv, batch), dim3(kShortThreads), 0, s, a);
    else if (bs == 32) hipLaunchKernelGGL((compress_short_kernel<D, 32>), dim3(hkv, batch), dim3(kShortThreads), 0, s, a);
    else hipLaunchKernelGGL((compress_short_kernel<D, 16>), dim3(hkv, batch), dim3(kShortThreads), 0, s, a);
    return check_launch("dgq_compress one-launch kernel");
  }
  const bool small = max_seq_len <= kSmallSeq && a.max_segments <= kMaxCuts + 1;
  if (max_seq_len > 0) {
    if (ragged) {
      hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(kMapThreads), 0, s, a, (int)map_tiles);
      st = check_launch("dgq_compress tile map kernel");
      if (st != DGQ_OK) return st;
    }
    hipLaunchKernelGGL(stats_kernel<D>, g64, dim3(256), 0, s, a);
    st = check_launch("dgq_compress stats kernel");
    if (st != DGQ_OK) return st;
    if (!small) {
      const dim3 gs(((max_seq_len + 255) / 256 + kScoreTiles - 1) / kScoreTiles, hkv, batch);
      hipLaunchKernelGGL(scores_kernel<D>, gs, dim3(256), 0, s, a);
      st = check_launch("dgq_compress scores kernel");
      if (st != DGQ_OK) return st;
    }
  }
  if (small && max_seq_len <= kSmallSeq / 2 && small_cuts_ok(small_waves<kSmallSeq / 2>(), a.max_segments))
    hipLaunchKernelGGL((select_small_kernel<D, kSmallSeq / 2>), dim3(hkv, batch), dim3(kSmallSeq / 2 / kPerThread), 0, s, a);
  else if (small)
    hipLaunchKernelGGL((select_small_kernel<D, kSmallSeq>), dim3(hkv, batch), dim3(kSmallSeq / kPerThread), 0, s, a);
  else hipLaunchKernelGGL(select_kernel<D>, dim3(hkv, batch), dim3(kSelThreads), 0, s, a);
  st = check_launch("dgq_compress select kernel");
  if (st != DGQ_OK) return st;
  if (max_seq_len == 0) return DGQ_OK;
  if (bs == 64) hipLaunchKernelGGL((encode_kernel<D, 64>), g64, dim3(256), 0, s, a);
  else if (bs == 32) hipLaunchKernelGGL((encode_kernel<D, 32>), g64, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((encode_kernel<D, 16>), g64, dim3(256), 0, s, a);
  return check_launch("dgq_compress encode kernel");
}

dgq_status_t launch_compress(const dgq_params_t *p, const uint16_t *k, const uint16_t *v,
                             int64_t stride_tok, int64_t stride_head, const int32_t *cu_seqlens,
                             int32_t batch, int32_t max_seq_len, int64_t total_tokens,
                             const int32_t *block_table, int32_t max_blocks,
                             const dgq_cache_t *cache, void *ws, hipStream_t stream) {
  const CompressLayout l = compress_layout(p, batch, total_tokens, max_seq_len);
  char *w = reinterpret_cast<char *>(ws);
  CompressArgs a;
  a.k = k;
  a.v = v;
  a.stride_tok = stride_tok;
  a.stride_head = stride_head;
  a.cu = cu_seqlens;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.hkv = p->num_kv_heads;
  a.batch = batch;
  a.max_segments = p->max_segments;
  a.seg_cap = p->seg_capacity;
  a.nsub = l.nsub;
  a.ntile = l.ntile;
  a.max_seq_len = max_seq_len;
  a.total = total_tokens;
  a.tau = p->tau;
  a.qfloor = variance_floor_q(p->min_var, p->head_dim);
  a.length_aware = (p->flags & DGQ_POLICY_LENGTH_AWARE) != 0;
  a.multipass = (p->flags & DGQ_COMPRESS_MULTIPASS) != 0;
  a.fmt = code_format(p);
  a.ws_a = reinterpret_cast<int32_t *>(w + l.a_off);
  a.ws_b = reinterpret_cast<int64_t *>(w + l.b_off);
  a.ws_score = reinterpret_cast<double *>(w + l.score_off);
  a.ws_ext = reinterpret_cast<float4 *>(w + l.ext_off);
  a.ws_tile = reinterpret_cast<double2 *>(w + l.tile_off);
  a.ws_text = reinterpret_cast<float4 *>(w + l.text_off);
  const int64_t padded = (int64_t)((max_seq_len + 63) / 64) * batch;
  const bool ragged = batch <= kMapThreads && l.map_tiles <= INT_MAX && 5 * l.map_tiles < 4 * padded;
  a.tile_map = ragged ? reinterpret_cast<int4 *>(w + l.map_off) : nullptr;
  a.cache = *cache;
  if (p->head_dim == 128) return launch_all<128>(a, p->block_size, max_seq_len, l.map_tiles, stream);
  return launch_all<64>(a, p->block_size, max_seq_len, l.map_tiles, stream);
}

}  // namespace dgq
