// Device helpers shared by the libdspark kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11).  Ten rounds of the 4x64 S-box: the two even words are
// multiplied by the round multipliers, the 128-bit products' high halves are
// crossed over and mixed with the odd words and the round key, the low
// halves become the new odd words.  The key advances by the Weyl constants
// between rounds.
// ---------------------------------------------------------------------------
struct Philox4 {
  uint64_t w[4];
};

__device__ __forceinline__ Philox4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                                 uint64_t key0, uint64_t key1) {
  constexpr uint64_t kMulA = 0xD2E7470EE14C6C93ull;
  constexpr uint64_t kMulB = 0xCA5A826395121157ull;
  constexpr uint64_t kWeylA = 0x9E3779B97F4A7C15ull;
  constexpr uint64_t kWeylB = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t hiA = __umul64hi(kMulA, c0), loA = kMulA * c0;
    const uint64_t hiB = __umul64hi(kMulB, c2), loB = kMulB * c2;
    const uint64_t n0 = hiB ^ c1 ^ key0;
    const uint64_t n2 = hiA ^ c3 ^ key1;
    c0 = n0;
    c1 = loB;
    c2 = n2;
    c3 = loA;
    key0 += kWeylA;
    key1 += kWeylB;
  }
  Philox4 r;
  r.w[0] = c0;
  r.w[1] = c1;
  r.w[2] = c2;
  r.w[3] = c3;
  return r;
}

// Random stream ids of the counter layout (round, position, stream, index).
enum : uint64_t { kStreamDraft = 0, kStreamAccept = 1, kStreamResidual = 2, kStreamFallback = 3 };

__device__ __forceinline__ Philox4 draw_block(uint64_t seed, uint64_t round, uint64_t pos,
                                              uint64_t stream, uint64_t index) {
  return philox4x64_10(round, pos, stream, index, seed, 0);
}

// A 64-bit word to the double ((w >> 12) + 0.5) * 2^-52: exact, inside (0, 1).
__device__ __forceinline__ double unit_uniform(uint64_t w) {
  return ((double)(w >> 12) + 0.5) * 0x1p-52;
}

// ---------------------------------------------------------------------------
// Reductions.  Wave-wide ones use cross-lane shuffles; block-wide ones go
// through a small LDS array of one slot per wave.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Argmax pair: larger value wins, the lower index on equal values.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(i, o);
    argmax_merge(v, i, ov, oi);
  }
}

// Inclusive prefix sum across a wave (Hillis-Steele).
__device__ __forceinline__ double wave_inclusive_scan(double x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// ---------------------------------------------------------------------------
// Wave reductions and scans through DPP lane moves (VALU operations, a few
// cycles each) instead of LDS permutes (an LDS round trip each): the rows of
// 16 lanes first, then the four rows.  The orders of the additions differ
// from the shuffle versions above, so sums may differ in the last bits.
// ---------------------------------------------------------------------------
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppRowShr = 0x110;       // + n: row_shr:n
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
constexpr int kDppRowRor8 = 0x128;      // row_ror:8, lane i of a row reads lane i ^ 8

// src moved by a DPP pattern; lanes without a source (or outside kRowMask)
// read 0.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)src, kCtrl, kRowMask, 0xF, true);
}
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp_f32(float src) {
  return __uint_as_float(dpp_u32<kCtrl, kRowMask>(__float_as_uint(src)));
}
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ double dpp_f64(double src) {
  const uint64_t u = (uint64_t)__double_as_longlong(src);
  const uint32_t lo = dpp_u32<kCtrl, kRowMask>((uint32_t)u);
  const uint32_t hi = dpp_u32<kCtrl, kRowMask>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// The value of lane l (l wave-uniform).
__device__ __forceinline__ float lane_f32(float x, int l) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(x), l));
}
__device__ __forceinline__ double lane_f64(double x, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ int lane_i32(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// Maximum over the wave, returned to every lane.
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadSwap2>(x));
  x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  return fmaxf(fmaxf(lane_f32(x, 0), lane_f32(x, 16)), fmaxf(lane_f32(x, 32), lane_f32(x, 48)));
}

// Inclusive prefix sum across the wave: Hillis-Steele within each row of 16
// lanes, then row 1 (3) adds the total of row 0 (2), then rows 2 and 3 add
// the total of rows 0 and 1.
__device__ __forceinline__ double wave_inclusive_scan_dpp(double x) {
  x += dpp_f64<kDppRowShr + 1>(x);
  x += dpp_f64<kDppRowShr + 2>(x);
  x += dpp_f64<kDppRowShr + 4>(x);
  x += dpp_f64<kDppRowShr + 8>(x);
  x += dpp_f64<kDppRowBcast15, 0xA>(x);
  x += dpp_f64<kDppRowBcast31, 0xC>(x);
  return x;
}

// Block-wide helpers for blockDim.x == kBlock (a multiple of 64, <= 1024).
// `scratch` must hold kBlock / 64 elements; the functions synchronise.
template <int kBlock>
__device__ __forceinline__ float block_max(float x, float* scratch) {
  constexpr int kWaves = kBlock / kWave;
  x = wave_max(x);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = x;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, scratch[i]);
  __syncthreads();
  return r;
}

template <int kBlock, typename T>
__device__ __forceinline__ T block_sum(T x, T* scratch) {
  constexpr int kWaves = kBlock / kWave;
  x = wave_sum(x);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = x;
  __syncthreads();
  T r = scratch[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r += scratch[i];
  __syncthreads();
  return r;
}

template <int kBlock>
__device__ __forceinline__ void block_argmax(float& v, int& idx, float* sv, int* si) {
  constexpr int kWaves = kBlock / kWave;
  wave_argmax(v, idx);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sv[w] = v;
    si[w] = idx;
  }
  __syncthreads();
  v = sv[0];
  idx = si[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) argmax_merge(v, idx, sv[i], si[i]);
  __syncthreads();
}

// Exclusive block prefix sum in thread order; also returns the block total.
// `scratch` holds kBlock / 64 doubles.
template <int kBlock>
__device__ __forceinline__ double block_exclusive_scan(double x, double* scratch, double& total) {
  constexpr int kWaves = kBlock / kWave;
  const double incl = wave_inclusive_scan(x);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == kWave - 1) scratch[w] = incl;
  __syncthreads();
  double before = 0.0;
  total = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    if (i < w) before += scratch[i];
    total += scratch[i];
  }
  __syncthreads();
  return before + incl - x;
}

// bf16 bit pattern to float (exact).
// Nearest bf16 of a finite float (ties to even).
__device__ __forceinline__ uint16_t bf16_round(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// 2^x for the softmax terms: the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Merges of per-lane partial summaries and the transposing wave reduction
// built from them.
// ---------------------------------------------------------------------------
// (max, sum of 2^((x - max) cf)) pairs: merge (m, s) with (om, os).
struct MergeMS {
  float cf;
  __device__ __forceinline__ void operator()(float& m, float& s, float om, float os) const {
    const float M = fmaxf(m, om);
    const float lo = fminf(m, om);
    const float e = M == -__builtin_inff() ? 0.0f : fast_exp2((lo - M) * cf);
    const float sh = m >= om ? s : os;
    const float sl = m >= om ? os : s;
    s = sh + sl * e;
    m = M;
  }
};

// (value, index as float bits): larger value, lower index on ties.
struct MergeArgmax {
  __device__ __forceinline__ void operator()(float& v, float& ib, float ov, float oib) const {
    int i = __float_as_int(ib);
    argmax_merge(v, i, ov, __float_as_int(oib));
    ib = __int_as_float(i);
  }
};

struct MergeSum {
  __device__ __forceinline__ void operator()(float& v, float& u, float ov, float ou) const {
    v += ov;
    u += ou;
  }
};

// One exchange of the transposing reduction: with H = half the live count,
// a lane keeps elements [0, H) or [H, 2H) (by its bit `o`) merged with the
// partner's copy of the same elements.
template <int H, int N, class M>
__device__ __forceinline__ void xstep(float (&a)[N], float (&b)[N], int lane, int o, const M& merge) {
  static_assert(2 * H <= N, "live count");
  const bool hi = (lane & o) != 0;
#pragma unroll
  for (int j = 0; j < H; ++j) {
    float ka = hi ? a[j + H] : a[j], kb = hi ? b[j + H] : b[j];
    const float sa = hi ? a[j] : a[j + H], sb = hi ? b[j] : b[j + H];
    const float ra = __shfl_xor(sa, o), rb = __shfl_xor(sb, o);
    merge(ka, kb, ra, rb);
    a[j] = ka;
    b[j] = kb;
  }
}

// Lane exchanges of gfx950's v_permlane32_swap / v_permlane16_swap.  After
// swap32(x, y), lanes 0-31 of x keep x and lanes 32-63 of x hold y's lanes
// 0-31, while y holds x's lanes 32-63 in its lanes 0-31 and keeps its own
// lanes 32-63.  swap16 does the same between the odd 16-lane rows of x and
// the even rows of y.  In both, a lane's two results are its own value and
// the partner's (lane ^ 32, lane ^ 16): x's value in the lower lanes, y's in
// the upper ones.
__device__ __forceinline__ void swap32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// Transposing wave reduction of eight per-lane pairs (a[j], b[j]) under a
// commutative merge.  On return every lane holds in a[0], b[0] element
// 4 * bit5 + 2 * bit4 + bit3 of its lane index, merged over all 64 lanes.
// The exchanges are lane swaps and DPP moves: no LDS.
template <class M>
__device__ __forceinline__ void wave_transpose8(float (&a)[8], float (&b)[8], int lane, const M& merge) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // lanes l, l ^ 32: element j below, j + 4 above
    swap32(a[j], a[j + 4]);
    swap32(b[j], b[j + 4]);
    merge(a[j], b[j], a[j + 4], b[j + 4]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // lanes l, l ^ 16: element j or j + 2
    swap16(a[j], a[j + 2]);
    swap16(b[j], b[j + 2]);
    merge(a[j], b[j], a[j + 2], b[j + 2]);
  }
  {  // lanes l, l ^ 8: element 0 or 1
    const bool hi = (lane & 8) != 0;
    float ka = hi ? a[1] : a[0], kb = hi ? b[1] : b[0];
    const float sa = hi ? a[0] : a[1], sb = hi ? b[0] : b[1];
    merge(ka, kb, dpp_f32<kDppRowRor8>(sa), dpp_f32<kDppRowRor8>(sb));
    a[0] = ka;
    b[0] = kb;
  }
  // the eight lanes of each group: quad neighbours, then the other quad
  merge(a[0], b[0], dpp_f32<kDppQuadSwap1>(a[0]), dpp_f32<kDppQuadSwap1>(b[0]));
  merge(a[0], b[0], dpp_f32<kDppQuadSwap2>(a[0]), dpp_f32<kDppQuadSwap2>(b[0]));
  merge(a[0], b[0], dpp_f32<kDppRowHalfMirror>(a[0]), dpp_f32<kDppRowHalfMirror>(b[0]));
}

// The same reduction for eight per-lane sums: s[0] ends with the total of
// element 4 * bit5 + 2 * bit4 + bit3 of the lane index.
__device__ __forceinline__ void wave_transpose_sum8(float (&s)[8], int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    swap32(s[j], s[j + 4]);
    s[j] += s[j + 4];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    swap16(s[j], s[j + 2]);
    s[j] += s[j + 2];
  }
  const bool hi = (lane & 8) != 0;
  s[0] = (hi ? s[1] : s[0]) + dpp_f32<kDppRowRor8>(hi ? s[0] : s[1]);
  s[0] += dpp_f32<kDppQuadSwap1>(s[0]);
  s[0] += dpp_f32<kDppQuadSwap2>(s[0]);
  s[0] += dpp_f32<kDppRowHalfMirror>(s[0]);
}

}  // namespace dspark
