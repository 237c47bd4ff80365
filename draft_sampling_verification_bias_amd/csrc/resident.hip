// The device-resident block loop of dspark_markov_draft: all gamma positions
// of the left-to-right sampler of the DSpark technical review ("The
// Sequential Correction", Eq. 4, with the Markov head of "Instantiation 1:
// The Markov Head", Eq. 5; the decode-round pseudocode's draft loop) in ONE
// launch, with W2 held on chip for the whole call.
//
// One workgroup of eight waves per compute unit, all co-resident
// (cooperative launch).  All but kResSelWg of them are tile workgroups; the
// others are selector workgroups.
//
// Tile workgroups.  The vocabulary is cut into 16-column sub-blocks and every
// tile wave owns a contiguous range of at most five of them; the wave's slice
// of W2 -- its columns for all r = 256 rows, up to 40 KB -- is loaded once,
// from the vocabulary-major copy W2T, into MFMA operand registers (A
// fragments of v_mfma_f32_16x16x32_bf16: lane l holds column l % 16 of a
// sub-block, k = 8 (l / 16) .. + 7 of a 32-wide k step; 160 VGPRs) and stays
// there for all positions.  The loop runs over steps t = (position k,
// 16-row group g), position-major: E rows of the group (the W1 rows of the
// previous tokens, 8 KB, one DMA per wave) and each wave's U_k block (16
// rows x its columns, 5 KB) arrive in LDS by global -> LDS DMA, U three
// steps ahead and E two steps ahead; 40 MFMAs per wave form bias^T = W2^T E^T
// for the wave's columns (exact bf16 products, fp32 accumulation); the
// epilogue adds U and reduces each row of the wave's range to (max, sum of
// 2^((l - max) log2(e) / T)) plus one partial sum per sub-block (argmax at
// T = 0), written to LDS; at the next step the control wave (the one wave
// that issues no DMAs) copies the workgroup's summaries of the step to the
// global arrays.  Per position the only HBM stream is U_k.
//
// The rows are split into two halves (the first ceil(G / 2) groups and the
// rest).  A tile workgroup announces each finished half of a position on its
// flag once the copies of the half's last step are complete; the selector
// workgroups wait for all tile workgroups on a half, pick that half's tokens
// (one wave per request: float64 search over the row's range summaries
// grouped by tile workgroup, then over the chosen workgroup's eight ranges
// and the chosen range's sub-block sums, then a rescan of one 16-column
// sub-block with W2T rows -- the stream-0 inverse CDF) and write W1[x_k] as
// the request's next E row, then announce the half on their flags.  A tile
// workgroup checks those flags only before its first E DMA of a half of the
// next position, so the selections of one half run while the tiles stream
// the other half.
//
// Flags are words written with release semantics at agent scope and polled by
// one wave with acquire semantics; every wait is bounded in time, and a wait
// that times out sets an error word, the workgroup drains its DMAs and exits,
// and a follow-up kernel marks every request invalid (-1 / NaN), so no launch
// can hang.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace dspark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void res_lds_void;

constexpr int kResThreads = 512;
constexpr int kResWaves = kResThreads / kWave;      // 8: two per SIMD
constexpr int kResR = 256;                          // Markov rank of this path
constexpr int kResSub = 5;                          // 16-column sub-blocks per wave (at most)
constexpr int kResKSteps = kResR / 32;              // k steps of 32
constexpr int kResRows = 16;                        // rows per group
constexpr int kResStages = 3;                       // U blocks in flight per wave
constexpr int kResStageBytes = kResSub * 1024;      // one U block: 16 rows x 80 columns
constexpr int kResWaveU = kResStages * kResStageBytes;
constexpr int kResEBytes = kResKSteps * 1024;       // E rows of one group in fragment order
constexpr int kResESlots = 3;                       // E(t) is issued two steps ahead
constexpr int kResLdsE = kResWaves * kResWaveU;     // tile: 120 KB of U stages, then the E slots
constexpr int kResSelStage = 16 * 1024;             // selector: per wave, summaries then W2T rows
constexpr int kResSelReq = 4;                       // selector: requests per wave (two per half)
constexpr int kResLdsSelE = kResWaves * kResSelStage;  // selector: then their E rows
constexpr int kResLdsCtlU = 144 * 1024;              // tile: the fourth U stage of the control wave
constexpr int kResLdsMisc = kResLdsCtlU + kResStageBytes;  // the ok word
// tile: the workgroup's summaries of one step, two buffers: range summaries
// [16 rows][8 waves] float2, then sub-block sums [16 rows][kResWgSub] float
constexpr int kResPartBytes = kResRows * kResWaves * 8;
constexpr int kResSsumBytes = kResRows * kResWaves * kResSub * 4;
constexpr int kResLdsSum = kResLdsMisc + 64;
constexpr int kResLds = kResLdsSum + 2 * (kResPartBytes + kResSsumBytes);
constexpr int kResCtl = kResWaves - 1;              // tile: the control wave (no DMAs of its own)
constexpr int kResEHelper = kResSub;                // tile: issues the control wave's E chunk
static_assert(kResSub < kResCtl && kResEHelper < kResCtl, "helpers of the control wave");
constexpr int kResMaxWg = 256;
constexpr int kResSelWg = 16;                       // selector workgroups
constexpr int kResSelWaves = kResSelWg * kResWaves;
constexpr int kResMaxNW = kResWaves * kResMaxWg;    // range summaries per row (bound)
constexpr int kResSumPerLane = kResMaxNW / kWave;   // 32
constexpr int kResWgSub = kResWaves * kResSub;      // sub-block sums per row per workgroup (slots)
constexpr int kResErr = kResMaxWg;                  // index of the error word among the flags
constexpr int kResSelSteps = 7;                     // tile: a half's selections, in tile steps (measured best)

static_assert(kResLdsE + kResESlots * kResEBytes <= kResLdsCtlU, "tile LDS");
static_assert(kResLdsSelE + kResWaves * kResSelReq * 512 <= kResLdsMisc, "selector LDS");
static_assert(kResLds <= 160 * 1024, "LDS budget");

struct ResArgs {
  const float* U;
  const uint16_t* W1;
  const uint16_t* W2T;
  const int32_t* x0;
  const uint64_t* seeds;
  uint64_t round;
  int B, gamma, V, nsb;
  int nt;          // tile workgroups (the first nt of the grid)
  int NW;          // tile waves: 8 nt
  int G, G0;       // groups of 16 rows; the first half is groups [0, G0)
  float cf;        // log2(e) / T (0 at T == 0)
  double inv_t;    // 1 / T
  int32_t* tokens;
  float* prob;
  float* lse;
  float2* part;    // [G][nt][16][8]: range summaries; one workgroup writes 1 KB per group
  float* ssum;     // [G][nt][16][40]: sub-block sums (relative to the range maximum)
  uint16_t* eops;  // [B][256] W1 row of each request's previous token
  uint32_t* flags; // [nt] tile phases, [nt, nt + kResSelWg) selector phases; [kResErr] the error word
  long long timeout;  // ticks of the 100 MHz real-time counter
};

// ---------------------------------------------------------------------------
// Low-level helpers
// ---------------------------------------------------------------------------
// One 16-byte global -> LDS DMA per lane (lane l writes LDS [dst + 16 l, +16)).
// The compiler does not see it: callers order it with explicit vmcnt waits
// and barriers.
__device__ __forceinline__ void res_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// LDS address of the dynamic shared array (taken once per kernel).
__device__ __forceinline__ uint32_t res_lds_base(unsigned char* smem) {
  return __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)((res_lds_void*)smem));
}

template <int N>
__device__ __forceinline__ void res_wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void res_wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0) only

__device__ __forceinline__ long long res_clock() { return (long long)__builtin_amdgcn_s_memrealtime(); }

// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 that hold one
// row in the MFMA result layout, with the gfx950 row swaps (no LDS): after
// v_permlane16_swap (v, v) the two results hold, in every lane, the values
// of l and l ^ 16; after v_permlane32_swap those of l and l ^ 32.
__device__ __forceinline__ float res_max_rows(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float res_sum_rows(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// (value, column) argmax over the same four lanes: larger value, then lower
// column.  Both lanes of a pair merge the same two candidates.
__device__ __forceinline__ void res_argmax_rows(float& v, int& c) {
  auto rv = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  auto rc = __builtin_amdgcn_permlane16_swap((unsigned)c, (unsigned)c, false, false);
  v = __uint_as_float(rv[0]);
  c = (int)rc[0];
  argmax_merge(v, c, __uint_as_float(rv[1]), (int)rc[1]);
  rv = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  rc = __builtin_amdgcn_permlane32_swap((unsigned)c, (unsigned)c, false, false);
  v = __uint_as_float(rv[0]);
  c = (int)rc[0];
  argmax_merge(v, c, __uint_as_float(rv[1]), (int)rc[1]);
}

// Data that crosses workgroups (summaries, E rows) is written with
// agent-scope stores, which write through to the device's coherence point:
// once such a store has completed (vmcnt), every agent-scope reader that
// acquires afterwards sees it, without an L2 write-back.
__device__ __forceinline__ void res_put(float2* p, float2 v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                     ((unsigned long long)__float_as_uint(v.y) << 32) | __float_as_uint(v.x), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void res_put(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void res_put(uint2* p, uint2 v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), ((unsigned long long)v.y << 32) | v.x,
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Flag arrival: every store the flag publishes was made with res_put and has
// completed (the caller made sure of it, for every wave of the workgroup,
// before a workgroup barrier), so a plain agent-scope store of the phase
// suffices: no write-back of the L2 and no wait for this wave's DMAs.
__device__ __forceinline__ void res_arrive(uint32_t* flag, uint32_t phase) {
  __hip_atomic_store(flag, phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (one wave) until flags[0, n) all reach `phase` (n <= 256); false on
// the error word or on timeout (then the error word is set).  Acquire on
// success.
__device__ bool res_wait_flags(const uint32_t* flags, int n, uint32_t phase, uint32_t* err, long long timeout) {
  const int lane = threadIdx.x & (kWave - 1);
  const long long t0 = res_clock();
  for (;;) {
    // the flags and the error word in one batch of loads (one round trip)
    uint32_t f[kResMaxWg / kWave];
#pragma unroll
    for (int j = 0; j < kResMaxWg / kWave; ++j) {
      const int i = lane + j * kWave;
      f[j] = i < n ? __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0xffffffffu;
    }
    const uint32_t e = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t mn = 0xffffffffu;
#pragma unroll
    for (int j = 0; j < kResMaxWg / kWave; ++j) mn = f[j] < mn ? f[j] : mn;
    if (__ballot(mn < phase) == 0) break;
    if (e != 0u) return false;
    if (res_clock() - t0 > timeout) {
      if (lane == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

// ---------------------------------------------------------------------------
// Column ranges: tile wave gw (of NW) owns sub-blocks [sb0, sb0 + n) of
// the V / 16, n <= kResSub.
// ---------------------------------------------------------------------------
struct Range {
  int sb0, n;
};

// (gw + 1) nsb <= NW * 5 NW < 2^32: 32-bit unsigned arithmetic is exact
__device__ __forceinline__ Range res_range(const ResArgs& a, int gw) {
  Range r;
  r.sb0 = (int)((uint32_t)gw * (uint32_t)a.nsb / (uint32_t)a.NW);
  r.n = (int)((uint32_t)(gw + 1) * (uint32_t)a.nsb / (uint32_t)a.NW) - r.sb0;
  return r;
}

// U block of (position k, group g) for the wave owning range `rg`: kResSub
// DMAs, sub-block s from lane l: row 16 g + l % 16 (clamped to B - 1),
// columns 16 (sb0 + s) + 4 (l / 16) .. + 3 (sub-blocks past the range repeat
// the first one; their values are never used).
//
// With real == false the same number of DMAs is issued, every lane reading
// the first 16 bytes of U (one cache line): the wait counts of the group
// loop then do not depend on the group, and the stage receives values that
// are never read.
__device__ __forceinline__ void res_issue_u(const ResArgs& a, Range rg, int k, int g, uint32_t stage,
                                            bool real = true) {
  const int lane = threadIdx.x & (kWave - 1);
  int row = kResRows * g + (lane & 15);
  row = row < a.B ? row : a.B - 1;
  const int cbase = rg.n > 0 ? 16 * rg.sb0 : 0;
  const uint32_t rowoff = (uint32_t)row * (uint32_t)a.gamma * (uint32_t)a.V + (uint32_t)(k - 1) * (uint32_t)a.V;
#pragma unroll
  for (int s = 0; s < kResSub; ++s) {
    const int se = s < rg.n ? s : 0;
    const uint32_t off = real ? (rowoff + (uint32_t)(cbase + 16 * se + 4 * (lane >> 4))) * 4u : 0u;
    res_dma16(a.U, off, stage + (uint32_t)(s * 1024));
  }
}

// Sub-block s of the same U block (one DMA).
__device__ __forceinline__ void res_issue_u1(const ResArgs& a, Range rg, int k, int g, uint32_t stage, bool real,
                                             int s) {
  const int lane = threadIdx.x & (kWave - 1);
  int row = kResRows * g + (lane & 15);
  row = row < a.B ? row : a.B - 1;
  const int cbase = rg.n > 0 ? 16 * rg.sb0 : 0;
  const int se = s < rg.n ? s : 0;
  const uint32_t rowoff = (uint32_t)row * (uint32_t)a.gamma * (uint32_t)a.V + (uint32_t)(k - 1) * (uint32_t)a.V;
  const uint32_t off = real ? (rowoff + (uint32_t)(cbase + 16 * se + 4 * (lane >> 4))) * 4u : 0u;
  res_dma16(a.U, off, stage + (uint32_t)(s * 1024));
}

// E rows of group g (the previous tokens' W1 rows): k steps ks0 .. ks0 +
// nks - 1, from lane l row 16 g + l % 16, k = 32 ks + 8 (l / 16) .. + 7.
// real == false as for res_issue_u (the first 16 bytes of the E rows).
__device__ __forceinline__ void res_issue_e(const ResArgs& a, int g, uint32_t ebuf, bool real, int ks0, int nks) {
  const int lane = threadIdx.x & (kWave - 1);
  int row = kResRows * g + (lane & 15);
  row = row < a.B ? row : a.B - 1;
  for (int ks = ks0; ks < ks0 + nks; ++ks) {
    const uint32_t off = real ? ((uint32_t)row * kResR + 32u * ks + 8u * (lane >> 4)) * 2u : 0u;
    res_dma16(a.eops, off, ebuf + (uint32_t)(ks * 1024));
  }
}

// ---------------------------------------------------------------------------
// Selection of one request's token at position k by one selector wave.
// `erow` is the request's current E row (W1[x_{k-1}], 512 B of LDS), which
// the call replaces with W1[x_k]; `stage` (16 KB of LDS) receives the row's
// range summaries and then the rescan's W2T rows.
// ---------------------------------------------------------------------------
template <bool kGreedy>
__device__ void res_select(const ResArgs& a, int b, int k, int& prev, unsigned char* erow, const unsigned char* stage,
                           uint32_t stage_lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nwg = a.nt;
  const size_t out = (size_t)b * a.gamma + (k - 1);
  if (prev < 0) {  // invalid anchor or earlier position
    if (lane == 0) {
      a.tokens[out] = -1;
      a.prob[out] = __builtin_nanf("");
      a.lse[out] = __builtin_nanf("");
    }
    return;
  }
  const uint32_t g = (uint32_t)b >> 4, n = (uint32_t)b & 15u;
  // The row's NW = 8 nt range summaries into the stage: the 64 bytes of tile
  // workgroup w (its eight ranges) sit at part[g][w][n][0..7]; DMA i gathers
  // workgroups 16 i .. 16 i + 15, four lanes each, so workgroup w lands at
  // byte 64 w and lane l's workgroups 4 l .. 4 l + 3 at [256 l, 256 l + 256).
  for (int i = 0; i < (nwg + 15) / 16; ++i) {
    uint32_t w = (uint32_t)(16 * i) + ((uint32_t)lane >> 2);
    w = w < (uint32_t)nwg ? w : 0u;
    const uint32_t off = (((g * (uint32_t)nwg + w) * 16u + n) * 8u) * 8u + 16u * ((uint32_t)lane & 3u);
    res_dma16(a.part, off, stage_lds + (uint32_t)(1024 * i));
  }
  res_wait_vmem<0>();
  // Chunk c (16 bytes: two ranges) of lane l is read at step (c - l) mod 16:
  // the 16 lanes of each quarter-wave then hit 16 different bank groups.
  // Workgroups past nt read as (-inf, no column / 0).
  constexpr int kWgPerLane = kResMaxWg / kWave;
  const float4* lane_chunks = reinterpret_cast<const float4*>(stage) + 16 * lane;
  auto chunk = [&](int step, int& c) -> float4 {
    c = (step + lane) & 15;
    const float4 q = lane_chunks[c];
    const bool live = kWgPerLane * lane + (c >> 2) < nwg;
    const float dead = kGreedy ? __int_as_float(0x7fffffff) : 0.0f;
    return live ? q : make_float4(-__builtin_inff(), dead, -__builtin_inff(), dead);
  };
  int x;
  if constexpr (kGreedy) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll 4
    for (int st = 0; st < 16; ++st) {
      int c;
      const float4 q = chunk(st, c);
      argmax_merge(bv, bi, q.x, __float_as_int(q.y));
      argmax_merge(bv, bi, q.z, __float_as_int(q.w));
    }
    wave_argmax(bv, bi);
    x = bi;
    if (lane == 0) {
      a.tokens[out] = x;
      a.prob[out] = 1.0f;
      a.lse[out] = 0.0f;
    }
  } else {
    float lm = -__builtin_inff();
#pragma unroll 4
    for (int st = 0; st < 16; ++st) {
      int c;
      const float4 q = chunk(st, c);
      lm = fmaxf(lm, fmaxf(q.x, q.z));
    }
    const float M = wave_max_dpp(lm);
    auto weight = [&](float mj, float sj) -> double {
      return mj != -__builtin_inff() ? (double)sj * (double)fast_exp2((mj - M) * a.cf) : 0.0;
    };
    // level 1: the weight of each of the lane's four workgroups (the sum of
    // its eight range weights)
    double wwg[kWgPerLane] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int st = 0; st < 16; ++st) {
      int c;
      const float4 q = chunk(st, c);
      const double w2 = weight(q.x, q.y) + weight(q.z, q.w);
#pragma unroll
      for (int qq = 0; qq < kWgPerLane; ++qq) wwg[qq] += (c >> 2) == qq ? w2 : 0.0;
    }
    double local = 0.0;
#pragma unroll
    for (int c = 0; c < kWgPerLane; ++c) local += wwg[c];
    const double incl = wave_inclusive_scan_dpp(local);
    const double total = lane_f64(incl, kWave - 1);
    const double u = unit_uniform(draw_block(a.seeds[b], a.round, (uint64_t)k, kStreamDraft, 0).w[0]);
    const double q = u * total;
    const unsigned long long cross = __ballot(local > 0.0 && incl > q);
    const unsigned long long pos = __ballot(local > 0.0);
    const int owner = cross ? __ffsll((long long)cross) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
    // the workgroup: first positive weight whose inclusive sum exceeds q,
    // else the last positive one (every lane finds its candidate, the
    // owner's is taken)
    int wsel = -1, lastc = -1;
    double base = 0.0, lastbase = 0.0;
    {
      double cum = incl - local;
#pragma unroll
      for (int c = 0; c < kWgPerLane; ++c) {
        const bool posw = wwg[c] > 0.0;
        const bool hit = posw && wsel < 0 && cum + wwg[c] > q;
        lastc = posw ? c : lastc;
        lastbase = posw ? cum : lastbase;
        wsel = hit ? c : wsel;
        base = hit ? cum : base;
        cum += wwg[c];
      }
      const bool none = wsel < 0;
      wsel = kWgPerLane * lane + (none ? (lastc < 0 ? 0 : lastc) : wsel);
      base = none ? (lastc < 0 ? 0.0 : lastbase) : base;
    }
    wsel = lane_i32(wsel, owner);
    base = lane_f64(base, owner);
    // level 2: that workgroup's eight ranges (lanes 0-7, from the stage), in
    // vocabulary order
    const float2 pv = lane < kResWaves ? reinterpret_cast<const float2*>(stage)[kResWaves * wsel + lane]
                                       : make_float2(-__builtin_inff(), 0.0f);
    const double wr = lane < kResWaves ? weight(pv.x, pv.y) : 0.0;
    const double rincl = wave_inclusive_scan_dpp(wr);
    const double qr = q - base;
    const unsigned long long rcross = __ballot(wr > 0.0 && rincl > qr);
    const unsigned long long rpos = __ballot(wr > 0.0);
    const int rj = rcross ? __ffsll((long long)rcross) - 1 : (rpos ? 63 - __clzll((long long)rpos) : 0);
    base += lane_f64(rincl - wr, rj);
    const int ri = kResWaves * wsel + rj;
    const float mi = lane_f32(pv.x, rj);
    const double scale = (double)fast_exp2((mi - M) * a.cf);
    const size_t wrow = ((size_t)g * nwg + wsel) * 16 + n;
    const float sv = lane < kResWgSub ? a.ssum[wrow * kResWgSub + lane] : 0.0f;
    // the sub-block of the range (its sums are relative to mi), from the
    // slots already loaded
    const Range rg = res_range(a, ri);
    const int loc = rg.sb0 - res_range(a, wsel * kResWaves).sb0;
    const float sbl = __shfl(sv, (loc + lane) & (kWave - 1));
    const float sbv = lane < rg.n ? sbl : 0.0f;
    const double wb = lane < rg.n ? (double)sbv * scale : 0.0;
    const double bincl = wave_inclusive_scan_dpp(wb);
    const double q1 = q - base;
    const unsigned long long bcross = __ballot(wb > 0.0 && bincl > q1);
    const unsigned long long bpos = __ballot(wb > 0.0);
    const int bj = bcross ? __ffsll((long long)bcross) - 1 : (bpos ? 63 - __clzll((long long)bpos) : 0);
    const double base1 = lane_f64(bincl - wb, bj);
    const int c0 = 16 * (rg.sb0 + bj);
    res_wait_lgkm0();  // every LDS read of the summaries is done before the stage is overwritten
    // Rescan of sub-block bj: the logits U + W1[x_{k-1}] . W2[:, c] of its 16
    // columns.  Its W2T rows (16 x 512 B) arrive in the stage (DMA i: columns
    // 2 i, 2 i + 1); lane l owns column l % 16 and the 64-wide k quarter
    // l / 16 (16-byte chunks read in a rotated order against bank conflicts).
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = ((uint32_t)(c0 + 2 * i + (lane >> 5)) * kResR + 8u * (lane & 31)) * 2u;
      res_dma16(a.W2T, off, stage_lds + (uint32_t)(i * 1024));
    }
    const int cl = lane & 15, qk = lane >> 4;
    const float uval = a.U[((size_t)b * a.gamma + (k - 1)) * a.V + c0 + cl];
    res_wait_vmem<0>();
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ch = 8 * qk + ((i + cl) & 7);  // 16-byte chunk of the 512-byte row
      const uint4 wv = *reinterpret_cast<const uint4*>(stage + cl * 512 + ch * 16);
      const uint4 ev = *reinterpret_cast<const uint4*>(erow + ch * 16);
      const uint32_t we[4] = {wv.x, wv.y, wv.z, wv.w};
      const uint32_t ee[4] = {ev.x, ev.y, ev.z, ev.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc = fmaf(__uint_as_float(ee[t] << 16), __uint_as_float(we[t] << 16), acc);
        acc = fmaf(__uint_as_float(ee[t] & 0xffff0000u), __uint_as_float(we[t] & 0xffff0000u), acc);
      }
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    const float l = uval + acc;
    const bool lv = lane < 16 && l != -__builtin_inff();
    const double wc = lv ? (double)fast_exp2((l - mi) * a.cf) * scale : 0.0;
    const double cincl = wave_inclusive_scan_dpp(wc);
    const double q2 = q1 - base1;
    const unsigned long long ccross = __ballot(wc > 0.0 && cincl > q2);
    const unsigned long long cpos = __ballot(wc > 0.0);
    const int cj = ccross ? __ffsll((long long)ccross) - 1 : (cpos ? 63 - __clzll((long long)cpos) : 0);
    x = c0 + cj;
    const float lx = lane_f32(l, cj);
    if (lane == 0) {
      a.tokens[out] = x;
      a.prob[out] = (float)((double)fast_exp2((lx - M) * a.cf) / total);
      // hardware log2 (about 1 ulp of log2(total)): the double library log
      // would hold its polynomial constants in registers across the kernel
      a.lse[out] = (float)((double)M * a.inv_t + 0.6931471805599453 * (double)__builtin_amdgcn_logf((float)total));
    }
  }
  if ((unsigned)x >= (unsigned)a.V) {  // only an all -inf row (outside the preconditions) gets here
    if (lane == 0) {
      a.tokens[out] = -1;
      a.prob[out] = __builtin_nanf("");
      a.lse[out] = __builtin_nanf("");
    }
    prev = -1;
    return;
  }
  prev = x;
  // W1[x] is the next position's E row: in the shared array for the tile
  // workgroups and in this wave's LDS for its own next rescan
  if (k < a.gamma) {
    const uint2 v = reinterpret_cast<const uint2*>(a.W1 + (size_t)x * kResR)[lane];
    res_put(reinterpret_cast<uint2*>(a.eops + (size_t)b * kResR) + lane, v);
    res_wait_lgkm0();  // the rescan's reads of the old row are done
    reinterpret_cast<uint2*>(erow)[lane] = v;
  }
}

// ---------------------------------------------------------------------------
// Tile workgroups
// ---------------------------------------------------------------------------
// Phase of half h of position k on the flags: tile workgroups set it when
// their summaries of the half are written; selector workgroups set 2 k + h + 1
// when the half's tokens are chosen and its E rows for position k + 1 written
// (2 after writing the E rows of position 1).  E rows of half h of position k
// are ready once every selector flag is >= res_phase(k, h).
__device__ __forceinline__ uint32_t res_phase(int k, int h) { return (uint32_t)(2 * (k - 1) + h + 1); }

template <bool kGreedy>
__device__ void res_tile(const ResArgs& a, unsigned char* smem) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wg = blockIdx.x, nt = a.nt;
  const int gw = wg * kResWaves + wave;
  const Range my = res_range(a, gw);
  const int cbase = my.n > 0 ? 16 * my.sb0 : 0;
  const int myloc = my.sb0 - res_range(a, wg * kResWaves).sb0;  // first sub-block slot of the wave in its workgroup
  const uint32_t lds = res_lds_base(smem);
  const uint32_t ebufs_l = lds + (uint32_t)kResLdsE;
  const unsigned char* ebufs = smem + kResLdsE;
  // The control wave (7) issues no DMAs: its polls and releases then wait for
  // nothing but its own stores.  Waves 0-4 issue one sub-block each of its U
  // blocks, into four stages (they cannot see when the control wave has read
  // a stage, so the stage they refill is the one of the step before, which
  // the workgroup barrier has retired), and wave 5 its E chunk.
  const bool ctl = wave == kResCtl;
  const Range ctl_rg = res_range(a, wg * kResWaves + kResCtl);
  const int nstage = ctl ? 4 : kResStages;
  auto stage_off = [&](int w, int st) -> int {
    return (w == kResCtl && st == kResStages) ? kResLdsCtlU : w * kResWaveU + st * kResStageBytes;
  };
  auto ustage_of = [&](int t) -> const unsigned char* { return smem + stage_off(wave, t % nstage); };
  auto ctl_stage_l = [&](int t) -> uint32_t { return lds + (uint32_t)stage_off(kResCtl, t % 4); };
  volatile int* ok_flag = reinterpret_cast<volatile int*>(smem + kResLdsMisc);
  uint32_t* err = a.flags + kResErr;
  const uint32_t* sel_flags = a.flags + nt;
  // the summaries of step t: written to LDS by every wave, copied to the
  // global arrays by the control wave at the next step (whole 512-byte runs
  // per store instruction, the other waves' vector-memory queues holding
  // only their DMAs)
  auto spart = [&](int t) { return reinterpret_cast<float2*>(smem + kResLdsSum + (t & 1) * kResPartBytes); };
  auto sssum = [&](int t) {
    return reinterpret_cast<float*>(smem + kResLdsSum + 2 * kResPartBytes + (t & 1) * kResSsumBytes);
  };
  const int G = a.G, G0 = a.G0, T = a.gamma * G;
  const int n16 = lane & 15, q4 = lane >> 4;

  auto pos_of = [&](int t) { return t / G + 1; };
  auto grp_of = [&](int t) { return t % G; };
  auto half_of = [&](int g) { return g < G0 ? 0 : 1; };
  // the last step of the half whose selections the E rows of step t need
  // (-1 for position 1: its E rows are written before any step)
  auto dep_of = [&](int t) {
    const int k = pos_of(t), g = grp_of(t);
    if (k == 1) return -1;
    return (k - 2) * G + (half_of(g) == 0 ? G0 - 1 : G - 1);
  };
  // E(t) is issued at step t - 2 (or depends on no selection) if the
  // selections it depends on are expected to be finished by then: announced
  // at the step after the half's last step, they take up to kResSelSteps
  // steps (the lead that measured fastest from B = 32 to 256).  Otherwise it
  // is issued at step t itself, which exposes one E load instead of stalling
  // the workgroup two steps early.
  const int e_lead = 3 + kResSelSteps;
  auto e_early = [&](int t) { return pos_of(t) == 1 || dep_of(t) <= t - e_lead; };
  auto half_end = [&](int t) { const int g = grp_of(t); return g == G0 - 1 || g == G - 1; };
  // the flag phase of the half that ends at step t
  auto end_phase = [&](int t) { return res_phase(pos_of(t), grp_of(t) == G - 1 ? 1 : 0); };
  uint32_t released = 0;   // tile phase already announced by this workgroup (uniform)
  uint32_t confirmed = 0;  // selector phase already observed by this workgroup (uniform)
  auto release = [&](uint32_t phase) {
    if (phase <= released) return;
    released = phase;
    if (ctl && lane == 0) res_arrive(a.flags + wg, phase);
  };
  // The control wave copies step tc's summaries to the global arrays.  The
  // copies are the only vector-memory operations of the control wave apart
  // from its polls (which it waits for itself), so its vmcnt counts them.
  auto flush = [&](int tc) {
    if (!ctl) return;
    const size_t blk = (size_t)grp_of(tc) * nt + wg;
    const uint2* sp = reinterpret_cast<const uint2*>(spart(tc));
    uint2* gp = reinterpret_cast<uint2*>(a.part) + blk * (kResPartBytes / 8);
#pragma unroll
    for (int i = 0; i < kResPartBytes / 512; ++i) res_put(gp + 64 * i + lane, sp[64 * i + lane]);
    if constexpr (!kGreedy) {
      const uint2* ss = reinterpret_cast<const uint2*>(sssum(tc));
      uint2* gs = reinterpret_cast<uint2*>(a.ssum) + blk * (kResSsumBytes / 8);
#pragma unroll
      for (int i = 0; i < kResSsumBytes / 512; ++i) res_put(gs + 64 * i + lane, ss[64 * i + lane]);
    }
  };
  // The control wave waits for the E rows of step t (the ok word reports a
  // failed wait; true if it polled).  The selectors need this workgroup's
  // announcement of the half that those rows depend on, which the top of
  // each step makes as soon as the half's copies are complete; should it be
  // missing, it is made here (every step up to now - 1 has been copied).
  auto check = [&](int t, int now) -> bool {
    const uint32_t need = res_phase(pos_of(t), half_of(grp_of(t)));
    if (need <= confirmed) return false;
    confirmed = need;
    // this workgroup's phase for that half of the previous position (none
    // at position 1, whose E rows the selectors write before any step)
    if (need > 2 && released < need - 2) {
      if (ctl) res_wait_vmem<0>();
      int last = now - 1;
      while (last > 0 && !half_end(last)) --last;
      release(end_phase(last));
    }
    if (ctl) {
      const bool ok = res_wait_flags(sel_flags, kResSelWg, need, err, a.timeout);
      if (lane == 0) *ok_flag = ok ? 1 : 0;
    }
    return true;
  };
  auto e_slot = [&](int t) -> uint32_t { return ebufs_l + (uint32_t)((t % kResESlots) * kResEBytes); };
  auto issue_e = [&](int t, bool real) {
    if (!ctl) res_issue_e(a, grp_of(t), e_slot(t), real, wave, 1);
    if (wave == kResEHelper) res_issue_e(a, grp_of(t), e_slot(t), real, kResCtl, 1);
  };
  // U of step t (real or not) for this wave and, from waves 0-4, one
  // sub-block each for the control wave
  auto issue_u = [&](int t, uint32_t own_stage) {
    const bool real = t < T;
    const int tt = real ? t : 0;
    if (!ctl) res_issue_u(a, my, pos_of(tt), grp_of(tt), own_stage, real);
    if (wave < kResSub) res_issue_u1(a, ctl_rg, pos_of(tt), grp_of(tt), ctl_stage_l(t), real, wave);
  };

  if (threadIdx.x == 0) *ok_flag = 1;
  // U of steps 0..2 stream in while W2 is loaded
  for (int t = 0; t < kResStages; ++t) issue_u(t, lds + (uint32_t)stage_off(wave, t));

  // the wave's slice of W2 as MFMA A fragments, for the whole call
  bf16x8 wf[kResSub][kResKSteps];
#pragma unroll
  for (int s = 0; s < kResSub; ++s) {
    const int se = s < my.n ? s : 0;
    const uint16_t* src = a.W2T + (size_t)(cbase + 16 * se + (lane & 15)) * kResR + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < kResKSteps; ++ks) wf[s][ks] = *reinterpret_cast<const bf16x8*>(src + 32 * ks);
  }

  // E of steps 0 and 1
  check(0, 0);
  if (T > 1 && e_early(1)) check(1, 0);
  __syncthreads();
  if (!*ok_flag) {
    res_wait_vmem<0>();
    return;
  }
  issue_e(0, true);
  issue_e(1, T > 1 && e_early(1));

  for (int t = 0; t < T; ++t) {
    // E(t) and the U blocks of step t this wave issued have landed.  Issue
    // order per step: e E DMAs at its start (E(t + 2), real or not), then u
    // U DMAs (U of step t + 3, real or not), with (e, u) = (1, 6) for waves
    // 0-4, (2, 5) for wave 5 and (1, 5) for wave 6; so after E(t) come e at
    // t = 0, e + u at t = 1 and 2 u + e at t >= 2.  U(t) is issued before
    // E(t).  An E issued late (at its own step) is waited for there, and
    // drains only make these counts safer.  The control wave issues no DMAs.
    __builtin_amdgcn_sched_barrier(0);
    if (ctl) {
    } else if (wave < kResSub) {
      if (t == 0) {
        res_wait_vmem<1>();
      } else if (t == 1) {
        res_wait_vmem<kResSub + 2>();
      } else {
        res_wait_vmem<2 * kResSub + 3>();
      }
    } else if (wave == kResEHelper) {
      if (t == 0) {
        res_wait_vmem<2>();
      } else if (t == 1) {
        res_wait_vmem<kResSub + 2>();
      } else {
        res_wait_vmem<2 * kResSub + 2>();
      }
    } else {
      if (t == 0) {
        res_wait_vmem<1>();
      } else if (t == 1) {
        res_wait_vmem<kResSub + 1>();
      } else {
        res_wait_vmem<2 * kResSub + 1>();
      }
    }
    // every wave's summaries of step t - 1 are in LDS
    __syncthreads();
    if (t >= 1) flush(t - 1);
    // A half is announced as soon as the control wave's copies of its last
    // step are complete (the control wave waits for them here; the other
    // waves meet it at the next barrier), so that its selections start one
    // step after its last tile step.
    if (t >= 1 && half_end(t - 1) && released < end_phase(t - 1)) {
      if (ctl) res_wait_vmem<0>();
      release(end_phase(t - 1));
    }
    const bool late = !e_early(t);
    bool polled = false;
    if (late) polled = check(t, t);
    if (t + 2 < T && e_early(t + 2)) polled = check(t + 2, t) || polled;
    if (polled) {
      __syncthreads();
      if (!*ok_flag) {
        res_wait_vmem<0>();
        return;
      }
    }
    if (late) {
      issue_e(t, true);
      if (!ctl) res_wait_vmem<0>();
      __syncthreads();
    }
    issue_e(t + 2, t + 2 < T && e_early(t + 2));

    // bias^T of the wave's columns for the group's 16 rows
    f32x4 acc[kResSub];
    {
      const unsigned char* ebuf = ebufs + (t % kResESlots) * kResEBytes;
      bf16x8 ev[kResKSteps];
#pragma unroll
      for (int ks = 0; ks < kResKSteps; ++ks) ev[ks] = *reinterpret_cast<const bf16x8*>(ebuf + ks * 1024 + 16 * lane);
#pragma unroll
      for (int s = 0; s < kResSub; ++s) acc[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < kResKSteps; ++ks) {
#pragma unroll
        for (int s = 0; s < kResSub; ++s)
          acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[s][ks], ev[ks], acc[s], 0, 0, 0);
      }
      // schedule: the eight LDS reads, then the MFMAs five at a time (left
      // alone, the scheduler re-reads one fragment per k step to save
      // registers)
      __builtin_amdgcn_sched_group_barrier(0x100, kResKSteps, 0);
#pragma unroll
      for (int ks = 0; ks < kResKSteps; ++ks) __builtin_amdgcn_sched_group_barrier(0x008, kResSub, 0);
    }

    // epilogue: acc[s][i] + U is the logit of row 16 g + l % 16, column
    // 16 (sb0 + s) + 4 (l / 16) + i (U added to the finished bias, not
    // accumulated through it: the float32 rounding then stays at the bias's
    // magnitude, as in the selection's rescan).  Sub-blocks past the range
    // repeat sub-block 0 (same columns, same values): they leave maxima
    // unchanged and are dropped from sums.
    {
      const unsigned char* ub = ustage_of(t);
#pragma unroll
      for (int s = 0; s < kResSub; ++s) {
        const float4 u = *reinterpret_cast<const float4*>(ub + s * 1024 + 16 * lane);
        acc[s][0] += u.x;
        acc[s][1] += u.y;
        acc[s][2] += u.z;
        acc[s][3] += u.w;
      }
      res_wait_lgkm0();
      // U of step t + 3 into the stage just read (waves 0-4 also refill the
      // control wave's stage of step t - 1)
      issue_u(t + kResStages, lds + (uint32_t)stage_off(wave, t % nstage));
    }
    if constexpr (kGreedy) {
      float bv = -__builtin_inff();
      int bc = 0x7fffffff;
#pragma unroll
      for (int s = 0; s < kResSub; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // ascending columns within the lane and strict comparison: the
          // lowest index wins ties, and a repeated sub-block never wins
          const bool better = acc[s][i] > bv;
          bv = better ? acc[s][i] : bv;
          bc = better ? cbase + 16 * s + 4 * q4 + i : bc;
        }
      }
      res_argmax_rows(bv, bc);
      if (my.n == 0) bv = -__builtin_inff(), bc = 0x7fffffff;
      if (lane < 16) spart(t)[n16 * kResWaves + wave] = make_float2(bv, __int_as_float(bc));
    } else {
      float m = -__builtin_inff();
#pragma unroll
      for (int s = 0; s < kResSub; ++s) m = fmaxf(m, fmaxf(fmaxf(acc[s][0], acc[s][1]), fmaxf(acc[s][2], acc[s][3])));
      m = res_max_rows(m);  // the row's maximum over the four lanes that hold it
      // with m = -inf every logit is -inf and every term 2^-inf = 0
      const float mc = m == -__builtin_inff() ? 0.0f : m * a.cf;
      float bp[kResSub];
#pragma unroll
      for (int s = 0; s < kResSub; ++s) {
        const float v = (fast_exp2(fmaf(acc[s][0], a.cf, -mc)) + fast_exp2(fmaf(acc[s][1], a.cf, -mc))) +
                        (fast_exp2(fmaf(acc[s][2], a.cf, -mc)) + fast_exp2(fmaf(acc[s][3], a.cf, -mc)));
        bp[s] = res_sum_rows(s < my.n ? v : 0.0f);
      }
      const float S = (((bp[0] + bp[1]) + bp[2]) + bp[3]) + bp[4];
      if (lane < 16) spart(t)[n16 * kResWaves + wave] = make_float2(my.n > 0 ? m : -__builtin_inff(), S);
      const float bq = q4 == 0 ? bp[0] : q4 == 1 ? bp[1] : q4 == 2 ? bp[2] : bp[3];
      float* ss = sssum(t) + n16 * kResWgSub + myloc;
      if (q4 < my.n) ss[q4] = bq;
      if (q4 == 0 && my.n > 4) ss[4] = bp[4];
    }

  }
  // the last step's summaries, then the halves not announced yet
  __syncthreads();
  flush(T - 1);
  res_wait_vmem<0>();
  release(res_phase(a.gamma, 1));
}

// ---------------------------------------------------------------------------
// Selector workgroups
// ---------------------------------------------------------------------------
// Selector wave sw (of kResSelWaves) owns, in half h, the requests
// R_h + sw + i kResSelWaves (i = 0, 1) below R_{h + 1}, with R_0 = 0,
// R_1 = min(B, 16 G0), R_2 = B; when both halves hold at most
// kResSelWaves / 2 requests, the one request R_h + sw - h kResSelWaves / 2
// instead (waves of the other half own none).
template <bool kGreedy>
__device__ void res_selector(const ResArgs& a, unsigned char* smem) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;

  const uint32_t lds = res_lds_base(smem);
  unsigned char* stage = smem + wave * kResSelStage;
  const uint32_t stage_l = lds + (uint32_t)(wave * kResSelStage);
  volatile int* ok_flag = reinterpret_cast<volatile int*>(smem + kResLdsMisc);
  uint32_t* err = a.flags + kResErr;
  uint32_t* my_flag = a.flags + a.nt + (blockIdx.x - a.nt);
  const int R1 = a.B < kResRows * a.G0 ? a.B : kResRows * a.G0;
  // Halves of at most kResSelWaves / 2 requests each (B <= 128) go to
  // disjoint waves, one request per wave: the selections of one half then
  // never queue behind those of the other, which matters when a half is only
  // a step or two of tile work.  Larger halves use every wave, up to two
  // requests per wave.
  constexpr int kHalfWaves = kResSelWaves / 2;
  const bool split = R1 <= kHalfWaves && a.B - R1 <= kHalfWaves;
  // Selector wave number: with split halves, wave-major, so that consecutive
  // requests land on different workgroups (each selection DMAs 15 KB of
  // summaries, and the selections of a short half are the critical path);
  // otherwise workgroup-major, so that a workgroup's waves take neighbouring
  // rows, whose summaries share cache lines.
  const int wgi = (int)blockIdx.x - a.nt;
  const int sw = split ? wave * kResSelWg + wgi : wgi * kResWaves + wave;
  auto req = [&](int h, int i) {
    return split ? (h == 0 ? 0 : R1) + sw - h * kHalfWaves : (h == 0 ? 0 : R1) + sw + i * kResSelWaves;
  };
  auto live = [&](int h, int i) {
    if (split && (i != 0 || sw < h * kHalfWaves)) return false;
    return req(h, i) < (h == 0 ? R1 : a.B);
  };
  auto erow = [&](int h, int i) { return smem + kResLdsSelE + (wave * kResSelReq + 2 * h + i) * 512; };

  // E rows of position 1: W1[x_0] (zero rows for invalid anchors)
  int prev[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      prev[h][i] = -1;
      if (live(h, i)) {
        const int b = req(h, i);
        const int x0 = a.x0[b];
        prev[h][i] = (unsigned)x0 < (unsigned)a.V ? x0 : -1;
        uint2 v = make_uint2(0u, 0u);
        if (prev[h][i] >= 0) v = reinterpret_cast<const uint2*>(a.W1 + (size_t)prev[h][i] * kResR)[lane];
        res_put(reinterpret_cast<uint2*>(a.eops + (size_t)b * kResR) + lane, v);
        reinterpret_cast<uint2*>(erow(h, i))[lane] = v;
      }
    }
  }
  res_wait_vmem<0>();
  __syncthreads();
  if (threadIdx.x == 0) res_arrive(my_flag, 2u);

  for (int k = 1; k <= a.gamma; ++k) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (wave == 0) {
        const bool ok = res_wait_flags(a.flags, a.nt, res_phase(k, h), err, a.timeout);
        if (lane == 0) *ok_flag = ok ? 1 : 0;
      }
      __syncthreads();
      if (!*ok_flag) {
        res_wait_vmem<0>();
        return;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (live(h, i)) res_select<kGreedy>(a, req(h, i), k, prev[h][i], erow(h, i), stage, stage_l);
      res_wait_vmem<0>();
      __syncthreads();
      if (threadIdx.x == 0) res_arrive(my_flag, (uint32_t)(2 * k + h + 1));
    }
  }
}

template <bool kGreedy>
__global__ __launch_bounds__(kResThreads, 1) void draft_resident_kernel(ResArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  if ((int)blockIdx.x < a.nt)
    res_tile<kGreedy>(a, smem);
  else
    res_selector<kGreedy>(a, smem);
}

// Outputs of every request become invalid (-1 / NaN) when the resident loop
// reported a failed wait.
__global__ void resident_fixup_kernel(const uint32_t* err, int32_t* tokens, float* prob, float* lse, int n) {
  if (*err == 0u) return;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    tokens[i] = -1;
    prob[i] = __builtin_nanf("");
    lse[i] = __builtin_nanf("");
  }
}

__global__ void resident_clear_kernel(uint32_t* flags, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) flags[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct ResLayout {
  size_t part, ssum, eops, flags, total;
};

static ResLayout res_layout(int B) {
  ResLayout l;
  const size_t rows = (size_t)(B + kResRows - 1) / kResRows * kResRows;  // whole groups
  l.part = 0;
  l.ssum = align256(rows * kResMaxNW * sizeof(float2));
  l.eops = l.ssum + align256(rows * kResMaxWg * kResWgSub * sizeof(float));
  l.flags = l.eops + align256((size_t)B * kResR * sizeof(uint16_t));
  l.total = l.flags + align256((size_t)(kResMaxWg + 1) * sizeof(uint32_t));
  return l;
}

size_t resident_workspace(int B, int gamma, int V, int r) {
  (void)gamma;
  if (r != kResR || V % 16 != 0) return 0;
  return res_layout(B).total;
}

template <bool kGreedy>
static hipError_t res_prepare(int& max_blocks) {
  static hipError_t state = hipErrorNotReady;
  static int blocks = 0;
  if (state == hipErrorNotReady) {
    state = hipFuncSetAttribute((const void*)draft_resident_kernel<kGreedy>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kResLds);
    if (state == hipSuccess)
      state = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, (const void*)draft_resident_kernel<kGreedy>,
                                                           kResThreads, kResLds);
  }
  max_blocks = blocks;
  return state;
}

bool resident_draft_applies(const DraftArgs& a, bool bf16) {
  if (!bf16 || a.W2T == nullptr || a.r != kResR || a.V % 16 != 0) return false;
  if (a.conf != nullptr) return false;  // the confidence head runs in the per-position selections
  const int nwg = compute_units_of_device();
  if (nwg > kResMaxWg || nwg <= kResSelWg) return false;
  const long long NW = (long long)(nwg - kResSelWg) * kResWaves;
  const long long nsb = a.V / 16;
  if ((nsb + NW - 1) / NW > kResSub) return false;                     // W2 slice fits the registers
  if ((long long)a.B > 2LL * 2 * kResSelWaves) return false;           // two requests per selector wave per half
  if ((double)a.B * a.gamma * a.V * 4.0 >= 4294967296.0) return false;  // 32-bit DMA offsets
  return true;
}

// Launches the resident loop; *launched is false (and nothing was enqueued)
// when the device cannot hold the grid, so the caller can use the per-position
// launches instead.
hipError_t launch_resident_draft(const DraftArgs& d, hipStream_t s, bool* launched) {
  *launched = false;
  const bool greedy = d.temperature == 0.0f;
  int maxb = 0;
  hipError_t e = greedy ? res_prepare<true>(maxb) : res_prepare<false>(maxb);
  if (e != hipSuccess || maxb < 1) return hipSuccess;
  const int nwg = compute_units_of_device();
  const ResLayout L = res_layout(d.B);
  char* ws = reinterpret_cast<char*>(d.ws);
  ResArgs a = {};
  a.U = d.U;
  a.W1 = reinterpret_cast<const uint16_t*>(d.W1);
  a.W2T = reinterpret_cast<const uint16_t*>(d.W2T);
  a.x0 = d.x0;
  a.seeds = d.seeds;
  a.round = d.round;
  a.B = d.B;
  a.gamma = d.gamma;
  a.V = d.V;
  a.nsb = d.V / 16;
  a.nt = nwg - kResSelWg;
  a.NW = a.nt * kResWaves;
  a.G = (d.B + kResRows - 1) / kResRows;
  a.G0 = (a.G + 1) / 2;
  a.cf = greedy ? 0.0f : (float)(1.4426950408889634 / (double)d.temperature);
  a.inv_t = greedy ? 0.0 : 1.0 / (double)d.temperature;
  a.tokens = d.tokens;
  a.prob = d.prob;
  a.lse = d.lse;
  a.part = reinterpret_cast<float2*>(ws + L.part);
  a.ssum = reinterpret_cast<float*>(ws + L.ssum);
  a.eops = reinterpret_cast<uint16_t*>(ws + L.eops);
  a.flags = reinterpret_cast<uint32_t*>(ws + L.flags);
  a.timeout = 20000000;  // 0.2 s at 100 MHz: orders of magnitude above a normal wait
  hipLaunchKernelGGL(resident_clear_kernel, dim3(1), dim3(256), 0, s, a.flags, kResMaxWg + 1);
  void* args[] = {&a};
  {
    ProfScope prof(s, kProfResidentDraft);  // the resident kernel alone
    e = hipLaunchCooperativeKernel(greedy ? (const void*)draft_resident_kernel<true>
                                          : (const void*)draft_resident_kernel<false>,
                                   dim3(nwg), dim3(kResThreads), args, kResLds, s);
    if (e != hipSuccess) prof.discard();
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hipSuccess;  // not launched: the caller falls back (the clear kernel is harmless)
  }
  *launched = true;
  const int n = d.B * d.gamma;
  hipLaunchKernelGGL(resident_fixup_kernel, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), dim3(256), 0, s,
                     a.flags + kResErr, d.tokens, d.prob, d.lse, n);
  return hipGetLastError();
}

}  // namespace dspark
