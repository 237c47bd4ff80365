// dspark_markov_draft: the left-to-right block sampler of the DSpark technical
// review, "The Sequential Correction" (Eq. 4) with the Markov head of
// "Instantiation 1: The Markov Head" (Eq. 5).
//
// Each block position k is one tile pass (bias MFMA + U stream + per-tile
// softmax summaries for all B requests) followed by one selection kernel
// (one workgroup per request) that normalises over the tile summaries in
// float64, draws the stream-0 uniform, finds the tile holding the draw and
// rescans that one tile.  The drafted token is written straight into the
// output array, where the next position's tile pass reads it as x_{k-1}.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace dspark {

constexpr int kSelThreads = 256;
constexpr int kCachedTiles = 4096;   // tile summaries kept in LDS up to V = 524288
constexpr int kPerThread = 8;        // summaries loaded per thread before the first use

struct SelectArgs {
  const float* U;
  const void* W1;
  const void* W2;
  const int32_t* x0;
  const uint64_t* seeds;
  uint64_t round;
  const float2* partials;
  int B, gamma, V, r, ntiles, k;  // k is 1-based
  float cf;
  double inv_t;
  int32_t* tokens;
  float* prob;
  float* lse;
  double* u_next;  // [2][B] stream-0 uniforms drawn one position ahead
  uint4* esw;      // optional: the drafted token's W1 row for the next tile pass
  // optional confidence head (conf != null), see conf_hidden below
  const float* ch;
  const float* cw;
  const float* csts;
  int cd;
  float* conf;
};

// Store W1 row x (bf16, r = 256) in the ring tile pass's operand layout for
// request row b; thread c < 32 copies chunk c.
template <bool kBf16>
__device__ __forceinline__ void store_ring_operand(const SelectArgs& a, int b, int x, int c) {
  if constexpr (kBf16) {
    if (a.esw != nullptr && c < 32 && (unsigned)x < (unsigned)a.V) {
      const uint4 v = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.W1) + (size_t)x * 256)[c];
      a.esw[ring_operand_index(b, c)] = v;
    }
  }
}

template <bool kBf16>
__device__ __forceinline__ float w2_at(const void* W2, size_t idx) {
  if constexpr (kBf16) {
    return bf16_to_float(reinterpret_cast<const uint16_t*>(W2)[idx]);
  } else {
    return reinterpret_cast<const float*>(W2)[idx];
  }
}

template <bool kBf16>
__device__ __forceinline__ float w1_at(const void* W1, size_t idx) {
  if constexpr (kBf16) {
    return bf16_to_float(reinterpret_cast<const uint16_t*>(W1)[idx]);
  } else {
    return reinterpret_cast<const float*>(W1)[idx];
  }
}

// Element j of W1 row `row`.  kParts == 1: a token's row.  kParts == 2: W1 is
// a table of operand rows (row b * gamma + k - 1) of two parts of r values,
// summed.
template <bool kBf16, int kParts>
__device__ __forceinline__ float opnd_at(const SelectArgs& a, int row, int j) {
  const size_t base = (size_t)row * kParts * a.r + j;
  float v = w1_at<kBf16>(a.W1, base);
  if constexpr (kParts == 2) v += w1_at<kBf16>(a.W1, base + a.r);
  return v;
}

// ---------------------------------------------------------------------------
// The confidence head of "The Confidence Head" (Eq. 7) with the per-position
// temperatures of Sequential Temperature Scaling (same section), fused into
// the selection:
//   c_{b,kk} = sigma((w_h . h_{b,kk} + w_e . W1[x_{kk-1}]) / t_kk).
// The selection of position k draws x_k and reads its W1 row for the next
// position's operand, so it emits c_{k+1}; the first selection also emits
// c_1 from the anchor.  The hidden part depends on no drafted token, so its
// loads go out at the start of the selection.  The float32 products are
// exact in float64 and summed there.  A position whose previous token is
// outside [0, V) gets NaN.
// ---------------------------------------------------------------------------

// This thread's share of w_h . h_{b,kk} (elements tid, tid + nthr, ...).
__device__ __forceinline__ double conf_hidden(const SelectArgs& a, int b, int kk, int tid, int nthr) {
  const float* hrow = a.ch + ((size_t)b * a.gamma + (kk - 1)) * a.cd;
  double s = 0.0;
  if ((a.cd & 3) == 0) {  // rows 16-byte aligned
    for (int i = 4 * tid; i < a.cd; i += 4 * nthr) {
      const float4 x = *reinterpret_cast<const float4*>(hrow + i);
      const float4 y = *reinterpret_cast<const float4*>(a.cw + i);
      s += (double)x.x * (double)y.x + (double)x.y * (double)y.y + (double)x.z * (double)y.z +
           (double)x.w * (double)y.w;
    }
  } else {
    for (int i = tid; i < a.cd; i += nthr) s += (double)hrow[i] * (double)a.cw[i];
  }
  return s;
}

// This thread's share of w_e . W1[x] for a token x in [0, V).
template <bool kBf16>
__device__ __forceinline__ double conf_embed(const SelectArgs& a, int x, int tid, int nthr) {
  double s = 0.0;
  for (int j = tid; j < a.r; j += nthr) s += (double)w1_at<kBf16>(a.W1, (size_t)x * a.r + j) * (double)a.cw[a.cd + j];
  return s;
}

__device__ __forceinline__ void conf_store(const SelectArgs& a, int b, int kk, double z) {
  const double t = a.csts ? (double)a.csts[kk - 1] : 1.0;
  a.conf[(size_t)b * a.gamma + (kk - 1)] = (float)(1.0 / (1.0 + exp(-z / t)));
}

// Invalid previous token at position k (x_{k-1} outside [0, V)): x_k is not
// drawn, so c_{k+1} (and at k == 1, c_1) are NaN.
__device__ __forceinline__ void conf_invalid(const SelectArgs& a, int b) {
  if (a.conf == nullptr) return;
  if (a.k < a.gamma) a.conf[(size_t)b * a.gamma + a.k] = __builtin_nanf("");
  if (a.k == 1) a.conf[(size_t)b * a.gamma] = __builtin_nanf("");
}

template <bool kGreedy, bool kBf16, int kParts = 1>
__global__ __launch_bounds__(kSelThreads) void draft_select_kernel(SelectArgs a) {
  __shared__ PickScratch ps;
  __shared__ float sw1[512];
  __shared__ float2 spart[kCachedTiles];
  __shared__ float sbias[8][kTileCols];
  __shared__ float sl[kTileCols];
  __shared__ double sterm[kTileCols];
  __shared__ float sv[kSelThreads / kWave];
  __shared__ int si[kSelThreads / kWave];
  __shared__ double sred[kSelThreads / kWave];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t out = (size_t)b * a.gamma + (a.k - 1);
  // The tile summaries are loaded up front (all loads of a thread in flight
  // together) while the previous token is fetched.
  const float2* P = a.partials + (size_t)b * a.ntiles;
  float2 pr[kPerThread];
  if constexpr (!kGreedy) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int t = tid + j * kSelThreads;
      pr[j] = t < a.ntiles ? P[t] : make_float2(-__builtin_inff(), 0.0f);
    }
  }
  const int ptok = a.k == 1 ? a.x0[b] : a.tokens[(size_t)b * a.gamma + a.k - 2];
  const int prev = kParts > 1 ? b * a.gamma + a.k - 1 : ptok;  // the W1 row
  if (ptok < 0 || ptok >= a.V) {  // invalid anchor or earlier position: propagate
    if (tid == 0) {
      a.tokens[out] = -1;
      a.prob[out] = __builtin_nanf("");
      a.lse[out] = __builtin_nanf("");
      conf_invalid(a, b);
    }
    return;
  }
  // confidence head: this thread's shares of the hidden part of c_{k+1} and
  // of the whole logit of c_1
  double c_next = 0.0, c_first = 0.0;
  if (a.conf != nullptr) {
    if (a.k < a.gamma) c_next = conf_hidden(a, b, a.k + 1, tid, kSelThreads);
    if (a.k == 1) c_first = conf_hidden(a, b, 1, tid, kSelThreads) + conf_embed<kBf16>(a, ptok, tid, kSelThreads);
  }
  // emits the confidences once x_k is known (every thread holds it)
  auto emit_conf = [&](int x) {
    if (a.conf == nullptr) return;
    if (a.k == 1) {
      const double z1 = block_sum<kSelThreads, double>(c_first, sred);
      if (tid == 0) conf_store(a, b, 1, z1);
    }
    if (a.k < a.gamma) {
      const double z = block_sum<kSelThreads, double>(c_next + conf_embed<kBf16>(a, x, tid, kSelThreads), sred);
      if (tid == 0) conf_store(a, b, a.k + 1, z);
    }
  };

  if constexpr (kGreedy) {
    float bv = -__builtin_inff();
    int bi = INT_MAX;
    for (int t = tid; t < a.ntiles; t += kSelThreads) {
      const float2 p = P[t];
      argmax_merge(bv, bi, p.x, __float_as_int(p.y));
    }
    block_argmax<kSelThreads>(bv, bi, sv, si);
    if (tid == 0) {
      a.tokens[out] = bi;
      a.prob[out] = 1.0f;
      a.lse[out] = 0.0f;
    }
    store_ring_operand<kBf16>(a, b, bi, tid);
    emit_conf(bi);
    return;
  } else {
    // One read of the tile summaries (kept in LDS when they fit) together
    // with the W1 row of the previous token.
    const bool cached = a.ntiles <= kCachedTiles;
    float w1v[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = tid + q * kSelThreads;
      const float v = opnd_at<kBf16, kParts>(a, prev, j < a.r ? j : 0);  // clamped: no branch
      w1v[q] = j < a.r ? v : 0.0f;
    }
    float lm = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int t = tid + j * kSelThreads;
      if (t < a.ntiles) {
        if (cached) spart[t] = pr[j];
        lm = fmaxf(lm, pr[j].x);
      }
    }
    for (int t = tid + kPerThread * kSelThreads; t < a.ntiles; t += kSelThreads) {
      const float2 p = P[t];
      if (cached) spart[t] = p;
      lm = fmaxf(lm, p.x);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = tid + q * kSelThreads;
      if (j < a.r) sw1[j] = w1v[q];
    }
    const float M = block_max<kSelThreads>(lm, sv);
    const double cf = (double)a.cf;
    auto weight_of = [&](float2 p) -> double {
      return p.x == -__builtin_inff() ? 0.0 : (double)p.y * (double)fast_exp2((p.x - M) * a.cf);
    };
    const double u = unit_uniform(draw_block(a.seeds[b], a.round, a.k, kStreamDraft, 0).w[0]);
    double total = 0.0, base = 0.0;
    int ts;
    if (cached) {
      ts = block_pick_uniform<kSelThreads>(a.ntiles, [&](int t) { return weight_of(spart[t]); }, u, ps, &base,
                                           &total);
    } else {
      ts = block_pick_uniform<kSelThreads>(a.ntiles, [&](int t) { return weight_of(P[t]); }, u, ps, &base, &total);
    }
    if (ts < 0) ts = 0;
    const double q = u * total;
    const float mt = cached ? spart[ts].x : P[ts].x;
    const double scale = exp2((double)(mt - M) * cf);

    // Rescan tile ts: rebuild its 128 logits.  Thread t owns columns
    // 4 (t % 32) .. +3 and one of 8 slices of the r products; each thread keeps
    // its whole slice of W2 loads in flight, then the slices are summed in LDS
    // in a fixed order.
    {
      const int quad = tid & 31, slice = tid >> 5;
      const int kslice = a.r / 8;                 // r % 16 == 0, so kslice is even
      const int c = ts * kTileCols + 4 * quad;
      const bool vec = kBf16 && (c + 4 <= a.V) && ((a.V & 3) == 0);
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      const int jend = (slice + 1) * kslice;
      // Loads use clamped indices so that every load of a chunk is issued
      // before the first use; out-of-range terms are zeroed afterwards.
      for (int j0 = slice * kslice; j0 < jend; j0 += 32) {
        float w[32][4];
        if (vec) {
#pragma unroll
          for (int jj = 0; jj < 32; ++jj) {
            const int j = min(j0 + jj, jend - 1);
            const uint2 p = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.W2) + (size_t)j * a.V + c);
            w[jj][0] = __uint_as_float(p.x << 16);
            w[jj][1] = __uint_as_float(p.x & 0xffff0000u);
            w[jj][2] = __uint_as_float(p.y << 16);
            w[jj][3] = __uint_as_float(p.y & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < 32; ++jj) {
            const int j = min(j0 + jj, jend - 1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int cc = c + q < a.V ? c + q : a.V - 1;
              const float v = w2_at<kBf16>(a.W2, (size_t)j * a.V + cc);
              w[jj][q] = c + q < a.V ? v : 0.0f;
            }
          }
        }
#pragma unroll
        for (int jj = 0; jj < 32; ++jj) {
          const float e = (j0 + jj < jend) ? sw1[j0 + jj] : 0.0f;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] = fmaf(e, w[jj][q], acc[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) sbias[slice][4 * quad + q] = acc[q];
    }
    __syncthreads();
    if (tid < kTileCols) {
      const int v = ts * kTileCols + tid;
      float bias = 0.0f;
#pragma unroll
      for (int g = 0; g < 8; ++g) bias += sbias[g][tid];
      float l = -__builtin_inff();
      if (v < a.V) l = a.U[((size_t)b * a.gamma + (a.k - 1)) * a.V + v] + bias;
      const float e = l == -__builtin_inff() ? 0.0f : fast_exp2((l - mt) * a.cf);
      sl[tid] = l;
      sterm[tid] = (double)e * scale;
    }
    __syncthreads();
    auto col_weight = [&](int c) -> double { return sterm[c]; };
    int c = block_pick_target<kSelThreads>(kTileCols, col_weight, q - base, ps, nullptr);
    if (c < 0) c = 0;
    if (tid == 0) {
      const float l = sl[c];
      a.tokens[out] = ts * kTileCols + c;
      a.prob[out] = (float)(exp2((double)(l - M) * cf) / total);
      a.lse[out] = (float)((double)M * a.inv_t + log(total));
    }
    store_ring_operand<kBf16>(a, b, ts * kTileCols + c, tid);
    emit_conf(ts * kTileCols + c);
  }
}

// ---------------------------------------------------------------------------
// Sampling select for rows of at most kWaveTiles tile summaries: the same draw
// as draft_select_kernel with wave-level searches and one barrier.
//
// Every wave runs the tile search on its own (lane l owns the contiguous
// summaries [l cs, l cs + cs)), so the search needs only cross-lane shuffles.
// The rescan of the picked tile is split by k over the four waves: a lane
// owns 8 columns and every fourth k of its wave's quarter, with all of its
// W2 loads (and the W1 and U values it needs) issued together.  The quarters
// meet in LDS and wave 0 draws the column.
// ---------------------------------------------------------------------------
// The stream-0 uniform of position k, out of line: the draw is needed only
// at the first position (later ones read the look-ahead value), and inline
// the compiler evaluates it on every position to select the result.
__device__ __noinline__ double draft_uniform(uint64_t seed, uint64_t round, int k) {
  return unit_uniform(draw_block(seed, round, k, kStreamDraft, 0).w[0]);
}

constexpr int kWaveTiles = 2048;                 // up to V = 262144
constexpr int kMaxRQuarter = 512 / 4;             // k per wave (r <= 512)

// kWavePer: summaries per lane, the smallest instantiated count that covers
// the row (the searches are unrolled over it, and they sit on the critical
// path of every position).
template <bool kBf16, int kWavePer, int kParts = 1>
__global__ __launch_bounds__(kSelThreads) void draft_select_wave_kernel(SelectArgs a) {
  __shared__ float sbias[4][kTileCols];
  __shared__ double sconf[2][4];  // per wave: hidden part of c_{k+1}, logit of c_1
  const int b = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const size_t out = (size_t)b * a.gamma + (a.k - 1);
  const int nt = a.ntiles;
  const int cs = (nt + kWave - 1) / kWave;
  const int t0 = min(nt, lane * cs);
  const int t1 = min(nt, t0 + cs);
  const float2* P = a.partials + (size_t)b * nt;

  // batch 1: this lane's summaries (clamped indices, all loads in flight),
  // the previous token, the key
  float2 pr[kWavePer];
#pragma unroll
  for (int j = 0; j < kWavePer; ++j) {
    const int t = t0 + j;
    pr[j] = P[t < t1 ? t : (t1 > 0 ? t1 - 1 : 0)];
  }
  const int ptok = a.k == 1 ? a.x0[b] : a.tokens[(size_t)b * a.gamma + a.k - 2];
  const int prev = kParts > 1 ? b * a.gamma + a.k - 1 : ptok;  // the W1 row
  const uint64_t seed = a.seeds[b];
  const double u_pre = a.k == 1 ? 0.0 : a.u_next[(size_t)((a.k - 1) & 1) * a.B + b];
  if (ptok < 0 || ptok >= a.V) {  // invalid anchor or earlier position: propagate
    if (threadIdx.x == 0) {
      a.tokens[out] = -1;
      a.prob[out] = __builtin_nanf("");
      a.lse[out] = __builtin_nanf("");
      conf_invalid(a, b);
    }
    return;
  }
  // confidence head: this thread's shares of the hidden part of c_{k+1} and
  // of the whole logit of c_1 (summed over the waves before the barrier)
  double c_next = 0.0, c_first = 0.0;
  if (a.conf != nullptr) {
    if (a.k < a.gamma) c_next = conf_hidden(a, b, a.k + 1, threadIdx.x, kSelThreads);
    if (a.k == 1)
      c_first = conf_hidden(a, b, 1, threadIdx.x, kSelThreads) + conf_embed<kBf16>(a, ptok, threadIdx.x, kSelThreads);
  }

  // row max, tile weights, their lane prefix, the picked tile
  // (selects rather than branches: every lane runs every j)
  float lm = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kWavePer; ++j) lm = t0 + j < t1 ? fmaxf(lm, pr[j].x) : lm;
  const float M = wave_max_dpp(lm);
  double pw[kWavePer];  // the lane's tile weights, kept for the owner's search
  double local = 0.0;
#pragma unroll
  for (int j = 0; j < kWavePer; ++j) {
    const float e = fast_exp2((pr[j].x - M) * a.cf);
    const bool live = t0 + j < t1 && pr[j].x != -__builtin_inff();
    pw[j] = live ? (double)pr[j].y * (double)e : 0.0;
    local += pw[j];
  }
  const double incl = wave_inclusive_scan_dpp(local);
  const double excl = incl - local;
  const double total = lane_f64(incl, kWave - 1);
  // the stream-0 uniform of this position: drawn by the previous position's
  // select (see below), or here at the first position
  const double u = a.k == 1 ? draft_uniform(seed, a.round, 1) : u_pre;
  const double q = u * total;
  const unsigned long long cross = __ballot(local > 0.0 && incl > q);
  const unsigned long long pos = __ballot(local > 0.0);
  const int owner = cross ? __ffsll((long long)cross) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
  // The owner's search, in selects rather than branches (every lane runs
  // it, the owner's result is taken): the first positive tile whose
  // inclusive cumulative weight exceeds q, else the last positive tile.
  // pw[j] is 0 past the lane's last tile.
  int ts = -1, lastpos = -1;
  double base = 0.0, lastbase = 0.0;
  float mt = 0.0f, lastm = 0.0f;
  {
    double cum = excl;
#pragma unroll
    for (int j = 0; j < kWavePer; ++j) {
      const double w = pw[j];
      const bool posw = w > 0.0;
      const bool hit = posw && ts < 0 && cum + w > q;
      lastpos = posw ? t0 + j : lastpos;
      lastbase = posw ? cum : lastbase;
      lastm = posw ? pr[j].x : lastm;
      ts = hit ? t0 + j : ts;
      base = hit ? cum : base;
      mt = hit ? pr[j].x : mt;
      cum += w;
    }
    const bool none = ts < 0;
    ts = none ? (lastpos < 0 ? 0 : lastpos) : ts;
    base = none ? (lastpos < 0 ? 0.0 : lastbase) : base;
    mt = none ? (lastpos < 0 ? M : lastm) : mt;
  }
  ts = lane_i32(ts, owner);
  base = lane_f64(base, owner);
  mt = lane_f32(mt, owner);

  // batch 2: the wave's quarter of the bias of tile ts.  Lane (cg, kr) owns
  // columns c .. c+7 and k = kq wave + kr + 4 i.
  const int kq = a.r / 4;  // r % 16 == 0
  const int nk = kq / 4;
  const int cg = lane & 15, kr = lane >> 4;
  const int c = ts * kTileCols + 8 * cg;
  const size_t V = (size_t)a.V;
  const float* urow = a.U + ((size_t)b * a.gamma + (a.k - 1)) * V;
  const int uc = ts * kTileCols + 2 * lane;  // wave 0: columns uc, uc + 1
  const float u0 = uc < a.V ? urow[uc] : 0.0f;
  const float u1 = uc + 1 < a.V ? urow[uc + 1] : 0.0f;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  const bool vec = c + 8 <= a.V && (a.V & 7) == 0;
  for (int i0 = 0; i0 < nk; i0 += 16) {
    float e[16];
    float w[16][8];
    // clamped k: every load of the chunk is issued before the first use
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = opnd_at<kBf16, kParts>(a, prev, wave * kq + kr + 4 * min(i0 + i, nk - 1));
    if (kBf16 && vec) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = wave * kq + kr + 4 * min(i0 + i, nk - 1);
        const uint4 p = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.W2) + (size_t)k * V + c);
        w[i][0] = __uint_as_float(p.x << 16);
        w[i][1] = __uint_as_float(p.x & 0xffff0000u);
        w[i][2] = __uint_as_float(p.y << 16);
        w[i][3] = __uint_as_float(p.y & 0xffff0000u);
        w[i][4] = __uint_as_float(p.z << 16);
        w[i][5] = __uint_as_float(p.z & 0xffff0000u);
        w[i][6] = __uint_as_float(p.w << 16);
        w[i][7] = __uint_as_float(p.w & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = wave * kq + kr + 4 * min(i0 + i, nk - 1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int cc = c + j < a.V ? c + j : a.V - 1;
          const float v = w2_at<kBf16>(a.W2, (size_t)k * V + cc);
          w[i][j] = c + j < a.V ? v : 0.0f;
        }
      }
    }
    if (i0 == 0 && threadIdx.x == 0 && a.k < a.gamma) {
      // the next position's uniform, drawn while the loads above are in
      // flight (two buffers: the next select reads one, writes the other)
      a.u_next[(size_t)(a.k & 1) * a.B + b] = unit_uniform(draw_block(seed, a.round, a.k + 1, kStreamDraft, 0).w[0]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float ei = i0 + i < nk ? e[i] : 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(ei, w[i][j], acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc[j] += __shfl_xor(acc[j], 16);
    acc[j] += __shfl_xor(acc[j], 32);
  }
  if (kr == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sbias[wave][8 * cg + j] = acc[j];
  }
  if (a.conf != nullptr) {
    c_next = wave_sum(c_next);
    c_first = wave_sum(c_first);
    if (lane == 0) {
      sconf[0][wave] = c_next;
      sconf[1][wave] = c_first;
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // wave 0: the two columns of each lane, the column draw within tile ts
  const double cf = (double)a.cf;
  const double scale = exp2((double)(mt - M) * cf);
  float l2[2];
  double term[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cc = 2 * lane + h;
    const float bias = ((sbias[0][cc] + sbias[1][cc]) + sbias[2][cc]) + sbias[3][cc];
    const float uv = h == 0 ? u0 : u1;
    const float l = uc + h < a.V ? uv + bias : -__builtin_inff();
    const float e = l == -__builtin_inff() ? 0.0f : fast_exp2((l - mt) * a.cf);
    l2[h] = l;
    term[h] = (double)e * scale;
  }
  const double loc2 = term[0] + term[1];
  const double inc2 = wave_inclusive_scan_dpp(loc2);
  const double exc2 = inc2 - loc2;
  const double q2 = q - base;
  const unsigned long long cross2 = __ballot(loc2 > 0.0 && inc2 > q2);
  const unsigned long long pos2 = __ballot(loc2 > 0.0);
  const int own2 = cross2 ? __ffsll((long long)cross2) - 1 : (pos2 ? 63 - __clzll((long long)pos2) : 0);
  int mytok = 0;
  if (lane == own2) {
    int h;
    if (cross2) {
      h = (term[0] > 0.0 && exc2 + term[0] > q2) ? 0 : 1;
    } else {
      h = term[1] > 0.0 ? 1 : 0;
    }
    const float l = l2[h];
    mytok = ts * kTileCols + 2 * lane + h;
    a.tokens[out] = mytok;
    a.prob[out] = (float)(exp2((double)(l - M) * cf) / total);
    a.lse[out] = (float)((double)M * a.inv_t + log(total));
  }
  const int xk = lane_i32(mytok, own2);
  store_ring_operand<kBf16>(a, b, xk, lane);
  if (a.conf != nullptr) {
    const double emb = wave_sum(a.k < a.gamma ? conf_embed<kBf16>(a, xk, lane, kWave) : 0.0);
    if (lane == 0) {
      if (a.k < a.gamma) conf_store(a, b, a.k + 1, ((sconf[0][0] + sconf[0][1]) + (sconf[0][2] + sconf[0][3])) + emb);
      if (a.k == 1) conf_store(a, b, 1, (sconf[1][0] + sconf[1][1]) + (sconf[1][2] + sconf[1][3]));
    }
  }
}

template <bool kBf16, int kParts = 1>
static hipError_t launch_select_wave(const SelectArgs& sa, hipStream_t s) {
  const int per = (sa.ntiles + kWave - 1) / kWave;
  ProfScope prof(s, kProfDraftSelect);
  if (per <= 8) {
    hipLaunchKernelGGL((draft_select_wave_kernel<kBf16, 8, kParts>), dim3(sa.B), dim3(kSelThreads), 0, s, sa);
  } else if (per <= 16) {
    hipLaunchKernelGGL((draft_select_wave_kernel<kBf16, 16, kParts>), dim3(sa.B), dim3(kSelThreads), 0, s, sa);
  } else if (per <= 20) {
    hipLaunchKernelGGL((draft_select_wave_kernel<kBf16, 20, kParts>), dim3(sa.B), dim3(kSelThreads), 0, s, sa);
  } else {
    static_assert(kWaveTiles == 32 * kWave, "largest instantiation covers kWaveTiles");
    hipLaunchKernelGGL((draft_select_wave_kernel<kBf16, 32, kParts>), dim3(sa.B), dim3(kSelThreads), 0, s, sa);
  }
  return hipGetLastError();
}

size_t draft_workspace(int B, int gamma, int V, int r) {
  // per-position launches: tile summaries, look-ahead uniforms, ring-kernel
  // operands (r = 256 only); the resident loop carves its own layout from the
  // same bytes
  const size_t launches = align256((size_t)B * tiles_of(V, kTileCols) * sizeof(float2)) +
                          align256((size_t)2 * B * sizeof(double)) + (r == 256 ? align256(ring_operand_bytes(B)) : 0);
  const size_t resident = resident_workspace(B, gamma, V, r);
  return launches > resident ? launches : resident;
}

template <bool kGreedy, bool kBf16, int kParts = 1>
static hipError_t launch_select(const SelectArgs& s, hipStream_t st) {
  ProfScope prof(st, kProfDraftSelect);
  hipLaunchKernelGGL((draft_select_kernel<kGreedy, kBf16, kParts>), dim3(s.B), dim3(kSelThreads), 0, st, s);
  return hipGetLastError();
}

hipError_t launch_draft(const DraftArgs& a, bool bf16, hipStream_t s) {
  if (resident_draft_applies(a, bf16)) {
    bool launched = false;
    const hipError_t e = launch_resident_draft(a, s, &launched);
    if (e != hipSuccess || launched) return e;
  }
  const bool greedy = a.temperature == 0.0f;
  const int ntiles = tiles_of(a.V, kTileCols);
  float2* partials = reinterpret_cast<float2*>(a.ws);
  const float cf = greedy ? 0.0f : (float)(1.4426950408889634 / (double)a.temperature);

  TileArgs t = {};
  t.U = a.U;
  t.W1 = a.W1;
  t.W2 = a.W2;
  t.x0 = a.x0;
  t.tokens = a.tokens;
  t.partials = partials;
  t.nrows = a.B;
  t.kper = 1;
  t.B = a.B;
  t.gamma = a.gamma;
  t.V = a.V;
  t.r = a.r;
  t.ntiles = ntiles;
  t.cf = cf;

  SelectArgs sa = {};
  sa.U = a.U;
  sa.W1 = a.W1;
  sa.W2 = a.W2;
  sa.x0 = a.x0;
  sa.seeds = a.seeds;
  sa.round = a.round;
  sa.partials = partials;
  sa.B = a.B;
  sa.gamma = a.gamma;
  sa.V = a.V;
  sa.r = a.r;
  sa.ntiles = ntiles;
  sa.cf = cf;
  sa.inv_t = greedy ? 0.0 : 1.0 / (double)a.temperature;
  sa.tokens = a.tokens;
  sa.prob = a.prob;
  sa.lse = a.lse;
  sa.ch = a.ch;
  sa.cw = a.cw;
  sa.csts = a.csts;
  sa.cd = a.cd;
  sa.conf = a.conf;
  sa.u_next = reinterpret_cast<double*>(reinterpret_cast<char*>(a.ws) +
                                        align256((size_t)a.B * ntiles * sizeof(float2)));
  // When the tile passes run the ring kernel, each selection also stores the
  // drafted token's W1 row in that kernel's operand layout, and the next
  // position's tile pass reads it instead of gathering W1 rows itself.
  const int mode = greedy ? kModeGreedy : kModeSample;
  uint4* esw = nullptr;
  if (a.r == 256 && tile_pass_uses_ring(t, mode, bf16))
    esw = reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.ws) + align256((size_t)a.B * ntiles * sizeof(float2)) +
                                   align256((size_t)2 * a.B * sizeof(double)));

  for (int k = 1; k <= a.gamma; ++k) {
    t.k0 = k - 1;
    t.esw = k >= 2 ? esw : nullptr;
    hipError_t e = launch_tile_pass(t, mode, bf16, s);
    if (e != hipSuccess) return e;
    sa.k = k;
    sa.esw = k < a.gamma ? esw : nullptr;
    if (greedy) {
      e = bf16 ? launch_select<true, true>(sa, s) : launch_select<true, false>(sa, s);
    } else if (ntiles <= kWaveTiles) {
      e = bf16 ? launch_select_wave<true>(sa, s) : launch_select_wave<false>(sa, s);
    } else {
      e = bf16 ? launch_select<false, true>(sa, s) : launch_select<false, false>(sa, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}


// ---------------------------------------------------------------------------
// Block sampling with the RNN head (DSpark, "Instantiation 2: The RNN Head",
// Eq. 6).  Per request s_0 = 0 and, for k = 1..gamma,
//   (g, c, o) = Wp [s_{k-1}; W1[x_{k-1}]] + hp_k
//   s_k = sigmoid(g) s_{k-1} + (1 - sigmoid(g)) tanh(c),   e_k = tanh(o)
// and the logits of position k are U_k + e_k W2, sampled exactly as the Markov
// head's.  hp_k = Wp[:, 2r:] h_k depends on no drafted token, so the caller
// brings it precomputed from the parallel stage.
//
// One cell launch per position: workgroup (request group, slice of jn state
// units) stages z = [s_{k-1}; W1[x_{k-1}]] of its requests in LDS and streams
// its rows of Wp through LDS in column chunks; two threads (one per half of
// the columns of z) form the three projections of one (request, unit).  The
// cell computes in float32, the
// precision of its inputs Wp and hp.  e_k goes to the operand table as two
// bf16 parts (hi = bf16(e), lo = bf16(e - hi)), so that the bf16 MFMA tile
// pass multiplies W2 by hi + lo, which is e to about 2^-18 relative.  The
// state is double-buffered (position k reads buffer (k - 1) & 1 and writes
// k & 1).
// ---------------------------------------------------------------------------

struct CellArgs {
  const void* W1;
  const float* Wp;     // [3r][2r]
  const float* hp;     // [B][gamma][3r]
  const int32_t* x0;
  const int32_t* tokens;
  float* state;        // [2][B][r]
  uint16_t* opnd;      // [B * gamma][2r]: bf16 hi parts, then lo parts
  float* e_out;        // optional [B][gamma][r]
  int B, gamma, V, r, k;
};

// The cell's workgroup owns 16 requests and 16 state units: per gate
// (g, c, o) a 16 x 16 block of [B x 2r] . [2r x 3r], the product z W_p^T
// with z = [s_{k-1}; W1[x_{k-1}]], on the float32 MFMA
// v_mfma_f32_16x16x4_f32.  Six waves: (gate, half of z), the state half
// (columns 0..r-1) and the token half (r..2r-1); the halves' blocks meet in
// LDS, where one thread per (request, unit) finishes the cell.
constexpr int kCellReq = 16;
constexpr int kCellUnits = 16;
constexpr int kCellWaves = 6;
constexpr int kCellThreads = kCellWaves * kWave;
constexpr int kCellChunks = 16;  // 16-column k chunks loaded together (all of a half at r <= 256)

typedef float cellx4 __attribute__((ext_vector_type(4)));

// One wave's half of z against its gate's W_p rows.  Lane l: request row
// l % 16 of z (zrow, at column 4 (l / 16) of the half) and unit row l % 16 of
// W_p (wrow, likewise).  The k order inside a 16-column chunk m is chosen so
// that each lane loads four consecutive columns: MFMA i of the chunk takes
// column 16 m + 4 (l / 16) + i from both operands.  Every load of a pass is
// issued before the first MFMA.  kZbf: z is a bf16 row (the token half with
// bf16 weights), else float32.  zrow_of(zrow, zmask) gives the lane's z row
// and a mask ANDed into its bits (0: this lane's z is zero); it is called
// after the first W_p loads are issued, so that a token load overlaps them.
template <bool kZbf, class ZRowOf>
__device__ __forceinline__ void cell_half(ZRowOf zrow_of, const float* wrow, int nchunk, cellx4& acc0,
                                          cellx4& acc1) {
  const void* zrow = nullptr;
  uint32_t zmask = 0;
  for (int p0 = 0; p0 < nchunk; p0 += kCellChunks) {
    // chunks past the end repeat the last one (loaded, not used)
    float4 w[kCellChunks];
    uint4 z[kCellChunks];  // float32 bits
#pragma unroll
    for (int q = 0; q < kCellChunks; ++q) w[q] = *reinterpret_cast<const float4*>(wrow + 16 * min(p0 + q, nchunk - 1));
    if (p0 == 0) zrow_of(zrow, zmask);
    if constexpr (kZbf) {
      uint2 zr[kCellChunks];
#pragma unroll
      for (int q = 0; q < kCellChunks; ++q)
        zr[q] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(zrow) + 16 * min(p0 + q, nchunk - 1));
#pragma unroll
      for (int q = 0; q < kCellChunks; ++q) {
        // a bf16 value is the high half of its float32
        const uint32_t x = zr[q].x & zmask, y = zr[q].y & zmask;
        z[q] = make_uint4(x << 16, x & 0xffff0000u, y << 16, y & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < kCellChunks; ++q) {
        const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(zrow) + 16 * min(p0 + q, nchunk - 1));
        z[q] = make_uint4(v.x & zmask, v.y & zmask, v.z & zmask, v.w & zmask);
      }
    }
#pragma unroll
    for (int q = 0; q < kCellChunks; ++q) {
      if (p0 + q < nchunk) {
        // two accumulators: no MFMA waits on the one just issued
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(z[q].x), w[q].x, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(z[q].y), w[q].y, acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(z[q].z), w[q].z, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(z[q].w), w[q].w, acc1, 0, 0, 0);
      }
    }
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kCellThreads) void rnn_cell_kernel(CellArgs a) {
  __shared__ float part[kCellWaves][kCellReq][kCellUnits + 1];
  const int r = a.r;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int lane = threadIdx.x & (kWave - 1);
  const int gate = wave >> 1, zh = wave & 1;
  const int b0 = blockIdx.x * kCellReq, j0 = blockIdx.y * kCellUnits;
  const float* sprev = a.state + (size_t)((a.k - 1) & 1) * a.B * r;
  float* snext = a.state + (size_t)(a.k & 1) * a.B * r;

  // lane l: request b0 + l % 16 (rows past B repeat the last request and are
  // not stored) and unit j0 + l % 16 (r % 16 == 0: every unit exists)
  const int lr = lane & 15, kq = 4 * (lane >> 4);
  const int bl = min(b0 + lr, a.B - 1);
  const float* wrow = a.Wp + ((size_t)gate * r + j0 + lr) * (size_t)(2 * r) + (size_t)zh * r + kq;

  // the finishing thread's inputs, loaded before the products: thread t <
  // 256 finishes (request b0 + t / 16, unit j0 + t % 16)
  const int t = threadIdx.x;
  const int ri = (t / kCellUnits) & (kCellReq - 1), ui = t & (kCellUnits - 1);
  const int b = b0 + ri, j = j0 + ui;
  const bool fin = t < kCellReq * kCellUnits && b < a.B;
  const size_t row = (size_t)min(b, a.B - 1) * a.gamma + a.k - 1;
  float hg = 0.0f, hc = 0.0f, ho = 0.0f, sp = 0.0f;
  if (fin) {
    const float* h = a.hp + row * 3 * r;
    hg = h[j];
    hc = h[r + j];
    ho = h[2 * r + j];
    if (a.k > 1) sp = sprev[(size_t)b * r + j];
  }

  cellx4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
  if (zh == 0) {
    // the state half; zero at k = 1 (s_0 = 0)
    auto srow = [&](const void*& zrow, uint32_t& zmask) {
      zrow = sprev + (size_t)bl * r + kq;
      zmask = 0xffffffffu;
    };
    if (a.k > 1) cell_half<false>(srow, wrow, r / 16, acc0, acc1);
  } else {
    // the token half: W1[x_{k-1}], zero for an out-of-range token (its
    // request is reported invalid by the selection)
    auto trow = [&](const void*& zrow, uint32_t& zmask) {
      const int x = a.k == 1 ? a.x0[bl] : a.tokens[(size_t)bl * a.gamma + a.k - 2];
      const bool bad = (unsigned)x >= (unsigned)a.V;
      const size_t xo = (bad ? 0 : (size_t)x * r) + kq;
      zmask = bad ? 0u : 0xffffffffu;
      if constexpr (kBf16) {
        zrow = reinterpret_cast<const uint16_t*>(a.W1) + xo;
      } else {
        zrow = reinterpret_cast<const float*>(a.W1) + xo;
      }
    };
    cell_half<kBf16>(trow, wrow, r / 16, acc0, acc1);
  }
  // lane l holds rows (requests) 4 (l / 16) + i, column (unit) l % 16
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][kq + i][lr] = acc0[i] + acc1[i];
  __syncthreads();

  // one thread per (request, unit): g, c, o of both halves plus h^p
  if (!fin) return;
  const float g = part[0][ri][ui] + part[1][ri][ui] + hg;
  const float c = part[2][ri][ui] + part[3][ri][ui] + hc;
  const float o = part[4][ri][ui] + part[5][ri][ui] + ho;
  const float sg = 1.0f / (1.0f + expf(-g));
  snext[(size_t)b * r + j] = sg * sp + (1.0f - sg) * tanhf(c);
  const float e = tanhf(o);
  const uint16_t hi = bf16_round(e);
  const uint16_t lo = bf16_round(e - bf16_to_float(hi));
  a.opnd[row * 2 * r + j] = hi;
  a.opnd[row * 2 * r + r + j] = lo;
  if (a.e_out) a.e_out[row * r + j] = e;
}

size_t rnn_draft_workspace(int B, int gamma, int V, int r) {
  // the Markov draft's buffers without the ring operands, then the state
  // and the operand table
  return align256((size_t)B * tiles_of(V, kTileCols) * sizeof(float2)) + align256((size_t)2 * B * sizeof(double)) +
         align256((size_t)2 * B * r * sizeof(float)) + align256((size_t)B * gamma * 2 * r * sizeof(uint16_t));
}

hipError_t launch_rnn_draft(const RnnDraftArgs& a, hipStream_t s) {
  const bool greedy = a.temperature == 0.0f;
  const int ntiles = tiles_of(a.V, kTileCols);
  char* ws = reinterpret_cast<char*>(a.ws);
  float2* partials = reinterpret_cast<float2*>(ws);
  ws += align256((size_t)a.B * ntiles * sizeof(float2));
  double* u_next = reinterpret_cast<double*>(ws);
  ws += align256((size_t)2 * a.B * sizeof(double));
  float* state = reinterpret_cast<float*>(ws);
  ws += align256((size_t)2 * a.B * a.r * sizeof(float));
  uint16_t* opnd = reinterpret_cast<uint16_t*>(ws);
  const float cf = greedy ? 0.0f : (float)(1.4426950408889634 / (double)a.temperature);

  CellArgs ca = {};
  ca.W1 = a.W1;
  ca.Wp = a.Wp;
  ca.hp = a.hp;
  ca.x0 = a.x0;
  ca.tokens = a.tokens;
  ca.state = state;
  ca.opnd = opnd;
  ca.e_out = a.e_out;
  ca.B = a.B;
  ca.gamma = a.gamma;
  ca.V = a.V;
  ca.r = a.r;
  if (a.r % 16 != 0) return hipErrorInvalidValue;  // whole 16-unit blocks and 16-column k chunks
  const dim3 cgrid((a.B + kCellReq - 1) / kCellReq, a.r / kCellUnits);

  TileArgs t = {};
  t.U = a.U;
  t.W1 = opnd;
  t.W2 = a.W2;
  t.x0 = a.x0;
  t.tokens = a.tokens;
  t.partials = partials;
  t.nrows = a.B;
  t.kper = 1;
  t.B = a.B;
  t.gamma = a.gamma;
  t.V = a.V;
  t.r = a.r;
  t.ntiles = ntiles;
  t.cf = cf;
  t.opnd_rows = 2;

  SelectArgs sa = {};
  sa.U = a.U;
  sa.W1 = opnd;
  sa.W2 = a.W2;
  sa.x0 = a.x0;
  sa.seeds = a.seeds;
  sa.round = a.round;
  sa.partials = partials;
  sa.B = a.B;
  sa.gamma = a.gamma;
  sa.V = a.V;
  sa.r = a.r;
  sa.ntiles = ntiles;
  sa.cf = cf;
  sa.inv_t = greedy ? 0.0 : 1.0 / (double)a.temperature;
  sa.tokens = a.tokens;
  sa.prob = a.prob;
  sa.lse = a.lse;
  sa.u_next = u_next;

  const int mode = greedy ? kModeGreedy : kModeSample;
  for (int k = 1; k <= a.gamma; ++k) {
    ca.k = k;
    {
      ProfScope prof(s, kProfRnnCell);
      hipLaunchKernelGGL(rnn_cell_kernel<true>, cgrid, dim3(kCellThreads), 0, s, ca);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    t.k0 = k - 1;
    e = launch_tile_pass(t, mode, true, s);
    if (e != hipSuccess) return e;
    sa.k = k;
    if (greedy) {
      e = launch_select<true, true, 2>(sa, s);
    } else if (ntiles <= kWaveTiles) {
      e = launch_select_wave<true, 2>(sa, s);
    } else {
      e = launch_select<false, true, 2>(sa, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dspark
