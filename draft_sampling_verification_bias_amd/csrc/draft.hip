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
};

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

template <bool kGreedy, bool kBf16>
__global__ __launch_bounds__(kSelThreads) void draft_select_kernel(SelectArgs a) {
  __shared__ PickScratch ps;
  __shared__ float sw1[512];
  __shared__ float sbias[2][kTileCols];
  __shared__ float sl[kTileCols];
  __shared__ double sterm[kTileCols];
  __shared__ float sv[kSelThreads / kWave];
  __shared__ int si[kSelThreads / kWave];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t out = (size_t)b * a.gamma + (a.k - 1);
  const int prev = a.k == 1 ? a.x0[b] : a.tokens[(size_t)b * a.gamma + a.k - 2];
  if (prev < 0 || prev >= a.V) {  // invalid anchor or earlier position: propagate
    if (tid == 0) {
      a.tokens[out] = -1;
      a.prob[out] = __builtin_nanf("");
      a.lse[out] = __builtin_nanf("");
    }
    return;
  }
  const float2* P = a.partials + (size_t)b * a.ntiles;

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
    return;
  } else {
    float lm = -__builtin_inff();
    for (int t = tid; t < a.ntiles; t += kSelThreads) lm = fmaxf(lm, P[t].x);
    const float M = block_max<kSelThreads>(lm, sv);
    const double cf = (double)a.cf;
    auto tile_weight = [&](int t) -> double {
      const float2 p = P[t];
      return p.x == -__builtin_inff() ? 0.0 : (double)p.y * exp2((double)(p.x - M) * cf);
    };
    const double u = unit_uniform(draw_block(a.seeds[b], a.round, a.k, kStreamDraft, 0).w[0]);
    double total = 0.0, base = 0.0;
    int ts = block_pick_uniform<kSelThreads>(a.ntiles, tile_weight, u, ps, &base, &total);
    if (ts < 0) ts = 0;
    const double q = u * total;
    const float mt = P[ts].x;
    const double scale = exp2((double)(mt - M) * cf);

    // Rescan tile ts: rebuild the 128 logits with a VALU dot product per column.
    for (int j = tid; j < a.r; j += kSelThreads) sw1[j] = w1_at<kBf16>(a.W1, (size_t)prev * a.r + j);
    __syncthreads();
    {
      const int col = tid % kTileCols, half = tid / kTileCols;
      const int v = ts * kTileCols + col;
      const int kh = a.r / 2;
      float acc = 0.0f;
      if (v < a.V) {
        for (int j = half * kh; j < (half + 1) * kh; ++j) acc = fmaf(sw1[j], w2_at<kBf16>(a.W2, (size_t)j * a.V + v), acc);
      }
      sbias[half][col] = acc;
    }
    __syncthreads();
    if (tid < kTileCols) {
      const int v = ts * kTileCols + tid;
      float l = -__builtin_inff();
      if (v < a.V) l = a.U[((size_t)b * a.gamma + (a.k - 1)) * a.V + v] + (sbias[0][tid] + sbias[1][tid]);
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
  }
}

size_t draft_workspace(int B, int gamma, int V, int r) {
  (void)gamma;
  (void)r;
  return align256((size_t)B * tiles_of(V, kTileCols) * sizeof(float2));
}

template <bool kGreedy, bool kBf16>
static hipError_t launch_select(const SelectArgs& s, hipStream_t st) {
  ProfScope prof(st, kProfDraftSelect);
  hipLaunchKernelGGL((draft_select_kernel<kGreedy, kBf16>), dim3(s.B), dim3(kSelThreads), 0, st, s);
  return hipGetLastError();
}

hipError_t launch_draft(const DraftArgs& a, bool bf16, hipStream_t s) {
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

  for (int k = 1; k <= a.gamma; ++k) {
    t.k0 = k - 1;
    hipError_t e = launch_tile_pass(t, greedy ? kModeGreedy : kModeSample, bf16, s);
    if (e != hipSuccess) return e;
    sa.k = k;
    if (greedy) {
      e = bf16 ? launch_select<true, true>(sa, s) : launch_select<true, false>(sa, s);
    } else {
      e = bf16 ? launch_select<false, true>(sa, s) : launch_select<false, false>(sa, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dspark
