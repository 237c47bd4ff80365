// dspark_verify: lossless rejection-sampling verification.
//
// Follows the DSpark technical review, "Speculative Decoding: Draft, Then
// Verify" (step 3: accept x_k with probability min(1, p_t^k(x_k)/p_d^k(x_k)),
// the first rejection ends the block) and "Speculative decoding, from zero to
// DSpark", section 2 (on rejection draw from norm(max(0, p_t - p_d)); if all
// positions pass, a bonus token from the position after the block).  At
// temperature 0 acceptance is the exact argmax match of "Common Questions
// Answered".
//
// Positions are processed in order with early exit: phase k only streams the
// target rows of requests that are still alive at k (their list is built by
// phase k-1), so each request reads target rows 1..n+1 and no more.  A phase is
// one target-statistics kernel (per-tile max / exp-sum over 1024 columns) and
// one decision kernel (one workgroup per request).  Residual draws propose
// from p_t with the tile summaries and need p_d at one token only, rebuilt by
// an r-term dot product; the rare exact-residual fallback runs two more
// kernels over only the requests that need it.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace dspark {

constexpr int kVThreads = 256;
constexpr int kRowsPerPhase = 2;   // block positions verified per phase
constexpr int kColsPerThread = kTgtCols / kVThreads;  // 4

struct FallbackInfo {
  int j;        // rejected position (1-based)
  int prev;     // x_{j-1}
  int phase_row;  // row of position j within its phase's summaries
  double M, Z;  // target row max and exp-sum (base 2, scaled by cf)
  double pdx;   // p_d^j(x_j)
  double lx;    // draft logit of x_j (U + bias), float64
};

struct VerifyWs {
  float2* tpart;        // [B][kRowsPerPhase][ntv] target tile summaries of the current phase
  int* lists;           // [gamma + 2][B] request lists per phase (index ph = 1, 2, ...)
  int* counts;          // [gamma + 2]: counts[ph] phase sizes, counts[0] fallback count
  int* fb_list;         // [B]
  FallbackInfo* fb;     // [B] indexed by request
  double* fb_part;      // [B][ntv] residual mass per tile
};

static VerifyWs carve_verify(void* ws, int B, int gamma, int V) {
  const int ntv = tiles_of(V, kTgtCols);
  char* p = reinterpret_cast<char*>(ws);
  VerifyWs w;
  w.tpart = reinterpret_cast<float2*>(p);
  p += align256((size_t)B * kRowsPerPhase * ntv * sizeof(float2));
  w.lists = reinterpret_cast<int*>(p);
  p += align256((size_t)(gamma + 2) * B * sizeof(int));
  w.counts = reinterpret_cast<int*>(p);
  p += align256((size_t)(gamma + 2) * sizeof(int));
  w.fb_list = reinterpret_cast<int*>(p);
  p += align256((size_t)B * sizeof(int));
  w.fb = reinterpret_cast<FallbackInfo*>(p);
  p += align256((size_t)B * sizeof(FallbackInfo));
  w.fb_part = reinterpret_cast<double*>(p);  // [B][ceil(V / kResCols)]
  return w;
}

size_t verify_workspace(int B, int gamma, int V, int r) {
  (void)r;
  const int ntv = tiles_of(V, kTgtCols);
  return align256((size_t)B * kRowsPerPhase * ntv * sizeof(float2)) + align256((size_t)(gamma + 2) * B * sizeof(int)) +
         align256((size_t)(gamma + 2) * sizeof(int)) + align256((size_t)B * sizeof(int)) +
         align256((size_t)B * sizeof(FallbackInfo)) + align256((size_t)B * tiles_of(V, 256) * sizeof(double));
}

template <bool kBf16>
__device__ __forceinline__ double wval(const void* W, size_t idx) {
  if constexpr (kBf16) {
    return (double)bf16_to_float(reinterpret_cast<const uint16_t*>(W)[idx]);
  } else {
    return (double)reinterpret_cast<const float*>(W)[idx];
  }
}

// ---------------------------------------------------------------------------
// Target-row statistics, shared with dspark_survival.
//   list mode (list != null): row li is request list[li] at block position
//     kk0; summaries go to row b of tpart.
//   all mode: row R = b * gamma + kk for kk < gamma; summaries go to row R.
// Sample mode writes (max t, sum 2^((t - max) * cf)); greedy mode (max t,
// argmax bits).
// ---------------------------------------------------------------------------
constexpr int kTilesPerItem = 4;

// Each work item is kTilesPerItem consecutive 1024-column tiles of one row:
// every thread issues its four 16-byte loads at once and the four tiles share
// one set of block reductions.
template <bool kGreedy>
__global__ __launch_bounds__(kVThreads) void target_stats_kernel(TStatsArgs a) {
  constexpr int kWaves = kVThreads / kWave;
  __shared__ float sv[kWaves][kTilesPerItem];
  __shared__ float ss[kWaves][kTilesPerItem];
  __shared__ int si[kWaves][kTilesPerItem];
  const int nrows = a.list ? *a.count * a.rows_per_req : a.nall;
  const int ngrp = (a.ntv + kTilesPerItem - 1) / kTilesPerItem;
  const long long items = (long long)nrows * ngrp;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const int li = (int)(it / ngrp);
    const int tg = (int)(it - (long long)li * ngrp);
    int b, kk, orow;
    if (a.list) {
      const int req = li / a.rows_per_req, row = li - req * a.rows_per_req;
      b = a.list[req];
      kk = a.kk0 + row;
      orow = b * a.orow_stride + row;
    } else {
      b = li / a.gamma;
      kk = li - b * a.gamma;
      orow = li;
    }
    const float* row = a.target + ((size_t)b * (a.gamma + 1) + kk) * (size_t)a.V;
    float x[kTilesPerItem][kColsPerThread];
#pragma unroll
    for (int j = 0; j < kTilesPerItem; ++j) {
      const int c0 = (tg * kTilesPerItem + j) * kTgtCols + threadIdx.x * kColsPerThread;
      if (c0 + kColsPerThread <= a.V && (a.V & 3) == 0) {
        const float4 q = *reinterpret_cast<const float4*>(row + c0);
        x[j][0] = q.x; x[j][1] = q.y; x[j][2] = q.z; x[j][3] = q.w;
      } else {
#pragma unroll
        for (int e = 0; e < kColsPerThread; ++e) x[j][e] = c0 + e < a.V ? row[c0 + e] : -__builtin_inff();
      }
    }
    if constexpr (kGreedy) {
      float bv[kTilesPerItem];
      int bi[kTilesPerItem];
#pragma unroll
      for (int j = 0; j < kTilesPerItem; ++j) {
        const int c0 = (tg * kTilesPerItem + j) * kTgtCols + threadIdx.x * kColsPerThread;
        bv[j] = x[j][0];
        bi[j] = c0;
#pragma unroll
        for (int e = 1; e < kColsPerThread; ++e) {
          if (x[j][e] > bv[j]) {
            bv[j] = x[j][e];
            bi[j] = c0 + e;
          }
        }
        wave_argmax(bv[j], bi[j]);
        if (lane == 0) {
          sv[wave][j] = bv[j];
          si[wave][j] = bi[j];
        }
      }
      __syncthreads();
      if (threadIdx.x < kTilesPerItem) {
        const int j = threadIdx.x, t = tg * kTilesPerItem + j;
        float v = sv[0][j];
        int i = si[0][j];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) argmax_merge(v, i, sv[w][j], si[w][j]);
        if (t < a.ntv) a.tpart[(size_t)orow * a.ntv + t] = make_float2(v, __int_as_float(i));
      }
      __syncthreads();
    } else {
      float m[kTilesPerItem];
#pragma unroll
      for (int j = 0; j < kTilesPerItem; ++j) {
        m[j] = wave_max(fmaxf(fmaxf(x[j][0], x[j][1]), fmaxf(x[j][2], x[j][3])));
        if (lane == 0) sv[wave][j] = m[j];
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kTilesPerItem; ++j) {
        float M = sv[0][j];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sv[w][j]);
        float sum = 0.0f;
        if (M != -__builtin_inff()) {
#pragma unroll
          for (int e = 0; e < kColsPerThread; ++e) sum += fast_exp2((x[j][e] - M) * a.cf);
        }
        m[j] = M;
        sum = wave_sum(sum);
        if (lane == 0) ss[wave][j] = sum;
      }
      __syncthreads();
      if (threadIdx.x < kTilesPerItem) {
        const int j = threadIdx.x, t = tg * kTilesPerItem + j;
        float S = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) S += ss[w][j];
        if (t < a.ntv) a.tpart[(size_t)orow * a.ntv + t] = make_float2(m[j], S);
      }
      __syncthreads();
    }
  }
}

hipError_t launch_target_stats(const TStatsArgs& a, bool greedy, int max_rows, hipStream_t s) {
  const long long items = (long long)max_rows * ((a.ntv + kTilesPerItem - 1) / kTilesPerItem);
  const int grid = (int)(items < 16384 ? items : 16384);
  if (grid <= 0) return hipSuccess;
  ProfScope prof(s, kProfTargetStats);
  if (greedy) {
    hipLaunchKernelGGL((target_stats_kernel<true>), dim3(grid), dim3(kVThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((target_stats_kernel<false>), dim3(grid), dim3(kVThreads), 0, s, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Initialisation: outputs to their "not reached" values, validity check of
// every request's tokens, and the ordered list of phase 1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kVThreads) void verify_init_kernel(VerifyArgs a, VerifyWs w) {
  __shared__ PickScratch ps;
  const int g = a.gamma;
  if (threadIdx.x < g + 2) w.counts[threadIdx.x] = 0;
  int running = 0;
  for (int base = 0; base < a.B; base += kVThreads) {
    const int b = base + threadIdx.x;
    int valid = 0;
    if (b < a.B) {
      valid = a.x0[b] >= 0 && a.x0[b] < a.V;
      for (int k = 0; k < g; ++k) {
        const int t = a.draft_tokens[(size_t)b * g + k];
        valid &= (t >= 0 && t < a.V);
        if (a.accept_prob) a.accept_prob[(size_t)b * g + k] = __builtin_nanf("");
      }
      for (int k = 0; k <= g; ++k) a.out_tokens[(size_t)b * (g + 1) + k] = -1;
      a.accept_len[b] = -1;
    }
    double tot;
    const double ex = block_exclusive_scan<kVThreads>((double)valid, ps.red, tot);
    if (valid) w.lists[(size_t)1 * a.B + running + (int)ex] = b;
    running += (int)tot;
  }
  __syncthreads();
  if (threadIdx.x == 0) w.counts[1] = running;
}

// ---------------------------------------------------------------------------
// Decision kernel of phase k.
// ---------------------------------------------------------------------------
struct DecideCtx {
  const float2* P;   // tile summaries of the request's target row
  const float* trow; // target row
  float M;           // row max
  double cf;
  int ntv, V;
};

// Categorical draw from p_t with uniform u: tile search over the summaries,
// then a rescan of one 1024-column tile.  `sterm` holds kTgtCols doubles.
__device__ int sample_target(const DecideCtx& c, double u, PickScratch& ps, double* sterm,
                             double* total_out) {
  auto tile_weight = [&](int t) -> double {
    const float2 p = c.P[t];
    return p.x == -__builtin_inff() ? 0.0 : (double)p.y * exp2((double)(p.x - c.M) * c.cf);
  };
  double base = 0.0, total = 0.0;
  int ts = block_pick_uniform<kVThreads>(c.ntv, tile_weight, u, ps, &base, &total);
  if (ts < 0) ts = 0;
  const double q = u * total;
  const float mt = c.P[ts].x;
  const double scale = exp2((double)(mt - c.M) * c.cf);
  const float cff = (float)c.cf;
  for (int j = threadIdx.x; j < kTgtCols; j += kVThreads) {
    const int v = ts * kTgtCols + j;
    const float x = v < c.V ? c.trow[v] : -__builtin_inff();
    const float e = x == -__builtin_inff() ? 0.0f : fast_exp2((x - mt) * cff);
    sterm[j] = (double)e * scale;
  }
  __syncthreads();
  auto col_weight = [&](int j) -> double { return sterm[j]; };
  int col = block_pick_target<kVThreads>(kTgtCols, col_weight, q - base, ps, nullptr);
  if (col < 0) col = 0;
  if (total_out) *total_out = total;
  return ts * kTgtCols + col;
}

// Draft logit U[v] + W1[prev] . W2[:, v] in float64 (all threads receive it).
template <bool kBf16>
__device__ double draft_logit(const VerifyArgs& a, const float* urow, const double* sw1, int v, double* red) {
  double s = 0.0;
  for (int j = threadIdx.x; j < a.r; j += kVThreads) s += sw1[j] * wval<kBf16>(a.W2, (size_t)j * a.V + v);
  s = block_sum<kVThreads, double>(s, red);
  return (double)urow[v] + s;
}

// ---------------------------------------------------------------------------
// Wave-level draw from p_t for the fast path (at most kPrefixMax tiles): the
// cumulative tile weights are in LDS (scum[t] = weight of tiles < t), so a draw
// is a binary search plus a rescan of one 1024-column tile by one wave, 16
// consecutive columns per lane.  Same rule as the block search: the first
// column whose cumulative weight exceeds q; the last positive one if rounding
// leaves none.
// ---------------------------------------------------------------------------
constexpr int kPrefixMax = 1024;

__device__ int wave_sample_target(const DecideCtx& c, const double* scum, int last_pos_tile, double q) {
  const int lane = threadIdx.x & (kWave - 1);
  // first tile t with scum[t + 1] > q
  int lo = 0, hi = c.ntv;  // answer in [0, ntv]; ntv means "none"
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (scum[mid + 1] > q) hi = mid; else lo = mid + 1;
  }
  const int ts = lo < c.ntv ? lo : last_pos_tile;
  const double base = scum[ts];
  const double ql = q - base;
  const float mt = c.P[ts].x;
  const double scale = exp2((double)(mt - c.M) * c.cf);
  const float cff = (float)c.cf;
  const int c0 = ts * kTgtCols + lane * 16;
  float x[16];
  if (c0 + 16 <= c.V && (c.V & 3) == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v4 = *reinterpret_cast<const float4*>(c.trow + c0 + 4 * j);
      x[4 * j] = v4.x; x[4 * j + 1] = v4.y; x[4 * j + 2] = v4.z; x[4 * j + 3] = v4.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = c0 + j < c.V ? c.trow[c0 + j] : -__builtin_inff();
  }
  double term[16];
  double local = 0.0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float e = x[j] == -__builtin_inff() ? 0.0f : fast_exp2((x[j] - mt) * cff);
    term[j] = (double)e * scale;
    local += term[j];
  }
  const double incl = wave_inclusive_scan(local);
  const double excl = incl - local;
  const unsigned long long cross = __ballot(local > 0.0 && excl + local > ql);
  const unsigned long long pos = __ballot(local > 0.0);
  const int owner = cross ? __ffsll((long long)cross) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
  int col = -1;
  if (lane == owner) {
    double cum = excl;
    int lastp = -1;
    for (int j = 0; j < 16; ++j) {
      if (term[j] > 0.0) {
        lastp = j;
        if (col < 0 && cum + term[j] > ql) col = j;
      }
      cum += term[j];
    }
    if (col < 0) col = lastp < 0 ? 0 : lastp;
    col += lane * 16;
  }
  col = __shfl(col, owner);
  return ts * kTgtCols + col;
}

// W1[prev] . W2[:, v] + U[v] in float64, summed by one wave.
template <bool kBf16>
__device__ double wave_draft_logit(const VerifyArgs& a, const float* urow, const double* sw1, int v) {
  const int lane = threadIdx.x & (kWave - 1);
  double s = 0.0;
  for (int j = lane; j < a.r; j += kWave) s += sw1[j] * wval<kBf16>(a.W2, (size_t)j * a.V + v);
  s = wave_sum(s);
  return (double)urow[v] + s;
}

// Decision kernel for rows of more than kPrefixMax tiles: the same decisions
// as verify_decide_kernel below, with block-wide searches over the tile
// summaries in global memory.
template <bool kGreedy, bool kBf16>
__global__ __launch_bounds__(kVThreads) void verify_decide_generic_kernel(VerifyArgs a, VerifyWs w, int ph,
                                                                         float cf_f, int ntv) {
  __shared__ PickScratch ps;
  __shared__ double sterm[kTgtCols];
  __shared__ double sw1[512];
  __shared__ double sred[kVThreads / kWave];
  __shared__ float sv[kVThreads / kWave];
  __shared__ int si[kVThreads / kWave];
  const int g = a.gamma;
  const int k0 = 2 * ph - 1, k1 = min(2 * ph, g + 1);
  const int count = w.counts[ph];
  const double cf = (double)cf_f;
  for (int li = blockIdx.x; li < count; li += gridDim.x) {
    const int b = w.lists[(size_t)ph * a.B + li];
    for (int k = k0; k <= k1; ++k) {
      const float2* P = w.tpart + ((size_t)b * kRowsPerPhase + (k - k0)) * ntv;
      const float* trow = a.target + ((size_t)b * (g + 1) + (k - 1)) * (size_t)a.V;
      bool accepted = false;
      if constexpr (kGreedy) {
        float bv = -__builtin_inff();
        int bi = INT_MAX;
        for (int t = threadIdx.x; t < ntv; t += kVThreads) argmax_merge(bv, bi, P[t].x, __float_as_int(P[t].y));
        block_argmax<kVThreads>(bv, bi, sv, si);
        if (k <= g) {
          const int x = a.draft_tokens[(size_t)b * g + k - 1];
          accepted = bi == x;
          if (threadIdx.x == 0) {
            if (a.accept_prob) a.accept_prob[(size_t)b * g + k - 1] = accepted ? 1.0f : 0.0f;
            a.out_tokens[(size_t)b * (g + 1) + k - 1] = accepted ? x : bi;
            if (!accepted) a.accept_len[b] = k - 1;
          }
        } else if (threadIdx.x == 0) {
          a.out_tokens[(size_t)b * (g + 1) + g] = bi;
          a.accept_len[b] = g;
        }
      } else {
        float lm = -__builtin_inff();
        for (int t = threadIdx.x; t < ntv; t += kVThreads) lm = fmaxf(lm, P[t].x);
        DecideCtx c;
        c.P = P;
        c.trow = trow;
        c.M = block_max<kVThreads>(lm, sv);
        c.cf = cf;
        c.ntv = ntv;
        c.V = a.V;
        const uint64_t seed = a.seeds[b];
        auto tile_weight = [&](int t) -> double {
          const float2 p = P[t];
          return p.x == -__builtin_inff() ? 0.0 : (double)p.y * exp2((double)(p.x - c.M) * cf);
        };
        const double Z = block_total<kVThreads>(ntv, tile_weight, ps);
        if (k > g) {  // bonus token from the position after the block
          const double u = unit_uniform(draw_block(seed, a.round, g + 1, kStreamResidual, 0).w[0]);
          const int y = sample_target(c, u, ps, sterm, nullptr);
          if (threadIdx.x == 0) {
            a.out_tokens[(size_t)b * (g + 1) + g] = y;
            a.accept_len[b] = g;
          }
        } else {
          const int x = a.draft_tokens[(size_t)b * g + k - 1];
          const double ptx = exp2((double)(trow[x] - c.M) * cf) / Z;
          const double pdx = (double)a.draft_prob[(size_t)b * g + k - 1];
          const double alpha = fmin(1.0, ptx / pdx);
          const double u = unit_uniform(draw_block(seed, a.round, k, kStreamAccept, 0).w[0]);
          accepted = u < alpha;
          if (threadIdx.x == 0) {
            if (a.accept_prob) a.accept_prob[(size_t)b * g + k - 1] = (float)alpha;
            if (accepted) a.out_tokens[(size_t)b * (g + 1) + k - 1] = x;
          }
          if (!accepted) {
            const int prev = k == 1 ? a.x0[b] : a.draft_tokens[(size_t)b * g + k - 2];
            for (int j = threadIdx.x; j < a.r; j += kVThreads) sw1[j] = wval<kBf16>(a.W1, (size_t)prev * a.r + j);
            __syncthreads();
            const float* urow = a.U + ((size_t)b * g + (k - 1)) * (size_t)a.V;
            const double lx = draft_logit<kBf16>(a, urow, sw1, x, sred);
            int found = -1;
            for (int i = 0; i < DSPARK_MAX_RESIDUAL_PROPOSALS; ++i) {
              const Philox4 d = draw_block(seed, a.round, k, kStreamResidual, (uint64_t)i);
              const double up = unit_uniform(d.w[0]);
              const double ua = unit_uniform(d.w[1]);
              const int v = sample_target(c, up, ps, sterm, nullptr);
              const double ptv = exp2((double)(trow[v] - c.M) * cf) / Z;
              const double lv = draft_logit<kBf16>(a, urow, sw1, v, sred);
              const double pdv = pdx * exp((lv - lx) * a.inv_t_d);
              const double keep = fmax(0.0, 1.0 - pdv / ptv);
              if (ua < keep) {
                found = v;
                break;
              }
            }
            if (threadIdx.x == 0) {
              a.accept_len[b] = k - 1;
              if (found >= 0) {
                a.out_tokens[(size_t)b * (g + 1) + k - 1] = found;
              } else {
                FallbackInfo f;
                f.j = k;
                f.prev = prev;
                f.phase_row = k - k0;
                f.M = (double)c.M;
                f.Z = Z;
                f.pdx = pdx;
                f.lx = lx;
                w.fb[b] = f;
                const int pos = atomicAdd(&w.counts[0], 1);
                w.fb_list[pos] = b;
              }
            }
          }
        }
      }
      __syncthreads();
      if (!accepted) break;
      if (k == k1 && threadIdx.x == 0) {
        const int pos = atomicAdd(&w.counts[ph + 1], 1);
        w.lists[(size_t)(ph + 1) * a.B + pos] = b;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decision kernel for rows of at most kPrefixMax tiles.  The loads are issued
// in three dependent batches -- the request id; then everything that depends
// only on the request (its tile summaries, drafted and previous tokens, p_d,
// key); then everything that depends on those tokens (target logit, base
// logit, W1 row, W2 column of the drafted token) -- so an accepted position
// costs three memory round trips and a rejection two more per batch of four
// residual proposals.
// ---------------------------------------------------------------------------
constexpr int kTilesPerThreadFast = kPrefixMax / kVThreads;  // 4

// W1[prev] . W2[:, v] + U[v] in float64, summed by one wave; the W2 loads of a
// lane are issued together (clamped indices, zeroed terms).
template <bool kBf16>
__device__ double wave_draft_logit_batched(const VerifyArgs& a, const float* urow, const float* sw1, int v) {
  const int lane = threadIdx.x & (kWave - 1);
  float wv[512 / kWave];
  const float uv = urow[v];
#pragma unroll
  for (int m = 0; m < 512 / kWave; ++m) {
    const int j = lane + m * kWave;
    wv[m] = (float)wval<kBf16>(a.W2, (size_t)(j < a.r ? j : 0) * a.V + v);
  }
  double s = 0.0;
#pragma unroll
  for (int m = 0; m < 512 / kWave; ++m) {
    const int j = lane + m * kWave;
    if (j < a.r) s += (double)sw1[j] * (double)wv[m];
  }
  s = wave_sum(s);
  return (double)uv + s;
}

template <bool kGreedy, bool kBf16>
__global__ __launch_bounds__(kVThreads) void verify_decide_kernel(VerifyArgs a, VerifyWs w, int ph, float cf_f,
                                                                 int ntv) {
  constexpr int kWaves = kVThreads / kWave;
  __shared__ PickScratch ps;
  __shared__ double scum[kPrefixMax + 1];
  __shared__ float sw1[512];
  __shared__ double sred[kWaves];
  __shared__ float sv[kWaves];
  __shared__ int si[kWaves];
  __shared__ int s_pass[kWaves], s_tok[kWaves], s_lastpos;
  const int g = a.gamma;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
  const int k0 = 2 * ph - 1, k1 = min(2 * ph, g + 1);
  const int count = w.counts[ph];
  const double cf = (double)cf_f;
  for (int li = blockIdx.x; li < count; li += gridDim.x) {
    const int b = w.lists[(size_t)ph * a.B + li];
    const uint64_t seed = kGreedy ? 0 : a.seeds[b];
    for (int k = k0; k <= k1; ++k) {
      const float2* P = w.tpart + ((size_t)b * kRowsPerPhase + (k - k0)) * ntv;
      const float* trow = a.target + ((size_t)b * (g + 1) + (k - 1)) * (size_t)a.V;
      // batch 1: the row's tile summaries and the tokens of position k
      float2 pv[kTilesPerThreadFast];
#pragma unroll
      for (int j = 0; j < kTilesPerThreadFast; ++j) {
        const int t = tid * kTilesPerThreadFast + j;
        pv[j] = P[t < ntv ? t : ntv - 1];
      }
      int x = 0, prev = 0;
      double pdx = 1.0;
      if (k <= g) {
        x = a.draft_tokens[(size_t)b * g + k - 1];
        prev = k == 1 ? a.x0[b] : a.draft_tokens[(size_t)b * g + k - 2];
        if constexpr (!kGreedy) pdx = (double)a.draft_prob[(size_t)b * g + k - 1];
      }
      bool accepted = false;  // uniform across the block
      if constexpr (kGreedy) {
        float bv = -__builtin_inff();
        int bi = INT_MAX;
#pragma unroll
        for (int j = 0; j < kTilesPerThreadFast; ++j) {
          const int t = tid * kTilesPerThreadFast + j;
          if (t < ntv) argmax_merge(bv, bi, pv[j].x, __float_as_int(pv[j].y));
        }
        block_argmax<kVThreads>(bv, bi, sv, si);
        if (k <= g) {
          accepted = bi == x;
          if (tid == 0) {
            if (a.accept_prob) a.accept_prob[(size_t)b * g + k - 1] = accepted ? 1.0f : 0.0f;
            a.out_tokens[(size_t)b * (g + 1) + k - 1] = accepted ? x : bi;
            if (!accepted) a.accept_len[b] = k - 1;
          }
        } else if (tid == 0) {
          a.out_tokens[(size_t)b * (g + 1) + g] = bi;
          a.accept_len[b] = g;
        }
      } else {
        // batch 2: depends on the drafted and previous tokens
        const float* urow = a.U + ((size_t)b * g + (k - 1)) * (size_t)a.V;
        float tx = 0.0f, ux = 0.0f, w1v[2] = {0.0f, 0.0f}, w2v[2] = {0.0f, 0.0f};
        if (k <= g) {
          tx = trow[x];
          ux = urow[x];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int j = tid + q * kVThreads;
            const int jc = j < a.r ? j : 0;
            w1v[q] = (float)wval<kBf16>(a.W1, (size_t)prev * a.r + jc);
            w2v[q] = (float)wval<kBf16>(a.W2, (size_t)jc * a.V + x);
          }
        }
        // normaliser and cumulative tile weights
        float lm = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < kTilesPerThreadFast; ++j) {
          const int t = tid * kTilesPerThreadFast + j;
          if (t < ntv) lm = fmaxf(lm, pv[j].x);
        }
        const float M = block_max<kVThreads>(lm, sv);
        double wt[kTilesPerThreadFast], local = 0.0;
#pragma unroll
        for (int j = 0; j < kTilesPerThreadFast; ++j) {
          const int t = tid * kTilesPerThreadFast + j;
          wt[j] = (t < ntv && pv[j].x != -__builtin_inff())
                      ? (double)pv[j].y * (double)fast_exp2((pv[j].x - M) * cf_f)
                      : 0.0;
          local += wt[j];
        }
        if (tid == 0) s_lastpos = 0;
        double Z;
        const double excl = block_exclusive_scan<kVThreads>(local, ps.red, Z);
        {
          double cum = excl;
#pragma unroll
          for (int j = 0; j < kTilesPerThreadFast; ++j) {
            const int t = tid * kTilesPerThreadFast + j;
            cum += wt[j];
            if (t < ntv) {
              scum[t + 1] = cum;
              if (wt[j] > 0.0) atomicMax(&s_lastpos, t);
            }
          }
          if (tid == 0) scum[0] = 0.0;
        }
        __syncthreads();
        DecideCtx c;
        c.P = P;
        c.trow = trow;
        c.M = M;
        c.cf = cf;
        c.ntv = ntv;
        c.V = a.V;
        if (k > g) {  // bonus token from the position after the block
          const double u = unit_uniform(draw_block(seed, a.round, g + 1, kStreamResidual, 0).w[0]);
          if (wave == 0) {
            const int y = wave_sample_target(c, scum, s_lastpos, u * Z);
            if (lane == 0) {
              a.out_tokens[(size_t)b * (g + 1) + g] = y;
              a.accept_len[b] = g;
            }
          }
        } else {
          const double ptx = exp2((double)(tx - M) * cf) / Z;
          const double alpha = fmin(1.0, ptx / pdx);
          const double u = unit_uniform(draw_block(seed, a.round, k, kStreamAccept, 0).w[0]);
          accepted = u < alpha;
          if (tid == 0) {
            if (a.accept_prob) a.accept_prob[(size_t)b * g + k - 1] = (float)alpha;
            if (accepted) a.out_tokens[(size_t)b * (g + 1) + k - 1] = x;
          }
          if (!accepted) {
            // Rejected at k: residual draw by proposals from p_t, one per wave.
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int j = tid + q * kVThreads;
              if (j < a.r) sw1[j] = w1v[q];
            }
            double part = 0.0;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int j = tid + q * kVThreads;
              if (j < a.r) part += (double)w1v[q] * (double)w2v[q];
            }
            const double lx = (double)ux + block_sum<kVThreads, double>(part, sred);
            int found = -1;
            for (int i0 = 0; i0 < DSPARK_MAX_RESIDUAL_PROPOSALS && found < 0; i0 += kWaves) {
              const int i = i0 + wave;
              int pass = 0, v = -1;
              if (i < DSPARK_MAX_RESIDUAL_PROPOSALS) {
                const Philox4 d = draw_block(seed, a.round, k, kStreamResidual, (uint64_t)i);
                const double up = unit_uniform(d.w[0]);
                const double ua = unit_uniform(d.w[1]);
                v = wave_sample_target(c, scum, s_lastpos, up * Z);
                const float tv = trow[v];
                const double lv = wave_draft_logit_batched<kBf16>(a, urow, sw1, v);
                const double ptv = exp2((double)(tv - M) * cf) / Z;
                const double pdv = pdx * exp((lv - lx) * a.inv_t_d);
                const double keep = fmax(0.0, 1.0 - pdv / ptv);
                pass = ua < keep;
              }
              if (lane == 0) {
                s_pass[wave] = pass;
                s_tok[wave] = v;
              }
              __syncthreads();
#pragma unroll
              for (int ww = 0; ww < kWaves; ++ww) {
                if (found < 0 && s_pass[ww]) found = s_tok[ww];
              }
              __syncthreads();
            }
            if (tid == 0) {
              a.accept_len[b] = k - 1;
              if (found >= 0) {
                a.out_tokens[(size_t)b * (g + 1) + k - 1] = found;
              } else {
                FallbackInfo f;
                f.j = k;
                f.prev = prev;
                f.phase_row = k - k0;
                f.M = (double)M;
                f.Z = Z;
                f.pdx = pdx;
                f.lx = lx;
                w.fb[b] = f;
                const int pos = atomicAdd(&w.counts[0], 1);
                w.fb_list[pos] = b;
              }
            }
          }
        }
      }
      __syncthreads();
      if (!accepted) break;  // rejection, or the bonus token: the request is finished
      if (k == k1) {         // accepted the last position of this phase: alive in the next one
        if (tid == 0) {
          const int pos = atomicAdd(&w.counts[ph + 1], 1);
          w.lists[(size_t)(ph + 1) * a.B + pos] = b;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Exact residual fallback: mass of max(0, p_t - p_d) per 256-column chunk,
// then one inverse-CDF draw with the stream-3 uniform.  p_d needs the bias at
// every column of the row, so each chunk rebuilds 256 bias values: thread t
// owns columns 4 (t % 64) .. +3 of the chunk and a quarter of the r products,
// with all of its W2 loads in flight; the quarters are summed in LDS in a
// fixed order, so both kernels obtain bit-identical residual terms.
// ---------------------------------------------------------------------------
constexpr int kResCols = 256;

template <bool kBf16>
__device__ double residual_term(const VerifyArgs& a, const FallbackInfo& f, int b, int chunk, const float* sw1f,
                                float (*sbias)[kResCols], double cf) {
  const int g = a.gamma;
  const int quad = threadIdx.x & 63, slice = threadIdx.x >> 6;
  const int kq = a.r / 4;  // r % 16 == 0
  const int c = chunk * kResCols + 4 * quad;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const bool vec = kBf16 && (c + 4 <= a.V) && ((a.V & 3) == 0);
  for (int j0 = slice * kq; j0 < (slice + 1) * kq; j0 += 32) {
    float wv[32][4];
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
      const int j = j0 + jj;
      if (j < (slice + 1) * kq && vec) {
        const uint2 p = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.W2) + (size_t)j * a.V + c);
        wv[jj][0] = __uint_as_float(p.x << 16);
        wv[jj][1] = __uint_as_float(p.x & 0xffff0000u);
        wv[jj][2] = __uint_as_float(p.y << 16);
        wv[jj][3] = __uint_as_float(p.y & 0xffff0000u);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          wv[jj][q] = (j < (slice + 1) * kq && c + q < a.V) ? (float)wval<kBf16>(a.W2, (size_t)j * a.V + c + q) : 0.0f;
      }
    }
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
      const float e = j0 + jj < (slice + 1) * kq ? sw1f[j0 + jj] : 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(e, wv[jj][q], acc[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) sbias[slice][4 * quad + q] = acc[q];
  __syncthreads();
  const int v = chunk * kResCols + threadIdx.x;
  double res = 0.0;
  if (v < a.V) {
    const float bias = (sbias[0][threadIdx.x] + sbias[1][threadIdx.x]) + (sbias[2][threadIdx.x] + sbias[3][threadIdx.x]);
    const float t = a.target[((size_t)b * (g + 1) + (f.j - 1)) * (size_t)a.V + v];
    const float uu = a.U[((size_t)b * g + (f.j - 1)) * (size_t)a.V + v];
    const double pt = t == -__builtin_inff() ? 0.0 : exp2((double)(t - (float)f.M) * cf) / f.Z;
    const double pd = uu == -__builtin_inff() ? 0.0 : f.pdx * exp(((double)uu + (double)bias - f.lx) * a.inv_t_d);
    res = fmax(0.0, pt - pd);
  }
  __syncthreads();
  return res;
}

template <bool kBf16>
__global__ __launch_bounds__(kVThreads) void residual_stats_kernel(VerifyArgs a, VerifyWs w, float cf_f, int ntr) {
  __shared__ float sw1f[512];
  __shared__ float sbias[4][kResCols];
  __shared__ double sred[kVThreads / kWave];
  const int count = w.counts[0];
  const long long items = (long long)count * ntr;
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const int li = (int)(it / ntr);
    const int chunk = (int)(it - (long long)li * ntr);
    const int b = w.fb_list[li];
    const FallbackInfo f = w.fb[b];
    for (int j = threadIdx.x; j < a.r; j += kVThreads) sw1f[j] = (float)wval<kBf16>(a.W1, (size_t)f.prev * a.r + j);
    __syncthreads();
    const double res = residual_term<kBf16>(a, f, b, chunk, sw1f, sbias, (double)cf_f);
    const double s = block_sum<kVThreads, double>(res, sred);
    if (threadIdx.x == 0) w.fb_part[(size_t)b * ntr + chunk] = s;
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kVThreads) void residual_select_kernel(VerifyArgs a, VerifyWs w, float cf_f, int ntv,
                                                                   int ntr) {
  __shared__ PickScratch ps;
  __shared__ double sterm[kTgtCols];
  __shared__ float sw1f[512];
  __shared__ float sbias[4][kResCols];
  const int count = w.counts[0];
  const int g = a.gamma;
  for (int li = blockIdx.x; li < count; li += gridDim.x) {
    const int b = w.fb_list[li];
    const FallbackInfo f = w.fb[b];
    const double u = unit_uniform(draw_block(a.seeds[b], a.round, f.j, kStreamFallback, 0).w[0]);
    const double* FP = w.fb_part + (size_t)b * ntr;
    auto chunk_mass = [&](int t) -> double { return FP[t]; };
    double base = 0.0, total = 0.0;
    const int ts = block_pick_uniform<kVThreads>(ntr, chunk_mass, u, ps, &base, &total);
    int y;
    if (total > 0.0 && ts >= 0) {
      for (int j = threadIdx.x; j < a.r; j += kVThreads) sw1f[j] = (float)wval<kBf16>(a.W1, (size_t)f.prev * a.r + j);
      __syncthreads();
      const double res = residual_term<kBf16>(a, f, b, ts, sw1f, sbias, (double)cf_f);
      sterm[threadIdx.x] = res;
      __syncthreads();
      auto col_weight = [&](int j) -> double { return sterm[j]; };
      int col = block_pick_target<kVThreads>(kResCols, col_weight, u * total - base, ps, nullptr);
      if (col < 0) col = 0;
      y = ts * kResCols + col;
    } else {
      // No residual mass (possible only through rounding): draw from p_t.
      DecideCtx c;
      c.P = w.tpart + ((size_t)b * kRowsPerPhase + f.phase_row) * ntv;
      c.trow = a.target + ((size_t)b * (g + 1) + (f.j - 1)) * (size_t)a.V;
      c.M = (float)f.M;
      c.cf = (double)cf_f;
      c.ntv = ntv;
      c.V = a.V;
      y = sample_target(c, u, ps, sterm, nullptr);
    }
    if (threadIdx.x == 0) a.out_tokens[(size_t)b * (g + 1) + f.j - 1] = y;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_verify(const VerifyArgs& a_in, bool bf16, hipStream_t s) {
  VerifyArgs a = a_in;
  const bool greedy = a.temperature == 0.0f;
  a.inv_t_d = greedy ? 0.0 : 1.0 / (double)a.temperature;
  const int ntv = tiles_of(a.V, kTgtCols);
  const float cf = greedy ? 0.0f : (float)(1.4426950408889634 / (double)a.temperature);
  VerifyWs w = carve_verify(a.ws, a.B, a.gamma, a.V);

  {
    ProfScope prof(s, kProfVerifyInit);
    hipLaunchKernelGGL(verify_init_kernel, dim3(1), dim3(kVThreads), 0, s, a, w);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int dgrid = a.B < 2048 ? a.B : 2048;
  const int nph = (a.gamma + 1 + kRowsPerPhase - 1) / kRowsPerPhase;
  for (int ph = 1; ph <= nph; ++ph) {
    const int k0 = kRowsPerPhase * (ph - 1) + 1;
    TStatsArgs t = {};
    t.target = a.target;
    t.list = w.lists + (size_t)ph * a.B;
    t.count = w.counts + ph;
    t.kk0 = k0 - 1;
    t.rows_per_req = min(kRowsPerPhase, a.gamma + 2 - k0);
    t.orow_stride = kRowsPerPhase;
    t.gamma = a.gamma;
    t.V = a.V;
    t.ntv = ntv;
    t.cf = cf;
    t.tpart = w.tpart;
    e = launch_target_stats(t, greedy, a.B * t.rows_per_req, s);
    if (e != hipSuccess) return e;
    ProfScope prof(s, kProfVerifyDecide);
    if (ntv <= kPrefixMax) {
      if (greedy) {
        hipLaunchKernelGGL((verify_decide_kernel<true, true>), dim3(dgrid), dim3(kVThreads), 0, s, a, w, ph, cf, ntv);
      } else if (bf16) {
        hipLaunchKernelGGL((verify_decide_kernel<false, true>), dim3(dgrid), dim3(kVThreads), 0, s, a, w, ph, cf, ntv);
      } else {
        hipLaunchKernelGGL((verify_decide_kernel<false, false>), dim3(dgrid), dim3(kVThreads), 0, s, a, w, ph, cf,
                           ntv);
      }
    } else if (greedy) {
      hipLaunchKernelGGL((verify_decide_generic_kernel<true, true>), dim3(dgrid), dim3(kVThreads), 0, s, a, w, ph, cf,
                         ntv);
    } else if (bf16) {
      hipLaunchKernelGGL((verify_decide_generic_kernel<false, true>), dim3(dgrid), dim3(kVThreads), 0, s, a, w, ph,
                         cf, ntv);
    } else {
      hipLaunchKernelGGL((verify_decide_generic_kernel<false, false>), dim3(dgrid), dim3(kVThreads), 0, s, a, w, ph,
                         cf, ntv);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!greedy) {
    const int ntr = tiles_of(a.V, kResCols);
    const long long items = (long long)a.B * ntr;
    const int sgrid = (int)(items < 1024 ? items : 1024);
    {
      ProfScope prof(s, kProfResidualStats);
      if (bf16) {
        hipLaunchKernelGGL((residual_stats_kernel<true>), dim3(sgrid), dim3(kVThreads), 0, s, a, w, cf, ntr);
      } else {
        hipLaunchKernelGGL((residual_stats_kernel<false>), dim3(sgrid), dim3(kVThreads), 0, s, a, w, cf, ntr);
      }
    }
    {
      ProfScope prof(s, kProfResidualSelect);
      if (bf16) {
        hipLaunchKernelGGL((residual_select_kernel<true>), dim3(dgrid), dim3(kVThreads), 0, s, a, w, cf, ntv, ntr);
      } else {
        hipLaunchKernelGGL((residual_select_kernel<false>), dim3(dgrid), dim3(kVThreads), 0, s, a, w, cf, ntv, ntr);
      }
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dspark
