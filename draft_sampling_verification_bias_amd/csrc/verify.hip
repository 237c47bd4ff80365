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
// one target-statistics kernel (per-tile max / exp-sum over 256 columns) and
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
constexpr int kPreRows = 2;        // block positions of a phase whose inputs the decision kernel loads up front
constexpr int kPropPre = 16;       // residual proposals whose uniforms are drawn ahead, per position

struct FallbackInfo {
  int j;        // rejected position (1-based)
  int prev;     // x_{j-1}
  int phase_row;  // row of position j within its phase's summaries
  double M, Z;  // target row max and exp-sum (base 2, scaled by cf)
  double pdx;   // p_d^j(x_j)
  double lx;    // draft logit of x_j (U + bias), float64
};

struct VerifyWs {
  int lmax;             // longest phase (block positions)
  float2* tpart;        // [B][lmax][ntv] target tile summaries of the current phase
  int* lists;           // [gamma + 2][B] request lists per phase (index ph = 1, 2, ...)
  int* counts;          // [gamma + 2]: counts[ph] phase sizes, counts[0] fallback count
  int* fb_list;         // [B]
  FallbackInfo* fb;     // [B] indexed by request
  double* fb_part;      // [B][ntv] residual mass per tile
  float* txv;           // [B][lmax] target logit of the drafted token, current phase
  int* alive;           // [B] the phase in which the request is still undecided (0: none)
  double* lxv;          // [B][gamma] draft logit U[x_k] + W1[x_{k-1}] . W2[:, x_k] of every drafted token
  double* u_acc;        // [B][gamma] acceptance uniforms (stream 1)
  double2* u_prop;      // [B][gamma + 1][kPropPre] words 0, 1 of the first residual proposals (stream 2)
};

// Phase schedule of the block positions 1..gamma+1.  Sampling verifies
// position 1 alone (about half of the requests end there), then positions 2
// and 3, then the rest; greedy verification goes two positions at a time.
// Each phase streams the target rows of the requests still undecided.
struct Phases {
  int n;
  int k0[40], k1[40];
};

static Phases phase_schedule(int gamma, bool greedy) {
  Phases p;
  p.n = 0;
  int k = 1;
  const int last = gamma + 1;
  while (k <= last) {
    int len;
    if (greedy) {
      len = 2;
    } else {
      len = p.n == 0 ? 1 : (p.n == 1 ? 2 : last - k + 1);
    }
    p.k0[p.n] = k;
    p.k1[p.n] = min(last, k + len - 1);
    k = p.k1[p.n] + 1;
    ++p.n;
  }
  return p;
}

// Longest phase of either schedule.
static int max_phase_rows(int gamma) { return max(2, gamma + 1 - 3); }

static VerifyWs carve_verify(void* ws, int B, int gamma, int V) {
  const int ntv = tiles_of(V, kTgtCols);
  char* p = reinterpret_cast<char*>(ws);
  VerifyWs w;
  w.lmax = max_phase_rows(gamma);
  w.tpart = reinterpret_cast<float2*>(p);
  p += align256((size_t)B * w.lmax * ntv * sizeof(float2));
  w.lists = reinterpret_cast<int*>(p);
  p += align256((size_t)(gamma + 2) * B * sizeof(int));
  w.counts = reinterpret_cast<int*>(p);
  p += align256((size_t)(gamma + 2) * sizeof(int));
  w.fb_list = reinterpret_cast<int*>(p);
  p += align256((size_t)B * sizeof(int));
  w.fb = reinterpret_cast<FallbackInfo*>(p);
  p += align256((size_t)B * sizeof(FallbackInfo));
  w.fb_part = reinterpret_cast<double*>(p);  // [B][ceil(V / kResCols)]
  p += align256((size_t)B * tiles_of(V, 256) * sizeof(double));
  w.txv = reinterpret_cast<float*>(p);
  p += align256((size_t)B * w.lmax * sizeof(float));
  w.alive = reinterpret_cast<int*>(p);
  p += align256((size_t)B * sizeof(int));
  w.lxv = reinterpret_cast<double*>(p);
  p += align256((size_t)B * gamma * sizeof(double));
  w.u_acc = reinterpret_cast<double*>(p);
  p += align256((size_t)B * gamma * sizeof(double));
  w.u_prop = reinterpret_cast<double2*>(p);
  return w;
}

size_t verify_workspace(int B, int gamma, int V, int r) {
  (void)r;
  const int ntv = tiles_of(V, kTgtCols);
  const int lmax = max_phase_rows(gamma);
  return align256((size_t)B * lmax * ntv * sizeof(float2)) + align256((size_t)(gamma + 2) * B * sizeof(int)) +
         align256((size_t)(gamma + 2) * sizeof(int)) + align256((size_t)B * sizeof(int)) +
         align256((size_t)B * sizeof(FallbackInfo)) + align256((size_t)B * tiles_of(V, 256) * sizeof(double)) +
         align256((size_t)B * lmax * sizeof(float)) + align256((size_t)B * sizeof(int)) +
         align256((size_t)B * gamma * sizeof(double)) + align256((size_t)B * gamma * sizeof(double)) +
         align256((size_t)B * (gamma + 1) * kPropPre * sizeof(double2));
}

template <bool kBf16>
__device__ __forceinline__ double wval(const void* W, size_t idx) {
  if constexpr (kBf16) {
    return (double)bf16_to_float(reinterpret_cast<const uint16_t*>(W)[idx]);
  } else {
    return (double)reinterpret_cast<const float*>(W)[idx];
  }
}

// Element j of the draft's operand row at block position k (1-based) of
// request b: the RNN head's e_k (float32, "Instantiation 2: The RNN Head",
// Eq. 6) when the draft's rows are given, else the Markov head's W1[prev]
// (Eq. 5).
template <bool kBf16>
__device__ __forceinline__ double opnd_val(const VerifyArgs& a, int b, int k, int prev, int j) {
  if (a.E != nullptr) return (double)a.E[((size_t)b * a.gamma + (k - 1)) * a.r + j];
  return wval<kBf16>(a.W1, (size_t)prev * a.r + j);
}

// ---------------------------------------------------------------------------
// Target-row statistics, shared with dspark_survival.
//   list mode (list != null): row li is request list[li / rows_per_req] at
//     block position kk0 + li % rows_per_req; summaries of (b, row) go to row
//     b * orow_stride + row of tpart.
//   request mode (list == null, nreq > 0): the same rows and summary layout
//     for every request b < nreq, with no list to look up.
//   all mode: row R = b * gamma + kk for kk < gamma; summaries go to row R.
// Sample mode writes (m, sum 2^((t - m) * cf)) with m the maximum over the
// eight tiles of the tile's wave (any m >= the tile's own maximum gives the
// same tile weight); greedy mode (max t, argmax bits).
// ---------------------------------------------------------------------------
constexpr int kStatBlocksPerCU = 16;
constexpr int kStatWaveTiles = 8;                                   // tiles per wave per item
constexpr int kStatItemTiles = kStatWaveTiles * (kVThreads / kWave);  // 32 tiles = 8192 columns

// Each work item is kStatItemTiles consecutive kTgtCols-column tiles of one
// row; a wave owns kStatWaveTiles of them, a lane four consecutive columns of
// each (one 16-byte load per tile, all issued together), and every reduction
// is a wave reduction.  With tx_out set (list mode), the lane holding the
// row's drafted token also stores its target logit.  In list mode the count
// and the item's list entry are loaded together (the entry speculatively,
// from inside the list buffer), so an item waits for two dependent loads:
// those, then its row.
template <bool kGreedy>
__global__ __launch_bounds__(kVThreads) void target_stats_kernel(TStatsArgs a) {
  const int ngrp = (a.ntv + kStatItemTiles - 1) / kStatItemTiles;
  const long long items_max = (long long)a.max_rows * ngrp;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const bool full_rows = (a.V & 3) == 0;

  struct Item {
    const float* row;
    int x, orow, tw;
    bool ok;
    bool skip;  // a row past the request's scheduled bonus row: not read
  };
  // Item `it`: its row, output row, drafted token and first tile; ok is false
  // past the last row (list mode: past the device count, and so for every
  // later item of this workgroup too, the items being in row order).
  auto resolve = [&](long long it) -> Item {
    Item m;
    m.ok = it < items_max;
    m.skip = false;
    if (!m.ok) return m;
    const int li = (int)(it / ngrp);
    const int tg = (int)(it - (long long)li * ngrp);
    int b, kk;
    if (a.list) {
      const int req = li / a.rows_per_req, row = li - req * a.rows_per_req;
      const int cnt = *a.count;                        // these two loads
      b = a.list[req < a.nreq ? req : a.nreq - 1];     // go out together
      m.ok = req < cnt;
      kk = a.kk0 + row;
      m.orow = b * a.orow_stride + row;
      // with scheduled lengths, the phase's rows past the bonus row l_b + 1
      // are never decided
      m.skip = m.ok && a.lengths != nullptr && kk > a.lengths[b];
    } else if (a.nreq > 0) {
      b = li / a.rows_per_req;
      const int row = li - b * a.rows_per_req;
      kk = a.kk0 + row;
      m.orow = b * a.orow_stride + row;
    } else {
      b = li / a.gamma;
      kk = li - b * a.gamma;
      m.orow = li;
    }
    m.row = a.target + ((size_t)b * (a.gamma + 1) + kk) * (size_t)a.V;
    m.x = (m.ok && !m.skip && a.tx_out && kk < a.gamma) ? a.draft_tokens[(size_t)b * a.gamma + kk] : -1;
    m.tw = tg * kStatItemTiles + wave * kStatWaveTiles;  // first tile of this wave
    return m;
  };
  auto load = [&](const Item& m, float (&v)[kStatWaveTiles][4]) {
    if (m.skip) return;
#pragma unroll
    for (int j = 0; j < kStatWaveTiles; ++j) {
      const int c0 = (m.tw + j) * kTgtCols + 4 * lane;
      if (full_rows && c0 + 4 <= a.V) {
        const float4 q = *reinterpret_cast<const float4*>(m.row + c0);
        v[j][0] = q.x; v[j][1] = q.y; v[j][2] = q.z; v[j][3] = q.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[j][e] = c0 + e < a.V ? m.row[c0 + e] : -__builtin_inff();
      }
    }
  };
  auto reduce_store = [&](const Item& m, const float (&v)[kStatWaveTiles][4]) {
    if (m.skip) return;  // the same for every wave of the workgroup
    // per lane: one (max, sum) or (value, index) pair per tile; the drafted
    // token's logit from the lane that holds it
    float pa[kStatWaveTiles], pb[kStatWaveTiles];
    {
      // the drafted token's logit: one wave-uniform test per item, then the
      // lane that holds it picks it out with selects (no dynamic indexing)
      const int rel = m.x - m.tw * kTgtCols;
      if ((unsigned)rel < (unsigned)(kStatWaveTiles * kTgtCols)) {
        const int jx = rel / kTgtCols, cx = rel - jx * kTgtCols;
        float val = 0.0f;
#pragma unroll
        for (int j = 0; j < kStatWaveTiles; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) val = (j == jx && e == (cx & 3)) ? v[j][e] : val;
        if (lane == (cx >> 2)) a.tx_out[m.orow] = val;
      }
    }
    static_assert(kStatWaveTiles == 8, "the transposing reductions take eight tiles");
    if constexpr (kGreedy) {
#pragma unroll
      for (int j = 0; j < kStatWaveTiles; ++j) {
        const int c0 = (m.tw + j) * kTgtCols + 4 * lane;
        float bv = v[j][0];
        int bi = c0;
#pragma unroll
        for (int e = 1; e < 4; ++e) {
          if (v[j][e] > bv) {
            bv = v[j][e];
            bi = c0 + e;
          }
        }
        pa[j] = bv;
        pb[j] = __int_as_float(bi);
      }
      wave_transpose8(pa, pb, lane, MergeArgmax{});
    } else {
      // One shift for all of the wave's tiles, the wave's maximum M: every
      // tile's sum is taken relative to it, so merging sums is plain
      // addition.  A term more than 126 / cf below M may flush to zero; it
      // is below 2^-126 of the maximum's own term.
      float lm = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < kStatWaveTiles; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) lm = fmaxf(lm, v[j][e]);
      const float M = wave_max_dpp(lm);
      const float mc = M == -__builtin_inff() ? 0.0f : M * a.cf;
#pragma unroll
      for (int j = 0; j < kStatWaveTiles; ++j) {
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) sum += fast_exp2(fmaf(v[j][e], a.cf, -mc));
        pb[j] = sum;
      }
      wave_transpose_sum8(pb, lane);
      pa[0] = M;
    }
    const int t = m.tw + 4 * ((lane >> 5) & 1) + 2 * ((lane >> 4) & 1) + ((lane >> 3) & 1);
    if ((lane & 7) == 0 && t < a.ntv) a.tpart[(size_t)m.orow * a.ntv + t] = make_float2(pa[0], pb[0]);
  };

  // Grid-stride over the items with the next item's loads in flight while
  // the current one is reduced (two register sets, roles swapped each turn).
  long long it = blockIdx.x;
  Item ca = resolve(it);
  if (!ca.ok) return;
  float va[kStatWaveTiles][4], vb[kStatWaveTiles][4];
  load(ca, va);
  for (;;) {
    it += gridDim.x;
    const Item cb = resolve(it);
    if (cb.ok) load(cb, vb);
    reduce_store(ca, va);
    if (!cb.ok) return;
    it += gridDim.x;
    ca = resolve(it);
    if (ca.ok) load(ca, va);
    reduce_store(cb, vb);
    if (!ca.ok) return;
  }
}

hipError_t launch_target_stats(const TStatsArgs& a, bool greedy, int max_rows, hipStream_t s) {
  const long long items = (long long)max_rows * ((a.ntv + kStatItemTiles - 1) / kStatItemTiles);
  // a few resident workgroups per CU, each walking many items
  const long long cap = (long long)kStatBlocksPerCU * compute_units_of_device();
  const int grid = (int)(items < cap ? items : cap);
  if (grid <= 0) return hipSuccess;
  ProfScope prof(s, kProfTargetStats);
  TStatsArgs g = a;
  g.max_rows = max_rows;
  if (greedy) {
    hipLaunchKernelGGL((target_stats_kernel<true>), dim3(grid), dim3(kVThreads), 0, s, g);
  } else {
    hipLaunchKernelGGL((target_stats_kernel<false>), dim3(grid), dim3(kVThreads), 0, s, g);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Initialisation: outputs to their "not reached" values, validity check of
// every request's tokens, and the ordered list of phase 1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kVThreads) void verify_init_kernel(VerifyArgs a, VerifyWs w, int wbf16) {
  __shared__ PickScratch ps;
  const int g = a.gamma;
  const int per_req = g + (g + 1) * kPropPre;
  const int draw_blocks = (a.B * per_req + kVThreads - 1) / kVThreads;
  if (blockIdx.x > draw_blocks) {
    // The draft logit of every drafted token (needed after a rejection), one
    // wave per (request, position): l = U[x] + e . W2[:, x] with float64
    // products of the exact weights, e = W1[x_prev] or the RNN draft's e_k.
    const int item = (blockIdx.x - 1 - draw_blocks) * (kVThreads / kWave) + threadIdx.x / kWave;
    if (item >= a.B * g) return;
    const int b = item / g, k = item - b * g;  // k 0-based
    const int lane = threadIdx.x & (kWave - 1);
    const int x = a.draft_tokens[(size_t)b * g + k];
    const int prev = k == 0 ? a.x0[b] : a.draft_tokens[(size_t)b * g + k - 1];
    if ((unsigned)x >= (unsigned)a.V || (unsigned)prev >= (unsigned)a.V) return;  // invalid request
    const float* urow = a.U + ((size_t)b * g + k) * (size_t)a.V;
    double sum = 0.0;
    for (int j0 = 0; j0 < a.r; j0 += 4 * kWave) {
      float e[4], wv[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int j = j0 + lane + m * kWave;
        const int jc = j < a.r ? j : 0;
        e[m] = a.E ? a.E[((size_t)b * g + k) * a.r + jc]
                   : wbf16 ? bf16_to_float(reinterpret_cast<const uint16_t*>(a.W1)[(size_t)prev * a.r + jc])
                           : reinterpret_cast<const float*>(a.W1)[(size_t)prev * a.r + jc];
        const size_t wi = a.W2T ? (size_t)x * a.r + jc : (size_t)jc * a.V + x;
        const void* W2x = a.W2T ? a.W2T : a.W2;
        wv[m] = wbf16 ? bf16_to_float(reinterpret_cast<const uint16_t*>(W2x)[wi])
                      : reinterpret_cast<const float*>(W2x)[wi];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (j0 + lane + m * kWave < a.r) sum += (double)e[m] * (double)wv[m];
    }
    sum = wave_sum(sum);
    if (lane == 0) w.lxv[(size_t)b * g + k] = (double)urow[x] + sum;
    return;
  }
  if (blockIdx.x > 0) {
    // The random numbers of the decisions, drawn ahead so that no decision
    // waits for a Philox evaluation: per (request, position) the acceptance
    // uniform and the first kPropPre residual proposals (both words), the
    // latter also at position gamma+1 (proposal 0 there is the bonus draw).
    const int id = (blockIdx.x - 1) * kVThreads + threadIdx.x;
    if (id >= a.B * per_req) return;
    const int b = id / per_req, j = id - b * per_req;
    const uint64_t seed = a.seeds[b];
    if (j < g) {
      w.u_acc[(size_t)b * g + j] = unit_uniform(draw_block(seed, a.round, j + 1, kStreamAccept, 0).w[0]);
    } else {
      const int kk = (j - g) / kPropPre, i = (j - g) - kk * kPropPre;
      const Philox4 d = draw_block(seed, a.round, kk + 1, kStreamResidual, (uint64_t)i);
      w.u_prop[((size_t)b * (g + 1) + kk) * kPropPre + i] = make_double2(unit_uniform(d.w[0]), unit_uniform(d.w[1]));
    }
    return;
  }
  if (threadIdx.x < g + 2) w.counts[threadIdx.x] = 0;
  int running = 0;
  for (int base = 0; base < a.B; base += kVThreads) {
    const int b = base + threadIdx.x;
    int valid = 0;
    if (b < a.B) {
      valid = a.x0[b] >= 0 && a.x0[b] < a.V;
      if (a.lengths) valid &= a.lengths[b] >= 0 && a.lengths[b] <= g;
      for (int k = 0; k < g; ++k) {
        const int t = a.draft_tokens[(size_t)b * g + k];
        valid &= (t >= 0 && t < a.V);
        if (a.accept_prob) a.accept_prob[(size_t)b * g + k] = __builtin_nanf("");
      }
      for (int k = 0; k <= g; ++k) a.out_tokens[(size_t)b * (g + 1) + k] = -1;
      a.accept_len[b] = -1;
      w.alive[b] = valid ? 1 : 0;
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
// then a rescan of one kTgtCols-column tile.  `sterm` holds kTgtCols doubles.
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

// Draft logit U[v] + e . W2[:, v] in float64 with the operand row e staged in
// sw1 (all threads receive it).
template <bool kBf16>
__device__ double draft_logit(const VerifyArgs& a, const float* urow, const double* sw1, int v, double* red) {
  double s = 0.0;
  for (int j = threadIdx.x; j < a.r; j += kVThreads) s += sw1[j] * wval<kBf16>(a.W2, (size_t)j * a.V + v);
  s = block_sum<kVThreads, double>(s, red);
  return (double)urow[v] + s;
}

constexpr int kPrefixMax = 1024;  // target tiles per row on the fast decision path (V <= 262144)

// ---------------------------------------------------------------------------
// Decision kernel for rows of more than kPrefixMax tiles: the same decisions
// as verify_decide_kernel below, with block-wide searches over the tile
// summaries in global memory.
template <bool kGreedy, bool kBf16>
__global__ __launch_bounds__(kVThreads) void verify_decide_generic_kernel(VerifyArgs a, VerifyWs w, int ph, int k0,
                                                                         int k1, float cf_f, int ntv) {
  __shared__ PickScratch ps;
  __shared__ double sterm[kTgtCols];
  __shared__ double sw1[512];
  __shared__ double sred[kVThreads / kWave];
  __shared__ float sv[kVThreads / kWave];
  __shared__ int si[kVThreads / kWave];
  const int g = a.gamma;
  const int count = w.counts[ph];
  const double cf = (double)cf_f;
  for (int li = blockIdx.x; li < count; li += gridDim.x) {
    const int b = w.lists[(size_t)ph * a.B + li];
    const int lb = a.lengths ? a.lengths[b] : g;  // scheduled length (validated by the init kernel)
    for (int k = k0; k <= k1; ++k) {
      const float2* P = w.tpart + ((size_t)b * w.lmax + (k - k0)) * ntv;
      const float* trow = a.target + ((size_t)b * (g + 1) + (k - 1)) * (size_t)a.V;
      bool accepted = false;
      if constexpr (kGreedy) {
        float bv = -__builtin_inff();
        int bi = INT_MAX;
        for (int t = threadIdx.x; t < ntv; t += kVThreads) argmax_merge(bv, bi, P[t].x, __float_as_int(P[t].y));
        block_argmax<kVThreads>(bv, bi, sv, si);
        if (k <= lb) {
          const int x = a.draft_tokens[(size_t)b * g + k - 1];
          accepted = bi == x;
          if (threadIdx.x == 0) {
            if (a.accept_prob) a.accept_prob[(size_t)b * g + k - 1] = accepted ? 1.0f : 0.0f;
            a.out_tokens[(size_t)b * (g + 1) + k - 1] = accepted ? x : bi;
            if (!accepted) a.accept_len[b] = k - 1;
          }
        } else if (threadIdx.x == 0) {  // bonus token from the position after the scheduled block
          a.out_tokens[(size_t)b * (g + 1) + lb] = bi;
          a.accept_len[b] = lb;
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
        if (k > lb) {  // bonus token from the position after the scheduled block
          const double u = unit_uniform(draw_block(seed, a.round, lb + 1, kStreamResidual, 0).w[0]);
          const int y = sample_target(c, u, ps, sterm, nullptr);
          if (threadIdx.x == 0) {
            a.out_tokens[(size_t)b * (g + 1) + lb] = y;
            a.accept_len[b] = lb;
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
            for (int j = threadIdx.x; j < a.r; j += kVThreads) sw1[j] = opnd_val<kBf16>(a, b, k, prev, j);
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
        w.alive[b] = ph + 1;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decision kernel for rows of at most kPrefixMax target tiles: one workgroup
// per listed request.  Every wave takes the same decisions from the same data
// (no barrier on the acceptance path): one batch of loads brings the tile
// summaries of the phase's rows, the drafted tokens, p_d(x) and the target
// logits t(x) recorded by the statistics kernel; a second batch the draft
// logits of the drafted tokens (needed only after a rejection, loaded
// anyway).  A lane owns a contiguous share of the summaries, so the searches
// over them are ballots and shuffles.  After a rejection the residual
// proposals are evaluated 16 at a time -- four per wave, 16 lanes each --
// and the waves agree on the lowest kept proposal through LDS.
// ---------------------------------------------------------------------------
constexpr int kLaneTilesMax = kPrefixMax / kWave;                 // 16 summaries per lane
constexpr int kPropBatch = 4 * (kVThreads / kWave);               // proposals per batch

// Weight of a tile summary relative to the row maximum M (cf = log2(e) / T).
__device__ __forceinline__ double tile_weight(const float2& p, float M, float cf) {
  return p.x == -__builtin_inff() ? 0.0 : (double)p.y * (double)fast_exp2((p.x - M) * cf);
}

// The lane's share [t0, t1) of a row's tile summaries and the row's
// normaliser: M = max, Z = sum of the tile weights, incl / excl = the
// cumulative weight through / before this lane's share.
template <int kLT>
struct RowScan {
  float2 p[kLT];
  int t0, t1;
  float M;
  double local, excl, incl, Z;
};

// (Selects rather than branches, and DPP lane moves for the wave max and
// scan: this sits on the critical path of every decision.)
template <int kLT>
__device__ __forceinline__ void row_scan(RowScan<kLT>& s, float cf, double (&cumi)[kLT], unsigned& wmask) {
  float lm = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kLT; ++j) lm = s.t0 + j < s.t1 ? fmaxf(lm, s.p[j].x) : lm;
  s.M = wave_max_dpp(lm);
  double loc = 0.0;
  wmask = 0u;
#pragma unroll
  for (int j = 0; j < kLT; ++j) {
    const float e = fast_exp2((s.p[j].x - s.M) * cf);
    const bool live = s.t0 + j < s.t1 && s.p[j].x != -__builtin_inff();
    const double wt = live ? (double)s.p[j].y * (double)e : 0.0;
    wmask |= wt > 0.0 ? 1u << j : 0u;
    loc += wt;
    cumi[j] = wt;
  }
  s.local = loc;
  s.incl = wave_inclusive_scan_dpp(loc);
  s.excl = s.incl - loc;
  s.Z = lane_f64(s.incl, kWave - 1);
  double cum = s.excl;  // the lane's inclusive cumulative weights, in tile order
#pragma unroll
  for (int j = 0; j < kLT; ++j) {
    cum += cumi[j];
    cumi[j] = cum;
  }
}

// Tile of the first cumulative weight above q among positive tiles (the last
// positive tile if rounding leaves none), the cumulative weight before it
// and its maximum.  q is the same on every lane; so are the results.
template <int kLT>
__device__ __forceinline__ void tile_search(const RowScan<kLT>& s, const double (&cumi)[kLT], unsigned wmask,
                                            double q, int& ts_o, double& base_o, float& mt_o) {
  const unsigned long long cross = __ballot(s.local > 0.0 && s.incl > q);
  const unsigned long long pos = __ballot(s.local > 0.0);
  const int owner = cross ? __ffsll((long long)cross) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
  // every lane runs the owner's search (selects, no branches); the owner's
  // result is taken
  int jp = -1, jl = -1;
#pragma unroll
  for (int j = 0; j < kLT; ++j) {
    const bool on = (wmask >> j) & 1u;
    jl = on ? j : jl;
    jp = (jp < 0 && on && cumi[j] > q) ? j : jp;
  }
  const int jj = jp >= 0 ? jp : jl;
  int t = 0;
  double bb = 0.0;
  float m = s.M;
#pragma unroll
  for (int j = 0; j < kLT; ++j) {
    const bool sel = j == jj;
    t = sel ? s.t0 + j : t;
    bb = sel ? (j == 0 ? s.excl : cumi[j > 0 ? j - 1 : 0]) : bb;
    m = sel ? s.p[j].x : m;
  }
  ts_o = lane_i32(t, owner);
  base_o = lane_f64(bb, owner);
  mt_o = lane_f32(m, owner);
}

// Within each group of kW lanes (16 or 64): the column of target tile ts
// (kTgtCols columns, kTgtCols / kW per lane) whose cumulative weight first
// exceeds ql (the last positive one if none), and its target logit.  ts, mt,
// ql may differ between groups.
template <int kW>
__device__ __forceinline__ void col_draw(const float* trow, int V, int ts, float mt, float M, float cf_f, double cf,
                                         double ql, int& v_out, float& x_out) {
  constexpr int kC = kTgtCols / kW;  // columns per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane & (kW - 1), gbase = lane & ~(kW - 1);
  const int c0 = ts * kTgtCols + kC * li;
  float x[kC];
  if ((V & 3) == 0 && c0 + kC <= V) {
#pragma unroll
    for (int j = 0; j < kC / 4; ++j) {
      const float4 q = *reinterpret_cast<const float4*>(trow + c0 + 4 * j);
      x[4 * j] = q.x; x[4 * j + 1] = q.y; x[4 * j + 2] = q.z; x[4 * j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      const int c = c0 + j < V ? c0 + j : V - 1;
      const float v = trow[c];
      x[j] = c0 + j < V ? v : -__builtin_inff();
    }
  }
  const double scale = exp2((double)(mt - M) * cf);
  float e[kC];
  double local = 0.0;
#pragma unroll
  for (int j = 0; j < kC; ++j) {
    e[j] = x[j] == -__builtin_inff() ? 0.0f : fast_exp2((x[j] - mt) * cf_f);
    local += (double)e[j] * scale;
  }
  double incl = local;
#pragma unroll
  for (int o = 1; o < kW; o <<= 1) {
    const double y = __shfl_up(incl, o);
    if (li >= o) incl += y;
  }
  const double excl = incl - local;
  const unsigned long long gmask = kW == 64 ? ~0ull : (((1ull << kW) - 1ull) << gbase);
  const unsigned long long cross = __ballot(local > 0.0 && incl > ql) & gmask;
  const unsigned long long pos = __ballot(local > 0.0) & gmask;
  const int owner = cross ? __ffsll((long long)cross) - 1 : (pos ? 63 - __clzll((long long)pos) : gbase);
  int col = -1;
  float xc = 0.0f;
  if (lane == owner) {
    double cum = excl;
    int lastp = -1;
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      const double t = (double)e[j] * scale;
      if (t > 0.0) {
        lastp = j;
        if (col < 0 && cum + t > ql) col = j;
      }
      cum += t;
    }
    if (col < 0) col = lastp < 0 ? 0 : lastp;
#pragma unroll
    for (int j = 0; j < kC; ++j)
      if (j == col) xc = x[j];
    col += c0;
  }
  v_out = __shfl(col, owner);
  x_out = __shfl(xc, owner);
}

// Draft logit U[v] + e . W2[:, v] in float64, summed by a group of kW lanes
// (lane li takes k = li + kW m); v may differ between groups.  e is the RNN
// draft's operand row erow when given, else W1[prev].
template <int kW, bool kBf16>
__device__ __forceinline__ double draft_logit_at(const VerifyArgs& a, const float* urow, const float* erow, int prev,
                                                 int v) {
  constexpr int kCh = 256 / kW;  // products per lane per 256 k
  const int li = threadIdx.x & (kW - 1);
  const float uv = urow[v];
  double s = 0.0;
  for (int k0 = 0; k0 < a.r; k0 += 256) {
    float e[kCh], wv[kCh];
#pragma unroll
    for (int m = 0; m < kCh; ++m) {
      const int k = k0 + li + kW * m;
      const int kc = k < a.r ? k : 0;  // clamped: all loads issued before the first use
      e[m] = erow ? erow[kc] : (float)wval<kBf16>(a.W1, (size_t)prev * a.r + kc);
      // with the transposed copy, the k of one load instruction are contiguous
      wv[m] = a.W2T ? (float)wval<kBf16>(a.W2T, (size_t)v * a.r + kc) : (float)wval<kBf16>(a.W2, (size_t)kc * a.V + v);
    }
#pragma unroll
    for (int m = 0; m < kCh; ++m)
      if (k0 + li + kW * m < a.r) s += (double)e[m] * (double)wv[m];
  }
#pragma unroll
  for (int o = 1; o < kW; o <<= 1) s += __shfl_xor(s, o);
  return (double)uv + s;
}

// Words 0 and 1 of residual proposal i as uniforms (kept out of line: only
// proposals past the first batch, which are rare, evaluate it here).
__device__ __noinline__ double2 proposal_uniforms(uint64_t seed, uint64_t round, int k, int i) {
  const Philox4 d = draw_block(seed, round, k, kStreamResidual, (uint64_t)i);
  return make_double2(unit_uniform(d.w[0]), unit_uniform(d.w[1]));
}

template <bool kGreedy, bool kBf16, int kLT>
__global__ __launch_bounds__(kVThreads) void verify_decide_kernel(VerifyArgs a, VerifyWs w, int ph, int k0, int k1,
                                                                 float cf_f, int ntv) {
  constexpr int kWaves = kVThreads / kWave;
  __shared__ int s_idx[kWaves], s_tok[kWaves], s_last;
  __shared__ double s_cum[kPrefixMax];  // inclusive cumulative tile weights (later proposal batches)
  __shared__ float s_m[kPrefixMax];     // tile maxima
  const int g = a.gamma;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int b = blockIdx.x;
  const int cs = (ntv + kWave - 1) / kWave;
  const int t0 = min(ntv, lane * cs), t1 = min(ntv, t0 + cs);

  // One batch of loads, all addressed by the request id: whether the request
  // is undecided in this phase, the summaries of the phase's rows, tokens,
  // p_d(x), t(x) and the draft logit of x, and the uniforms drawn ahead.
  const int alive = w.alive[b];
  const int lb = a.lengths ? a.lengths[b] : g;  // scheduled length (validated by the init kernel)
  // The inputs of one block position of the phase (row rr of the phase's
  // summaries); positions past k1 are clamped so that every load stays in
  // bounds (their values are not used).
  struct RowIn {
    int x, prev;
    float pdx, tx;
    double ua, lx;
    double2 up;  // lane l: proposal l % 16 of the row (proposal 0 of row gamma+1: the bonus)
  };
  auto load_row = [&](int rr, RowScan<kLT>& rsr, RowIn& in) {
    const int rc = min(rr, w.lmax - 1);
    const float2* P = w.tpart + ((size_t)b * w.lmax + rc) * ntv;
    rsr.t0 = t0;
    rsr.t1 = t1;
#pragma unroll
    for (int j = 0; j < kLT; ++j) {
      const int t = t0 + j;
      rsr.p[j] = P[t < t1 ? t : (t1 > 0 ? t1 - 1 : 0)];
    }
    const int kc = min(k0 + rr, g);
    in.x = a.draft_tokens[(size_t)b * g + kc - 1];
    if constexpr (!kGreedy) {
      in.prev = kc == 1 ? a.x0[b] : a.draft_tokens[(size_t)b * g + kc - 2];
      in.pdx = a.draft_prob[(size_t)b * g + kc - 1];
      in.tx = w.txv[(size_t)b * w.lmax + rc];
      in.lx = w.lxv[(size_t)b * g + kc - 1];
      in.ua = w.u_acc[(size_t)b * g + kc - 1];
      const int kp = min(k0 + rr, g + 1);
      in.up = w.u_prop[((size_t)b * (g + 1) + kp - 1) * kPropPre + (lane & (kPropPre - 1))];
    }
  };
  RowScan<kLT> rs[kPreRows];
  RowIn rin[kPreRows];
#pragma unroll
  for (int rr = 0; rr < kPreRows; ++rr) load_row(rr, rs[rr], rin[rr]);
  if (alive != ph) return;

  // accepted through the last position of the phase: undecided in the next
  auto carry_on = [&]() {
    if (threadIdx.x == 0) {
      const int pos = atomicAdd(&w.counts[ph + 1], 1);
      w.lists[(size_t)(ph + 1) * a.B + pos] = b;
      w.alive[b] = ph + 1;
    }
  };

  if constexpr (kGreedy) {  // greedy phases have at most kPreRows positions
#pragma unroll
    for (int rr = 0; rr < kPreRows; ++rr) {
      const int k = k0 + rr;
      if (k > k1) break;
      float bv = -__builtin_inff();
      int bi = INT_MAX;
#pragma unroll
      for (int j = 0; j < kLT; ++j)
        if (t0 + j < t1) argmax_merge(bv, bi, rs[rr].p[j].x, __float_as_int(rs[rr].p[j].y));
      wave_argmax(bv, bi);
      bool accepted = false;
      if (k <= lb) {
        accepted = bi == rin[rr].x;
        if (threadIdx.x == 0) {
          if (a.accept_prob) a.accept_prob[(size_t)b * g + k - 1] = accepted ? 1.0f : 0.0f;
          a.out_tokens[(size_t)b * (g + 1) + k - 1] = accepted ? rin[rr].x : bi;
          if (!accepted) a.accept_len[b] = k - 1;
        }
      } else if (threadIdx.x == 0) {  // bonus token from the position after the scheduled block
        a.out_tokens[(size_t)b * (g + 1) + lb] = bi;
        a.accept_len[b] = lb;
      }
      if (!accepted) return;
      if (k == k1) carry_on();
    }
  } else {
    const uint64_t seed = a.seeds[b];
    const double cf = (double)cf_f;
    // One block position; returns true when the request is finished (a
    // rejection, or the bonus token).
    auto position = [&](int rr, RowScan<kLT>& s, int x, int prev, float pdxf, float tx, double lx, double uacc,
                        double2 up0) -> bool {
      const int k = k0 + rr;
      double cumi[kLT];
      unsigned wmask;
      row_scan(s, cf_f, cumi, wmask);
      const float* trow = a.target + ((size_t)b * (g + 1) + (k - 1)) * (size_t)a.V;
      if (k > lb) {  // bonus token from the position after the scheduled block
        const double q = __shfl(up0.x, 0) * s.Z;
        int ts;
        double base;
        float mt;
        tile_search(s, cumi, wmask, q, ts, base, mt);
        int y;
        float ty;
        col_draw<kWave>(trow, a.V, ts, mt, s.M, cf_f, cf, q - base, y, ty);
        if (threadIdx.x == 0) {
          a.out_tokens[(size_t)b * (g + 1) + lb] = y;
          a.accept_len[b] = lb;
        }
        return true;
      }
      const double ptx = exp2((double)(tx - s.M) * cf) / s.Z;
      const double pdx = (double)pdxf;
      const double alpha = fmin(1.0, ptx / pdx);
      const bool accepted = uacc < alpha;
      if (threadIdx.x == 0) {
        if (a.accept_prob) a.accept_prob[(size_t)b * g + k - 1] = (float)alpha;
        if (accepted) a.out_tokens[(size_t)b * (g + 1) + k - 1] = x;
      }
      if (accepted) {
        if (k == k1) carry_on();
        return false;
      }

      // Rejected at k: residual draw by proposals from p_t.  Proposal i is
      // kept with probability max(0, 1 - p_d(v) / p_t(v)); the lowest kept i
      // wins.  Proposals go in batches of 16, four per wave (16 lanes each):
      // with the acceptance rates of typical drafts a batch of 16 almost
      // always holds a kept proposal, so a second batch (another three
      // dependent memory round trips) is rare.
      const float* urow = a.U + ((size_t)b * g + (k - 1)) * (size_t)a.V;
      const float* erow = a.E ? a.E + ((size_t)b * g + (k - 1)) * a.r : nullptr;
      auto keep_test = [&](double ua, int v, float tv, double lv) -> bool {
        const double ptv = exp2((double)(tv - s.M) * cf) / s.Z;
        const double pdv = pdx * exp((lv - lx) * a.inv_t_d);
        return ua < fmax(0.0, 1.0 - pdv / ptv);
      };
      // lowest kept proposal index over the waves (every wave receives it)
      auto agree = [&](int idx, int tok, int& best, int& btok) {
        if (lane == 0) {
          s_idx[wave] = idx;
          s_tok[wave] = tok;
        }
        __syncthreads();
        best = INT_MAX;
        btok = -1;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          if (s_idx[ww] < best) {
            best = s_idx[ww];
            btok = s_tok[ww];
          }
        }
        __syncthreads();
      };
      int found = INT_MAX, ytok = -1;
      const int grp = lane >> 4;
      // Each group's tile search is a binary search over an LDS copy of the
      // cumulative weights: the first tile whose inclusive cumulative weight
      // exceeds q (it has positive weight), else the last positive tile --
      // the rule of tile_search.
      if (wave == 0) {
#pragma unroll
        for (int j = 0; j < kLT; ++j) {
          if (s.t0 + j < s.t1) {
            s_cum[s.t0 + j] = cumi[j];
            s_m[s.t0 + j] = s.p[j].x;
          }
        }
        const unsigned long long pl = __ballot(wmask != 0u);
        const int lw = pl ? 63 - __clzll((long long)pl) : 0;
        if (lane == lw) s_last = wmask ? s.t0 + 31 - __clz(wmask) : 0;
      }
      __syncthreads();
      for (int i0 = 0; found == INT_MAX && i0 < DSPARK_MAX_RESIDUAL_PROPOSALS; i0 += kPropBatch) {
        // uniforms of the batch: lane l holds proposal i0 + l % 16
        const int ip = i0 + (lane & 15);
        const double sx = __shfl(up0.x, ip & (kPropPre - 1)), sy = __shfl(up0.y, ip & (kPropPre - 1));
        double2 pb = make_double2(sx, sy);
        if (ip >= kPropPre) pb = proposal_uniforms(seed, a.round, k, ip);
        // this group's proposal: i0 + 4 wave + grp
        const int il = 4 * wave + grp;
        const double q = __shfl(pb.x, il) * s.Z;
        const double ua = __shfl(pb.y, il);
        int lo = 0, hi = ntv;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s_cum[mid] > q) hi = mid; else lo = mid + 1;
        }
        const int ts = lo < ntv ? lo : s_last;
        const double ql = q - (ts > 0 ? s_cum[ts - 1] : 0.0);
        const float mt = s_m[ts];
        int v;
        float tv;
        col_draw<16>(trow, a.V, ts, mt, s.M, cf_f, cf, ql, v, tv);
        const double lv = draft_logit_at<16, kBf16>(a, urow, erow, prev, v);
        const int i = i0 + 4 * wave + grp;
        const bool pass = i < DSPARK_MAX_RESIDUAL_PROPOSALS && keep_test(ua, v, tv, lv);
        const unsigned long long kept = __ballot(pass && (lane & 15) == 0);
        const int gi = kept ? (__ffsll((long long)kept) - 1) >> 4 : -1;
        const int tok = __shfl(v, gi < 0 ? 0 : 16 * gi);
        agree(gi < 0 ? INT_MAX : i0 + 4 * wave + gi, tok, found, ytok);
      }
      if (threadIdx.x == 0) {
        a.accept_len[b] = k - 1;
        if (found != INT_MAX) {
          a.out_tokens[(size_t)b * (g + 1) + k - 1] = ytok;
        } else {
          FallbackInfo f;
          f.j = k;
          f.prev = prev;
          f.phase_row = rr;
          f.M = (double)s.M;
          f.Z = s.Z;
          f.pdx = pdx;
          f.lx = lx;
          w.fb[b] = f;
          const int pos = atomicAdd(&w.counts[0], 1);
          w.fb_list[pos] = b;
        }
      }
      return true;
    };
    // Rows in a rolled loop over a selected copy of the row state (one copy
    // of the code; the selects stay in registers); positions past the first
    // kPreRows of the phase load their inputs when they are reached.
#pragma unroll 1
    for (int rr = 0; k0 + rr <= k1; ++rr) {
      RowScan<kLT> cur;
      RowIn in;
      if (rr < kPreRows) {
        const bool r1 = rr == 1;
#pragma unroll
        for (int j = 0; j < kLT; ++j) cur.p[j] = r1 ? rs[1].p[j] : rs[0].p[j];
        cur.t0 = t0;
        cur.t1 = t1;
        in = r1 ? rin[1] : rin[0];
      } else {
        load_row(rr, cur, in);
      }
      if (position(rr, cur, in.x, in.prev, in.pdx, in.tx, in.lx, in.ua, in.up)) return;
    }
  }
}

// ---------------------------------------------------------------------------
// Exact residual fallback: mass of max(0, p_t - p_d) per 256-column chunk,
// then one inverse-CDF draw with the stream-3 uniform.  p_d needs the bias at
// every column of the row, so each chunk rebuilds 256 bias values: thread t
// owns columns 4 (t % 64) .. +3 of the chunk and a quarter of the r products,
// kResBatch W2 rows of loads in flight at a time; the quarters are summed in
// LDS in a fixed order.  Up to kResGroup fallback requests share each W2 load (their
// biases are accumulated side by side, each in the same order as alone), and
// both kernels run this one function, so they obtain bit-identical residual
// terms.
// ---------------------------------------------------------------------------
constexpr int kResCols = 256;
constexpr int kResGroup = 4;  // fallback requests per residual-mass item
constexpr int kResBatch = 16;  // W2 rows per load batch of a thread

struct ResGroup {
  int n;                    // requests in the group (1..kResGroup)
  int b[kResGroup];
  FallbackInfo f[kResGroup];
};

// The operand rows of the group's requests into sw1f.
template <bool kBf16>
__device__ void residual_rows(const VerifyArgs& a, const ResGroup& rg, float (*sw1f)[512]) {
  for (int i = 0; i < rg.n; ++i)
    for (int j = threadIdx.x; j < a.r; j += kVThreads)
      sw1f[i][j] = (float)opnd_val<kBf16>(a, rg.b[i], rg.f[i].j, rg.f[i].prev, j);
  __syncthreads();
}

// Residual terms of column chunk * kResCols + threadIdx.x for the group's
// requests (res[i], i < rg.n); sw1f[i] holds request i's operand row.
template <bool kBf16>
__device__ void residual_terms(const VerifyArgs& a, const ResGroup& rg, int chunk, const float (*sw1f)[512],
                               float (*sbias)[4][kResCols], double cf, double (&res)[kResGroup]) {
  const int g = a.gamma;
  const int quad = threadIdx.x & 63, slice = threadIdx.x >> 6;
  const int kq = a.r / 4;  // r % 16 == 0
  const int c = chunk * kResCols + 4 * quad;
  float acc[kResGroup][4];
#pragma unroll
  for (int i = 0; i < kResGroup; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = 0.0f;
  const bool vec = kBf16 && (c + 4 <= a.V) && ((a.V & 3) == 0);
  for (int j0 = slice * kq; j0 < (slice + 1) * kq; j0 += kResBatch) {
    float wv[kResBatch][4];
#pragma unroll
    for (int jj = 0; jj < kResBatch; ++jj) {
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
    for (int i = 0; i < kResGroup; ++i) {
      if (i >= rg.n) break;
#pragma unroll
      for (int jj = 0; jj < kResBatch; ++jj) {
        const float e = j0 + jj < (slice + 1) * kq ? sw1f[i][j0 + jj] : 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(e, wv[jj][q], acc[i][q]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kResGroup; ++i) {
    if (i >= rg.n) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) sbias[i][slice][4 * quad + q] = acc[i][q];
  }
  __syncthreads();
  const int v = chunk * kResCols + threadIdx.x;
#pragma unroll
  for (int i = 0; i < kResGroup; ++i) {
    res[i] = 0.0;
    if (i >= rg.n || v >= a.V) continue;
    const int b = rg.b[i];
    const FallbackInfo& f = rg.f[i];
    const float bias = (sbias[i][0][threadIdx.x] + sbias[i][1][threadIdx.x]) +
                       (sbias[i][2][threadIdx.x] + sbias[i][3][threadIdx.x]);
    const float t = a.target[((size_t)b * (g + 1) + (f.j - 1)) * (size_t)a.V + v];
    const float uu = a.U[((size_t)b * g + (f.j - 1)) * (size_t)a.V + v];
    const double pt = t == -__builtin_inff() ? 0.0 : exp2((double)(t - (float)f.M) * cf) / f.Z;
    const double pd = uu == -__builtin_inff() ? 0.0 : f.pdx * exp(((double)uu + (double)bias - f.lx) * a.inv_t_d);
    res[i] = fmax(0.0, pt - pd);
  }
  __syncthreads();
}

// Items are (chunk, group of kResGroup fallback requests), numbered so that
// every group of one chunk has the same index mod 8: with a grid that is a
// multiple of 8 they run on one XCD (workgroups are dealt to the XCDs round
// robin), whose L2 then holds that chunk's W2 columns for all of them.
template <bool kBf16>
__global__ __launch_bounds__(kVThreads) void residual_stats_kernel(VerifyArgs a, VerifyWs w, float cf_f, int ntr) {
  __shared__ float sw1f[kResGroup][512];
  __shared__ float sbias[kResGroup][4][kResCols];
  __shared__ double sred[kVThreads / kWave];
  const int count = w.counts[0];
  const int ngroups = (count + kResGroup - 1) / kResGroup;
  const long long items = 8LL * ((ntr + 7) / 8) * ngroups;
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const long long y = it >> 3;
    const int chunk = (int)(y / ngroups) * 8 + (int)(it & 7);
    const int grp = (int)(y % ngroups);
    if (chunk >= ntr) continue;
    ResGroup rg;
    rg.n = min(kResGroup, count - grp * kResGroup);
    for (int i = 0; i < rg.n; ++i) {
      rg.b[i] = w.fb_list[grp * kResGroup + i];
      rg.f[i] = w.fb[rg.b[i]];
    }
    residual_rows<kBf16>(a, rg, sw1f);
    double res[kResGroup];
    residual_terms<kBf16>(a, rg, chunk, sw1f, sbias, (double)cf_f, res);
    for (int i = 0; i < rg.n; ++i) {
      const double s = block_sum<kVThreads, double>(res[i], sred);
      if (threadIdx.x == 0) w.fb_part[(size_t)rg.b[i] * ntr + chunk] = s;
    }
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kVThreads) void residual_select_kernel(VerifyArgs a, VerifyWs w, float cf_f, int ntv,
                                                                   int ntr) {
  __shared__ PickScratch ps;
  __shared__ double sterm[kTgtCols];
  __shared__ float sw1f[kResGroup][512];
  __shared__ float sbias[kResGroup][4][kResCols];
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
      // the chosen chunk's terms again, by the same function as the masses
      ResGroup rg;
      rg.n = 1;
      rg.b[0] = b;
      rg.f[0] = f;
      residual_rows<kBf16>(a, rg, sw1f);
      double res[kResGroup];
      residual_terms<kBf16>(a, rg, ts, sw1f, sbias, (double)cf_f, res);
      sterm[threadIdx.x] = res[0];
      __syncthreads();
      auto col_weight = [&](int j) -> double { return sterm[j]; };
      int col = block_pick_target<kVThreads>(kResCols, col_weight, u * total - base, ps, nullptr);
      if (col < 0) col = 0;
      y = ts * kResCols + col;
    } else {
      // No residual mass (possible only through rounding): draw from p_t.
      DecideCtx c;
      c.P = w.tpart + ((size_t)b * w.lmax + f.phase_row) * ntv;
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
// The decision kernel instantiated for the smallest summaries-per-lane count
// that covers ntv (its row searches are unrolled over that count).
template <bool kGreedy, bool kBf16>
static void launch_decide(const VerifyArgs& a, const VerifyWs& w, int ph, int k0, int k1, float cf, int ntv,
                          hipStream_t s) {
  const int per = (ntv + kWave - 1) / kWave;
  if (per <= 8) {
    hipLaunchKernelGGL((verify_decide_kernel<kGreedy, kBf16, 8>), dim3(a.B), dim3(kVThreads), 0, s, a, w, ph, k0, k1,
                       cf, ntv);
  } else if (per <= 10) {
    hipLaunchKernelGGL((verify_decide_kernel<kGreedy, kBf16, 10>), dim3(a.B), dim3(kVThreads), 0, s, a, w, ph, k0, k1,
                       cf, ntv);
  } else if (per <= 12) {
    hipLaunchKernelGGL((verify_decide_kernel<kGreedy, kBf16, 12>), dim3(a.B), dim3(kVThreads), 0, s, a, w, ph, k0, k1,
                       cf, ntv);
  } else {
    static_assert(kLaneTilesMax == 16, "largest instantiation covers kPrefixMax");
    hipLaunchKernelGGL((verify_decide_kernel<kGreedy, kBf16, 16>), dim3(a.B), dim3(kVThreads), 0, s, a, w, ph, k0, k1,
                       cf, ntv);
  }
}

hipError_t launch_verify(const VerifyArgs& a_in, bool bf16, hipStream_t s) {
  VerifyArgs a = a_in;
  const bool greedy = a.temperature == 0.0f;
  a.inv_t_d = greedy ? 0.0 : 1.0 / (double)a.temperature;
  const int ntv = tiles_of(a.V, kTgtCols);
  const float cf = greedy ? 0.0f : (float)(1.4426950408889634 / (double)a.temperature);
  VerifyWs w = carve_verify(a.ws, a.B, a.gamma, a.V);

  {
    ProfScope prof(s, kProfVerifyInit);
    // block 0: outputs and lists; then the uniforms; then the draft logits
    const long long draws = (long long)a.B * (a.gamma + (a.gamma + 1) * kPropPre);
    const long long draw_blocks = (draws + kVThreads - 1) / kVThreads;
    const long long lx_blocks = ((long long)a.B * a.gamma + kVThreads / kWave - 1) / (kVThreads / kWave);
    const int grid = greedy ? 1 : (int)(1 + draw_blocks + lx_blocks);
    hipLaunchKernelGGL(verify_init_kernel, dim3(grid), dim3(kVThreads), 0, s, a, w, bf16 ? 1 : 0);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int dgrid = a.B < 2048 ? a.B : 2048;
  const Phases sched = phase_schedule(a.gamma, greedy);
  for (int pi = 0; pi < sched.n; ++pi) {
    const int ph = pi + 1;
    const int k0 = sched.k0[pi], k1 = sched.k1[pi];
    TStatsArgs t = {};
    t.target = a.target;
    // phase 1 tests every valid request: read its rows without the list
    t.list = pi == 0 ? nullptr : w.lists + (size_t)ph * a.B;
    t.count = w.counts + ph;
    t.nreq = a.B;
    t.kk0 = k0 - 1;
    t.rows_per_req = k1 - k0 + 1;
    t.orow_stride = w.lmax;
    t.gamma = a.gamma;
    t.V = a.V;
    t.ntv = ntv;
    t.cf = cf;
    t.tpart = w.tpart;
    t.draft_tokens = a.draft_tokens;
    t.tx_out = greedy ? nullptr : w.txv;
    t.lengths = a.lengths;
    e = launch_target_stats(t, greedy, a.B * t.rows_per_req, s);
    if (e != hipSuccess) return e;
    ProfScope prof(s, kProfVerifyDecide);
    if (ntv <= kPrefixMax) {  // one workgroup per request (those not undecided in this phase exit)
      if (greedy) {
        launch_decide<true, true>(a, w, ph, k0, k1, cf, ntv, s);
      } else if (bf16) {
        launch_decide<false, true>(a, w, ph, k0, k1, cf, ntv, s);
      } else {
        launch_decide<false, false>(a, w, ph, k0, k1, cf, ntv, s);
      }
    } else if (greedy) {
      hipLaunchKernelGGL((verify_decide_generic_kernel<true, true>), dim3(dgrid), dim3(kVThreads), 0, s, a, w, ph, k0,
                         k1, cf, ntv);
    } else if (bf16) {
      hipLaunchKernelGGL((verify_decide_generic_kernel<false, true>), dim3(dgrid), dim3(kVThreads), 0, s, a, w, ph,
                         k0, k1, cf, ntv);
    } else {
      hipLaunchKernelGGL((verify_decide_generic_kernel<false, false>), dim3(dgrid), dim3(kVThreads), 0, s, a, w, ph,
                         k0, k1, cf, ntv);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!greedy) {
    const int ntr = tiles_of(a.V, kResCols);
    // the most items the fallback can have (every request falling back): a
    // multiple of 8, as the grid then is
    const long long items = 8LL * ((ntr + 7) / 8) * ((a.B + kResGroup - 1) / kResGroup);
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
