// dspark_survival: prefix survival products a_{b,k} = prod_{i<=k} c_{b,i} of
// the DSpark technical review, "The Hardware-Aware Prefix Scheduler".
//
// Confidence mode multiplies given confidences.  Analytical mode uses the
// acceptance probability c*_k = sum_v min(p_d^k(v), p_t^k(v)) of "Deriving the
// Acceptance-Rate Identity Behind Equation 8" (Eq. 8a), clamped to [0, 1] as
// the accept-rate label of the robotworld.top review is, at every block
// position along the drafted prefix:
//   1. target statistics for all B*gamma rows (per 1024-column tile);
//   2. per row, the target's log2 normaliser (or, at T == 0, the argmax
//      indicator x_k == argmax target_k);
//   3. the MFMA tile pass in overlap mode: bias + U for every (request,
//      position) row at once -- all drafted tokens are known, so the whole
//      (B*gamma) x r x V contraction is one dense pass -- fused with
//      sum min(p_d, p_t) over each 128-column tile.  The bias operand is the
//      Markov head's W1[x_{k-1}], or the RNN head's e_k ("Instantiation 2:
//      The RNN Head", Eq. 6) when the draft's operand rows are given: with
//      bf16 weights as two bf16 parts (hi = bf16(e), lo = bf16(e - hi)),
//      the split the RNN draft's own tile pass uses;
//   4. per request: float64 sums over tiles, clamp, cumulative product.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace dspark {

constexpr int kSThreads = 256;

struct SurvWs {
  float2* tpart;  // [B*gamma][ntv]
  float* lt2;     // [B*gamma] target log2 normaliser, or the greedy indicator
  float2* opart;  // [B*gamma][ntd]
  uint16_t* opnd; // [B*gamma][2r] two-part bf16 operand rows of an RNN draft
};

static SurvWs carve_survival(void* ws, int B, int gamma, int V) {
  const int ntv = tiles_of(V, kTgtCols);
  const size_t rows = (size_t)B * gamma;
  char* p = reinterpret_cast<char*>(ws);
  SurvWs w;
  w.tpart = reinterpret_cast<float2*>(p);
  p += align256(rows * ntv * sizeof(float2));
  w.lt2 = reinterpret_cast<float*>(p);
  p += align256(rows * sizeof(float));
  w.opart = reinterpret_cast<float2*>(p);
  p += align256(rows * tiles_of(V, kTileCols) * sizeof(float2));
  w.opnd = reinterpret_cast<uint16_t*>(p);
  return w;
}

size_t survival_workspace(int B, int gamma, int V, int r) {
  const size_t rows = (size_t)B * gamma;
  return align256(rows * tiles_of(V, kTgtCols) * sizeof(float2)) + align256(rows * sizeof(float)) +
         align256(rows * tiles_of(V, kTileCols) * sizeof(float2)) + align256(rows * 2 * r * sizeof(uint16_t));
}

// The RNN draft's operand rows e (float32) as two bf16 parts per element,
// row R = [hi(e_R) ; lo(e_R)], for the bf16 tile pass.
__global__ void split_rows_kernel(const float* E, long long n, int r, uint16_t* opnd) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const long long row = i / r;
  const int j = (int)(i - row * r);
  const float e = E[i];
  const uint16_t hi = bf16_round(e);
  const uint16_t lo = bf16_round(e - bf16_to_float(hi));
  opnd[row * 2 * r + j] = hi;
  opnd[row * 2 * r + r + j] = lo;
}

__device__ __forceinline__ bool request_valid(const int32_t* x0, const int32_t* dt, int b, int gamma, int V) {
  bool ok = x0[b] >= 0 && x0[b] < V;
  for (int k = 0; k < gamma; ++k) {
    const int t = dt[(size_t)b * gamma + k];
    ok = ok && t >= 0 && t < V;
  }
  return ok;
}

// Confidence mode: a_{b,k} = prod_{i<=k} conf_{b,i}, one thread per request.
__global__ void survival_conf_kernel(const float* conf, int B, int gamma, float* survival) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  double a = 1.0;
  for (int k = 0; k < gamma; ++k) {
    a *= (double)conf[(size_t)b * gamma + k];
    survival[(size_t)b * gamma + k] = (float)a;
  }
}

// Step 2: one workgroup per row R = b * gamma + kk.
template <bool kGreedy>
__global__ __launch_bounds__(kSThreads) void survival_tnorm_kernel(SurvivalArgs a, SurvWs w, int ntv, float cf_f) {
  __shared__ float sv[kSThreads / kWave];
  __shared__ int si[kSThreads / kWave];
  __shared__ double sred[kSThreads / kWave];
  const int R = blockIdx.x;
  const float2* P = w.tpart + (size_t)R * ntv;
  if constexpr (kGreedy) {
    float bv = -__builtin_inff();
    int bi = INT_MAX;
    for (int t = threadIdx.x; t < ntv; t += kSThreads) argmax_merge(bv, bi, P[t].x, __float_as_int(P[t].y));
    block_argmax<kSThreads>(bv, bi, sv, si);
    if (threadIdx.x == 0) w.lt2[R] = (bi == a.draft_tokens[R]) ? 1.0f : 0.0f;
  } else {
    float lm = -__builtin_inff();
    for (int t = threadIdx.x; t < ntv; t += kSThreads) lm = fmaxf(lm, P[t].x);
    const float M = block_max<kSThreads>(lm, sv);
    const double cf = (double)cf_f;
    double s = 0.0;
    for (int t = threadIdx.x; t < ntv; t += kSThreads) {
      const float2 p = P[t];
      if (p.x != -__builtin_inff()) s += (double)p.y * exp2((double)(p.x - M) * cf);
    }
    s = block_sum<kSThreads, double>(s, sred);
    if (threadIdx.x == 0) w.lt2[R] = (float)((double)M * cf + log2(s));
  }
}

// Step 4: one workgroup per request.
template <bool kGreedy>
__global__ __launch_bounds__(kSThreads) void survival_finish_kernel(SurvivalArgs a, SurvWs w, int ntd) {
  __shared__ double sred[kSThreads / kWave];
  const int b = blockIdx.x;
  const int g = a.gamma;
  const bool ok = request_valid(a.x0, a.draft_tokens, b, g, a.V);
  double prod = 1.0;
  for (int k = 0; k < g; ++k) {
    const size_t R = (size_t)b * g + k;
    double c;
    if constexpr (kGreedy) {
      c = (double)w.lt2[R];
    } else {
      double s = 0.0;
      for (int t = threadIdx.x; t < ntd; t += kSThreads) s += (double)w.opart[R * ntd + t].x;
      s = block_sum<kSThreads, double>(s, sred);
      c = fmin(1.0, fmax(0.0, s));
    }
    prod *= c;
    if (threadIdx.x == 0) {
      const float nanv = __builtin_nanf("");
      if (a.c_star) a.c_star[R] = ok ? (float)c : nanv;
      a.survival[R] = ok ? (float)prod : nanv;
    }
  }
}

hipError_t launch_survival(const SurvivalArgs& a, bool bf16, hipStream_t s) {
  if (a.conf) {
    const int threads = 256;
    ProfScope prof(s, kProfSurvivalConf);
    hipLaunchKernelGGL(survival_conf_kernel, dim3((a.B + threads - 1) / threads), dim3(threads), 0, s, a.conf, a.B,
                       a.gamma, a.survival);
    return hipGetLastError();
  }
  const bool greedy = a.temperature == 0.0f;
  const int ntv = tiles_of(a.V, kTgtCols);
  const int ntd = tiles_of(a.V, kTileCols);
  const int rows = a.B * a.gamma;
  const float cf = greedy ? 0.0f : (float)(1.4426950408889634 / (double)a.temperature);
  SurvWs w = carve_survival(a.ws, a.B, a.gamma, a.V);

  TStatsArgs t = {};
  t.target = a.target;
  t.nall = rows;
  t.rows_per_req = 1;
  t.orow_stride = 1;
  t.gamma = a.gamma;
  t.V = a.V;
  t.ntv = ntv;
  t.cf = cf;
  t.tpart = w.tpart;
  hipError_t e = launch_target_stats(t, greedy, rows, s);
  if (e != hipSuccess) return e;

  {
    ProfScope prof(s, kProfSurvivalTnorm);
    if (greedy) {
      hipLaunchKernelGGL((survival_tnorm_kernel<true>), dim3(rows), dim3(kSThreads), 0, s, a, w, ntv, cf);
    } else {
      hipLaunchKernelGGL((survival_tnorm_kernel<false>), dim3(rows), dim3(kSThreads), 0, s, a, w, ntv, cf);
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (!greedy) {
    TileArgs ta = {};
    ta.U = a.U;
    ta.W1 = a.W1;
    if (a.E != nullptr) {
      if (bf16) {
        const long long n = (long long)rows * a.r;
        hipLaunchKernelGGL(split_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.E, n, a.r,
                           w.opnd);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        ta.W1 = w.opnd;
        ta.opnd_rows = 2;
      } else {
        ta.W1 = a.E;
        ta.opnd_rows = 1;
      }
    }
    ta.W2 = a.W2;
    ta.x0 = a.x0;
    ta.tokens = a.draft_tokens;
    ta.target = a.target;
    ta.lse_d = a.draft_lse;
    ta.lt2 = w.lt2;
    ta.partials = w.opart;
    ta.nrows = rows;
    ta.kper = a.gamma;
    ta.k0 = 0;
    ta.B = a.B;
    ta.gamma = a.gamma;
    ta.V = a.V;
    ta.r = a.r;
    ta.ntiles = ntd;
    ta.cf = cf;
    e = launch_tile_pass(ta, kModeOverlap, bf16, s);
    if (e != hipSuccess) return e;
    ProfScope prof(s, kProfSurvivalFinish);
    hipLaunchKernelGGL((survival_finish_kernel<false>), dim3(a.B), dim3(kSThreads), 0, s, a, w, ntd);
  } else {
    ProfScope prof(s, kProfSurvivalFinish);
    hipLaunchKernelGGL((survival_finish_kernel<true>), dim3(a.B), dim3(kSThreads), 0, s, a, w, ntd);
  }
  return hipGetLastError();
}

}  // namespace dspark
