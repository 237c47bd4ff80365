// dspark_schedule: the hardware-aware prefix scheduler of the DSpark technical
// review, "The Hardware-Aware Prefix Scheduler" (Algorithm 1).
//
// Every (request r, position j) with survival a_{r,j} > 0 is a candidate.
// Taken in descending a (ties: lowest request, then lowest position), the
// m-th admission makes the verified batch B + m tokens and the expected
// accepted count tau(m) = B + (sum of the first m survivals); Theta(m) =
// tau(m) SPS(B + m).  The scan keeps admitting while Theta improves and stops
// at the first admission that does not (the non-anticipating early stop), so
// the admitted set is the longest prefix m* of the sorted candidates with
// Theta(0) < Theta(1) < ... < Theta(m*).  Each request's length is the largest
// position admitted for it; survivals that do not increase along a request's
// block make the admitted positions of every request contiguous from 1.
//
// One workgroup: candidate keys (descending survival, then index) are sorted
// in LDS by a bitonic network, the sorted survivals are summed in float64 by
// a block scan, every thread tests Theta at its own admission counts, and the
// first non-improving count is found by an LDS atomic minimum.
#include <limits.h>

#include "common.hpp"
#include "launch.hpp"

namespace dspark {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / kWave;

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const float* __restrict__ surv,
                                                                 const double* __restrict__ sps, int B, int gamma,
                                                                 int32_t* __restrict__ lengths, double* theta_out) {
  __shared__ unsigned long long key[kScheduleMax];
  __shared__ int len[kScheduleMax];
  __shared__ double wtot[kSchedWaves];
  __shared__ int s_valid, s_stop;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int n = B * gamma;
  int np2 = 1;
  while (np2 < n) np2 <<= 1;

  if (tid == 0) {
    s_valid = 0;
    s_stop = INT_MAX;
  }
  for (int i = tid; i < B; i += kSchedThreads) len[i] = 0;
  __syncthreads();
  // Key of candidate i = r gamma + (j - 1): the complemented bits of its
  // (positive) survival above its index, so ascending keys are descending
  // survivals with ties in index order.  Non-candidates (a <= 0 or NaN) and
  // the padding sort last.
  int mine = 0;
  for (int i = tid; i < np2; i += kSchedThreads) {
    unsigned long long k = ~0ull;
    if (i < n) {
      const float v = surv[i];
      if (v > 0.0f) {
        k = ((unsigned long long)(~__float_as_uint(v)) << 32) | (unsigned)i;
        ++mine;
      }
    }
    key[i] = k;
  }
  if (mine) atomicAdd(&s_valid, mine);
  __syncthreads();

  for (int k = 2; k <= np2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < np2; i += kSchedThreads) {
        const int p = i ^ j;
        if (p > i) {
          const unsigned long long x = key[i], y = key[p];
          if ((x > y) == ((i & k) == 0)) {
            key[i] = y;
            key[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }

  // Thread t owns the sorted candidates [t per, t per + per) of the M valid.
  const int M = s_valid;
  const int per = (M + kSchedThreads - 1) / kSchedThreads;
  const int c0 = min(M, tid * per), c1 = min(M, c0 + per);
  auto value = [&](int pos) -> double { return (double)__uint_as_float(~(unsigned)(key[pos] >> 32)); };
  double local = 0.0;
  for (int pos = c0; pos < c1; ++pos) local += value(pos);
  // exclusive block scan of the thread sums
  double incl = local;
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wtot[wave] = incl;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  const double S0 = base + incl - local;  // sum of the survivals sorted before c0

  // Theta(m) against Theta(m - 1) at this thread's admission counts m = pos + 1
  const double Bd = (double)B;
  double S = S0;
  double prev_theta = (Bd + S) * sps[B + c0];
  for (int pos = c0; pos < c1; ++pos) {
    S += value(pos);
    const double theta = (Bd + S) * sps[B + pos + 1];
    if (!(theta > prev_theta)) {
      atomicMin(&s_stop, pos + 1);
      break;
    }
    prev_theta = theta;
  }
  __syncthreads();
  const int mstar = s_stop == INT_MAX ? M : s_stop - 1;

  for (int pos = tid; pos < mstar; pos += kSchedThreads) {
    const unsigned idx = (unsigned)key[pos];
    atomicMax(&len[idx / (unsigned)gamma], (int)(idx % (unsigned)gamma) + 1);
  }
  // Theta_best = Theta(m*), summed in the order of the comparisons above by
  // the thread that owns candidate m* - 1
  if (theta_out != nullptr) {
    if (mstar == 0) {
      if (tid == 0) *theta_out = Bd * sps[B];
    } else if (c0 < mstar && mstar <= c1) {
      double s = S0;
      for (int pos = c0; pos < mstar; ++pos) s += value(pos);
      *theta_out = (Bd + s) * sps[B + mstar];
    }
  }
  __syncthreads();
  for (int i = tid; i < B; i += kSchedThreads) lengths[i] = len[i];
}

hipError_t launch_schedule(const float* survival, const double* sps, int B, int gamma, int32_t* lengths,
                           double* theta, hipStream_t s) {
  ProfScope prof(s, kProfSchedule);
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, s, survival, sps, B, gamma, lengths, theta);
  return hipGetLastError();
}

}  // namespace dspark
