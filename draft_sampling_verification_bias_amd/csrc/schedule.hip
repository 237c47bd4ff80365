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
// Two more modes serve the asynchronous adaptation of "The Asynchronous Fix,
// and Why It Stays Lossless": the capacity search takes the first maximum of
// Theta over every admission count (no early stop; run on earlier survival
// products), and the top-K mode admits the first K sorted candidates of the
// current products, K decided earlier.
//
// One workgroup: candidate keys (descending survival, then index) are sorted
// by a bitonic network held in registers (shuffles within a wave, LDS only for
// partners in other waves), the sorted survivals are summed in float64 by a
// block scan, every thread tests Theta at its own admission counts, and the
// first non-improving count is found by an LDS atomic minimum.  Up to 16 keys
// per lane (16384 candidates); the key array (up to 128 KB of LDS) is reused
// for the per-request lengths once the scan has read it.
#include <limits.h>

#include "common.hpp"
#include "launch.hpp"

namespace dspark {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kSchedPer = kScheduleMax / kSchedThreads;  // keys per lane at most (16)

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long x, int m) {
  const unsigned lo = __shfl_xor((unsigned)x, m), hi = __shfl_xor((unsigned)(x >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
}

// Compare-exchange of two keys: ascending order if up.
__device__ __forceinline__ void cmp_swap(unsigned long long& a, unsigned long long& b, bool up) {
  const unsigned long long lo = a < b ? a : b, hi = a < b ? b : a;
  a = up ? lo : hi;
  b = up ? hi : lo;
}

// kE keys per lane: the sort covers 1024 kE keys (kE = 1, 2, 4, 8 or 16),
// every stage of the network is resolved at compile time, and the dynamic LDS
// holds 1024 kE keys.
template <int kE>
__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const float* __restrict__ surv,
                                                                 const double* __restrict__ sps, int B, int gamma,
                                                                 int mode, const int32_t* __restrict__ cap_in,
                                                                 int32_t* __restrict__ cap_out,
                                                                 int32_t* __restrict__ lengths, double* theta_out) {
  extern __shared__ unsigned long long key[];
  __shared__ double wtot[kSchedWaves];
  __shared__ double s_bt[kSchedWaves];
  __shared__ int s_bm[kSchedWaves];
  __shared__ int s_valid, s_stop;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int n = B * gamma;
  constexpr int np2 = kSchedThreads * kE;
  constexpr int E = kE;
  // Lane `lane` of wave w holds the keys of indices w 64E + 64q + lane.
  auto idx = [&](int q) { return wave * kWave * E + q * kWave + lane; };

  if (tid == 0) {
    s_valid = 0;
    s_stop = INT_MAX;
  }
  // Key of candidate i = r gamma + (j - 1): the complemented bits of its
  // (positive) survival above its index, so ascending keys are descending
  // survivals with ties in index order.  Non-candidates (a <= 0 or NaN) and
  // the padding sort last.
  unsigned long long v[E];
  int mine = 0;
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const int i = idx(q);
    unsigned long long k = ~0ull;
    if (i < n) {
      const float a = surv[i];
      if (a > 0.0f) {
        k = ((unsigned long long)(~__float_as_uint(a)) << 32) | (unsigned)i;
        ++mine;
      }
    }
    v[q] = k;
  }
  __syncthreads();
  if (mine) atomicAdd(&s_valid, mine);
  __syncthreads();

  // This thread's share of the admission counts, and its throughput table
  // entries, loaded now so that they arrive during the sort (after it at 8
  // and 16 keys per lane, where holding them through the sort would spill).
  const int M = s_valid;
  const int per = (M + kSchedThreads - 1) / kSchedThreads;  // <= E
  const int c0 = min(M, tid * per), c1 = min(M, c0 + per);
  double sp[E + 1];
  auto load_sp = [&]() {
#pragma unroll
    for (int t = 0; t <= E; ++t) sp[t] = sps[B + min(c0 + t, c1)];
  };
  if constexpr (E <= 4) load_sp();

  // Bitonic sort, ascending.  Partners at distance j < 64 are in other lanes
  // of the wave (shuffles), 64 <= j < 64E in other registers of the lane,
  // j >= 64E in other waves (through LDS, two barriers).
#pragma unroll
  for (int k = 2; k <= np2; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= kWave * E) {
#pragma unroll
        for (int q = 0; q < E; ++q) key[idx(q)] = v[q];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < E; ++q) {
          const int i = idx(q), p = i ^ j;
          const unsigned long long y = key[p];
          const bool keep_min = ((i & k) == 0) == (i < p);
          v[q] = keep_min ? (v[q] < y ? v[q] : y) : (v[q] < y ? y : v[q]);
        }
        __syncthreads();
      } else if (j >= kWave) {  // 64 <= j < 64 E: registers q and q + j / 64 of the lane
        const int d = j / kWave;
#pragma unroll
        for (int q = 0; q < E; ++q)
          if ((q & d) == 0) cmp_swap(v[q], v[q + d], (idx(q) & k) == 0);
      } else {
#pragma unroll
        for (int q = 0; q < E; ++q) {
          const unsigned long long y = shfl_xor_u64(v[q], j);
          const int i = idx(q);
          const bool keep_min = ((i & k) == 0) == ((lane & j) == 0);
          v[q] = keep_min ? (v[q] < y ? v[q] : y) : (v[q] < y ? y : v[q]);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < E; ++q) key[idx(q)] = v[q];
  if constexpr (E > 4) load_sp();
  __syncthreads();

  // Thread t owns the sorted candidates [c0, c1) of the M valid.
  auto value = [&](int pos) -> double { return (double)__uint_as_float(~(unsigned)(key[pos] >> 32)); };
  double vals[E];
  double local = 0.0;
#pragma unroll
  for (int t = 0; t < E; ++t) {
    vals[t] = c0 + t < c1 ? value(c0 + t) : 0.0;
    local += vals[t];
  }
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

  const double Bd = (double)B;
  int mstar;
  if (mode == kScheduleEarlyStop) {
    // Theta(m) against Theta(m - 1) at this thread's admission counts m = c0 + t + 1
    double S = S0;
    double prev_theta = (Bd + S) * sp[0];
    bool going = true;
#pragma unroll
    for (int t = 0; t < E; ++t) {
      if (going && c0 + t < c1) {
        S += vals[t];
        const double theta = (Bd + S) * sp[t + 1];
        if (!(theta > prev_theta)) {
          atomicMin(&s_stop, c0 + t + 1);
          going = false;
        }
        prev_theta = theta;
      }
    }
    __syncthreads();
    mstar = s_stop == INT_MAX ? M : s_stop - 1;
  } else if (mode == kScheduleCapacity) {
    // The first maximum of Theta(m) over m = 0..M: this thread's counts
    // c0..c1 (Theta(c0) from the sum before c0), then a block argmax with
    // ties to the lower count.
    double S = S0;
    double bt = (Bd + S) * sp[0];
    int bm = c0;
#pragma unroll
    for (int t = 0; t < E; ++t) {
      if (c0 + t < c1) {
        S += vals[t];
        const double theta = (Bd + S) * sp[t + 1];
        if (theta > bt) {
          bt = theta;
          bm = c0 + t + 1;
        }
      }
    }
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const double ot = __shfl_xor(bt, o);
      const int om = __shfl_xor(bm, o);
      if (ot > bt || (ot == bt && om < bm)) {
        bt = ot;
        bm = om;
      }
    }
    if (lane == 0) {
      s_bt[wave] = bt;
      s_bm[wave] = bm;
    }
    __syncthreads();
    if (tid == 0) {
      double t0 = s_bt[0];
      int m0 = s_bm[0];
      for (int w = 1; w < kSchedWaves; ++w) {
        if (s_bt[w] > t0 || (s_bt[w] == t0 && s_bm[w] < m0)) {
          t0 = s_bt[w];
          m0 = s_bm[w];
        }
      }
      s_stop = m0;
      if (cap_out != nullptr) *cap_out = m0;
    }
    __syncthreads();
    mstar = s_stop;
  } else {  // kScheduleTopK: the capacity decided earlier, filled by the current ranking
    mstar = min(max(cap_in[0], 0), M);
  }

  // The candidate ids of the admitted positions this thread visits, then the
  // key array becomes the lengths (B <= 1024 E ints).
  unsigned ids[E];
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const int pos = tid + q * kSchedThreads;
    ids[q] = pos < mstar ? (unsigned)key[pos] : ~0u;
  }
  __syncthreads();
  int* len = reinterpret_cast<int*>(key);
  for (int i = tid; i < B; i += kSchedThreads) len[i] = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < E; ++q)
    if (ids[q] != ~0u) atomicMax(&len[ids[q] / (unsigned)gamma], (int)(ids[q] % (unsigned)gamma) + 1);
  // Theta(m*), summed in the order of the comparisons above by the thread
  // that owns candidate m* - 1
  if (theta_out != nullptr) {
    if (mstar == 0) {
      if (tid == 0) *theta_out = Bd * sps[B];
    } else if (c0 < mstar && mstar <= c1) {
      double S = S0, th = 0.0;
#pragma unroll
      for (int t = 0; t < E; ++t) {
        if (c0 + t < mstar) {
          S += vals[t];
          th = (Bd + S) * sp[t + 1];
        }
      }
      *theta_out = th;
    }
  }
  __syncthreads();
  for (int i = tid; i < B; i += kSchedThreads) lengths[i] = len[i];
}

template <int kE>
static hipError_t launch_schedule_e(const float* survival, const double* sps, int B, int gamma, int mode,
                                    const int32_t* cap_in, int32_t* cap_out, int32_t* lengths, double* theta,
                                    hipStream_t s) {
  const size_t lds = sizeof(unsigned long long) * kSchedThreads * kE;
  if (lds > 64 * 1024) {
    // once per instantiation (the attribute belongs to the kernel)
    static hipError_t state = hipErrorNotReady;
    if (state == hipErrorNotReady)
      state = hipFuncSetAttribute((const void*)schedule_kernel<kE>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
    if (state != hipSuccess) return state;
  }
  hipLaunchKernelGGL(schedule_kernel<kE>, dim3(1), dim3(kSchedThreads), lds, s, survival, sps, B, gamma, mode,
                     cap_in, cap_out, lengths, theta);
  return hipGetLastError();
}

hipError_t launch_schedule(const float* survival, const double* sps, int B, int gamma, int mode,
                           const int32_t* cap_in, int32_t* cap_out, int32_t* lengths, double* theta, hipStream_t s) {
  ProfScope prof(s, kProfSchedule);
  const int n = B * gamma;
  static_assert(kScheduleMax == 16 * kSchedThreads, "the largest instantiation covers kScheduleMax");
  if (n <= kSchedThreads) return launch_schedule_e<1>(survival, sps, B, gamma, mode, cap_in, cap_out, lengths, theta, s);
  if (n <= 2 * kSchedThreads)
    return launch_schedule_e<2>(survival, sps, B, gamma, mode, cap_in, cap_out, lengths, theta, s);
  if (n <= 4 * kSchedThreads)
    return launch_schedule_e<4>(survival, sps, B, gamma, mode, cap_in, cap_out, lengths, theta, s);
  if (n <= 8 * kSchedThreads)
    return launch_schedule_e<8>(survival, sps, B, gamma, mode, cap_in, cap_out, lengths, theta, s);
  return launch_schedule_e<16>(survival, sps, B, gamma, mode, cap_in, cap_out, lengths, theta, s);
}

}  // namespace dspark
