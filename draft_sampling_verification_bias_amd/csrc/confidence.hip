// dspark_confidence: the confidence head of the DSpark technical review, "The
// Confidence Head" (Eq. 7), c_k = sigma(w . [h_k ; W1[x_{k-1}]]), with the
// per-position temperatures of Sequential Temperature Scaling (same section)
// applied to the logit: c_k = sigma(z_k / t_k).  The previous token's Markov
// embedding is the row the draft gathers for position k (x_0 = the anchor).
//
// One workgroup per (request, position): the hidden part is read with 16-byte
// loads, the embedding row as r values; the float32 products are exact in
// float64 and summed there, so the logit differs from a float64 reference
// only by summation order.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace dspark {

constexpr int kConfThreads = 256;
constexpr int kConfWaves = kConfThreads / kWave;

// One workgroup per (request, position): every thread keeps all of its
// 16-byte hidden-state loads in flight, then one embedding element per k.
template <bool kBf16>
__global__ __launch_bounds__(kConfThreads) void confidence_kernel(ConfArgs a) {
  __shared__ double part[kConfWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const long long item = blockIdx.x;
  const int b = (int)(item / a.gamma), k = (int)(item - (long long)b * a.gamma);
  const int prev = k == 0 ? a.x0[b] : a.tokens[(size_t)b * a.gamma + k - 1];
  if ((unsigned)prev >= (unsigned)a.V) {  // invalid anchor or drafted token
    if (tid == 0) a.conf[item] = __builtin_nanf("");
    return;
  }
  const float* hrow = a.h + (size_t)item * a.d;
  double s = 0.0;
  if ((a.d & 3) == 0) {
#pragma unroll 4
    for (int i = 4 * tid; i < a.d; i += 4 * kConfThreads) {
      const float4 x = *reinterpret_cast<const float4*>(hrow + i);
      const float4 y = *reinterpret_cast<const float4*>(a.w + i);
      s += (double)x.x * (double)y.x + (double)x.y * (double)y.y + (double)x.z * (double)y.z +
           (double)x.w * (double)y.w;
    }
  } else {
    for (int i = tid; i < a.d; i += kConfThreads) s += (double)hrow[i] * (double)a.w[i];
  }
  for (int j = tid; j < a.r; j += kConfThreads) {
    const size_t wi = (size_t)prev * a.r + j;
    const float e = kBf16 ? bf16_to_float(reinterpret_cast<const uint16_t*>(a.W1)[wi])
                          : reinterpret_cast<const float*>(a.W1)[wi];
    s += (double)e * (double)a.w[a.d + j];
  }
  s = wave_sum(s);
  if (lane == 0) part[wave] = s;
  __syncthreads();
  if (tid == 0) {
    double z = 0.0;
#pragma unroll
    for (int w = 0; w < kConfWaves; ++w) z += part[w];
    const double t = a.sts ? (double)a.sts[k] : 1.0;
    a.conf[item] = (float)(1.0 / (1.0 + exp(-z / t)));
  }
}

hipError_t launch_confidence(const ConfArgs& a, bool bf16, hipStream_t s) {
  const int grid = a.B * a.gamma;  // B <= 65536, gamma <= 32
  ProfScope prof(s, kProfConfidence);
  if (bf16) {
    hipLaunchKernelGGL(confidence_kernel<true>, dim3(grid), dim3(kConfThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(confidence_kernel<false>, dim3(grid), dim3(kConfThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dspark
