// Weight layout helper: W2 [r][V] -> W2T [V][r] (the Markov projection of
// Eq. 5 of the DSpark technical review, "Instantiation 1: The Markov Head",
// stored vocabulary-major so that one token's column is one contiguous row).
#include "common.hpp"
#include "launch.hpp"

namespace dspark {

constexpr int kTrTile = 64;

// One 64 x 64 block through LDS: coalesced reads along V, coalesced writes
// along r.  Element type T is uint16_t (bf16 bits) or float.
template <typename T>
__global__ __launch_bounds__(256) void transpose_w2_kernel(const T* __restrict__ W2, int r, int V,
                                                           T* __restrict__ W2T) {
  __shared__ T tile[kTrTile][kTrTile + 1];
  const int v0 = blockIdx.x * kTrTile, j0 = blockIdx.y * kTrTile;
  const int tx = threadIdx.x & (kTrTile - 1), ty = threadIdx.x / kTrTile;  // 64 x 4
  for (int jj = ty; jj < kTrTile; jj += 4) {
    const int j = j0 + jj, v = v0 + tx;
    if (j < r && v < V) tile[jj][tx] = W2[(size_t)j * V + v];
  }
  __syncthreads();
  for (int vv = ty; vv < kTrTile; vv += 4) {
    const int v = v0 + vv, j = j0 + tx;
    if (j < r && v < V) W2T[(size_t)v * r + j] = tile[tx][vv];
  }
}

hipError_t launch_transpose_w2(const void* W2, bool bf16, int r, int V, void* W2T, hipStream_t s) {
  const dim3 grid((unsigned)(((long long)V + kTrTile - 1) / kTrTile), (r + kTrTile - 1) / kTrTile);
  if (bf16) {
    hipLaunchKernelGGL(transpose_w2_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(W2), r, V,
                       static_cast<uint16_t*>(W2T));
  } else {
    hipLaunchKernelGGL(transpose_w2_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(W2), r, V,
                       static_cast<float*>(W2T));
  }
  return hipGetLastError();
}

}  // namespace dspark
