// Block-wide inverse-CDF search used by every categorical draw of the library.
//
// A draw with uniform u from weights w_0..w_{n-1} (Z = sum w) takes the first
// index t, in ascending order, whose inclusive cumulative weight exceeds
// q = u * Z; when rounding leaves no such index, the last index with positive
// weight.  Threads own contiguous chunks of indices, so the cumulative order
// is the ascending order.  All cumulative sums are in float64.
#pragma once

#include <limits.h>

#include "common.hpp"

namespace dspark {

// Shared scratch of the search (one per block).
struct PickScratch {
  double red[16];
  double base;
  int first, last, pick;
};

// Sum of the weights over [0, n) (all threads receive it).  `weight(t)` must
// return the same double every time it is called with the same t.
template <int kBlock, class F>
__device__ double block_total(int n, F weight, PickScratch& ps) {
  const int cs = (n + kBlock - 1) / kBlock;
  const int t0 = min(n, (int)threadIdx.x * cs);
  const int t1 = min(n, t0 + cs);
  double local = 0.0;
  for (int t = t0; t < t1; ++t) local += weight(t);
  return block_sum<kBlock, double>(local, ps.red);
}

// Core of the search.  With `by_uniform` the target is q = uq * (sum of all
// weights), otherwise q = uq.  Returns the picked index (-1 if no weight is
// positive) to all threads, with the cumulative weight before it in *base_out
// and the total weight in *total_out (either may be null).
template <int kBlock, class F>
__device__ int block_pick_core(int n, F weight, bool by_uniform, double uq, PickScratch& ps,
                               double* base_out, double* total_out) {
  const int cs = (n + kBlock - 1) / kBlock;
  const int t0 = min(n, (int)threadIdx.x * cs);
  const int t1 = min(n, t0 + cs);
  double local = 0.0;
  for (int t = t0; t < t1; ++t) local += weight(t);
  double total;
  const double excl = block_exclusive_scan<kBlock>(local, ps.red, total);
  const double q = by_uniform ? uq * total : uq;
  if (threadIdx.x == 0) {
    ps.first = INT_MAX;
    ps.last = -1;
    ps.pick = -1;
    ps.base = 0.0;
  }
  __syncthreads();
  if (local > 0.0) {
    if (excl + local > q) atomicMin(&ps.first, (int)threadIdx.x);
    atomicMax(&ps.last, (int)threadIdx.x);
  }
  __syncthreads();
  const int owner = ps.first != INT_MAX ? ps.first : ps.last;
  if ((int)threadIdx.x == owner) {
    double cum = excl;
    int pick = -1, lastpos = -1;
    double pickbase = 0.0, lastbase = 0.0;
    for (int t = t0; t < t1; ++t) {
      const double w = weight(t);
      if (w > 0.0) {
        lastpos = t;
        lastbase = cum;
        if (pick < 0 && cum + w > q) {
          pick = t;
          pickbase = cum;
        }
      }
      cum += w;
    }
    if (pick < 0) {
      pick = lastpos;
      pickbase = lastbase;
    }
    ps.pick = pick;
    ps.base = pickbase;
  }
  __syncthreads();
  const int pick = ps.pick;
  if (base_out) *base_out = ps.base;
  if (total_out) *total_out = total;
  __syncthreads();
  return pick;
}

// Draw with uniform u in (0, 1): q = u * total.
template <int kBlock, class F>
__device__ int block_pick_uniform(int n, F weight, double u, PickScratch& ps, double* base_out,
                                  double* total_out) {
  return block_pick_core<kBlock>(n, weight, true, u, ps, base_out, total_out);
}

// Search for a given cumulative target q.
template <int kBlock, class F>
__device__ int block_pick_target(int n, F weight, double q, PickScratch& ps, double* base_out) {
  return block_pick_core<kBlock>(n, weight, false, q, ps, base_out, nullptr);
}

}  // namespace dspark
