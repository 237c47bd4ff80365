// The tile pass: Markov bias rows (Eq. 5 of the DSpark technical review,
// "Instantiation 1: The Markov Head") for a batch of logical rows, computed
// tile by tile over the vocabulary and consumed in registers:
//
//   l[R][v] = U[R][v] + sum_j W1[prev(R)][j] * W2[j][v]
//
// One workgroup owns one tile of kTileCols vocabulary columns for ALL rows, so
// each W2 tile is fetched from HBM once per pass and reused by every row.
// bf16 weights go through the gfx950 MFMA v_mfma_f32_32x32x16_bf16 (exact
// products, fp32 accumulation); float32 weights use VALU FMAs.  The bias is
// never written to HBM (except in bias mode): the epilogue adds the U tile,
// streamed once with coalesced loads, and reduces each row's 128 columns to
// one summary (see TileMode).
#include "common.hpp"
#include "launch.hpp"

namespace dspark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileThreads = 256;
constexpr int kNB = kTileCols / 32;  // 32-column MFMA blocks per tile
constexpr float kLog2e = 1.4426950408889634f;

struct RowInfo {
  int b, kk;
};

__device__ __forceinline__ RowInfo row_info(const TileArgs& a, int R) {
  RowInfo ri;
  if (a.kper == 1) {
    ri.b = R;
    ri.kk = a.k0;
  } else {
    ri.b = R / a.kper;
    ri.kk = R - ri.b * a.kper;
  }
  return ri;
}

__device__ __forceinline__ int prev_token(const TileArgs& a, RowInfo ri) {
  return ri.kk == 0 ? a.x0[ri.b] : a.tokens[(size_t)ri.b * a.gamma + ri.kk - 1];
}

// Half-wave (32-lane) reductions: lanes 0..31 and 32..63 reduce separately.
__device__ __forceinline__ float half_max(float x) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float half_sum(float x) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ void half_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(i, o);
    argmax_merge(v, i, ov, oi);
  }
}

// Stage W2[0:r][v0:v0+128] into LDS transposed, column-major with a padded
// pitch, so that each lane reads its 8 consecutive-k bf16 MFMA operand with one
// 16-byte LDS load.
__device__ __forceinline__ void stage_w2_tile(const uint16_t* __restrict__ W2, uint16_t* sW, int r,
                                              int V, int v0, int pitch) {
  const int items = (r / 2) * (kTileCols / 4);
  const bool full = (v0 + kTileCols <= V) && ((V & 3) == 0);
  for (int it = threadIdx.x; it < items; it += kTileThreads) {
    const int cq = it % (kTileCols / 4);
    const int kp = it / (kTileCols / 4);
    const int kA = 2 * kp;
    const int c = v0 + 4 * cq;
    uint16_t e0[4], e1[4];
    if (full) {
      const uint2 p0 = *reinterpret_cast<const uint2*>(W2 + (size_t)kA * V + c);
      const uint2 p1 = *reinterpret_cast<const uint2*>(W2 + (size_t)(kA + 1) * V + c);
      e0[0] = p0.x & 0xffff; e0[1] = p0.x >> 16; e0[2] = p0.y & 0xffff; e0[3] = p0.y >> 16;
      e1[0] = p1.x & 0xffff; e1[1] = p1.x >> 16; e1[2] = p1.y & 0xffff; e1[3] = p1.y >> 16;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = c + q < V;
        e0[q] = ok ? W2[(size_t)kA * V + c + q] : (uint16_t)0;
        e1[q] = ok ? W2[(size_t)(kA + 1) * V + c + q] : (uint16_t)0;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<uint32_t*>(sW + (size_t)(4 * cq + q) * pitch + kA) =
          (uint32_t)e0[q] | ((uint32_t)e1[q] << 16);
    }
  }
}

// Row index of accumulator register i for this lane in the 32x32 MFMA output.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

template <int kMode, bool kBf16>
__global__ __launch_bounds__(kTileThreads) void tile_pass_kernel(TileArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tile = blockIdx.x;
  const int v0 = tile * kTileCols;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int pitch = a.r + 8;
  uint16_t* sW = reinterpret_cast<uint16_t*>(smem);

  if constexpr (kBf16) {
    stage_w2_tile(reinterpret_cast<const uint16_t*>(a.W2), sW, a.r, a.V, v0, pitch);
    __syncthreads();
  }

  const int nrb = (a.nrows + 31) / 32;
  const int ksteps = a.r / 16;
  for (int rb = wave; rb < nrb; rb += kTileThreads / kWave) {
    f32x16 acc[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][i] = 0.0f;

    if constexpr (kBf16) {
      // A operand: the lane's row (lane % 32) of E = W1[prev], k-chunk lane / 32.
      const int arow = rb * 32 + (lane & 31);
      int prev = -1;
      if (arow < a.nrows) prev = prev_token(a, row_info(a, arow));
      const bool ok = prev >= 0 && prev < a.V;
      const uint16_t* w1row = reinterpret_cast<const uint16_t*>(a.W1) + (size_t)(ok ? prev : 0) * a.r;
      const int koff = 8 * (lane >> 5);
      const uint16_t* bcol = sW + (size_t)(lane & 31) * pitch + koff;
#pragma unroll 4
      for (int ks = 0; ks < ksteps; ++ks) {
        bf16x8 av;
        if (ok) {
          av = *reinterpret_cast<const bf16x8*>(w1row + ks * 16 + koff);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) av[j] = (__bf16)0.0f;
        }
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(bcol + (size_t)nb * 32 * pitch + ks * 16);
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[nb], 0, 0, 0);
        }
      }
    } else {
      // float32 weights: each lane forms its 16 rows x 4 columns directly.
      const float* W1f = reinterpret_cast<const float*>(a.W1);
      const float* W2f = reinterpret_cast<const float*>(a.W2);
      int prevs[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int R = rb * 32 + acc_row(i, lane);
        int p = -1;
        if (R < a.nrows) p = prev_token(a, row_info(a, R));
        prevs[i] = (p >= 0 && p < a.V) ? p : -1;
      }
      for (int kq = 0; kq < a.r; ++kq) {
        float w2v[kNB];
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const int c = v0 + nb * 32 + (lane & 31);
          w2v[nb] = c < a.V ? W2f[(size_t)kq * a.V + c] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = prevs[i] >= 0 ? W1f[(size_t)prevs[i] * a.r + kq] : 0.0f;
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) acc[nb][i] = fmaf(e, w2v[nb], acc[nb][i]);
        }
      }
    }

    // Epilogue: register i holds row acc_row(i, lane), column lane % 32 of each block.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int R = rb * 32 + acc_row(i, lane);
      const bool rok = R < a.nrows;
      const RowInfo ri = row_info(a, rok ? R : 0);
      const size_t urow = ((size_t)ri.b * a.gamma + ri.kk) * (size_t)a.V;
      if constexpr (kMode == kModeBias) {
        if (rok) {
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const int c = v0 + nb * 32 + (lane & 31);
            if (c < a.V) {
              const int p = a.x0[R];
              a.bias_out[(size_t)R * a.V + c] = (p >= 0 && p < a.V) ? acc[nb][i] : __builtin_nanf("");
            }
          }
        }
        continue;
      }
      float x[kNB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int c = v0 + nb * 32 + (lane & 31);
        x[nb] = (rok && c < a.V) ? acc[nb][i] + a.U[urow + c] : -__builtin_inff();
      }
      if constexpr (kMode == kModeSample) {
        float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = half_max(mx);
        float s = 0.0f;
        if (mx != -__builtin_inff()) {
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) s += fast_exp2((x[nb] - mx) * a.cf);
        }
        s = half_sum(s);
        if (rok && (lane & 31) == 0) a.partials[(size_t)R * a.ntiles + tile] = make_float2(mx, s);
      } else if constexpr (kMode == kModeGreedy) {
        float bv = x[0];
        int bi = v0 + (lane & 31);
#pragma unroll
        for (int nb = 1; nb < kNB; ++nb) {
          if (x[nb] > bv) {
            bv = x[nb];
            bi = v0 + nb * 32 + (lane & 31);
          }
        }
        half_argmax(bv, bi);
        if (rok && (lane & 31) == 0) a.partials[(size_t)R * a.ntiles + tile] = make_float2(bv, __int_as_float(bi));
      } else {  // kModeOverlap
        const size_t trow = ((size_t)ri.b * (a.gamma + 1) + ri.kk) * (size_t)a.V;
        const float ld2 = rok ? a.lse_d[(size_t)ri.b * a.gamma + ri.kk] * kLog2e : 0.0f;
        const float lt2 = rok ? a.lt2[R] : 0.0f;
        float s = 0.0f;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const int c = v0 + nb * 32 + (lane & 31);
          if (rok && c < a.V) {
            const float pd = fast_exp2(x[nb] * a.cf - ld2);
            const float pt = fast_exp2(a.target[trow + c] * a.cf - lt2);
            s += fminf(pd, pt);
          }
        }
        s = half_sum(s);
        if (rok && (lane & 31) == 0) a.partials[(size_t)R * a.ntiles + tile] = make_float2(s, 0.0f);
      }
    }
  }
}

template <int kMode, bool kBf16>
static hipError_t launch_mode(const TileArgs& a, hipStream_t s) {
  const size_t lds = kBf16 ? (size_t)kTileCols * (a.r + 8) * sizeof(uint16_t) : 0;
  ProfScope prof(s, kProfTileSample + kMode);
  hipLaunchKernelGGL((tile_pass_kernel<kMode, kBf16>), dim3(a.ntiles), dim3(kTileThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_tile_pass(const TileArgs& a, int mode, bool bf16, hipStream_t s) {
  switch (mode) {
    case kModeSample: return bf16 ? launch_mode<kModeSample, true>(a, s) : launch_mode<kModeSample, false>(a, s);
    case kModeGreedy: return bf16 ? launch_mode<kModeGreedy, true>(a, s) : launch_mode<kModeGreedy, false>(a, s);
    case kModeOverlap: return bf16 ? launch_mode<kModeOverlap, true>(a, s) : launch_mode<kModeOverlap, false>(a, s);
    case kModeBias: return bf16 ? launch_mode<kModeBias, true>(a, s) : launch_mode<kModeBias, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_markov_bias(const void* W1, const void* W2, bool bf16, const int32_t* tokens, int n,
                              int V, int r, float* out, hipStream_t s) {
  TileArgs a = {};
  a.W1 = W1;
  a.W2 = W2;
  a.x0 = tokens;
  a.bias_out = out;
  a.nrows = n;
  a.kper = 1;
  a.k0 = 0;
  a.B = n;
  a.gamma = 1;
  a.V = V;
  a.r = r;
  a.ntiles = tiles_of(V, kTileCols);
  return launch_tile_pass(a, kModeBias, bf16, s);
}

}  // namespace dspark
