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
constexpr int kRowsPerGroup = 128;   // rows of one workgroup: one 32-row block per wave

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

// The W1 row of row (b, kk): the previous token's, or with operand rows the
// table row b * gamma + kk.
__device__ __forceinline__ int prev_token(const TileArgs& a, RowInfo ri) {
  if (a.opnd_rows) return ri.b * a.gamma + ri.kk;
  return ri.kk == 0 ? a.x0[ri.b] : a.tokens[(size_t)ri.b * a.gamma + ri.kk - 1];
}

// Whether that row exists (a token id inside the vocabulary).
__device__ __forceinline__ bool prev_ok(const TileArgs& a, int prev) {
  return a.opnd_rows ? prev >= 0 : (unsigned)prev < (unsigned)a.V;
}

// ---------------------------------------------------------------------------
// Column mapping.  MFMA output block nb (0..3), column n (0..31) of a tile is
// vocabulary column v0 + 4 n + nb, so the four values a lane holds for one
// row are four consecutive columns: U and target rows are read with one
// 16-byte load per accumulator register, 512 contiguous bytes per half-wave.
// ---------------------------------------------------------------------------

// Stage W2[0:r][v0:v0+128] into LDS as [block nb][column n][k] (padded pitch),
// so each lane reads its 8 consecutive-k bf16 MFMA operand with one 16-byte
// LDS load.  A work item is 8 rows k of 4 columns: eight 8-byte global loads,
// all issued before any LDS store, then one 16-byte LDS store per column.
__device__ __forceinline__ void stage_w2_tile(const uint16_t* __restrict__ W2, uint16_t* sW, int r, int V, int v0,
                                              int pitch) {
  constexpr int kPerPass = 4;                        // items per thread per pass
  const int items = (r / 8) * (kTileCols / 4);       // (k octet, column quad)
  const bool full = (v0 + kTileCols <= V) && ((V & 3) == 0);
  for (int base = 0; base < items; base += kPerPass * kTileThreads) {
    uint2 p[kPerPass][8];
#pragma unroll
    for (int j = 0; j < kPerPass; ++j) {
      const int it = base + j * kTileThreads + threadIdx.x;
      const int n = it % (kTileCols / 4);
      const int k8 = 8 * (it / (kTileCols / 4));
      const int c = v0 + 4 * n;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if (it < items && full) {
          p[j][kk] = *reinterpret_cast<const uint2*>(W2 + (size_t)(k8 + kk) * V + c);
        } else if (it < items) {
          uint32_t e[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) e[q] = c + q < V ? W2[(size_t)(k8 + kk) * V + c + q] : 0u;
          p[j][kk] = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
        } else {
          p[j][kk] = make_uint2(0u, 0u);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kPerPass; ++j) {
      const int it = base + j * kTileThreads + threadIdx.x;
      if (it >= items) break;
      const int n = it % (kTileCols / 4);
      const int k8 = 8 * (it / (kTileCols / 4));
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        uint32_t h[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const uint32_t wrd = (nb < 2) ? p[j][kk].x : p[j][kk].y;
          h[kk] = (nb & 1) ? (wrd >> 16) : (wrd & 0xffffu);
        }
        const uint4 v = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
        *reinterpret_cast<uint4*>(sW + (size_t)(nb * 32 + n) * pitch + k8) = v;
      }
    }
  }
}

// Row index of accumulator register i for this lane in the 32x32 MFMA output.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// Four consecutive columns c..c+3 of a row, -inf past the end of the row.
__device__ __forceinline__ float4 load4(const float* __restrict__ row, int c, int V, bool full) {
  if (full) return *reinterpret_cast<const float4*>(row + c);
  float4 r;
  r.x = c < V ? row[c] : -__builtin_inff();
  r.y = c + 1 < V ? row[c + 1] : -__builtin_inff();
  r.z = c + 2 < V ? row[c + 2] : -__builtin_inff();
  r.w = c + 3 < V ? row[c + 3] : -__builtin_inff();
  return r;
}

__device__ __forceinline__ float comp(const float4& v, int q) { return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w; }

// Reduce 16 per-lane row values over the 32 lanes of each half-wave.  On
// return a[0], b[0] hold the result for register (lane & 31) >> 1 in both
// lanes of each even/odd pair.
template <class M>
__device__ __forceinline__ void transpose_reduce(float (&a)[16], float (&b)[16], int lane, const M& merge) {
  xstep<8>(a, b, lane, 16, merge);
  xstep<4>(a, b, lane, 8, merge);
  xstep<2>(a, b, lane, 4, merge);
  xstep<1>(a, b, lane, 2, merge);
  const float ra = __shfl_xor(a[0], 1), rb = __shfl_xor(b[0], 1);
  merge(a[0], b[0], ra, rb);
}

// Grid mapping: block -> (tile, row group).  With several row groups the
// groups of one tile go to blocks b, b+8, ... -- the same XCD under the
// round-robin dispatch of workgroups to the 8 XCDs -- so the W2 tile is
// re-read from that XCD's L2.
__device__ __forceinline__ bool block_tile(const TileArgs& a, int& tile, int& group) {
  const int b = blockIdx.x;
  if (a.ngroups == 1) {
    tile = b;
    group = 0;
  } else {
    const int slot = b / 8;
    tile = (slot / a.ngroups) * 8 + (b % 8);
    group = slot % a.ngroups;
  }
  const bool ok = tile < a.tile_count;
  tile += a.tile_begin;
  return ok;
}

// ---------------------------------------------------------------------------
// Fast path of the sample, argmax and overlap modes: bf16 weights, r = 256,
// full 128-column tiles of a vocabulary whose size is a multiple of 4, groups
// of 128 rows (the last one may be partial), and base-logit rows at a
// constant stride (one block position of every request, or all positions of
// consecutive requests).
//
// A workgroup owns one 128-row group and a contiguous range of tiles, walked
// as 64-column halves: while the MFMA and the epilogue of one half run, the
// W2 block of the next half is on its way into the other LDS buffer (global
// -> LDS DMA) and its U block into a second register set, so every workgroup
// keeps loads in flight instead of alternating between loading and computing.
// The W1 rows (the B operand) are loaded once per workgroup.
//
// LDS: two 256 x 64 bf16 buffers (32 KB each), rows of 128 bytes whose 16-byte
// chunks are permuted by an XOR with 4 ((k / 2) mod 2), which keeps the four
// rows of a transposing read on disjoint banks.
// ---------------------------------------------------------------------------
constexpr int kFastR = 256;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kHalfCols = 64;
constexpr int kHalfBytes = kFastR * kHalfCols * 2;  // 32 KB

__device__ __forceinline__ int w2h_slot(int row, int chunk) { return chunk ^ (4 * ((row >> 1) & 1)); }

// One 16-byte global -> LDS DMA per lane: lane l writes LDS bytes
// [dst + 16 l, dst + 16 l + 16) (dst wave-uniform, passed in M0).  Issued as
// a statement the compiler does not model, so it adds no wait of its own for
// the LDS destination: the caller orders the copy before the LDS reads with
// wait_vmem and a barrier.  The source is a wave-uniform base plus a per-lane
// byte offset below 2^32.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, unsigned char* dst) {
  const unsigned lds = (unsigned)(unsigned long)((lds_void*)dst);
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// vmcnt-only wait (expcnt, lgkmcnt left at their maxima); n <= 63.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Block -> (row group, column slice).  With the workgroup count a multiple of
// 8, consecutive indices are placed on one XCD (workgroups are dealt to the
// 8 XCDs round robin), so the row groups of a slice share that XCD's L2 copy
// of the W2 blocks.
__device__ __forceinline__ void pipe_block(int ngroups, int nslices, int& group, int& slice) {
  const int total = ngroups * nslices;
  const int b = blockIdx.x;
  const int idx = (total & 7) == 0 ? (b & 7) * (total >> 3) + (b >> 3) : b;
  group = idx % ngroups;
  slice = idx / ngroups;
}

template <int kMode>
__global__ __launch_bounds__(kTileThreads, kMode == kModeOverlap ? 1 : 2) void tile_pipe_kernel(TileArgs a,
                                                                                                 int nslices) {
  constexpr bool kOv = kMode == kModeOverlap;  // also streams the target rows
  extern __shared__ __align__(16) unsigned char smem[];
  int group, slice;
  pipe_block(a.ngroups, nslices, group, slice);
  const int t_begin = a.tile_begin + (int)((long long)slice * a.tile_count / nslices);
  const int t_end = a.tile_begin + (int)((long long)(slice + 1) * a.tile_count / nslices);
  if (t_begin >= t_end) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int n = lane & 31, hh = lane >> 5;
  const size_t V = (size_t)a.V;
  const uint16_t* W2 = reinterpret_cast<const uint16_t*>(a.W2);
  unsigned char* buf0 = smem;
  unsigned char* buf1 = smem + kHalfBytes;

  // Lane (n, hh) owns request row R; in a half starting at column c it holds
  // columns c + 32 nb + 8 q + 4 hh + 0..3 (nb = 0, 1; q = 0..3).
  // Rows at or past row_end (the last group may be partial) read a valid row
  // instead, are given no previous token and write nothing.
  const int R = group * kRowsPerGroup + 32 * wave + n;
  const bool rowok = R < a.row_end;
  const int Rc = rowok ? R : a.row_end - 1;
  const size_t rs = a.kper == 1 ? (size_t)a.gamma * V : V;
  const float* urow = a.U + (size_t)Rc * rs + (a.kper == 1 ? (size_t)a.k0 * V : 0) + 4 * hh;
  // overlap mode (rows b * gamma + kk, one per block position): the target row
  // of (b, kk) and the draft / target log2 normalisers of the row
  const float* tgrow = nullptr;
  float ld2 = 0.0f, lt2 = 0.0f;
  if constexpr (kOv) {
    const RowInfo ri = row_info(a, Rc);
    tgrow = a.target + ((size_t)ri.b * (a.gamma + 1) + ri.kk) * V + 4 * hh;
    ld2 = a.lse_d[(size_t)ri.b * a.gamma + ri.kk] * kLog2e;
    lt2 = a.lt2[Rc];
  }

  // Byte offset of this lane's 16-byte W2 chunk in the first DMA of a half:
  // row 64 wave + l / 8 (8 rows per instruction), slot l % 8 of the permuted
  // row (the XOR permutation is its own inverse and is the same for the rows
  // 8 i + l / 8 of every instruction i).
  const int w2row = 64 * wave + (lane >> 3);
  const uint32_t w2off = ((uint32_t)w2row * (uint32_t)V + 8u * (uint32_t)w2h_slot(w2row, lane & 7)) * 2u;

  // The lane's U values of the half, then W2[0:256][c:c+64] -> buf by DMA
  // (each wave 64 rows, 8 rows per instruction): 16 vector memory
  // instructions per wave, in this order (the DMA statements are volatile and
  // clobber memory, so the loads cannot be moved past them).
  auto issue = [&](int c, unsigned char* buf, float4 (&u)[2][4], float4 (&t)[2][4]) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) u[nb][q] = *reinterpret_cast<const float4*>(urow + c + 32 * nb + 8 * q);
    if constexpr (kOv) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) t[nb][q] = *reinterpret_cast<const float4*>(tgrow + c + 32 * nb + 8 * q);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rbase = 64 * wave + 8 * i;
      dma16(W2 + c, w2off + (uint32_t)(i * 16) * (uint32_t)V, buf + (size_t)rbase * 128);
    }
  };

  float4 uA[2][4], uB[2][4];
  float4 tA[2][4], tB[2][4];  // target values (overlap mode only)
  issue(t_begin * kTileCols, buf0, uA, tA);

  // B operand: row R of E = W1[prev], k-chunk hh of each 16-wide k step.
  const int prev = prev_token(a, row_info(a, Rc));
  const bool ok = rowok && prev_ok(a, prev);
  const uint16_t* w1row = reinterpret_cast<const uint16_t*>(a.W1) + (size_t)(ok ? prev : 0) * kFastR + 8 * hh;
  bf16x8 ev[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) ev[j] = *reinterpret_cast<const bf16x8*>(w1row + j * 16);
  if (!ok) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) ev[j][e] = (__bf16)0.0f;
  }

  const int trow = 8 * hh + ((lane & 15) >> 2);             // + 16 j + 4 h
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + 32 nb
  // bias^T of one half (A = W2^T by transposing LDS reads, B = E^T), plus U.
  auto logits = [&](const unsigned char* buf, const float4 (&u)[2][4], float (&x)[2][16]) {
    f32x16 acc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][i] = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        bf16x8 av;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 16 * j + 4 * h + trow;
          const int col = 32 * nb + tcol;
          const int addr = row * 128 + w2h_slot(row, col >> 3) * 16 + (col & 7) * 2;
          const bf16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(buf + addr));
#pragma unroll
          for (int e = 0; e < 4; ++e) av[4 * h + e] = t[e];
        }
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, ev[j], acc[nb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[nb][i] = acc[nb][i] + comp(u[nb][i >> 2], i & 3);
  };

  // Per half: wait for its loads (issued one half earlier) and for every wave
  // to be done with the other buffer, then issue the next half's loads into
  // the other buffer and register set, then compute.  After the full wait the
  // compiler knows the half's U registers are complete and adds no waits of
  // its own that would also cover the loads in flight.
  for (int tile = t_begin; tile < t_end; ++tile) {
    const int c0 = tile * kTileCols;
    float x[2][16];
    float m0, s0, bv0;
    int bp0;

    // first half (buf0, uA)
    __builtin_amdgcn_sched_barrier(0);  // keep the previous half's work before the wait
    wait_vmem<0>();
    __syncthreads();
    issue(c0 + kHalfCols, buf1, uB, tB);
    logits(buf0, uA, x);
    if constexpr (kOv) {
      float sum = 0.0f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sum += fminf(fast_exp2(x[nb][i] * a.cf - ld2), fast_exp2(comp(tA[nb][i >> 2], i & 3) * a.cf - lt2));
      s0 = sum;
      asm volatile("" : "+v"(s0));
    } else if constexpr (kMode == kModeSample) {
      float m = -__builtin_inff();
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, x[nb][i]);
      const float mc = m * a.cf;
      float sum = 0.0f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += fast_exp2(fmaf(x[nb][i], a.cf, -mc));
      m0 = m;
      s0 = m == -__builtin_inff() ? 0.0f : sum;
      asm volatile("" : "+v"(m0), "+v"(s0));  // finish this half's epilogue here, not in the next half
    } else {
      float bv = -__builtin_inff();
      int bpos = 0;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (x[nb][i] > bv) {  // ascending columns: the lowest index wins ties
            bv = x[nb][i];
            bpos = nb * 16 + i;
          }
      bv0 = bv;
      bp0 = bpos;
      asm volatile("" : "+v"(bv0), "+v"(bp0));
    }

    // second half (buf1, uB)
    __builtin_amdgcn_sched_barrier(0);
    wait_vmem<0>();
    __syncthreads();
    if (tile + 1 < t_end) issue(c0 + kTileCols, buf0, uA, tA);
    logits(buf1, uB, x);
    if constexpr (kOv) {
      float sum = s0;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sum += fminf(fast_exp2(x[nb][i] * a.cf - ld2), fast_exp2(comp(tB[nb][i >> 2], i & 3) * a.cf - lt2));
      sum += __shfl_xor(sum, 32);
      if (hh == 0 && rowok) a.partials[(size_t)R * a.ntiles + tile] = make_float2(sum, 0.0f);
    } else if constexpr (kMode == kModeSample) {
      float m = -__builtin_inff();
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, x[nb][i]);
      const float mc = m * a.cf;
      float sum = 0.0f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += fast_exp2(fmaf(x[nb][i], a.cf, -mc));
      if (m == -__builtin_inff()) sum = 0.0f;
      const MergeMS merge{a.cf};
      merge(m, sum, m0, s0);
      const float om = __shfl_xor(m, 32), os = __shfl_xor(sum, 32);
      merge(m, sum, om, os);
      if (hh == 0 && rowok) a.partials[(size_t)R * a.ntiles + tile] = make_float2(m, sum);
    } else {
      float bv = -__builtin_inff();
      int bpos = 0;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (x[nb][i] > bv) {
            bv = x[nb][i];
            bpos = nb * 16 + i;
          }
      const int cb = c0 + 4 * hh;
      int b0 = cb + 32 * (bp0 >> 4) + 8 * ((bp0 >> 2) & 3) + (bp0 & 3);
      const int b1 = cb + kHalfCols + 32 * (bpos >> 4) + 8 * ((bpos >> 2) & 3) + (bpos & 3);
      float bvm = bv0;
      argmax_merge(bvm, b0, bv, b1);
      const float ov = __shfl_xor(bvm, 32);
      const int oi = __shfl_xor(b0, 32);
      argmax_merge(bvm, b0, ov, oi);
      if (hh == 0 && rowok) a.partials[(size_t)R * a.ntiles + tile] = make_float2(bvm, __int_as_float(b0));
    }
  }
}

// ---------------------------------------------------------------------------
// Wide variant of the fast path for launches of at least 192 rows (sample and
// argmax modes).  One 8-wave workgroup per CU owns a group of 256 rows, so a
// W2 half block staged in LDS serves twice as many rows, and the W2 blocks go
// through a ring of three LDS buffers.  Step j (one 64-column half):
//   wait until W2(j) and U(j) have landed (the loads of half j + 1 stay in
//   flight), barrier, DMA W2(j + 2) into the buffer of half j - 1,
//   MFMA and epilogue of half j,
//   load U(j + 2) into the register set of half j.
// The MFMA and epilogue of a half thus run with the loads of the next two
// halves in flight; the two-buffer kernel waits for all of its loads at every
// half and so leaves the memory system idle while it computes.
//
// Wait counts.  Per wave a half is kDma DMA instructions (which the
// compiler does not see) and 8 U loads (which it does), issued in the order
// W2(j+2) ... U(j+2), so at the start of step j the operations issued after
// U(j) are W2(j+1) and U(j+1) (when half j+1 exists) and at most one summary
// store; a vmcnt of (DMA instructions) + 8 lets exactly those stay in flight (a store
// among them only makes the wait one operation stricter).  The compiler adds
// its own waits for the U registers from the loads it sees; those are always
// sufficient and at most somewhat stricter.
// ---------------------------------------------------------------------------
//
// Two-part operand rows (kParts == 2, the RNN head's e_hi, e_lo) are
// multiplied by the same W2 fragments; their second operand set fills the
// register file of eight waves (252 VGPRs).  A four-wave form (groups of 128
// rows, one workgroup per CU) serves launches whose 256-row groups would be
// mostly empty: two-part rows below 3/4 of a group, and single-part
// launches of at most 64 rows.
// ---------------------------------------------------------------------------
constexpr int kRingWaves = 8;
constexpr int kRingThreads = kWave * kRingWaves;
constexpr int kRingRows = 32 * kRingWaves;            // rows per group
constexpr int kRingStages = 3;                        // W2 buffers in LDS
constexpr int kRing2Waves = 4;                        // waves of the two-part variant

template <int kMode, int kWaves = kRingWaves, int kParts = 1>
__global__ __launch_bounds__(kWave * kWaves) void tile_ring_kernel(TileArgs a, int nslices) {
  static_assert(kMode == kModeSample || kMode == kModeGreedy, "ring kernel modes");
  static_assert(kParts == 1 || kParts == 2, "one or two operand parts");
  constexpr int kRows = 32 * kWaves;            // rows per group
  constexpr int kKPerWave = kFastR / kWaves;    // W2 rows k staged per wave
  constexpr int kDma = kKPerWave / 8;           // DMA instructions per wave per half
  constexpr int kWait = kDma + 8;               // ops of one later half
  extern __shared__ __align__(16) unsigned char smem[];
  int group, slice;
  pipe_block(a.ngroups, nslices, group, slice);
  const int t_begin = a.tile_begin + (int)((long long)slice * a.tile_count / nslices);
  const int t_end = a.tile_begin + (int)((long long)(slice + 1) * a.tile_count / nslices);
  if (t_begin >= t_end) return;
  const int H = 2 * (t_end - t_begin);  // halves of this workgroup

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int n = lane & 31, hh = lane >> 5;
  const size_t V = (size_t)a.V;
  const uint16_t* W2 = reinterpret_cast<const uint16_t*>(a.W2);

  // Lane (n, hh) of wave w owns request row R = 256 group + 32 w + n and, in a
  // half starting at column c, columns c + 32 nb + 8 q + 4 hh + 0..3.  Rows at
  // or past row_end read a valid row, get no previous token and write nothing.
  const int R = group * kRows + 32 * wave + n;
  const bool rowok = R < a.row_end;
  const int Rc = rowok ? R : a.row_end - 1;
  const size_t rs = a.kper == 1 ? (size_t)a.gamma * V : V;
  const float* urow = a.U + (size_t)Rc * rs + (a.kper == 1 ? (size_t)a.k0 * V : 0) + 4 * hh;

  // DMA lane mapping: wave w stages rows k = 32 w .. 32 w + 31, 8 per
  // instruction, lane l the 16-byte slot l % 8 of row 32 w + 8 i + l / 8 (the
  // XOR permutation depends on (k / 2) mod 2 only, the same for every i).
  const int w2row = kKPerWave * wave + (lane >> 3);
  const uint32_t w2off = ((uint32_t)w2row * (uint32_t)V + 8u * (uint32_t)w2h_slot(w2row, lane & 7)) * 2u;
  const int c00 = t_begin * kTileCols;
  auto bufp = [&](int j) -> unsigned char* { return smem + (size_t)(j % kRingStages) * kHalfBytes; };
  auto issue_w2 = [&](int j) {
    unsigned char* buf = bufp(j);
    const int c = c00 + kHalfCols * j;
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      const int rbase = kKPerWave * wave + 8 * i;
      dma16(W2 + c, w2off + (uint32_t)(i * 16) * (uint32_t)V, buf + (size_t)rbase * 128);
    }
  };
  auto issue_u = [&](int j, float4 (&u)[2][4]) {
    const int c = c00 + kHalfCols * j;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) u[nb][q] = *reinterpret_cast<const float4*>(urow + c + 32 * nb + 8 * q);
  };

  // Issue order: the previous token, alone (waiting for it then waits for
  // nothing else), the W1 row, W2(0), U(0), W2(1), U(1).  Everything a
  // workgroup needs for step 0 is thus requested before the bulk of the
  // kernel's loads, and the W1 row ahead of the halves.
  bf16x8 ev[kParts][16];
  float4 uA[2][4], uB[2][4];
  bool stored = false;
  if constexpr (kParts == 1 && kWaves == kRingWaves) {
    if (a.esw) {
      // The operand stored by the previous position's selection: 16
      // fully-coalesced 1 KB loads per wave, no dependence on the previous
      // token.  (Rows whose previous token was invalid read a stale operand;
      // their summaries are never used, the selection propagating the
      // invalid token.)
      const uint4* ew = a.esw + ((size_t)group * kRingWaves + wave) * 16 * kWave + lane;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint4 v = ew[(size_t)j * kWave];
        ev[0][j] = __builtin_bit_cast(bf16x8, v);
      }
      issue_w2(0);
      issue_u(0, uA);
      stored = true;
    }
  }
  if (!stored) {
    // the W1 row of the previous token, or operand-table row b gamma + kk of
    // kParts parts
    const int prev = prev_token(a, row_info(a, Rc));
    const bool ok = rowok && prev_ok(a, prev);
    const uint16_t* w1row =
        reinterpret_cast<const uint16_t*>(a.W1) + (size_t)(ok ? prev : 0) * kParts * kFastR + 8 * hh;
#pragma unroll
    for (int p = 0; p < kParts; ++p)
#pragma unroll
      for (int j = 0; j < 16; ++j) ev[p][j] = *reinterpret_cast<const bf16x8*>(w1row + p * kFastR + j * 16);
    issue_w2(0);
    issue_u(0, uA);
    if (!ok) {
#pragma unroll
      for (int p = 0; p < kParts; ++p)
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) ev[p][j][e] = (__bf16)0.0f;
    }
  }
  issue_w2(1);
  issue_u(1, uB);

  const int trow = 8 * hh + ((lane & 15) >> 2);             // + 16 j + 4 h
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + 32 nb
  auto logits = [&](const unsigned char* buf, const float4 (&u)[2][4], float (&x)[2][16]) {
    f32x16 acc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][i] = 0.0f;
    auto w2frag = [&](int j, int nb) -> bf16x8 {
      bf16x8 av;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 16 * j + 4 * h + trow;
        const int col = 32 * nb + tcol;
        const int addr = row * 128 + w2h_slot(row, col >> 3) * 16 + (col & 7) * 2;
        const bf16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(buf + addr));
#pragma unroll
        for (int e = 0; e < 4; ++e) av[4 * h + e] = t[e];
      }
      return av;
    };
    if constexpr (kParts == 1) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const bf16x8 av = w2frag(j, nb);
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, ev[0][j], acc[nb], 0, 0, 0);
        }
      }
    } else {
      // both parts against the same W2 fragments; the accumulators alternate
      // so that no MFMA waits on the one just issued
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bf16x8 av0 = w2frag(j, 0), av1 = w2frag(j, 1);
#pragma unroll
        for (int p = 0; p < kParts; ++p) {
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av0, ev[p][j], acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av1, ev[p][j], acc[1], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[nb][i] = acc[nb][i] + comp(u[nb][i >> 2], i & 3);
  };

  // One tile = steps j, j + 1.
  for (int tile = t_begin; tile < t_end; ++tile) {
    const bool more = tile + 1 < t_end;  // halves j + 2, j + 3 exist
    const int j = 2 * (tile - t_begin);
    const int c0 = tile * kTileCols;
    float x[2][16];
    float m0, s0, bv0;
    int bp0;

    // first half: step j (uA); half j + 1 always exists
    __builtin_amdgcn_sched_barrier(0);
    wait_vmem<kWait>();
    __syncthreads();
    if (more) issue_w2(j + 2);
    logits(bufp(j), uA, x);
    if constexpr (kMode == kModeSample) {
      float m = -__builtin_inff();
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, x[nb][i]);
      const float mc = m * a.cf;
      float sum = 0.0f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += fast_exp2(fmaf(x[nb][i], a.cf, -mc));
      m0 = m;
      s0 = m == -__builtin_inff() ? 0.0f : sum;
      asm volatile("" : "+v"(m0), "+v"(s0));
    } else {
      float bv = -__builtin_inff();
      int bpos = 0;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (x[nb][i] > bv) {  // ascending columns: the lowest index wins ties
            bv = x[nb][i];
            bpos = nb * 16 + i;
          }
      bv0 = bv;
      bp0 = bpos;
      asm volatile("" : "+v"(bv0), "+v"(bp0));
    }
    __builtin_amdgcn_sched_barrier(0);
    // past the last half the loads are still issued (of half j again, whose
    // lines are still cached, values unused): the loop keeps one shape and
    // every path carries the same loads
    issue_u(more ? j + 2 : j, uA);

    // second half: step j + 1 (uB)
    __builtin_amdgcn_sched_barrier(0);
    // after U(j + 1): W2(j + 2) if it exists, then the eight loads into uA
    if (more) {
      wait_vmem<kWait>();
    } else {
      wait_vmem<8>();
    }
    __syncthreads();
    if (more) issue_w2(j + 3);
    logits(bufp(j + 1), uB, x);
    if constexpr (kMode == kModeSample) {
      float m = -__builtin_inff();
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, x[nb][i]);
      const float mc = m * a.cf;
      float sum = 0.0f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += fast_exp2(fmaf(x[nb][i], a.cf, -mc));
      if (m == -__builtin_inff()) sum = 0.0f;
      const MergeMS merge{a.cf};
      merge(m, sum, m0, s0);
      const float om = __shfl_xor(m, 32), os = __shfl_xor(sum, 32);
      merge(m, sum, om, os);
      if (hh == 0 && rowok) a.partials[(size_t)R * a.ntiles + tile] = make_float2(m, sum);
    } else {
      float bv = -__builtin_inff();
      int bpos = 0;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (x[nb][i] > bv) {
            bv = x[nb][i];
            bpos = nb * 16 + i;
          }
      const int cb = c0 + 4 * hh;
      int b0 = cb + 32 * (bp0 >> 4) + 8 * ((bp0 >> 2) & 3) + (bp0 & 3);
      const int b1 = cb + kHalfCols + 32 * (bpos >> 4) + 8 * ((bpos >> 2) & 3) + (bpos & 3);
      float bvm = bv0;
      argmax_merge(bvm, b0, bv, b1);
      const float ov = __shfl_xor(bvm, 32);
      const int oi = __shfl_xor(b0, 32);
      argmax_merge(bvm, b0, ov, oi);
      if (hh == 0 && rowok) a.partials[(size_t)R * a.ntiles + tile] = make_float2(bvm, __int_as_float(b0));
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_u(more ? j + 3 : j + 1, uB);
  }
}

template <int kMode, bool kBf16>
__global__ __launch_bounds__(kTileThreads, kMode == kModeOverlap ? 1 : 2) void tile_pass_kernel(TileArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  int tile, group;
  if (!block_tile(a, tile, group)) return;
  const int v0 = tile * kTileCols;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int pitch = a.r + 8;
  const int n = lane & 31;
  const int c4 = v0 + 4 * n;                       // first of this lane's 4 columns
  const bool full = (v0 + kTileCols <= a.V) && ((a.V & 3) == 0);
  uint16_t* sW = reinterpret_cast<uint16_t*>(smem);

  const int row0 = a.row_begin + group * a.rows_per_group;
  const int row1 = min(a.row_end, row0 + a.rows_per_group);
  const int nrb = (row1 - row0 + 31) / 32;
  const int ksteps = a.r / 16;

  // The epilogue's row loads of a row block are issued before anything that
  // waits: for the first row block even before the W2 tile is staged.
  float4 u4[16];
  float4 t4[kMode == kModeOverlap ? 16 : 1];
  auto issue_rows = [&](int rb) {
    const int R0 = row0 + rb * 32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int R = R0 + acc_row(i, lane);
      if (rb < nrb && R < row1 && kMode != kModeBias) {
        const RowInfo ri = row_info(a, R);
        u4[i] = load4(a.U + ((size_t)ri.b * a.gamma + ri.kk) * (size_t)a.V, c4, a.V, full);
        if constexpr (kMode == kModeOverlap)
          t4[i] = load4(a.target + ((size_t)ri.b * (a.gamma + 1) + ri.kk) * (size_t)a.V, c4, a.V, full);
      } else {
        u4[i] = make_float4(-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff());
        if constexpr (kMode == kModeOverlap) t4[i] = u4[i];
      }
    }
  };
  issue_rows(wave);

  if constexpr (kBf16) {
    stage_w2_tile(reinterpret_cast<const uint16_t*>(a.W2), sW, a.r, a.V, v0, pitch);
    __syncthreads();
  }

  for (int rb = wave; rb < nrb; rb += kTileThreads / kWave) {
    const int R0 = row0 + rb * 32;
    if (rb != wave) issue_rows(rb);

    f32x16 acc[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][i] = 0.0f;

    if constexpr (kBf16) {
      // A operand: the lane's row (lane % 32) of E = W1[prev], k-chunk lane / 32.
      const int arow = R0 + (lane & 31);
      int prev = -1;
      if (arow < row1) prev = prev_token(a, row_info(a, arow));
      const bool ok = arow < row1 && prev_ok(a, prev);
      // Operand rows may hold several parts of r values (a bf16 value and its
      // bf16 remainder); every part multiplies the same staged W2 tile.
      const int parts = a.opnd_rows > 0 ? a.opnd_rows : 1;
      const uint16_t* w1base = reinterpret_cast<const uint16_t*>(a.W1) + (size_t)(ok ? prev : 0) * parts * a.r;
      const int koff = 8 * (lane >> 5);
      const uint16_t* bcol = sW + (size_t)(lane & 31) * pitch + koff;
      for (int part = 0; part < parts; ++part)
      for (int k0 = 0; k0 < ksteps; k0 += 16) {
        const uint16_t* w1row = w1base + (size_t)part * a.r;
        bf16x8 av[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (ok && k0 + j < ksteps) {
            av[j] = *reinterpret_cast<const bf16x8*>(w1row + (k0 + j) * 16 + koff);
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) av[j][q] = (__bf16)0.0f;
          }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (k0 + j < ksteps) {
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
              const bf16x8 bv = *reinterpret_cast<const bf16x8*>(bcol + (size_t)nb * 32 * pitch + (k0 + j) * 16);
              acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[j], bv, acc[nb], 0, 0, 0);
            }
          }
        }
      }
    } else {
      // float32 weights: each lane forms its 16 rows x 4 columns directly.
      const float* W1f = reinterpret_cast<const float*>(a.W1);
      const float* W2f = reinterpret_cast<const float*>(a.W2);
      const int parts = a.opnd_rows > 0 ? a.opnd_rows : 1;
      int prevs[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int R = R0 + acc_row(i, lane);
        int p = -1;
        if (R < row1) p = prev_token(a, row_info(a, R));
        prevs[i] = (R < row1 && prev_ok(a, p)) ? p : -1;
      }
      for (int kq = 0; kq < a.r; ++kq) {
        float w2v[kNB];
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) w2v[nb] = c4 + nb < a.V ? W2f[(size_t)kq * a.V + c4 + nb] : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float e = 0.0f;
          if (prevs[i] >= 0)
            for (int part = 0; part < parts; ++part) e += W1f[((size_t)prevs[i] * parts + part) * a.r + kq];
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) acc[nb][i] = fmaf(e, w2v[nb], acc[nb][i]);
        }
      }
    }

    if constexpr (kMode == kModeBias) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int R = R0 + acc_row(i, lane);
        if (R >= row1) continue;
        const int p = a.x0[R];
        const float nanv = __builtin_nanf("");
        const bool ok = p >= 0 && p < a.V;
        float* orow = a.bias_out + (size_t)R * a.V;
        if (full) {
          *reinterpret_cast<float4*>(orow + c4) =
              ok ? make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]) : make_float4(nanv, nanv, nanv, nanv);
        } else {
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb)
            if (c4 + nb < a.V) orow[c4 + nb] = ok ? acc[nb][i] : nanv;
        }
      }
      continue;
    }

    // Epilogue: register i holds row acc_row(i, lane), columns c4..c4+3.
    float ra[16], rb2[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x[kNB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) x[nb] = acc[nb][i] + comp(u4[i], nb);  // -inf stays -inf
      if constexpr (kMode == kModeSample) {
        const float m = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        float sum = 0.0f;
        if (m != -__builtin_inff()) {
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) sum += fast_exp2((x[nb] - m) * a.cf);
        }
        ra[i] = m;
        rb2[i] = sum;
      } else if constexpr (kMode == kModeGreedy) {
        float bv = x[0];
        int bi = c4;
#pragma unroll
        for (int nb = 1; nb < kNB; ++nb) {
          if (x[nb] > bv) {
            bv = x[nb];
            bi = c4 + nb;
          }
        }
        ra[i] = bv;
        rb2[i] = __int_as_float(bi);
      } else {  // kModeOverlap
        const int R = R0 + acc_row(i, lane);
        float sum = 0.0f;
        if (R < row1) {
          const RowInfo ri = row_info(a, R);
          const float ld2 = a.lse_d[(size_t)ri.b * a.gamma + ri.kk] * kLog2e;
          const float lt2 = a.lt2[R];
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const float pd = fast_exp2(x[nb] * a.cf - ld2);
            const float pt = fast_exp2(comp(t4[kMode == kModeOverlap ? i : 0], nb) * a.cf - lt2);
            sum += fminf(pd, pt);
          }
        }
        ra[i] = sum;
        rb2[i] = 0.0f;
      }
    }
    if constexpr (kMode == kModeSample) {
      transpose_reduce(ra, rb2, lane, MergeMS{a.cf});
    } else if constexpr (kMode == kModeGreedy) {
      transpose_reduce(ra, rb2, lane, MergeArgmax{});
    } else {
      transpose_reduce(ra, rb2, lane, MergeSum{});
    }
    const int R = R0 + acc_row((lane & 31) >> 1, lane);
    if ((lane & 1) == 0 && R < row1) a.partials[(size_t)R * a.ntiles + tile] = make_float2(ra[0], rb2[0]);
  }
}

// Compute units of the current device (cached per device).
int compute_units_of_device() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// The ring kernel's LDS (96 KB) is above the default dynamic limit: raise the
// limit once per process for each instantiation (the attribute belongs to the
// kernel, not to a device).
template <int kMode, int kWaves = kRingWaves, int kParts = 1>
static hipError_t ring_lds_attribute(size_t lds) {
  static hipError_t state = hipErrorNotReady;
  if (state == hipErrorNotReady)
    state = hipFuncSetAttribute((const void*)tile_ring_kernel<kMode, kWaves, kParts>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  return state;
}

// Rows [row_begin, row_end) x tiles [tile_begin, tile_begin + tile_count) with
// the one-tile-per-workgroup kernel.
template <int kMode, bool kBf16>
static void launch_tiles(const TileArgs& a, int row_begin, int row_end, int tile_begin, int tile_count,
                         hipStream_t s) {
  if (row_end <= row_begin || tile_count <= 0) return;
  const size_t lds = kBf16 ? (size_t)kTileCols * (a.r + 8) * sizeof(uint16_t) : 0;
  TileArgs g = a;
  g.rows_per_group = kRowsPerGroup;
  g.ngroups = (row_end - row_begin + kRowsPerGroup - 1) / kRowsPerGroup;
  g.row_begin = row_begin;
  g.row_end = row_end;
  g.tile_begin = tile_begin;
  g.tile_count = tile_count;
  const int blocks = g.ngroups == 1 ? tile_count : ((tile_count + 7) / 8) * 8 * g.ngroups;
  hipLaunchKernelGGL((tile_pass_kernel<kMode, kBf16>), dim3(blocks), dim3(kTileThreads), lds, s, g);
}

// Full 128-column tiles of the vocabulary on the fast paths (V % 4 == 0).
static int fast_full_tiles(const TileArgs& a) { return (a.V & 3) == 0 ? a.V / kTileCols : 0; }

// The fast paths: bf16 weights, r = 256, W1 rows of previous tokens (or
// two-part operand rows, pipelined kernel only), at least one full tile, rows
// at a constant stride, and W2 addressed with 32-bit byte offsets (2 r V < 2^32).
static bool fast_path(const TileArgs& a, int mode, bool bf16) {
  // two-part operand rows: sample and argmax modes, one block position per
  // launch (the ring kernels)
  return bf16 && (mode == kModeSample || mode == kModeGreedy || mode == kModeOverlap) && a.r == kFastR &&
         (a.opnd_rows == 0 || (a.opnd_rows == 2 && mode != kModeOverlap && a.kper == 1)) &&
         (a.kper == 1 || a.kper == a.gamma) && fast_full_tiles(a) > 0 &&
         (size_t)2 * kFastR * (size_t)a.V < ((size_t)1 << 32);
}

// The eight-wave ring's 256-row groups are at least 3/4 filled.
static bool ring_wide(const TileArgs& a) {
  const int rgroups = (a.nrows + kRingRows - 1) / kRingRows;
  return 4 * a.nrows >= 3 * rgroups * kRingRows;
}

bool tile_pass_uses_ring(const TileArgs& a, int mode, bool bf16) {
  // the eight-wave ring with W1 rows (whose previous position's selection can
  // store them in the ring's operand layout)
  return fast_path(a, mode, bf16) && (mode == kModeSample || mode == kModeGreedy) && a.kper == 1 &&
         a.opnd_rows == 0 && ring_wide(a);
}

// The full tiles of all rows on tile_ring_kernel<kMode, kWaves, kParts>: one
// workgroup per CU, the column slices of every row group together filling
// the CUs once.
template <int kMode, int kWaves, int kParts>
static hipError_t launch_ring(const TileArgs& a, int full_tiles, hipStream_t s) {
  constexpr int kRows = 32 * kWaves;
  const int rgroups = (a.nrows + kRows - 1) / kRows;
  const size_t lds = (size_t)kRingStages * kHalfBytes;
  const hipError_t e = ring_lds_attribute<kMode, kWaves, kParts>(lds);
  if (e != hipSuccess) return e;
  TileArgs g = a;
  g.ngroups = rgroups;
  g.rows_per_group = kRows;
  g.row_begin = 0;
  g.row_end = a.nrows;
  g.tile_begin = 0;
  g.tile_count = full_tiles;
  int nslices = compute_units_of_device() / rgroups;
  if (nslices >= 8) nslices &= ~7;
  nslices = nslices < 1 ? 1 : (nslices > full_tiles ? full_tiles : nslices);
  hipLaunchKernelGGL((tile_ring_kernel<kMode, kWaves, kParts>), dim3(rgroups * nslices), dim3(kWave * kWaves), lds, s,
                     g, nslices);
  return hipGetLastError();
}

template <int kMode, bool kBf16>
static hipError_t launch_mode(const TileArgs& a, hipStream_t s) {
  ProfScope prof(s, kProfTileSample + kMode);
  const int groups = (a.nrows + kRowsPerGroup - 1) / kRowsPerGroup;  // the last one may be partial
  const int full_tiles = fast_full_tiles(a);
  if (!fast_path(a, kMode, kBf16)) {
    launch_tiles<kMode, kBf16>(a, 0, a.nrows, 0, a.ntiles, s);
    return hipGetLastError();
  }
  if constexpr (kBf16 && (kMode == kModeSample || kMode == kModeGreedy)) {
    // The ring kernels (one launch of rows at a constant stride):
    //   eight waves (256-row groups) when those groups are at least 3/4
    //   filled, for W1 rows and for two-part operand rows alike;
    //   otherwise four waves (128-row groups) for two-part operand rows, and
    //   for single-part launches of at most 64 rows (most of a 128-row group
    //   idle: the W2 stream sets the time, and the ring keeps more of it in
    //   flight than two two-buffer workgroups do).
    hipError_t e = hipSuccess;
    bool ring = a.kper == 1;
    if (ring && a.opnd_rows == 0 && ring_wide(a)) {
      e = launch_ring<kMode, kRingWaves, 1>(a, full_tiles, s);
    } else if (ring && a.opnd_rows == 2 && ring_wide(a)) {
      e = launch_ring<kMode, kRingWaves, 2>(a, full_tiles, s);
    } else if (ring && a.opnd_rows == 2) {
      e = launch_ring<kMode, kRing2Waves, 2>(a, full_tiles, s);
    } else if (ring && a.opnd_rows == 0 && a.nrows <= 64) {
      e = launch_ring<kMode, kRing2Waves, 1>(a, full_tiles, s);
    } else {
      ring = false;
    }
    if (ring) {
      if (e != hipSuccess) return e;
      launch_tiles<kMode, kBf16>(a, 0, a.nrows, full_tiles, a.ntiles - full_tiles, s);
      return hipGetLastError();
    }
  }
  if constexpr (kBf16 && (kMode == kModeSample || kMode == kModeGreedy || kMode == kModeOverlap)) {
    TileArgs g = a;
    g.ngroups = groups;
    g.rows_per_group = kRowsPerGroup;
    g.row_begin = 0;
    g.row_end = a.nrows;
    g.tile_begin = 0;
    g.tile_count = full_tiles;
    // Two resident workgroups per CU (64 KB of LDS each; one in overlap mode,
    // whose waves also hold the target values); the column slices of every
    // row group together fill them once.
    const bool one_per_cu = kMode == kModeOverlap;
    int nslices = (one_per_cu ? 1 : 2) * compute_units_of_device() / groups;
    if (nslices >= 8) nslices &= ~7;
    nslices = nslices < 1 ? 1 : (nslices > full_tiles ? full_tiles : nslices);
    const size_t lds = 2 * (size_t)kHalfBytes;
    hipLaunchKernelGGL((tile_pipe_kernel<kMode>), dim3(groups * nslices), dim3(kTileThreads), lds, s, g, nslices);
  }
  // The partial last tile, all rows.
  launch_tiles<kMode, kBf16>(a, 0, a.nrows, full_tiles, a.ntiles - full_tiles, s);
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
