// Decode-form expert GEMV passes (dense fp32 / bf16 weights), shared by ffn.hip.
//
// A pass computes, for every routed group in the work list and every row r
// of its weight matrix W [rows, K] (K contiguous), the dot products of r with
// the group's activation rows:
//   pass 1 (SWIGLU): W = W13 of the slot (row 2n = gate n, row 2n+1 = up n),
//            activations = tokens x[perm[p] / k]; epilogue h[p][n] = SiLU(g) * u
//   pass 2:  W = W2 of the slot (row = output feature), activations = h[p];
//            epilogue y[p][row] = dot.
// AF is the activation format (tokens: fp32 or bf16; h: fp32); NTL marks
// the weight loads non-temporal (streamed once, kept out of the caches).
// Work decomposition (256 threads = 4 waves per workgroup):
//   - a workgroup owns RPW * (4 / KS) consecutive rows of one group;
//   - KS waves share a row block and split K: wave slice s takes the 512-
//     element chunks s, s + KS, s + 2 KS, ... (lane l holds elements
//     chunk * 512 + 8 l .. + 7, one 16-byte load for bf16);
//   - U chunks are loaded before they are used, so every lane keeps
//     RPW * U 16-byte weight loads in flight;
//   - activations are read per chunk for a tile of NT <= MAXNT rows, so a
//     weight row is streamed once per tile; fp32 FMA accumulation;
//   - wave reduction by xor shuffles, then the KS partial sums meet in LDS.
#pragma once

#include "common.h"
#include "ffn_internal.h"

namespace gemv {

template <int FMT>
__device__ __forceinline__ void load8(const void* base, size_t elem, float out[8]) {
  if constexpr (FMT == MOE_BF16) {
    u32x4 v = ld16(static_cast<const uint16_t*>(base) + elem);
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
    out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
    out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
  } else {
    const float* p = static_cast<const float*>(base) + elem;
    u32x4 a = ld16(p), b = ld16(p + 4);
    out[0] = __uint_as_float(a.x); out[1] = __uint_as_float(a.y);
    out[2] = __uint_as_float(a.z); out[3] = __uint_as_float(a.w);
    out[4] = __uint_as_float(b.x); out[5] = __uint_as_float(b.y);
    out[6] = __uint_as_float(b.z); out[7] = __uint_as_float(b.w);
  }
}

// Raw 16-byte weight vector (8 bf16 or 4+4 fp32 in two loads).
template <int FMT>
struct WVec {
  u32x4 a, b;
};

template <int FMT, bool NTL>
__device__ __forceinline__ WVec<FMT> wload(const char* row, size_t elem) {
  WVec<FMT> v;
  if constexpr (FMT == MOE_BF16) {
    v.a = NTL ? ld16_stream(row + elem * 2) : ld16(row + elem * 2);
  } else {
    v.a = NTL ? ld16_stream(row + elem * 4) : ld16(row + elem * 4);
    v.b = NTL ? ld16_stream(row + elem * 4 + 16) : ld16(row + elem * 4 + 16);
  }
  return v;
}

template <int FMT>
__device__ __forceinline__ void wunpack(const WVec<FMT>& v, float w[8]) {
  if constexpr (FMT == MOE_BF16) {
    w[0] = bf16_lo(v.a.x); w[1] = bf16_hi(v.a.x);
    w[2] = bf16_lo(v.a.y); w[3] = bf16_hi(v.a.y);
    w[4] = bf16_lo(v.a.z); w[5] = bf16_hi(v.a.z);
    w[6] = bf16_lo(v.a.w); w[7] = bf16_hi(v.a.w);
  } else {
    w[0] = __uint_as_float(v.a.x); w[1] = __uint_as_float(v.a.y);
    w[2] = __uint_as_float(v.a.z); w[3] = __uint_as_float(v.a.w);
    w[4] = __uint_as_float(v.b.x); w[5] = __uint_as_float(v.b.y);
    w[6] = __uint_as_float(v.b.z); w[7] = __uint_as_float(v.b.w);
  }
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

// One tile of NT activation rows starting at sorted position prow.
template <int WF, int AF, int OF, int RPW, int KS, int U, int NT, bool SWIGLU, bool NTL>
__device__ __forceinline__ void tile(const char* __restrict__ wrows, size_t rowb, int K,
                                     const void* __restrict__ act, const int32_t* __restrict__ perm,
                                     int k, int prow, int r0, bool store, int out_ld,
                                     void* __restrict__ out, float* __restrict__ red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slice = wave % KS;
  size_t arow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) arow[t] = SWIGLU ? (size_t)(perm[prow + t] / k) : (size_t)(prow + t);
  float acc[RPW][NT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;

  const int nchunks = (K + 511) / 512;
  for (int c0 = slice; c0 < nchunks; c0 += KS * U) {
    WVec<WF> wv[U][RPW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * KS;
      const size_t e = (size_t)c * 512 + lane * 8;
      if (c < nchunks && e < (size_t)K) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) wv[u][r] = wload<WF, NTL>(wrows + r * rowb, e);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * KS;
      const size_t e = (size_t)c * 512 + lane * 8;
      if (c < nchunks && e < (size_t)K) {
        float xv[NT][8];
#pragma unroll
        for (int t = 0; t < NT; ++t) load8<AF>(act, arow[t] * K + e, xv[t]);
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          float w[8];
          wunpack<WF>(wv[u][r], w);
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[r][t] = fmaf(w[q], xv[t][q], acc[r][t]);
        }
      }
    }
  }
  // wave reduction, then the KS slices of a row block meet in LDS
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = wave_sum(acc[r][t]);
  if constexpr (KS > 1) {
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) red[(wave * RPW + r) * NT + t] = acc[r][t];
    }
    __syncthreads();
    if (slice == 0) {
#pragma unroll
      for (int s = 1; s < KS; ++s)
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[r][t] += red[((wave + s) * RPW + r) * NT + t];
    }
    __syncthreads();
  }
  if (store && slice == 0 && lane < NT) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (lane == t) {
        if constexpr (SWIGLU && OF == MOE_BF16) {
          uint16_t* o = static_cast<uint16_t*>(out) + (size_t)(prow + t) * out_ld;
#pragma unroll
          for (int r = 0; r < RPW; r += 2)
            o[(r0 + r) / 2] = f32_to_bf16_rne(silu(acc[r][t]) * acc[r + 1][t]);
        } else if constexpr (SWIGLU) {
          float* o = static_cast<float*>(out) + (size_t)(prow + t) * out_ld;
#pragma unroll
          for (int r = 0; r < RPW; r += 2) o[(r0 + r) / 2] = silu(acc[r][t]) * acc[r + 1][t];
        } else {
          float* o = static_cast<float*>(out) + (size_t)(prow + t) * out_ld;
#pragma unroll
          for (int r = 0; r < RPW; ++r) o[r0 + r] = acc[r][t];
        }
      }
    }
  }
}

// rows: rows of W per group; K: inputs per row; off: byte offset of W in a
// slot. Work unit u = (item u / row_blocks, row block u % row_blocks); the
// grid may be smaller than the number of units (each workgroup loops).
template <int WF, int AF, int OF, int RPW, int KS, int U, int MAXNT, bool SWIGLU, bool NTL>
__global__ __launch_bounds__(256) void pass_kernel(const void* __restrict__ act,
                                                   const int32_t* __restrict__ perm, int k,
                                                   const FfnItem* __restrict__ items,
                                                   const int32_t* __restrict__ n_items,
                                                   const char* __restrict__ pool, size_t stride,
                                                   size_t off, int rows, int K, int out_ld,
                                                   int row_blocks, void* __restrict__ out) {
  __shared__ float red[4 * RPW * MAXNT];
  constexpr int kBlocksPerWg = 4 / KS;
  constexpr size_t esz = (WF == MOE_BF16) ? 2 : 4;
  const size_t rowb = (size_t)K * esz;
  const int wave = threadIdx.x >> 6;
  const int units = n_items[0] * row_blocks;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int item = u / row_blocks;
    const int rb = u - item * row_blocks;
    const FfnItem it = items[item];
    // A row block past the end (rows not a multiple of the workgroup's rows)
    // still takes part in the LDS barriers: it re-reads block 0 and stores nothing.
    int r0 = (rb * kBlocksPerWg + wave / KS) * RPW;
    const bool store = r0 < rows;
    if (!store) r0 = 0;
    const char* wrows = pool + (size_t)it.slot * stride + off + (size_t)r0 * rowb;
    int done = 0;
    for (; it.rows - done >= MAXNT; done += MAXNT)
      tile<WF, AF, OF, RPW, KS, U, MAXNT, SWIGLU, NTL>(wrows, rowb, K, act, perm, k,
                                                       it.row_begin + done, r0, store, out_ld, out,
                                                       red);
    const int rest = it.rows - done, p = it.row_begin + done;
#define MOE_GEMV_TILE(NT_)                                                                       \
  tile<WF, AF, OF, RPW, KS, U, NT_, SWIGLU, NTL>(wrows, rowb, K, act, perm, k, p, r0, store, out_ld, \
                                                 out, red)
    if constexpr (MAXNT > 1) {
      if (rest == 1) MOE_GEMV_TILE(1);
    }
    if constexpr (MAXNT > 2) {
      if (rest == 2) MOE_GEMV_TILE(2);
      if (rest == 3) MOE_GEMV_TILE(3);
    }
    if constexpr (MAXNT > 4) {
      if (rest == 4) MOE_GEMV_TILE(4);
      if (rest == 5) MOE_GEMV_TILE(5);
      if (rest == 6) MOE_GEMV_TILE(6);
      if (rest == 7) MOE_GEMV_TILE(7);
    }
#undef MOE_GEMV_TILE
  }
}

// Workgroups along the rows of one group for a pass.
template <int RPW, int KS>
inline unsigned row_blocks(int rows) {
  const int per_wg = RPW * (4 / KS);
  return (unsigned)((rows + per_wg - 1) / per_wg);
}

}  // namespace gemv
