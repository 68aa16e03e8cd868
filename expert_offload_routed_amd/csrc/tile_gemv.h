// Decode-form expert GEMV passes over tile-major weights (bf16; int4; and the
// int4 + int4-residual and int8 forms of split-precision experts), shared by
// ffn.hip and ffn_int4.hip.
//
// Tile-major layout (moe_slot_layout): the weights of a 32-row block are
// consecutive 1 KB chunks; in chunk ks lane l holds row l % 32 and the K
// range ks * KC + half (l / 32), so one 16-byte load per lane reads 1 KB of
// contiguous memory. A pass computes, for every routed group in the work
// list and every row r of W [R, K], the dot products of r with the group's
// activation rows:
//   pass 1 (SWIGLU): W = W13 (row 2n = gate n, row 2n+1 = up n), activations
//            = tokens x[perm[p] / k]; epilogue h[p][n] = SiLU(g) * u (gate and
//            up rows sit in neighbouring lanes);
//   pass 2:  W = W2, activations = h[p]; epilogue y[p][row] = dot.
// A workgroup has NW waves; KS waves share RBW row blocks and split their
// chunks (chunk ks goes to wave slice ks % KS), U x RBW chunks in flight per
// lane; each activation load serves RBW rows. The two K halves of a row
// (lanes l, l + 32) meet through a shuffle, the KS slices in LDS. Each weight
// chunk is streamed once per tile of NT <= MAXNT rows.
#pragma once

#include "common.h"
#include "ffn_internal.h"

namespace tgemv {

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

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

// int4 codes to int8 bytes holding 16 q (exact, in [-128, 112]): a code moved to
// the high nibble of its byte keeps its sign. A 32-bit word holds codes c..c+3
// in its low nibbles and c+4..c+7 in its high nibbles.
__device__ __forceinline__ uint32_t q16_lo(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t q16_hi(uint32_t w) { return w & 0xF0F0F0F0u; }

// Final reduction and epilogue, shared by both formats. acc[b][t] holds this
// lane's partial dot of row (rb0 + b) * 32 + lane % 32 (one K half, one K slice).
template <int RBW, int NT, int KS, bool SWIGLU, int OF>
__device__ __forceinline__ void finish(float (&acc)[RBW][NT], const float* scale_t, int prow,
                                       int rb0, int nrb, int out_ld, void* __restrict__ out,
                                       float* __restrict__ red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slice = wave % KS;
#pragma unroll
  for (int b = 0; b < RBW; ++b)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[b][t] += __shfl_xor(acc[b][t], 32, 64);
  if constexpr (KS > 1) {
    if (lane < 32) {
#pragma unroll
      for (int b = 0; b < RBW; ++b)
#pragma unroll
        for (int t = 0; t < NT; ++t) red[((wave * RBW + b) * 32 + lane) * NT + t] = acc[b][t];
    }
    __syncthreads();
    if (slice == 0) {
#pragma unroll
      for (int s = 1; s < KS; ++s)
#pragma unroll
        for (int b = 0; b < RBW; ++b)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[b][t] += red[(((wave + s) * RBW + b) * 32 + (lane & 31)) * NT + t];
    }
    __syncthreads();
  }
  if (slice != 0) return;
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const bool store = rb0 + b < nrb;
    const int row = (rb0 + b) * 32 + (lane & 31);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float v = acc[b][t] * (scale_t ? scale_t[t] : 1.f);
      if constexpr (SWIGLU) {
        const float u = __shfl_xor(v, 1, 64);  // odd row = up of the same neuron
        if (store && lane < 32 && (lane & 1) == 0) {
          const float hv = silu(v) * u;
          if constexpr (OF == MOE_BF16)
            static_cast<uint16_t*>(out)[(size_t)(prow + t) * out_ld + (row >> 1)] = f32_to_bf16_rne(hv);
          else
            static_cast<float*>(out)[(size_t)(prow + t) * out_ld + (row >> 1)] = hv;
        }
      } else {
        if (store && lane < 32) static_cast<float*>(out)[(size_t)(prow + t) * out_ld + row] = v;
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 ---
template <int AF, int OF, int KS, int RBW, int U, int NT, bool SWIGLU>
__device__ __forceinline__ void tile_bf16(const char* __restrict__ wbase, int nks, int K,
                                          const void* __restrict__ act,
                                          const int32_t* __restrict__ perm, int k, int prow,
                                          int rb0, int nrb, int out_ld, void* __restrict__ out,
                                          float* __restrict__ red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slice = wave % KS;
  const int kh = 8 * (lane >> 5);
  size_t arow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) arow[t] = SWIGLU ? (size_t)(perm[prow + t] / k) : (size_t)(prow + t);
  float acc[RBW][NT];
#pragma unroll
  for (int b = 0; b < RBW; ++b)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[b][t] = 0.f;
  // block b's chunks; blocks past the end re-read the last block (their rows are not stored)
  const char* wl[RBW];
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const int rb = (rb0 + b < nrb) ? rb0 + b : nrb - 1;
    wl[b] = wbase + (size_t)rb * nks * 1024 + lane * 16;
  }
  for (int ks0 = slice; ks0 < nks; ks0 += KS * U) {
    u32x4 wv[U][RBW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = ks0 + u * KS;
      if (ks < nks) {
#pragma unroll
        for (int b = 0; b < RBW; ++b) wv[u][b] = ld16_stream(wl[b] + (size_t)ks * 1024);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = ks0 + u * KS;
      if (ks < nks) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float xv[8];
          load8<AF>(act, arow[t] * K + ks * 16 + kh, xv);
#pragma unroll
          for (int b = 0; b < RBW; ++b) {
            const u32x4& w = wv[u][b];
            acc[b][t] = fmaf(bf16_lo(w.x), xv[0], acc[b][t]);
            acc[b][t] = fmaf(bf16_hi(w.x), xv[1], acc[b][t]);
            acc[b][t] = fmaf(bf16_lo(w.y), xv[2], acc[b][t]);
            acc[b][t] = fmaf(bf16_hi(w.y), xv[3], acc[b][t]);
            acc[b][t] = fmaf(bf16_lo(w.z), xv[4], acc[b][t]);
            acc[b][t] = fmaf(bf16_hi(w.z), xv[5], acc[b][t]);
            acc[b][t] = fmaf(bf16_lo(w.w), xv[6], acc[b][t]);
            acc[b][t] = fmaf(bf16_hi(w.w), xv[7], acc[b][t]);
          }
        }
      }
    }
  }
  finish<RBW, NT, KS, SWIGLU, OF>(acc, nullptr, prow, rb0, nrb, out_ld, out, red);
}

// ------------------------------------------------------------------ int4 ---
// Codes expanded to bytes 16 q; the dot products are 16 sum q x (exact int32)
// and the group scale carries the factor 1/16 (exact in fp32).
__device__ __forceinline__ int dot64_int4(const u32x4& w, const u32x4& a0, const u32x4& a1) {
  int is = 0;
  is = __builtin_amdgcn_sdot4((int)q16_lo(w.x), (int)a0.x, is, false);
  is = __builtin_amdgcn_sdot4((int)q16_hi(w.x), (int)a0.y, is, false);
  is = __builtin_amdgcn_sdot4((int)q16_lo(w.y), (int)a0.z, is, false);
  is = __builtin_amdgcn_sdot4((int)q16_hi(w.y), (int)a0.w, is, false);
  is = __builtin_amdgcn_sdot4((int)q16_lo(w.z), (int)a1.x, is, false);
  is = __builtin_amdgcn_sdot4((int)q16_hi(w.z), (int)a1.y, is, false);
  is = __builtin_amdgcn_sdot4((int)q16_lo(w.w), (int)a1.z, is, false);
  is = __builtin_amdgcn_sdot4((int)q16_hi(w.w), (int)a1.w, is, false);
  return is;
}

// RES adds a second int4 matrix of the same layout (the residual W^R of a
// split-precision expert, codes at rbase, scales rscales) to the first: both
// group products are scaled and accumulated into the same fp32 sums.
// LDSA: the tile's NT activation rows are rows 0..NT-1 of aq / as (staged in
// LDS by stage_rows) instead of rows of the global int8 buffers.
template <int KS, int RBW, int U, int NT, bool SWIGLU, bool RES, bool LDSA = false>
__device__ __forceinline__ void tile_int4(const char* __restrict__ wbase,
                                          const uint16_t* __restrict__ scales,
                                          const char* __restrict__ rbase,
                                          const uint16_t* __restrict__ rscales, int nkc, int K,
                                          const int8_t* __restrict__ aq,
                                          const float* __restrict__ as,
                                          const int32_t* __restrict__ perm, int k, int prow,
                                          int rb0, int nrb, int out_ld, float* __restrict__ out,
                                          float* __restrict__ red) {
  constexpr int UR = RES ? U : 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slice = wave % KS;
  const int kh = 16 * (lane >> 5);
  const int gld = K / 128;
  int arow[NT];
  float sx[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    arow[t] = LDSA ? t : SWIGLU ? perm[prow + t] / k : prow + t;
    sx[t] = as[arow[t]];
  }
  float acc[RBW][NT];
#pragma unroll
  for (int b = 0; b < RBW; ++b)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[b][t] = 0.f;
  const char* wl[RBW];
  const uint16_t* srow[RBW];
  const char* rl[RBW];
  const uint16_t* rrow[RBW];
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const int rb = (rb0 + b < nrb) ? rb0 + b : nrb - 1;
    const size_t wo = (size_t)rb * nkc * 1024 + lane * 16;
    const size_t so = (size_t)(rb * 32 + (lane & 31)) * gld;
    wl[b] = wbase + wo;
    srow[b] = scales + so;
    if constexpr (RES) {
      rl[b] = rbase + wo;
      rrow[b] = rscales + so;
    }
  }
  for (int kc0 = slice; kc0 < nkc; kc0 += KS * U) {
    u32x4 cw[U][RBW];
    float sw[U][RBW];
    u32x4 cr[UR][RBW];
    float sr[UR][RBW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kc = kc0 + u * KS;
      if (kc < nkc) {
#pragma unroll
        for (int b = 0; b < RBW; ++b) {
          cw[u][b] = ld16_stream(wl[b] + (size_t)kc * 1024);
          sw[u][b] = bf16_to_f32(srow[b][kc >> 1]) * 0.0625f;
          if constexpr (RES) {
            cr[u][b] = ld16_stream(rl[b] + (size_t)kc * 1024);
            sr[u][b] = bf16_to_f32(rrow[b][kc >> 1]) * 0.0625f;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kc = kc0 + u * KS;
      if (kc < nkc) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int8_t* ap = aq + (size_t)arow[t] * K + kc * 64 + kh;
          const u32x4 a0 = ld16(ap), a1 = ld16(ap + 32);
#pragma unroll
          for (int b = 0; b < RBW; ++b) {
            acc[b][t] = fmaf((float)dot64_int4(cw[u][b], a0, a1), sw[u][b], acc[b][t]);
            if constexpr (RES)
              acc[b][t] = fmaf((float)dot64_int4(cr[u][b], a0, a1), sr[u][b], acc[b][t]);
          }
        }
      }
    }
  }
  finish<RBW, NT, KS, SWIGLU, MOE_F32>(acc, sx, prow, rb0, nrb, out_ld, out, red);
}

// ------------------------------------------------------------------ int8 ---
// 8-bit codes (the high-precision down projection W^H of a split-precision
// expert): tile-major 1 KB chunks of 32 rows x 32 codes, lane l holding the 16
// codes of row l % 32 at k offset 16 (l / 32); the integer sums are exact and
// the group (4 chunks) scale applies in fp32. Second pass only: the
// activation rows are the permuted rows of h.
template <int KS, int RBW, int U, int NT, bool LDSA = false>
__device__ __forceinline__ void tile_int8(const char* __restrict__ wbase,
                                          const uint16_t* __restrict__ scales, int nkc, int K,
                                          const int8_t* __restrict__ aq,
                                          const float* __restrict__ as, int prow, int rb0,
                                          int nrb, int out_ld, float* __restrict__ out,
                                          float* __restrict__ red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slice = wave % KS;
  const int kh = 16 * (lane >> 5);
  const int gld = K / 128;
  int arow[NT];
  float sx[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    arow[t] = LDSA ? t : prow + t;
    sx[t] = as[arow[t]];
  }
  float acc[RBW][NT];
#pragma unroll
  for (int b = 0; b < RBW; ++b)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[b][t] = 0.f;
  const char* wl[RBW];
  const uint16_t* srow[RBW];
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const int rb = (rb0 + b < nrb) ? rb0 + b : nrb - 1;
    wl[b] = wbase + (size_t)rb * nkc * 1024 + lane * 16;
    srow[b] = scales + (size_t)(rb * 32 + (lane & 31)) * gld;
  }
  for (int kc0 = slice; kc0 < nkc; kc0 += KS * U) {
    u32x4 cw[U][RBW];
    float sw[U][RBW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kc = kc0 + u * KS;
      if (kc < nkc) {
#pragma unroll
        for (int b = 0; b < RBW; ++b) {
          cw[u][b] = ld16_stream(wl[b] + (size_t)kc * 1024);
          sw[u][b] = bf16_to_f32(srow[b][kc >> 2]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kc = kc0 + u * KS;
      if (kc < nkc) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const u32x4 a = ld16(aq + (size_t)arow[t] * K + kc * 32 + kh);
#pragma unroll
          for (int b = 0; b < RBW; ++b) {
            const u32x4& w = cw[u][b];
            int is = 0;
            is = __builtin_amdgcn_sdot4((int)w.x, (int)a.x, is, false);
            is = __builtin_amdgcn_sdot4((int)w.y, (int)a.y, is, false);
            is = __builtin_amdgcn_sdot4((int)w.z, (int)a.z, is, false);
            is = __builtin_amdgcn_sdot4((int)w.w, (int)a.w, is, false);
            acc[b][t] = fmaf((float)is, sw[u][b], acc[b][t]);
          }
        }
      }
    }
  }
  finish<RBW, NT, KS, false, MOE_F32>(acc, sx, prow, rb0, nrb, out_ld, out, red);
}

// ---------------------------------------------------------------- kernels --
// Work unit u = (item u / units_per_item, row-block group u % units_per_item);
// a group is the NW / KS row blocks of one workgroup.
#define TGEMV_REST(CALL)                      \
  if constexpr (MAXNT > 1) {                  \
    if (rest == 1) CALL(1);                   \
  }                                           \
  if constexpr (MAXNT > 2) {                  \
    if (rest == 2) CALL(2);                   \
    if (rest == 3) CALL(3);                   \
  }

template <int AF, int OF, int KS, int RBW, int NW, int U, int MAXNT, bool SWIGLU>
__global__ __launch_bounds__(NW * 64) void bf16_kernel(
    const void* __restrict__ act, const int32_t* __restrict__ perm, int k,
    const FfnItem* __restrict__ items, const int32_t* __restrict__ n_items,
    const char* __restrict__ pool, size_t stride, size_t off, int R, int K, int out_ld,
    int units_per_item, void* __restrict__ out) {
  __shared__ float red[NW * RBW * 32 * MAXNT];
  const int wave = threadIdx.x >> 6;
  const int nks = K / 16;
  const int nrb = R / 32;
  const int units = n_items[0] * units_per_item;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int item = u / units_per_item;
    const int rb0 = ((u - item * units_per_item) * (NW / KS) + wave / KS) * RBW;
    const FfnItem it = items[item];
    const char* wbase = pool + (size_t)it.slot * stride + off;
    int done = 0;
    for (; it.rows - done >= MAXNT; done += MAXNT)
      tile_bf16<AF, OF, KS, RBW, U, MAXNT, SWIGLU>(wbase, nks, K, act, perm, k, it.row_begin + done,
                                                   rb0, nrb, out_ld, out, red);
    const int rest = it.rows - done, p = it.row_begin + done;
#define TGEMV_BF16(NT_)                                                                        \
  tile_bf16<AF, OF, KS, RBW, U, NT_, SWIGLU>(wbase, nks, K, act, perm, k, p, rb0, nrb, out_ld, out, \
                                             red)
    TGEMV_REST(TGEMV_BF16)
#undef TGEMV_BF16
  }
}

// Byte offsets inside a slot of the two weight forms a quantised pass reads:
// lo = the int4 codes and scales every group uses at low precision; hi = the
// second section of a high-precision group (pass 1: the int4 residual added to
// lo; pass 2: the 8-bit codes used instead of lo).
struct QuantOffsets {
  size_t lo, lo_s, hi, hi_s;
};

// The int8 rows of a tile, quantised by the workgroup into LDS: NT rows of K
// values (bf16 tokens x[perm[p] / k] when GATHER, else fp32 rows p of h),
// each with s = max|v| / 127 (1 for a zero row) and q = clip(rint(v / s),
// -127, 127), the rule of quant_rows_kernel, so the codes are the same.
template <bool GATHER, int NT>
__device__ __forceinline__ void stage_rows(const void* __restrict__ raw,
                                           const int32_t* __restrict__ perm, int k, int prow,
                                           int K, int8_t* q, float* s, float* wmax) {
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6;
  __syncthreads();  // the previous tile's readers are done with q and s
#pragma unroll 1
  for (int t = 0; t < NT; ++t) {
    const size_t row = GATHER ? (size_t)(perm[prow + t] / k) : (size_t)(prow + t);
    auto load8v = [&](int e0, float v[8]) {
      if constexpr (GATHER) {
        load8<MOE_BF16>(raw, row * K + e0, v);
      } else {
        load8<MOE_F32>(raw, row * K + e0, v);
      }
    };
    float amax = 0.f;
    for (int e0 = tid * 8; e0 < K; e0 += nthr * 8) {
      float v[8];
      load8v(e0, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = wave_max(amax);
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    float m = 0.f;
    for (int w = 0; w < (nthr >> 6); ++w) m = fmaxf(m, wmax[w]);
    const float sc = (m == 0.f) ? 1.f : m / 127.f;
    for (int e0 = tid * 8; e0 < K; e0 += nthr * 8) {
      float v[8];
      load8v(e0, v);
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float r = rintf(v[i] / sc);
        r = fminf(fmaxf(r, -127.f), 127.f);
        const uint32_t b = (uint32_t)((int)r & 0xFF);
        if (i < 4) w0 |= b << (8 * i); else w1 |= b << (8 * (i - 4));
      }
      *reinterpret_cast<uint2*>(q + (size_t)t * K + e0) = make_uint2(w0, w1);
    }
    if (tid == 0) s[t] = sc;
    __syncthreads();  // wmax is reused by the next row; q and s are complete
  }
}

// LDS of a workgroup that quantises its own activation rows (QIN).
struct StageLds {
  int8_t* q;    // [MAXNT][K]
  float* s;     // [MAXNT]
  float* wmax;  // [16]
};

// Item modes of the quantised passes: 0 = int4, 1 = int4 + int4 residual, 2 = int8.
// QIN: the activation rows are quantised per tile by the workgroup (stage_rows,
// from raw) instead of read from the int8 buffers aq / as.
// staged: the activation row held in the LDS stage when it holds one row (its row
// index in raw), else -1; a one-row tile of the same row is not quantised again.
template <int MODE, int KS, int RBW, int U, int MAXNT, bool SWIGLU, bool QIN>
__device__ __forceinline__ void quant_item(const char* slot, const QuantOffsets& o, int K,
                                           const int8_t* aq, const float* as, const void* raw,
                                           const StageLds& st, const int32_t* perm, int k,
                                           const FfnItem& it, int rb0, int nrb, int out_ld,
                                           float* out, float* red, int& staged) {
  const char* wb = slot + (MODE == 2 ? o.hi : o.lo);
  const uint16_t* ws = reinterpret_cast<const uint16_t*>(slot + (MODE == 2 ? o.hi_s : o.lo_s));
  const char* rb = slot + o.hi;
  const uint16_t* rs = reinterpret_cast<const uint16_t*>(slot + o.hi_s);
  const int nkc = MODE == 2 ? K / 32 : K / 64;
  // with the residual, two chunks per step: half the steps in flight keeps the bytes in flight
  constexpr int UQ = (MODE == 1 && U > 1) ? U / 2 : U;
#define TGEMV_Q(NT_, P_)                                                                       \
  do {                                                                                         \
    if constexpr (QIN) {                                                                       \
      const int key_ = NT_ == 1 ? (SWIGLU ? perm[P_] / k : (P_)) : -1;                         \
      if (key_ < 0 || key_ != staged)                                                          \
        stage_rows<SWIGLU, NT_>(raw, perm, k, P_, K, st.q, st.s, st.wmax);                     \
      staged = key_;                                                                           \
    }                                                                                          \
    const int8_t* aq_ = QIN ? st.q : aq;                                                       \
    const float* as_ = QIN ? st.s : as;                                                        \
    if constexpr (MODE == 2)                                                                   \
      tile_int8<KS, RBW, U, NT_, QIN>(wb, ws, nkc, K, aq_, as_, P_, rb0, nrb, out_ld, out,     \
                                      red);                                                    \
    else                                                                                       \
      tile_int4<KS, RBW, UQ, NT_, SWIGLU, MODE == 1, QIN>(wb, ws, rb, rs, nkc, K, aq_, as_,    \
                                                          perm, k, P_, rb0, nrb, out_ld, out,  \
                                                          red);                                \
  } while (0)
  int done = 0;
  for (; it.rows - done >= MAXNT; done += MAXNT) TGEMV_Q(MAXNT, it.row_begin + done);
  const int rest = it.rows - done, p = it.row_begin + done;
#define TGEMV_QR(NT_) TGEMV_Q(NT_, p)
  TGEMV_REST(TGEMV_QR)
#undef TGEMV_QR
#undef TGEMV_Q
}

// The quantised GEMV pass. SPLIT = false: every item on the int4 weights.
// SPLIT = true (split-precision experts): an item runs at high precision when
// it is a shared group (expert >= E), when mask is NULL, or when mask[expert]
// >= 2, else on the int4 weights; the choice is uniform over a workgroup.
// QIN: the workgroup quantises each tile's activation rows itself, from raw
// (bf16 tokens in the gate/up pass, fp32 h in the down pass), into
// MAXNT * K bytes of dynamic LDS; aq and as are then unused.
template <int KS, int RBW, int NW, int U, int MAXNT, bool SWIGLU, bool SPLIT, bool QIN>
__global__ __launch_bounds__(NW * 64) void int4_kernel(
    const int8_t* __restrict__ aq, const float* __restrict__ as, const void* __restrict__ raw,
    const int32_t* __restrict__ perm, int k, const FfnItem* __restrict__ items,
    const int32_t* __restrict__ n_items, const char* __restrict__ pool, size_t stride,
    QuantOffsets offs, const int32_t* __restrict__ mask, int E, int R, int K, int out_ld,
    int units_per_item, float* __restrict__ out) {
  __shared__ float red[NW * RBW * 32 * MAXNT];
  __shared__ float st_s[MAXNT];
  __shared__ float st_wmax[16];
  extern __shared__ __attribute__((aligned(16))) int8_t st_q[];
  const StageLds st{st_q, st_s, st_wmax};
  const int wave = threadIdx.x >> 6;
  const int nrb = R / 32;
  // One-row tiles (the launch holds only the resident workgroups): a contiguous range of
  // units per workgroup, so consecutive units mostly share an item and its staged row.
  // Otherwise one unit per workgroup in turn (grid-stride), the workgroups with work
  // first when fewer items are present than the grid was sized for.
  const int units = n_items[0] * units_per_item;
  const int ub = MAXNT == 1 ? (int)((long long)units * blockIdx.x / gridDim.x) : (int)blockIdx.x;
  const int ue = MAXNT == 1 ? (int)((long long)units * (blockIdx.x + 1) / gridDim.x) : units;
  const int us = MAXNT == 1 ? 1 : (int)gridDim.x;
  int staged = -1;
  for (int u = ub; u < ue; u += us) {
    const int item = u / units_per_item;
    const int rb0 = ((u - item * units_per_item) * (NW / KS) + wave / KS) * RBW;
    const FfnItem it = items[item];
    const char* slot = pool + (size_t)it.slot * stride;
    bool hi = false;
    if constexpr (SPLIT) hi = it.expert >= E || mask == nullptr || mask[it.expert] >= 2;
    if (hi)
      quant_item<SWIGLU ? 1 : 2, KS, RBW, U, MAXNT, SWIGLU, QIN>(
          slot, offs, K, aq, as, raw, st, perm, k, it, rb0, nrb, out_ld, out, red, staged);
    else
      quant_item<0, KS, RBW, U, MAXNT, SWIGLU, QIN>(slot, offs, K, aq, as, raw, st, perm, k, it,
                                                    rb0, nrb, out_ld, out, red, staged);
  }
}
#undef TGEMV_REST

// Launch split for a pass with row_blocks_total 32-row blocks (over all
// groups) of nchunks chunks each, measured on gfx950 for decode shapes:
// - RBW (row blocks per wave) reuses each activation load for RBW rows. For
//   bf16 it pays once tiles hold >= 2 activation rows; int4, whose int8
//   activations take twice the bytes of the codes they meet, uses 2 or 4.
// - KS (waves splitting one row block's K range) is raised until the pass has
//   ~8192 waves (bf16) while every wave keeps >= 8 chunks; the int4 split
//   follows the measured optimum for its two K extents.
struct Split {
  int rbw, ks;
};
inline Split choose_split_bf16(int row_blocks_total, int nchunks, int maxnt) {
  Split sp{1, 1};
  if (maxnt >= 2 && row_blocks_total >= 1024) sp.rbw = 2;
  const int ks_max = sp.rbw == 1 ? 16 : 8;
  const long long blocks = row_blocks_total / sp.rbw;
  while (sp.ks < ks_max && blocks * sp.ks < 8192 && nchunks / (sp.ks * 2) >= 8) sp.ks *= 2;
  return sp;
}
inline Split choose_split_int4(int row_blocks_total, int nchunks) {
  // long rows (the gate/up pass of wide experts): two row blocks per wave, 8 or 16 waves
  // per row block; a few hundred workgroups of 8 waves leave a second, mostly idle round
  // on part of the 256 CUs, so small passes take 16 waves (measured at 9 and 33 groups of
  // 4096 x 7168)
  if (nchunks >= 64) return Split{2, (row_blocks_total + 1) / 2 < 1024 ? 16 : 8};
  Split sp{4, 1};
  const long long blocks = (row_blocks_total + 3) / 4;
  if (blocks < 1024)
    while (sp.ks < 4 && nchunks / (sp.ks * 2) >= 8) sp.ks *= 2;
  return sp;
}

constexpr int kGridCap = 8192;

template <int KS>
inline unsigned grid_for(int units) {
  return (unsigned)(units < kGridCap ? units : kGridCap);
}

}  // namespace tgemv
