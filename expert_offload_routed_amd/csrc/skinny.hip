// Expert FFN passes on MFMA for groups of 2 to 32 rows (bf16), the decode-batch
// form of the SwiGLU expert of "RapidMoE: Exploiting Cross-Asymmetry via
// Adaptive Residual Offloading for Large-Scale MoE Inference", Eq. (7), read
// through the slot table of the SeqMoE summary page (Mechanism).
//
// A group's rows (at most 32) fill the 32 rows of one v_mfma_f32_32x32x16_bf16
// operand; the weights stream once, straight from their tile-major 1 KB chunks,
// which are that instruction's B operand as stored (lane l: weight row l % 32,
// K values 8 (l / 32) .. +7 of the 16-value chunk). Per chunk a lane loads the
// matching 16 bytes of its token row (row l % 32 of the group; rows past the
// group read its first row and their results are dropped) as the A operand, so
// the compute is one MFMA per 1 KB of weights and the pass is bound by the
// weight stream. A 128-row GEMM tile for such a group held at most a few
// hundred live workgroups over the whole pass; here every (group, row block)
// is a unit of its own.
//
// A workgroup has 4 waves: KS waves split the K chunks of one row block (chunk
// c to slice c % KS), the 4 / KS wave groups take consecutive row blocks; U
// chunks per lane in flight. The slices meet in LDS in a fixed order.
// Accumulator r of a lane holds token row 8 (r / 4) + 4 (l / 32) + r % 4 and
// weight row l % 32 of the block.
//
// The int4 form (group-128 codes with int8 rows, the same arithmetic as the
// int8 GEMM tiles of ffn_int4.hip): per scale group of 128 K values, four
// v_mfma_i32_32x32x32_i8 of the group's int8 rows (quantised beforehand, 16
// bytes per lane and K step) against the codes expanded to 16 q (two masks and
// a shift), the exact int32 sum folded into fp32 with scale / 16, the row scale
// applied at the end. Each wave takes two row blocks, so every activation
// fragment serves two MFMAs.
#include "common.h"
#include "ffn_internal.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int intx4;
typedef __attribute__((__vector_size__(16 * sizeof(int)))) int intx16;

constexpr int kSkinnyWaves = 4;

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

__device__ __forceinline__ bf16x8 ld_frag(const void* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 ld_frag_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
}

template <int KS, int U, bool SWIGLU>
__global__ __launch_bounds__(64 * kSkinnyWaves) void skinny_bf16_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ perm, int k,
    const FfnItem* __restrict__ items, const int32_t* __restrict__ n_items,
    const char* __restrict__ pool, size_t stride, size_t off, int R, int K, int out_ld,
    int units_per_item, void* __restrict__ out) {
  constexpr int GROUPS = kSkinnyWaves / KS;  // row blocks of a unit
  __shared__ floatx16 red[kSkinnyWaves][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slice = wave % KS, grp = wave / KS;
  const int nrb = R / 32, nkc = K / 16;
  const int units = n_items[0] * units_per_item;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int item = u / units_per_item;
    const int rb = (u - item * units_per_item) * GROUPS + grp;
    const bool rvalid = rb < nrb;
    const FfnItem it = items[item];
    const int t = lane & 31;
    const int p = it.row_begin + (t < it.rows ? t : 0);
    const size_t arow = SWIGLU ? (size_t)(perm[p] / k) : (size_t)p;
    const uint16_t* ap = act + arow * K + 8 * (lane >> 5);
    const char* wp = pool + (size_t)it.slot * stride + off +
                     (size_t)(rvalid ? rb : nrb - 1) * nkc * 1024 + lane * 16;
    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    for (int kc0 = slice; kc0 < nkc; kc0 += KS * U) {
      bf16x8 a[U], w[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int kc = kc0 + j * KS;
        if (kc < nkc) {
          w[j] = ld_frag_stream(wp + (size_t)kc * 1024);
          a[j] = ld_frag(ap + (size_t)kc * 16);
        }
      }
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (kc0 + j * KS < nkc) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], w[j], acc, 0, 0, 0);
    }
    if constexpr (KS > 1) {
      red[wave][lane] = acc;
      __syncthreads();
      if (slice == 0) {
#pragma unroll
        for (int s = 1; s < KS; ++s) {
          const floatx16 o = red[wave + s][lane];
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] += o[r];
        }
      }
      __syncthreads();  // red is rewritten by the next unit
    }
    if (slice != 0 || !rvalid) continue;
    const int n = rb * 32 + (lane & 31);
    auto row_of = [&](int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); };
    if constexpr (SWIGLU) {
      // lanes 2i and 2i+1 hold the gate and up rows of neuron n/2; after one exchange per
      // pair of elements the even lane forms elements r < 8, the odd lane elements r + 8
      const bool odd = lane & 1;
      uint16_t* h = static_cast<uint16_t*>(out);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float lo = acc[r], hi = acc[r + 8];
        const float got = __shfl_xor(odd ? lo : hi, 1, 64);
        const float g = odd ? got : lo, up = odd ? hi : got;
        const int m = row_of(odd ? r + 8 : r);
        if (m < it.rows) h[(size_t)(it.row_begin + m) * out_ld + (n >> 1)] = f32_to_bf16_rne(silu(g) * up);
      }
    } else {
      float* y = static_cast<float*>(out);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = row_of(r);
        if (m < it.rows) y[(size_t)(it.row_begin + m) * out_ld + n] = acc[r];
      }
    }
  }
}

// int4 codes with int8 rows; KS waves split the scale groups of two row blocks.
template <int KS, int U, bool SWIGLU>
__global__ __launch_bounds__(64 * kSkinnyWaves) void skinny_w4a8_kernel(
    const int8_t* __restrict__ aq, const float* __restrict__ as, const int32_t* __restrict__ perm,
    int k, const FfnItem* __restrict__ items, const int32_t* __restrict__ n_items,
    const char* __restrict__ pool, size_t stride, size_t off_codes, size_t off_scales, int R, int K,
    int out_ld, int units_per_item, float* __restrict__ out) {
  constexpr int GROUPS = kSkinnyWaves / KS;  // pairs of row blocks of a unit
  __shared__ floatx16 red[kSkinnyWaves][2][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slice = wave % KS, grp = wave / KS;
  const int nrb = R / 32, ng = K / 128, nkc = K / 64;
  const int units = n_items[0] * units_per_item;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int item = u / units_per_item;
    const int rb0 = ((u - item * units_per_item) * GROUPS + grp) * 2;
    const FfnItem it = items[item];
    const int t = lane & 31;
    const int p = it.row_begin + (t < it.rows ? t : 0);
    const size_t arow = SWIGLU ? (size_t)(perm[p] / k) : (size_t)p;
    const float my_sx = as[arow];  // row scale of this lane's token row
    const int8_t* ap = aq + arow * K + 16 * (lane >> 5);
    const char* slot = pool + (size_t)it.slot * stride;
    const char* wp[2];
    const uint16_t* sp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int rb = rb0 + b < nrb ? rb0 + b : nrb - 1;
      wp[b] = slot + off_codes + (size_t)rb * nkc * 1024 + lane * 16;
      sp[b] = reinterpret_cast<const uint16_t*>(slot + off_scales) + (size_t)(rb * 32 + t) * ng;
    }
    floatx16 accf[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) accf[b][r] = 0.f;
    for (int g0 = slice; g0 < ng; g0 += KS * U) {
      u32x4 cw[U][2][2];  // [group][row block][chunk]
      intx4 a[U][4];      // [group][k step of 32]
      uint16_t sc[U][2];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int g = g0 + j * KS;
        if (g < ng) {
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            cw[j][b][0] = ld16_stream(wp[b] + (size_t)(2 * g) * 1024);
            cw[j][b][1] = ld16_stream(wp[b] + (size_t)(2 * g + 1) * 1024);
            sc[j][b] = sp[b][g];
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) a[j][q] = *reinterpret_cast<const intx4*>(ap + (size_t)g * 128 + q * 32);
        }
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (g0 + j * KS < ng) {
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            intx16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              // k step q: chunk q / 2, its K half (q % 2) of the lane's 32 codes
              const u32x4& c = cw[j][b][q >> 1];
              const uint32_t w0 = (q & 1) ? c.z : c.x, w1 = (q & 1) ? c.w : c.y;
              intx4 bq;
              bq[0] = (int)((w0 << 4) & 0xF0F0F0F0u);
              bq[1] = (int)(w0 & 0xF0F0F0F0u);
              bq[2] = (int)((w1 << 4) & 0xF0F0F0F0u);
              bq[3] = (int)(w1 & 0xF0F0F0F0u);
              acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j][q], bq, acc, 0, 0, 0);
            }
            const float sw = bf16_to_f32(sc[j][b]) * 0.0625f;  // codes entered as 16 q
#pragma unroll
            for (int r = 0; r < 16; ++r) accf[b][r] = fmaf((float)acc[r], sw, accf[b][r]);
          }
        }
      }
    }
    if constexpr (KS > 1) {
      red[wave][0][lane] = accf[0];
      red[wave][1][lane] = accf[1];
      __syncthreads();
      if (slice == 0) {
#pragma unroll
        for (int s = 1; s < KS; ++s)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const floatx16 o = red[wave + s][b][lane];
#pragma unroll
            for (int r = 0; r < 16; ++r) accf[b][r] += o[r];
          }
      }
      __syncthreads();  // red is rewritten by the next unit
    }
    if (slice != 0) continue;
    auto row_of = [&](int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); };
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int rb = rb0 + b;
      if (rb >= nrb) continue;
      const int n = rb * 32 + t;
      if constexpr (SWIGLU) {
        // gate (even lane) and up (odd lane) rows of neuron n/2: the even lane forms
        // elements r < 8, the odd lane elements r + 8, after one exchange per pair
        const bool odd = lane & 1;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float lo = accf[b][r] * __shfl(my_sx, row_of(r), 64);
          const float hi = accf[b][r + 8] * __shfl(my_sx, row_of(r + 8), 64);
          const float got = __shfl_xor(odd ? lo : hi, 1, 64);
          const float g = odd ? got : lo, up = odd ? hi : got;
          const int m = row_of(odd ? r + 8 : r);
          if (m < it.rows) out[(size_t)(it.row_begin + m) * out_ld + (n >> 1)] = silu(g) * up;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = row_of(r);
          const float v = accf[b][r] * __shfl(my_sx, m, 64);
          if (m < it.rows) out[(size_t)(it.row_begin + m) * out_ld + n] = v;
        }
      }
    }
  }
}

template <int KS, bool SWIGLU>
void launch_ks(const void* act, const int32_t* perm, int k, const FfnItem* items,
               const int32_t* n_items, int max_items, const char* pool, size_t stride, size_t off,
               int R, int K, int out_ld, void* out, hipStream_t s) {
  constexpr int GROUPS = kSkinnyWaves / KS;
  constexpr int U = 4;
  const int upi = (R / 32 + GROUPS - 1) / GROUPS;
  const long long units = (long long)upi * max_items;
  const unsigned grid = (unsigned)(units < kSkinnyGridCap ? units : kSkinnyGridCap);
  if (grid == 0) return;
  hipLaunchKernelGGL((skinny_bf16_kernel<KS, U, SWIGLU>), dim3(grid), dim3(64 * kSkinnyWaves), 0,
                     s, static_cast<const uint16_t*>(act), perm, k, items, n_items, pool, stride,
                     off, R, K, out_ld, upi, out);
}

}  // namespace

void launch_skinny_bf16(int pass, const void* act, const int32_t* perm, int k,
                        const FfnItem* items, const int32_t* n_items, int max_items,
                        const char* pool, size_t stride, size_t off, int R, int K, int out_ld,
                        void* out, hipStream_t s) {
  // K slices per row block: each wave keeps at least 16 chunks of its row block
  const int nkc = K / 16;
  const int ks = nkc >= 64 ? 4 : nkc >= 32 ? 2 : 1;
#define MOE_SKINNY(KS_)                                                                         \
  do {                                                                                          \
    if (pass == 1)                                                                              \
      launch_ks<KS_, true>(act, perm, k, items, n_items, max_items, pool, stride, off, R, K,    \
                           out_ld, out, s);                                                     \
    else                                                                                        \
      launch_ks<KS_, false>(act, perm, k, items, n_items, max_items, pool, stride, off, R, K,   \
                            out_ld, out, s);                                                    \
  } while (0)
  if (ks == 4) MOE_SKINNY(4);
  else if (ks == 2) MOE_SKINNY(2);
  else MOE_SKINNY(1);
#undef MOE_SKINNY
}

void launch_skinny_w4a8(int pass, const int8_t* aq, const float* as, const int32_t* perm, int k,
                        const FfnItem* items, const int32_t* n_items, int max_items,
                        const char* pool, size_t stride, size_t off_codes, size_t off_scales,
                        int R, int K, int out_ld, float* out, hipStream_t s) {
  // K slices: each wave keeps at least 8 of the row blocks' scale groups
  const int ng = K / 128;
  const int ks = ng >= 32 ? 4 : ng >= 16 ? 2 : 1;
  constexpr int U = 2;
#define MOE_SKINNY_Q(KS_)                                                                         \
  do {                                                                                            \
    constexpr int GROUPS = kSkinnyWaves / KS_;                                                    \
    const int upi = (R / 32 + 2 * GROUPS - 1) / (2 * GROUPS);                                     \
    const long long units = (long long)upi * max_items;                                           \
    const unsigned grid = (unsigned)(units < kSkinnyGridCap ? units : kSkinnyGridCap);            \
    if (grid == 0) return;                                                                        \
    if (pass == 1)                                                                                \
      hipLaunchKernelGGL((skinny_w4a8_kernel<KS_, U, true>), dim3(grid), dim3(64 * kSkinnyWaves), \
                         0, s, aq, as, perm, k, items, n_items, pool, stride, off_codes,          \
                         off_scales, R, K, out_ld, upi, out);                                     \
    else                                                                                          \
      hipLaunchKernelGGL((skinny_w4a8_kernel<KS_, U, false>), dim3(grid),                        \
                         dim3(64 * kSkinnyWaves), 0, s, aq, as, perm, k, items, n_items, pool,    \
                         stride, off_codes, off_scales, R, K, out_ld, upi, out);                  \
  } while (0)
  if (ks == 4) MOE_SKINNY_Q(4);
  else if (ks == 2) MOE_SKINNY_Q(2);
  else MOE_SKINNY_Q(1);
#undef MOE_SKINNY_Q
}
