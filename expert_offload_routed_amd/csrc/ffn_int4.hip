// int4 group-128 expert weights with int8 per-row activations
// (moe_expert_ffn with MOE_INT4G128).
//
// The expert is the SwiGLU FFN of "RapidMoE: Exploiting Cross-Asymmetry via
// Adaptive Residual Offloading for Large-Scale MoE Inference", Eq. (7), read
// through the slot table of the SeqMoE summary page (Mechanism). Numerics:
//   W_hat[n][c] = q[n][c] * s[n][c / 128]      (q: signed 4-bit, s: bf16)
//   x_hat = rint(x / s_x) * s_x, s_x = max|x_row| / 127 (IEEE fp32 division)
//   y[n] = s_x * sum_g s[n][g] * sum_{c in g} q[n][c] * qx[c]
// The inner sums are exact int32 (int8 x int4 products); the group scales and
// the row scale are applied in fp32. The SwiGLU intermediate is formed in
// fp32 and quantised per row the same way before the down projection.
//
// Codes are used in offset form u = q + 8 (0..15: bytes that are valid
// non-negative int8 for sdot4 and the int8 MFMA); sum q x = sum u x - 8 sum x,
// where sum x over a 128-value group is precomputed per activation row.
// Slot word order (moe_slot_layout): a 32-bit word holds 8 consecutive codes,
// low nibbles = codes 0..3, high nibbles = codes 4..7, so
//   u_lo = (w ^ 0x88888888) & 0x0F0F0F0F, u_hi = ((w ^ 0x88888888) >> 4) & 0x0F0F0F0F
// are two words of 4 consecutive int8 values in natural order.
#include "common.h"
#include "ffn_internal.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int intx4;
typedef __attribute__((__vector_size__(16 * sizeof(int)))) int intx16;

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

__device__ __forceinline__ uint32_t u_lo(uint32_t w) { return (w ^ 0x88888888u) & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t u_hi(uint32_t w) { return ((w ^ 0x88888888u) >> 4) & 0x0F0F0F0Fu; }

// ------------------------------------------------------ row quantisation ---
// One workgroup per row of K values (K % 128 == 0): s = max|v| / 127,
// q = clip(rint(v / s), -127, 127), gsum[g] = sum of q over group g.
// With offsets != NULL, row p is skipped unless it belongs to a selected,
// resident group (the rows this call computes).
template <int IN>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const void* __restrict__ in, int K, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ lut, const int32_t* __restrict__ mask, int E, int num_slots,
    int8_t* __restrict__ q, float* __restrict__ s, int32_t* __restrict__ gsum) {
  __shared__ float s_max[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (offsets) {
    int lo = 0, hi = E;  // largest e with offsets[e] <= row
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= row) lo = mid; else hi = mid;
    }
    const int e = lo;
    if (row >= offsets[E]) return;
    if (mask && mask[e] == 0) return;
    const int slot = lut[e];
    if (slot < 0 || slot >= num_slots) return;
  }
  float v[4][8];
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e0 = c * 2048 + tid * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[c][i] = 0.f;
    if (e0 < K) {
      if constexpr (IN == MOE_BF16) {
        const u32x4 r = ld16(static_cast<const uint16_t*>(in) + (size_t)row * K + e0);
        v[c][0] = bf16_lo(r.x); v[c][1] = bf16_hi(r.x); v[c][2] = bf16_lo(r.y); v[c][3] = bf16_hi(r.y);
        v[c][4] = bf16_lo(r.z); v[c][5] = bf16_hi(r.z); v[c][6] = bf16_lo(r.w); v[c][7] = bf16_hi(r.w);
      } else {
        const float* p = static_cast<const float*>(in) + (size_t)row * K + e0;
        const u32x4 a = ld16(p), b = ld16(p + 4);
        v[c][0] = __uint_as_float(a.x); v[c][1] = __uint_as_float(a.y);
        v[c][2] = __uint_as_float(a.z); v[c][3] = __uint_as_float(a.w);
        v[c][4] = __uint_as_float(b.x); v[c][5] = __uint_as_float(b.y);
        v[c][6] = __uint_as_float(b.z); v[c][7] = __uint_as_float(b.w);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
    }
  }
  amax = wave_max(amax);
  if (lane == 0) s_max[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float sc = (amax == 0.f) ? 1.f : amax / 127.f;
  if (tid == 0) s[row] = sc;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e0 = c * 2048 + tid * 8;
    int part = 0;
    if (e0 < K) {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float r = rintf(v[c][i] / sc);
        r = fminf(fmaxf(r, -127.f), 127.f);
        const int qi = (int)r;
        part += qi;
        const uint32_t b = (uint32_t)(qi & 0xFF);
        if (i < 4) w0 |= b << (8 * i); else w1 |= b << (8 * (i - 4));
      }
      *reinterpret_cast<uint2*>(q + (size_t)row * K + e0) = make_uint2(w0, w1);
    }
    // 16 consecutive threads hold one 128-value group
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
    if (e0 < K && (tid & 15) == 0) gsum[(size_t)row * (K / 128) + e0 / 128] = part;
  }
}

// ------------------------------------------------------------- int4 GEMV ---
// Same decomposition as the dense decode GEMV: a workgroup owns RPW * (4/KS)
// rows; KS waves split K in 2048-value chunks (16 code bytes per lane).
template <int RPW, int KS, int NT, bool SWIGLU>
__device__ __forceinline__ void gemv_tile(const char* __restrict__ codes, size_t rowb,
                                          const uint16_t* __restrict__ scales, int sld, int K,
                                          const int8_t* __restrict__ aq,
                                          const float* __restrict__ as,
                                          const int32_t* __restrict__ ag,
                                          const int32_t* __restrict__ perm, int k, int prow,
                                          int r0, bool store, int out_ld, float* __restrict__ out,
                                          float* __restrict__ red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slice = wave % KS;
  int arow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) arow[t] = SWIGLU ? perm[prow + t] / k : prow + t;
  float acc[RPW][NT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;
  const int gld = K / 128;
  const int nchunks = (K + 2047) / 2048;
  for (int c = slice; c < nchunks; c += KS) {
    const int e = c * 2048 + lane * 32;
    if (e < K) {
      const int g = e >> 7;
      u32x4 cw[RPW];
      float sw[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        cw[r] = ld16_stream(codes + r * rowb + (e >> 1));
        sw[r] = bf16_to_f32(scales[(size_t)r * sld + g]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int8_t* ap = aq + (size_t)arow[t] * K + e;
        const u32x4 xa = ld16(ap), xb = ld16(ap + 16);
        const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
        const int gs = ((lane & 3) == 0) ? ag[(size_t)arow[t] * gld + g] : 0;
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const uint32_t w[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
          int is = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            is = __builtin_amdgcn_sdot4((int)u_lo(w[i]), (int)xw[2 * i], is, false);
            is = __builtin_amdgcn_sdot4((int)u_hi(w[i]), (int)xw[2 * i + 1], is, false);
          }
          acc[r][t] = fmaf((float)(is - 8 * gs), sw[r], acc[r][t]);
        }
      }
    }
  }
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
      for (int s2 = 1; s2 < KS; ++s2)
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[r][t] += red[((wave + s2) * RPW + r) * NT + t];
    }
    __syncthreads();
  }
  if (store && slice == 0 && lane < NT) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (lane == t) {
        const float sx = as[arow[t]];
        float* o = out + (size_t)(prow + t) * out_ld;
        if constexpr (SWIGLU) {
#pragma unroll
          for (int r = 0; r < RPW; r += 2) o[(r0 + r) / 2] = silu(acc[r][t] * sx) * (acc[r + 1][t] * sx);
        } else {
#pragma unroll
          for (int r = 0; r < RPW; ++r) o[r0 + r] = acc[r][t] * sx;
        }
      }
    }
  }
}

template <int RPW, int KS, int MAXNT, bool SWIGLU>
__global__ __launch_bounds__(256) void gemv_w4a8_kernel(
    const int8_t* __restrict__ aq, const float* __restrict__ as, const int32_t* __restrict__ ag,
    const int32_t* __restrict__ perm, int k, const FfnItem* __restrict__ items,
    const int32_t* __restrict__ n_items, const char* __restrict__ pool, size_t stride,
    size_t off_codes, size_t off_scales, int rows, int K, int out_ld, int row_blocks,
    float* __restrict__ out) {
  __shared__ float red[4 * RPW * MAXNT];
  constexpr int kBlocksPerWg = 4 / KS;
  const size_t rowb = (size_t)K / 2;
  const int sld = K / 128;
  const int wave = threadIdx.x >> 6;
  const int units = n_items[0] * row_blocks;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int item = u / row_blocks;
    const int rb = u - item * row_blocks;
    const FfnItem it = items[item];
    int r0 = (rb * kBlocksPerWg + wave / KS) * RPW;
    const bool store = r0 < rows;
    if (!store) r0 = 0;
    const char* slot = pool + (size_t)it.slot * stride;
    const char* codes = slot + off_codes + (size_t)r0 * rowb;
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(slot + off_scales) + (size_t)r0 * sld;
    int done = 0;
    for (; it.rows - done >= MAXNT; done += MAXNT)
      gemv_tile<RPW, KS, MAXNT, SWIGLU>(codes, rowb, scales, sld, K, aq, as, ag, perm, k,
                                        it.row_begin + done, r0, store, out_ld, out, red);
    const int rest = it.rows - done, p = it.row_begin + done;
#define MOE_W4_TILE(NT_)                                                                       \
  gemv_tile<RPW, KS, NT_, SWIGLU>(codes, rowb, scales, sld, K, aq, as, ag, perm, k, p, r0, store, \
                                  out_ld, out, red)
    if constexpr (MAXNT > 1) {
      if (rest == 1) MOE_W4_TILE(1);
    }
    if constexpr (MAXNT > 2) {
      if (rest == 2) MOE_W4_TILE(2);
      if (rest == 3) MOE_W4_TILE(3);
    }
#undef MOE_W4_TILE
  }
}

// -------------------------------------------------------- int8 MFMA GEMM ---
constexpr int QBM = kGemmBM;  // 64 activation rows
constexpr int QBN = 128;      // weight rows
constexpr int QBK = 128;      // one scale group
constexpr int A_LD = QBK + 16;      // bytes per staged activation row
constexpr int B_LD = QBK / 2 + 16;  // bytes per staged code row

template <int PASS>
__global__ __launch_bounds__(256) void gemm_w4a8_kernel(
    const int8_t* __restrict__ aq, const float* __restrict__ as, const int32_t* __restrict__ ag,
    const int32_t* __restrict__ perm, int k, const GemmTile* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, const char* __restrict__ pool, size_t stride,
    size_t off_codes, size_t off_scales, int N, int K, int out_ld, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) int8_t sA[2][QBM * A_LD];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][QBN * B_LD];
  __shared__ float sS[2][QBN];
  __shared__ int sG[2][QBM];
  if ((int)blockIdx.y >= n_tiles[0]) return;
  const GemmTile tl = tiles[blockIdx.y];
  const int n0 = blockIdx.x * QBN;
  if (n0 >= N) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gld = K / 128;

  // activation rows staged by this thread: (tid >> 3) + 32 i, 16 bytes at (tid & 7) * 16
  const int8_t* arow[2];
  bool avalid[2];
  int arowid[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = (tid >> 3) + 32 * i;
    avalid[i] = m < tl.rows;
    const int p = tl.row_begin + (avalid[i] ? m : 0);
    arowid[i] = (PASS == 1) ? perm[p] / k : p;
    arow[i] = aq + (size_t)arowid[i] * K;
  }
  // gsum row for the epilogue of a K tile: threads 0..63 own row tid
  int grow = 0;
  bool gvalid = false;
  if (tid < QBM) {
    gvalid = tid < tl.rows;
    const int p = tl.row_begin + (gvalid ? tid : 0);
    grow = (PASS == 1) ? perm[p] / k : p;
  }
  // code rows: (tid >> 2) + 64 i, 16 bytes at (tid & 3) * 16
  const char* slot = pool + (size_t)tl.slot * stride;
  const char* brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int n = n0 + (tid >> 2) + 64 * i;
    if (n >= N) n = N - 1;
    brow[i] = slot + off_codes + (size_t)n * (K / 2);
  }
  const uint16_t* scl = reinterpret_cast<const uint16_t*>(slot + off_scales);
  int sn = n0 + (tid & 127);
  if (sn >= N) sn = N - 1;

  u32x4 ra[2], rb[2];
  float rs = 0.f;
  int rg = 0;
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      ra[i] = avalid[i] ? ld16(arow[i] + kt * QBK + (tid & 7) * 16) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 2; ++i) rb[i] = ld16_stream(brow[i] + kt * (QBK / 2) + (tid & 3) * 16);
    if (tid < QBN) rs = bf16_to_f32(scl[(size_t)sn * gld + kt]);
    if (tid < QBM) rg = gvalid ? ag[(size_t)grow * gld + kt] : 0;
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(&sA[buf][((tid >> 3) + 32 * i) * A_LD + (tid & 7) * 16]) = ra[i];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(&sB[buf][((tid >> 2) + 64 * i) * B_LD + (tid & 3) * 16]) = rb[i];
    if (tid < QBN) sS[buf][tid] = rs;
    if (tid < QBM) sG[buf][tid] = rg;
  };

  float accf[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) accf[j][r] = 0.f;

  const int nk = K / QBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    intx16 acci[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acci[j][r] = 0;
#pragma unroll
    for (int ks = 0; ks < QBK / 32; ++ks) {
      const intx4 a = *reinterpret_cast<const intx4*>(
          &sA[buf][(wm * 32 + (lane & 31)) * A_LD + ks * 32 + 16 * (lane >> 5)]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint2 w = *reinterpret_cast<const uint2*>(
            &sB[buf][(wn * 64 + j * 32 + (lane & 31)) * B_LD + ks * 16 + 8 * (lane >> 5)]);
        intx4 b;
        b[0] = (int)u_lo(w.x);
        b[1] = (int)u_hi(w.x);
        b[2] = (int)u_lo(w.y);
        b[3] = (int)u_hi(w.y);
        acci[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acci[j], 0, 0, 0);
      }
    }
    // fold this scale group into fp32: (sum u x - 8 sum x) * s_w
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float sw = sS[buf][wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        accf[j][r] = fmaf((float)(acci[j][r] - 8 * sG[buf][m]), sw, accf[j][r]);
      }
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const bool ok = m < tl.rows;
      const int p = tl.row_begin + (ok ? m : 0);
      const float sx = as[(PASS == 1) ? perm[p] / k : p];
      const float v = accf[j][r] * sx;
      if constexpr (PASS == 1) {
        const float u = __shfl_xor(v, 1, 64);  // odd column = up of the same neuron
        if ((n & 1) == 0 && ok && n < N) out[(size_t)p * out_ld + (n >> 1)] = silu(v) * u;
      } else {
        if (ok && n < N) out[(size_t)p * out_ld + n] = v;
      }
    }
  }
}

template <int RPW, int KS, int MAXNT, bool SWIGLU>
void launch_gemv(const int8_t* aq, const float* as, const int32_t* ag, const int32_t* perm, int k,
                 const FfnItem* items, const int32_t* n_items, int max_items, const char* pool,
                 size_t stride, size_t off_codes, size_t off_scales, int rows, int K, int out_ld,
                 float* out, hipStream_t s) {
  const int per_wg = RPW * (4 / KS);
  const long long rb = (rows + per_wg - 1) / per_wg;
  const long long units = rb * max_items;
  const unsigned grid = (unsigned)(units < 8192 ? units : 8192);
  if (grid == 0) return;
  hipLaunchKernelGGL((gemv_w4a8_kernel<RPW, KS, MAXNT, SWIGLU>), dim3(grid), dim3(256), 0, s, aq,
                     as, ag, perm, k, items, n_items, pool, stride, off_codes, off_scales, rows, K,
                     out_ld, (int)rb, out);
}

template <int MAXNT>
void launch_gemv_pair(bool first, const int8_t* aq, const float* as, const int32_t* ag,
                      const int32_t* perm, int k, const FfnItem* items, const int32_t* n_items,
                      int max_items, const char* pool, size_t stride, const SlotLayout& lay, int H,
                      int F, float* out, hipStream_t s) {
  if (first) {
    // K = H: split K over 2 waves when a row spans several 2048-value chunks
    if (H > 2048)
      launch_gemv<4, 2, MAXNT, true>(aq, as, ag, perm, k, items, n_items, max_items, pool, stride,
                                     lay.off_w13, lay.off_s13, 2 * F, H, F, out, s);
    else
      launch_gemv<4, 1, MAXNT, true>(aq, as, ag, perm, k, items, n_items, max_items, pool, stride,
                                     lay.off_w13, lay.off_s13, 2 * F, H, F, out, s);
  } else {
    if (F > 2048)
      launch_gemv<4, 2, MAXNT, false>(aq, as, ag, perm, k, items, n_items, max_items, pool, stride,
                                      lay.off_w2, lay.off_s2, H, F, H, out, s);
    else
      launch_gemv<4, 1, MAXNT, false>(aq, as, ag, perm, k, items, n_items, max_items, pool, stride,
                                      lay.off_w2, lay.off_s2, H, F, H, out, s);
  }
}

void launch_gemv_any(bool first, int nt, const int8_t* aq, const float* as, const int32_t* ag,
                     const int32_t* perm, int k, const FfnItem* items, const int32_t* n_items,
                     int max_items, const char* pool, size_t stride, const SlotLayout& lay, int H,
                     int F, float* out, hipStream_t s) {
  if (nt <= 1)
    launch_gemv_pair<1>(first, aq, as, ag, perm, k, items, n_items, max_items, pool, stride, lay, H,
                        F, out, s);
  else if (nt <= 2)
    launch_gemv_pair<2>(first, aq, as, ag, perm, k, items, n_items, max_items, pool, stride, lay, H,
                        F, out, s);
  else
    launch_gemv_pair<4>(first, aq, as, ag, perm, k, items, n_items, max_items, pool, stride, lay, H,
                        F, out, s);
}

}  // namespace

int ffn_int4(const void* x, const int32_t* perm, const int32_t* offsets, const int32_t* lut,
             const int32_t* group_mask, const char* pool, size_t stride, int num_slots,
             const SlotLayout& lay, int T, int H, int F, int E, int k, float* y, int32_t* err,
             char* ws, const FfnWorkspace& wl, hipStream_t s) {
  int32_t* n_items = reinterpret_cast<int32_t*>(ws);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(ws + 4);
  FfnItem* items = reinterpret_cast<FfnItem*>(ws + wl.items);
  GemmTile* tiles = reinterpret_cast<GemmTile*>(ws + wl.tiles);
  float* hbuf = reinterpret_cast<float*>(ws + wl.h);
  int8_t* xq = reinterpret_cast<int8_t*>(ws + wl.xq);
  float* xs = reinterpret_cast<float*>(ws + wl.xs);
  int32_t* xg = reinterpret_cast<int32_t*>(ws + wl.xg);
  int8_t* hq = reinterpret_cast<int8_t*>(ws + wl.hq);
  float* hs = reinterpret_cast<float*>(ws + wl.hs);
  int32_t* hg = reinterpret_cast<int32_t*>(ws + wl.hg);
  if (H > 4 * 2048 || F > 4 * 2048) return MOE_EUNSUPPORTED;  // quant_rows covers 8192 values
  const long long tk = (long long)T * k;
  const int max_items = (int)(tk < E ? tk : E);
  const int max_tiles = (T > kGemvMaxRows) ? wl.max_tiles : 0;
  if (max_tiles > 65535) return MOE_EUNSUPPORTED;
  launch_ffn_plan(offsets, lut, group_mask, E, num_slots, kGemvMaxRows, items, n_items, tiles,
                  n_tiles, err, s);
  hipLaunchKernelGGL(quant_rows_kernel<MOE_BF16>, dim3(T), dim3(256), 0, s, x, H, nullptr, nullptr,
                     nullptr, 0, 0, xq, xs, xg);
  const int nt = T < kGemvMaxRows ? T : kGemvMaxRows;
  launch_gemv_any(true, nt, xq, xs, xg, perm, k, items, n_items, max_items, pool, stride, lay, H, F,
                  hbuf, s);
  if (max_tiles > 0)
    hipLaunchKernelGGL(gemm_w4a8_kernel<1>, dim3((2 * F + QBN - 1) / QBN, max_tiles), dim3(256), 0,
                       s, xq, xs, xg, perm, k, tiles, n_tiles, pool, stride, lay.off_w13,
                       lay.off_s13, 2 * F, H, F, hbuf);
  hipLaunchKernelGGL(quant_rows_kernel<MOE_F32>, dim3((unsigned)tk), dim3(256), 0, s, hbuf, F,
                     offsets, lut, group_mask, E, num_slots, hq, hs, hg);
  launch_gemv_any(false, nt, hq, hs, hg, perm, k, items, n_items, max_items, pool, stride, lay, H,
                  F, y, s);
  if (max_tiles > 0)
    hipLaunchKernelGGL(gemm_w4a8_kernel<2>, dim3((H + QBN - 1) / QBN, max_tiles), dim3(256), 0, s,
                       hq, hs, hg, perm, k, tiles, n_tiles, pool, stride, lay.off_w2, lay.off_s2, H,
                       F, H, y);
  return moe_launch_status();
}
