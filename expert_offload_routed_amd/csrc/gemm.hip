// Grouped bf16 GEMM tiles on MFMA for expert groups with many rows (prefill,
// large-batch decode), the dense-contraction form of the SwiGLU expert of
// "RapidMoE: Exploiting Cross-Asymmetry via Adaptive Residual Offloading for
// Large-Scale MoE Inference", Eq. (7), read through the slot table of the
// SeqMoE summary page (Mechanism).
//
// C[m][n] = sum_k A[m][k] * W[n][k] for one M-tile of a group:
//   pass 1: A = token rows x[perm[p] / k] (bf16), W = W13 of the slot
//           (rows 2n / 2n+1 = gate / up of neuron n), epilogue
//           h[p][n] = SiLU(gate) * up, stored bf16;
//   pass 2: A = h rows (bf16), W = W2 of the slot, epilogue y[p][n] fp32.
// Tiles: BM = 64 rows x BN = 128 weight rows x BK = 64, 4 waves in a 2x2
// layout, each wave 32 x 64 = two v_mfma_f32_32x32x16_bf16 accumulators.
// A and W tiles are staged through LDS (rows padded to 72 elements, 8 lanes
// per coalesced 128-byte row segment); global loads run kAhead K-tiles ahead
// through a ring of register stages, so each weight element is fetched from
// HBM once per M-tile and reused for the tile's 64 rows from LDS.
// Lane layouts (checked on gfx950): A/B operand lane l holds row l % 32,
// k = 8 (l / 32) .. +7; accumulator r holds row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.
#include "common.h"
#include "ffn_internal.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;

constexpr int BM = kGemmBM;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDS_LD = BK + 8;  // padded row (elements)
constexpr int kAhead = 3;       // K-tiles of global loads in flight per thread

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

template <int PASS>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ perm, int k,
    const GemmTile* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    const char* __restrict__ pool, size_t stride, size_t off, int N, int K, int out_ld,
    void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDS_LD];
  if ((int)blockIdx.y >= n_tiles[0]) return;
  const GemmTile tl = tiles[blockIdx.y];
  const int n0 = blockIdx.x * BN;
  if (n0 >= N) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves

  // global -> LDS assignment: 8 threads per 128-byte row chunk of 64 bf16
  const int lrow = tid >> 3, lcol = (tid & 7) * 8;
  // A rows this thread stages: lrow and lrow + 32 (BM = 64)
  const uint16_t* arow[2];
  bool avalid[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = lrow + 32 * i;
    avalid[i] = m < tl.rows;
    const int p = tl.row_begin + (avalid[i] ? m : 0);
    const size_t r = (PASS == 1) ? (size_t)(perm[p] / k) : (size_t)p;
    arow[i] = act + r * K;
  }
  // W rows this thread stages: lrow + 32 i, i < 4
  const char* wbase = pool + (size_t)tl.slot * stride + off;
  const uint16_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int n = n0 + lrow + 32 * i;
    if (n >= N) n = N - 1;
    brow[i] = reinterpret_cast<const uint16_t*>(wbase) + (size_t)n * K;
  }

  // register stages: tile kt + kAhead is loaded while tile kt is computed and
  // tile kt + 1 is written to LDS, so every global load has kAhead - 1 full
  // compute iterations to land
  struct Stage {
    u32x4 a[2], b[4];
  };
  Stage st[kAhead];
  auto gload = [&](Stage& r, int kt) {
    const int kk = kt * BK + lcol;
#pragma unroll
    for (int i = 0; i < 2; ++i) r.a[i] = avalid[i] ? ld16(arow[i] + kk) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) r.b[i] = ld16_stream(brow[i] + kk);
  };
  auto sstore = [&](const Stage& r, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(&sA[buf][(lrow + 32 * i) * LDS_LD + lcol]) = r.a[i];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&sB[buf][(lrow + 32 * i) * LDS_LD + lcol]) = r.b[i];
  };

  floatx16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  const int nk = K / BK;
#pragma unroll
  for (int s = 0; s < kAhead; ++s)
    if (s < nk) gload(st[s], s);
  sstore(st[0], 0);
  __syncthreads();
  // iteration kt: refill stage kt % kAhead with tile kt + kAhead, compute LDS
  // buffer kt % 2, write tile kt + 1 (stage (kt + 1) % kAhead) to the other buffer
  auto step = [&](Stage& mine, Stage& next, int kt) {
    const int buf = kt & 1;
    if (kt + kAhead < nk) gload(mine, kt + kAhead);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kc = ks * 16 + 8 * (lane >> 5);
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sA[buf][(wm * 32 + (lane & 31)) * LDS_LD + kc]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 b =
            *reinterpret_cast<const bf16x8*>(&sB[buf][(wn * 64 + j * 32 + (lane & 31)) * LDS_LD + kc]);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) sstore(next, buf ^ 1);
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += kAhead) {
#pragma unroll
    for (int s = 0; s < kAhead; ++s)
      if (kt + s < nk) step(st[s], st[(s + 1) % kAhead], kt + s);
  }

  // epilogue
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const float v = acc[j][r];
      if constexpr (PASS == 1) {
        const float u = __shfl_xor(v, 1, 64);  // odd column = up of the same neuron
        if ((n & 1) == 0 && m < tl.rows && n < N) {
          uint16_t* h = static_cast<uint16_t*>(out) + (size_t)(tl.row_begin + m) * out_ld;
          h[n >> 1] = f32_to_bf16_rne(silu(v) * u);
        }
      } else {
        if (m < tl.rows && n < N)
          static_cast<float*>(out)[(size_t)(tl.row_begin + m) * out_ld + n] = v;
      }
    }
  }
}

}  // namespace

void launch_gemm_bf16(int pass, const void* act, const int32_t* perm, int k, const GemmTile* tiles,
                      const int32_t* n_tiles, int max_tiles, const char* pool, size_t stride,
                      size_t off, int N, int K, int out_ld, void* out, hipStream_t s) {
  const dim3 grid((N + BN - 1) / BN, max_tiles);
  if (pass == 1)
    hipLaunchKernelGGL(gemm_bf16_kernel<1>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(act), perm, k, tiles, n_tiles, pool, stride, off,
                       N, K, out_ld, out);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<2>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(act), perm, k, tiles, n_tiles, pool, stride, off,
                       N, K, out_ld, out);
}
