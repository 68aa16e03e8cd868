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
// Tiles: BM = 128 activation rows x 128 weight rows, K steps of BK = 64. Each
// of the 4 waves owns one 32-row block of the tile-major weights (one
// v_mfma_f32_32x32x16_bf16 accumulator per 32 activation rows; fragments
// without rows are skipped): its operand fragments are whole 1 KB chunks of
// the slot, read with one contiguous 16-byte load per lane straight into
// registers. The loads stay cacheable so that the M-tiles of one group,
// which run side by side, share the chunks through L2.
// The activation tile, shared by the 4 waves, is staged through LDS (rows
// padded to 72 elements, 8 lanes per 128-byte row segment). Global loads run
// kAhead K-tiles ahead through a ring of register stages.
// Lane layouts (checked on gfx950): A/B operand lane l holds row l % 32,
// k = 8 (l / 32) .. +7; accumulator r holds row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.
#include "common.h"
#include "ffn_internal.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;

constexpr int BM = kGemmBM;
constexpr int MF = BM / 32;  // 32-row activation fragments per tile
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
  if ((int)blockIdx.y >= n_tiles[0]) return;
  const GemmTile tl = tiles[blockIdx.y];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrb = N / 32;
  if ((int)blockIdx.x * 4 >= nrb) return;

  // activation rows this thread stages: (tid >> 3) + 32 i, 16 bytes at (tid & 7) * 8 elements
  const int lrow = tid >> 3, lcol = (tid & 7) * 8;
  const uint16_t* arow[MF];
  bool avalid[MF];
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int m = lrow + 32 * i;
    avalid[i] = m < tl.rows;
    const int p = tl.row_begin + (avalid[i] ? m : 0);
    const size_t r = (PASS == 1) ? (size_t)(perm[p] / k) : (size_t)p;
    arow[i] = act + r * K;
  }
  // this wave's 32-row weight block; a block past N re-reads the last one and stores nothing
  int rb = blockIdx.x * 4 + wave;
  const bool nvalid = rb < nrb;
  if (!nvalid) rb = nrb - 1;
  const char* wchunks = pool + (size_t)tl.slot * stride + off + (size_t)rb * (K / 16) * 1024 + lane * 16;

  // register stages: tile kt + kAhead is loaded right after tile kt is used
  struct Stage {
    u32x4 a[MF], b[BK / 16];
  };
  Stage st[kAhead];
  auto gload = [&](Stage& r, int kt) {
    const int kk = kt * BK + lcol;
#pragma unroll
    for (int i = 0; i < MF; ++i) r.a[i] = avalid[i] ? ld16(arow[i] + kk) : u32x4{0u, 0u, 0u, 0u};
    // cacheable: the other M-tiles of the group read the same chunks
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) r.b[s] = ld16(wchunks + (size_t)(kt * (BK / 16) + s) * 1024);
  };
  auto astore = [&](const Stage& r, int buf) {
#pragma unroll
    for (int i = 0; i < MF; ++i)
      *reinterpret_cast<u32x4*>(&sA[buf][(lrow + 32 * i) * LDS_LD + lcol]) = r.a[i];
  };
  const int live = (tl.rows + 31) / 32;  // activation fragments holding rows

  floatx16 acc[MF];
#pragma unroll
  for (int j = 0; j < MF; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  const int nk = K / BK;
#pragma unroll
  for (int s = 0; s < kAhead; ++s)
    if (s < nk) gload(st[s], s);
  astore(st[0], 0);
  __syncthreads();
  auto step = [&](Stage& mine, Stage& next, int kt) {
    const int buf = kt & 1;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&mine.b[ks]);
#pragma unroll
      for (int j = 0; j < MF; ++j) {
        if (j < live) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              &sA[buf][(j * 32 + (lane & 31)) * LDS_LD + ks * 16 + 8 * (lane >> 5)]);
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
        }
      }
    }
    if (kt + kAhead < nk) gload(mine, kt + kAhead);
    if (kt + 1 < nk) astore(next, buf ^ 1);
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += kAhead) {
#pragma unroll
    for (int s = 0; s < kAhead; ++s)
      if (kt + s < nk) step(st[s], st[(s + 1) % kAhead], kt + s);
  }

  // epilogue: accumulator j covers rows 32 j .., weight row n of this lane
  const int n = rb * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < MF; ++j) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = j * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const float v = acc[j][r];
      if constexpr (PASS == 1) {
        const float u = __shfl_xor(v, 1, 64);  // odd row = up of the same neuron
        if ((n & 1) == 0 && m < tl.rows && nvalid) {
          uint16_t* h = static_cast<uint16_t*>(out) + (size_t)(tl.row_begin + m) * out_ld;
          h[n >> 1] = f32_to_bf16_rne(silu(v) * u);
        }
      } else {
        if (m < tl.rows && nvalid)
          static_cast<float*>(out)[(size_t)(tl.row_begin + m) * out_ld + n] = v;
      }
    }
  }
}

}  // namespace

void launch_gemm_bf16(int pass, const void* act, const int32_t* perm, int k, const GemmTile* tiles,
                      const int32_t* n_tiles, int max_tiles, const char* pool, size_t stride,
                      size_t off, int N, int K, int out_ld, void* out, hipStream_t s) {
  const dim3 grid((N / 32 + 3) / 4, max_tiles);
  if (pass == 1)
    hipLaunchKernelGGL(gemm_bf16_kernel<1>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(act), perm, k, tiles, n_tiles, pool, stride, off,
                       N, K, out_ld, out);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<2>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(act), perm, k, tiles, n_tiles, pool, stride, off,
                       N, K, out_ld, out);
}
