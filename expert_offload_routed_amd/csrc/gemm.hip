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
// Tile: 128 activation rows (one GemmTile) x 256 weight rows (eight 32-row
// blocks of the tile-major slot), K steps of 32. 8 waves; wave w computes
// rows 64 (w & 1) .. +63 against weight blocks 2 (w >> 1), +1: four
// v_mfma_f32_32x32x16_bf16 accumulators, so each LDS fragment feeds two MFMAs.
// Operands reach LDS through asynchronous global -> LDS copies (16 bytes per
// lane) in a ring of kStages stages, no register holding data in flight:
//   A: the stage's 128 rows x 32 K values (64 bytes a row), one copy
//      instruction per wave covering 16 whole rows (4 lanes a row). Row r's
//      16-byte chunk c lands in slot 4 (r % 16) + (c ^ ((r / 4) % 4)) of its
//      16-row KB, so the MFMA operand reads (lane l: row mf*32 + l%32, chunk
//      2 ks + l/32) of any 16 consecutive lanes hit 16 different 16-byte
//      groups of the 256 bytes the 64 LDS banks serve at once. (Copies of 32
//      rows x 32 bytes cost twice the cache-line requests and left the loop
//      bound by them.)
//   B: the 16 chunks of the tile's 8 weight blocks, as stored.
// Each wave issues 3 copies per stage; before computing stage kt it waits
// until only the later stages' copies are outstanding, then one barrier
// publishes the stage to all waves. A stage is 24 KB, so two workgroups share
// a CU (4 waves per SIMD).
// Lane layouts (checked on gfx950): A/B operand lane l holds row l % 32,
// k = 8 (l / 32) .. +7; accumulator r holds row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.
#include "common.h"
#include "ffn_internal.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;

constexpr int BM = kGemmBM;  // activation rows of a tile (128)
constexpr int BN = 256;      // weight rows of a tile
constexpr int BK = 32;       // K values of a stage
constexpr int kStages = 3;
constexpr int kStageBytes = 8192 + 16384;  // A, B
static_assert(BM == 128, "the 8-wave bf16 tile covers 128 activation rows");

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

// 16 bytes per lane from global memory into LDS at lds + 16 * lane (a device-only helper:
// called straight from the kernel's lambdas the builtin hides the host launch stub)
__device__ __forceinline__ void copy16_to_lds(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

template <int PASS>
__global__ __launch_bounds__(512) void gemm_bf16_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ perm, int k,
    const GemmTile* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    const char* __restrict__ pool, size_t stride, size_t off, int N, int K, int out_ld,
    void* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
  if ((int)blockIdx.y >= n_tiles[0]) return;
  const GemmTile tl = tiles[blockIdx.y];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mh = wave & 1, np = wave >> 1;
  const int nrb = N / 32;
  // copies of this wave per stage: rows 16 wave .. +15 of A (row m into slot `lane` of KB
  // `wave`, so chunk (lane % 4) ^ ((m / 4) % 4)); the 2 chunks of weight block `wave`
  const uint16_t* a_src;
  {
    const int m = 16 * wave + (lane >> 2);
    const int p = tl.row_begin + (m < tl.rows ? m : 0);  // rows past the tile read row 0
    const size_t r = (PASS == 1) ? (size_t)(perm[p] / k) : (size_t)p;
    a_src = act + r * K + 8 * ((lane & 3) ^ ((m >> 2) & 3));
  }
  // the lane's A operand of k step ks inside a 32-row block (row l%32, chunk 2 ks + l/32)
  int aoff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int r = lane & 31, c = 2 * ks + (lane >> 5);
    aoff[ks] = (r >> 4) * 1024 + (4 * (r & 15) + (c ^ ((r >> 2) & 3))) * 16;
  }
  int lrb = blockIdx.x * (BN / 32) + wave;
  if (lrb >= nrb) lrb = nrb - 1;
  const char* b_src = pool + (size_t)tl.slot * stride + off + (size_t)lrb * (K / 16) * 1024 + lane * 16;
  bool nvalid[2];
  int rbv[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    int rb = blockIdx.x * (BN / 32) + np * 2 + nb;
    nvalid[nb] = rb < nrb;
    rbv[nb] = nvalid[nb] ? rb : nrb - 1;
  }
  auto stage_a = [&](int buf) { return smem + buf * kStageBytes; };
  auto stage_b = [&](int buf) { return smem + buf * kStageBytes + 8192; };
  auto issue = [&](int kt, int buf) {
    copy16_to_lds(a_src + kt * BK, stage_a(buf) + wave * 1024);
    char* lb = stage_b(buf) + wave * 2048;
#pragma unroll
    for (int c = 0; c < 2; ++c) copy16_to_lds(b_src + (size_t)(2 * kt + c) * 1024, lb + c * 1024);
  };
  floatx16 acc[2][2];
#pragma unroll
  for (int mf = 0; mf < 2; ++mf)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mf][nb][r] = 0.f;
  const int nk = K / BK;
#pragma unroll
  for (int s2 = 0; s2 < kStages - 1; ++s2)
    if (s2 < nk) issue(s2, s2);
  auto step = [&](int kt, int buf) {
    // stages issued after kt: at most kStages - 2 = 1, of 3 copies each
    if (kt + 1 < nk) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
    // every wave has finished stage kt - 1, whose buffer is refilled now
    if (kt + kStages - 1 < nk) issue(kt + kStages - 1, (buf + kStages - 1) % kStages);
    const char* A = stage_a(buf);
    const char* Bs = stage_b(buf);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 b[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        b[nb] = *reinterpret_cast<const bf16x8*>(Bs + ((np * 2 + nb) * 2 + ks) * 1024 + lane * 16);
#pragma unroll
      for (int mf = 0; mf < 2; ++mf) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + (mh * 2 + mf) * 2048 + aoff[ks]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mf][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[nb], acc[mf][nb], 0, 0, 0);
      }
    }
  };
  for (int kt = 0; kt < nk; kt += kStages) {
#pragma unroll
    for (int j = 0; j < kStages; ++j)
      if (kt + j < nk) step(kt + j, j);
  }

  // epilogue: accumulator (mf, nb) covers rows (mh*2 + mf)*32 .., weight row n of this lane
#pragma unroll
  for (int mf = 0; mf < 2; ++mf) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = rbv[nb] * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = (mh * 2 + mf) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const float v = acc[mf][nb][r];
        if constexpr (PASS == 1) {
          const float u = __shfl_xor(v, 1, 64);  // odd row = up of the same neuron
          if ((n & 1) == 0 && m < tl.rows && nvalid[nb]) {
            uint16_t* h = static_cast<uint16_t*>(out) + (size_t)(tl.row_begin + m) * out_ld;
            h[n >> 1] = f32_to_bf16_rne(silu(v) * u);
          }
        } else {
          if (m < tl.rows && nvalid[nb])
            static_cast<float*>(out)[(size_t)(tl.row_begin + m) * out_ld + n] = v;
        }
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
    hipLaunchKernelGGL(gemm_bf16_kernel<1>, grid, dim3(512), 0, s,
                       static_cast<const uint16_t*>(act), perm, k, tiles, n_tiles, pool, stride, off,
                       N, K, out_ld, out);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<2>, grid, dim3(512), 0, s,
                       static_cast<const uint16_t*>(act), perm, k, tiles, n_tiles, pool, stride, off,
                       N, K, out_ld, out);
}
