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
// Codes are expanded to int8 bytes holding 16 q: a code moved to the high
// nibble of its byte keeps its sign, so the expansion is two masks and a shift
// and no correction term is needed. The integer sums are then 16 sum q x
// (exact) and the group scale carries the factor 1/16 (exact in fp32).
// Slot layout (moe_slot_layout): tile-major 1 KB chunks of 32 rows x 64 codes;
// a 32-bit word holds 8 consecutive codes, low nibbles = codes 0..3, high
// nibbles = codes 4..7, so
//   (w << 4) & 0xF0F0F0F0  and  w & 0xF0F0F0F0
// are two words of 4 consecutive int8 values (16 q) in natural order.
#include "common.h"
#include "ffn_internal.h"
#include "tile_gemv.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int intx4;
typedef __attribute__((__vector_size__(16 * sizeof(int)))) int intx16;

// SiLU of the MFMA tile epilogue: g / (1 + e^-g) from the hardware exp2 and
// reciprocal (about 1 ulp each; the result is quantised to int8 next)
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}


// ------------------------------------------------------ row quantisation ---
// One workgroup per row of K values (K % 128 == 0): s = max|v| / 127,
// q = clip(rint(v / s), -127, 127).
// With offsets != NULL, row p is skipped unless it belongs to a selected,
// resident group (the rows this call computes): groups 0..E-1 are routed
// (lut, mask), groups E..E+n_shared-1 shared (always computed).
template <int IN>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const void* __restrict__ in, int K, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ lut, const int32_t* __restrict__ mask, int E, int n_shared,
    int num_slots, int8_t* __restrict__ q, float* __restrict__ s) {
  __shared__ float s_max[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (offsets) {
    const int G = E + n_shared;
    int lo = 0, hi = G;  // largest e with offsets[e] <= row
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= row) lo = mid; else hi = mid;
    }
    const int e = lo;
    if (row >= offsets[G]) return;
    if (e < E) {
      if (mask && mask[e] == 0) return;
      const int slot = lut[e];
      if (slot < 0 || slot >= num_slots) return;
    }
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
    if (e0 < K) {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float r = rintf(v[c][i] / sc);
        r = fminf(fmaxf(r, -127.f), 127.f);
        const uint32_t b = (uint32_t)((int)r & 0xFF);
        if (i < 4) w0 |= b << (8 * i); else w1 |= b << (8 * (i - 4));
      }
      *reinterpret_cast<uint2*>(q + (size_t)row * K + e0) = make_uint2(w0, w1);
    }
  }
}

// -------------------------------------------------------- int8 MFMA GEMM ---
// Tile: 128 activation rows (one GemmTile) x 256 weight rows (eight 32-row
// blocks of the tile-major codes), K steps of 128 values = one scale group.
// 8 waves; wave w owns weight block w of the tile and computes all 128 rows
// against it: four v_mfma_i32_32x32x32_i8 accumulators (32-row blocks mf),
// only the blocks that hold rows of the tile (a 40-row tile computes two).
//
// Every operand reaches LDS by asynchronous global -> LDS copies (each lane
// copies 16 bytes to the instruction's LDS base + 16 lane):
//   A: the step's 128 rows x 128 int8 values (16 KB). One copy instruction
//      takes 8 whole rows (8 lanes per 128-byte row), and the eight waves
//      copy two each. Row r's 16-byte chunk c lands in slot
//      8 (r % 8) + (c ^ ((r / 2) % 8)) of its 8-row KB, so the MFMA operand
//      reads (lane l: row mf*32 + l%32, chunk 2 ks + l/32) of any 16
//      consecutive lanes hit 16 different 16-byte groups of the 256 bytes the
//      64 LDS banks serve at once.
//   B: the wave's own two 1 KB code chunks per step (no other wave reads
//      them), read back 16 bytes per lane and expanded to int8 with two masks
//      and a shift.
//   scales: the wave's 32 rows x K/128 bf16 group scales, copied once per
//      tile (contiguous in the slot) into a table read 2 bytes per lane and
//      step.
// Copies run three steps ahead into a ring of four 32 KB stages; one barrier
// per step publishes a stage and frees the oldest. Issuing 16-byte copies of
// 32 different rows, or one scale word per lane and step, cost four and eight
// times the cache lines per byte and left the loop bound by those requests.
// The int32 sums of a group are folded into fp32 (group scale / 16) just
// before the block's accumulator restarts on the next group, so each fold
// overlaps the other blocks' MFMAs.
constexpr int QBN = 256;          // weight rows of a tile
constexpr int QBK = 128;          // one scale group per K step
constexpr int kQABytes = kGemmBM * QBK;  // 16 KB of activations per step
constexpr int kQMaxGroups = 64;   // K <= 8192
constexpr int kQCorr = 4;         // K steps between offset corrections of the fold
static_assert(kGemmBM == 128, "the 8-wave int8 tile covers 128 activation rows");
// Per weight form WM (below): K steps of copies in flight, 1 KB code chunks per
// wave and step, scale tables, and the LDS of a workgroup: the ring of stages
// (activations, then each wave's code chunks), then the scale tables of the eight
// waves (32 rows x kQMaxGroups bf16 each).
__host__ __device__ constexpr int q_ahead(int wm) { return wm == 0 ? 3 : 1; }
__host__ __device__ constexpr int q_chunks(int wm) { return wm == 0 ? 2 : 4; }
__host__ __device__ constexpr int q_tables(int wm) { return wm == 1 ? 2 : 1; }
__host__ __device__ constexpr int q_stage_bytes(int wm) { return kQABytes + 8 * q_chunks(wm) * 1024; }
__host__ __device__ constexpr int q_table_bytes() { return 8 * 32 * kQMaxGroups * 2; }
__host__ __device__ constexpr int q_lds_bytes(int wm) {
  return (q_ahead(wm) + 1) * q_stage_bytes(wm) + q_tables(wm) * q_table_bytes();
}
static_assert(q_lds_bytes(0) <= 160 * 1024 && q_lds_bytes(1) <= 160 * 1024 &&
              q_lds_bytes(2) <= 160 * 1024, "a workgroup's LDS is at most 160 KB");

template <int N_>
__device__ __forceinline__ void vm_wait() {
  // s_waitcnt with only the vector-memory counter limited (N_ < 64)
  __builtin_amdgcn_s_waitcnt((N_ & 15) | ((N_ >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Asynchronous global -> LDS copy of the MFMA tile: 16 bytes per lane to
// lds + 16 lane (lds is the same for every lane of the wave), issued from
// inline assembly so that the compiler does not track it: it would otherwise
// wait for every copy in flight before each LDS read it cannot prove disjoint
// from them, which drains the copy ring every step. The caller orders the
// copies with explicit waits on the vector-memory counter (in-order
// completion) and barriers, and waits for all of them before the workgroup
// ends. The compiler's own waits stay correct: a copy it does not know about
// only makes them more conservative. m0 is listed as clobbered; the kernels
// that use these copies hold no other m0 value (their code writes m0 only right
// before each copy).
__device__ __forceinline__ void dma16_to_lds(const void* g, void* lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(l), "v"(g) : "memory", "m0");
}

// Weight forms of an MFMA tile: WM 0 = int4 codes (W^L, the int4 format);
// WM 1 = int4 codes plus the int4 residual W^R of a split-precision expert
// (gate/up at W^H: each K step runs the group's MFMAs twice, once per code
// set, each folded with its own scale); WM 2 = 8-bit codes (down at W^H:
// 1 KB chunks of 32 rows x 32 codes, already the MFMA operand, group scale
// without the factor 1/16). The forms with more code bytes per step keep one
// step of copies in flight instead of three, to stay within the LDS.
template <int PASS, int NMF, int WM>
__device__ __forceinline__ void w4a8_tile(
    int8_t* smem, const int8_t* __restrict__ aq, const float* __restrict__ as,
    const int32_t* __restrict__ perm, int k, const GemmTile& tl, const char* __restrict__ slot,
    size_t off_codes, size_t off_scales, size_t off_rcodes, size_t off_rscales, int N, int K,
    int out_ld, float* __restrict__ out) {
  constexpr int AH = q_ahead(WM);            // K steps of copies in flight
  constexpr int RING = AH + 1;
  constexpr int NB = q_chunks(WM);           // 1 KB code chunks per wave per K step
  constexpr int NT = q_tables(WM);           // scale tables (W^Q and W^R for WM 1)
  constexpr int kOps = 2 + NB;               // copies per wave per K step (2 for A)
  constexpr int kStage = q_stage_bytes(WM);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrb = N / 32;
  const int gld = K / 128;  // scale groups per weight row
  const int nk = K / QBK;
  int rb = blockIdx.x * (QBN / 32) + wave;
  const bool nvalid = rb < nrb;
  if (!nvalid) rb = nrb - 1;

  // the row scale of each tile row, held by thread m until the loop is over
  float my_rs = 0.f;
  if (tid < kGemmBM) {
    const int p = tl.row_begin + (tid < tl.rows ? tid : 0);
    my_rs = as[(PASS == 1) ? perm[p] / k : p];
  }
  // this lane's two A copies: row m = 16 wave + 8 q + lane/8 into slot lane of its KB,
  // so chunk (lane%8) ^ ((m / 2) % 8)
  const int8_t* a_src[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int m = 16 * wave + 8 * q + (lane >> 3);
    const int p = tl.row_begin + (m < tl.rows ? m : 0);  // rows past the tile read row 0
    a_src[q] = aq + (size_t)((PASS == 1) ? perm[p] / k : p) * K + 16 * ((lane & 7) ^ ((m >> 1) & 7));
  }
  // chunk c of K step kt: int4 (K / 64 chunks per block, 2 per step), int8 (K / 32, 4 per step)
  const size_t blk = (size_t)rb * (K / (WM == 2 ? 32 : 64)) * 1024 + lane * 16;
  const char* b_src = slot + off_codes + blk;
  const char* r_src = slot + off_rcodes + blk;
  int8_t* tables = smem + RING * kStage;
  // the scale tables: rows 32 rb .. 32 rb + 31 of [N, K/128] bf16, 64 gld contiguous bytes
  {
    const int tbytes = 64 * gld;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const char* src = slot + (t == 0 ? off_scales : off_rscales) + (size_t)rb * tbytes;
      int8_t* dst = tables + (t * 8 + wave) * (32 * kQMaxGroups * 2);
      for (int q = 0; q * 1024 < tbytes; ++q) {
        const int b = q * 1024 + lane * 16;
        dma16_to_lds(src + (b < tbytes ? b : tbytes - 16), dst + q * 1024);
      }
    }
  }
  const uint16_t* stab = reinterpret_cast<const uint16_t*>(tables + wave * (32 * kQMaxGroups * 2))
                         + (lane & 31) * gld;

  auto issue = [&](int kt, int buf) {
    int8_t* st = smem + buf * kStage;
    dma16_to_lds(a_src[0] + kt * QBK, st + (2 * wave) * 1024);
    dma16_to_lds(a_src[1] + kt * QBK, st + (2 * wave + 1) * 1024);
    int8_t* lb = st + kQABytes + wave * NB * 1024;
    if constexpr (WM == 2) {
#pragma unroll
      for (int c = 0; c < 4; ++c) dma16_to_lds(b_src + (size_t)(4 * kt + c) * 1024, lb + c * 1024);
    } else {
      dma16_to_lds(b_src + (size_t)(2 * kt) * 1024, lb);
      dma16_to_lds(b_src + (size_t)(2 * kt + 1) * 1024, lb + 1024);
      if constexpr (WM == 1) {
        dma16_to_lds(r_src + (size_t)(2 * kt) * 1024, lb + 2048);
        dma16_to_lds(r_src + (size_t)(2 * kt + 1) * 1024, lb + 3072);
      }
    }
  };
  // the lane's A operand of k step ks inside a 32-row block: row l%32 of the block,
  // chunk 2 ks + l/32, at the swizzled slot of its 8-row KB
  int aoff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int r = lane & 31, c = 2 * ks + (lane >> 5);  // row within the 32-row block
    aoff[ks] = (r >> 3) * 1024 + (8 * (r & 7) + (c ^ ((r >> 1) & 7))) * 16;
  }
  // Each group's int32 sum P is folded into the fp32 sums as fma(float(P), s, acc):
  // float(P) is exact (|P| <= 128 * 128 * 127 < 2^24) and so is P * s for the small
  // integer codes of a group, so a fold rounds once. (Starting P from the bit pattern of
  // 1.5 * 2^23 saves the conversion, but leaves an offset of 1.5 * 2^23 * s per group
  // in the sums, whose rounding then swamps the groups of a row with small scales.)
  constexpr bool MAGIC = false;
  constexpr int kMagicBits = MAGIC ? 0x4B400000 : 0;
  constexpr float kMagic = MAGIC ? 12582912.f : 0.f;
  // the MFMAs' C operand of a group's first k step, held in registers (a value the
  // compiler cannot see as a constant, so it is not rebuilt before every group)
  intx16 magic16 = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (MAGIC) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int v;
      asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(kMagicBits));
      magic16[r] = v;
    }
  }
  intx16 acc[4];
  float accf[4][16];
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
    acc[mf] = magic16;
#pragma unroll
    for (int r = 0; r < 16; ++r) accf[mf][r] = 0.f;
  }
  float pend = 0.f;  // scales folded since the last offset correction
  auto fold = [&](int mf, float sw) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      accf[mf][r] = fmaf(MAGIC ? __int_as_float(acc[mf][r]) : (float)acc[mf][r], sw, accf[mf][r]);
  };
  auto fold_corr = [&](int mf, float sw, float corr) {
    if constexpr (MAGIC) {
#pragma unroll
      for (int r = 0; r < 16; ++r) accf[mf][r] = fmaf(__int_as_float(acc[mf][r]), sw, accf[mf][r] - corr);
    } else {
      fold(mf, sw);
    }
  };
#pragma unroll
  for (int s2 = 0; s2 < AH; ++s2)
    if (s2 < nk) issue(s2, s2);
  float sprev = 0.f;  // the scale of the group in the accumulators (0 before the first)
  // the plain fold skips the first step's (empty) fold; the magic one must fold it to
  // count its kMagic out evenly, and it adds 0 there
  bool started = MAGIC;
  auto step = [&](int kt, int j) {
    // this wave's copies of step kt (and the scale tables) have landed once at most the
    // later steps' are outstanding
    const int after = nk - 1 - kt;
    if constexpr (AH >= 3) {
      if (after >= 2) vm_wait<2 * kOps>(); else if (after == 1) vm_wait<kOps>(); else vm_wait<0>();
    } else {
      vm_wait<0>();
    }
    __builtin_amdgcn_s_barrier();  // every wave's A copies of step kt; every wave is past step kt - 1
    if (kt + AH < nk) issue(kt + AH, (j + AH) % RING);
    const int8_t* A0 = smem + j * kStage;
    const u32x4* bq = reinterpret_cast<const u32x4*>(smem + j * kStage + kQABytes + wave * NB * 1024) + lane;
#pragma unroll
    for (int sub = 0; sub < (WM == 1 ? 2 : 1); ++sub) {
      // the residual pass reads its A fragments from LDS again rather than holding the
      // first pass's in registers (an offset of zero the compiler cannot see through)
      int zero = 0;
      if (sub > 0) asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
      const int8_t* A = A0 + zero;
      const uint32_t sb = (uint32_t)stab[sub * (8 * 32 * kQMaxGroups) + kt] << 16;
      const float scur = __uint_as_float(sb) * (WM == 2 ? 1.f : 0.0625f);  // int4 enters as 16 q
      // the B operand of k step ks: int8 chunks as they are; int4 words expanded to 16 q
      auto operand = [&](int ks) {
        intx4 b;
        if constexpr (WM == 2) {
          const u32x4 cw = bq[ks * 64];
          b[0] = (int)cw.x; b[1] = (int)cw.y; b[2] = (int)cw.z; b[3] = (int)cw.w;
        } else {
          const u32x4 cw = bq[(2 * sub + (ks >> 1)) * 64];
          const uint32_t w0 = (ks & 1) ? cw.z : cw.x, w1 = (ks & 1) ? cw.w : cw.y;
          b[0] = (int)((w0 << 4) & 0xF0F0F0F0u);
          b[1] = (int)(w0 & 0xF0F0F0F0u);
          b[2] = (int)((w1 << 4) & 0xF0F0F0F0u);
          b[3] = (int)(w1 & 0xF0F0F0F0u);
        }
        return b;
      };
      intx4 b[WM == 0 ? 4 : 1];  // the int4 form expands its four operands up front
      if constexpr (WM == 0) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) b[ks] = operand(ks);
      }
      // every kQCorr steps the fold of the previous group also removes the pending offsets
      const bool correct = MAGIC && (j % kQCorr) == 0 && sub == 0;
      const float corr = MAGIC ? kMagic * pend : 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const intx4 bk = WM == 0 ? b[WM == 0 ? ks : 0] : operand(ks);
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf) {
          // the previous group (or code set), before the accumulator restarts; before the
          // first group the accumulator holds kMagic and sprev is 0, so the fold adds 0
          if (ks == 0 && started) {
            if (correct) fold_corr(mf, sprev, corr); else fold(mf, sprev);
          }
          const intx4 a = *reinterpret_cast<const intx4*>(A + aoff[ks] + mf * 4096);
          acc[mf] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bk, ks == 0 ? magic16 : acc[mf], 0, 0, 0);
        }
      }
      if constexpr (MAGIC) pend = correct ? sprev : pend + sprev;
      sprev = scur;
      started = true;
    }
  };
  for (int kt0 = 0; kt0 < nk; kt0 += RING) {
#pragma unroll
    for (int j = 0; j < RING; ++j)
      if (kt0 + j < nk) step(kt0 + j, j);
  }
  {
    const float corr = MAGIC ? kMagic * pend : 0.f;
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf) fold_corr(mf, sprev, corr);
  }
  const float off = MAGIC ? kMagic * sprev : 0.f;  // the last group's offset
  // the row scales go to the first ring stage once every wave is done with it (the
  // last step's wait left no copy in flight)
  float* srow = reinterpret_cast<float*>(smem);
  __syncthreads();
  if (tid < kGemmBM) srow[tid] = my_rs;
  __syncthreads();

  const int n = rb * 32 + (lane & 31);
  // accumulator element r of block mf holds tile row mf*32 + 8(r/4) + 4(lane/32) + r%4
  auto row_of = [&](int mf, int r) { return mf * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); };
#pragma unroll
  for (int mf = 0; mf < NMF; ++mf) {
    if constexpr (PASS == 1) {
      // lanes 2i and 2i+1 hold the gate and up rows of neuron n/2; after one exchange per
      // pair of elements the even lane forms elements r < 8, the odd lane elements r + 8
      const bool odd = lane & 1;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float lo = (accf[mf][r] - off) * srow[row_of(mf, r)];
        const float hi = (accf[mf][r + 8] - off) * srow[row_of(mf, r + 8)];
        const float got = __shfl_xor(odd ? lo : hi, 1, 64);
        const float g = odd ? got : lo, u = odd ? hi : got;
        const int m = row_of(mf, odd ? r + 8 : r);
        if (m < tl.rows && nvalid)
          out[(size_t)(tl.row_begin + m) * out_ld + (n >> 1)] = silu_fast(g) * u;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = row_of(mf, r);
        if (m < tl.rows && nvalid)
          out[(size_t)(tl.row_begin + m) * out_ld + n] = (accf[mf][r] - off) * srow[m];
      }
    }
  }
}

// One MFMA pass over the tile list. HI = false: the tiles on W^L (every tile
// without split precision); HI = true: the tiles on W^H (WM 1 in the gate/up
// pass, WM 2 in the down pass). With split = 1 (split-precision experts) a
// tile is W^H when its group is shared (expert >= E), when mask is NULL or
// when mask[expert] >= 2; each kernel skips the other kind. o holds the W^L
// section (lo) and the W^H one (hi) of the pass.
template <int PASS, bool HI>
__global__ __launch_bounds__(512) void gemm_w4a8_kernel(
    const int8_t* __restrict__ aq, const float* __restrict__ as,
    const int32_t* __restrict__ perm, int k, const GemmTile* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, const char* __restrict__ pool, size_t stride,
    tgemv::QuantOffsets o, const int32_t* __restrict__ mask, int E, int split, int N, int K,
    int out_ld, float* __restrict__ out) {
  constexpr int WM = HI ? (PASS == 1 ? 1 : 2) : 0;
  __shared__ __attribute__((aligned(1024))) int8_t smem[q_lds_bytes(WM)];
  if ((int)blockIdx.y >= n_tiles[0]) return;
  const GemmTile tl = tiles[blockIdx.y];
  const char* slot = pool + (size_t)tl.slot * stride;
  const int nmf = (tl.rows + 31) >> 5;  // 32-row blocks holding rows of the tile
  const bool hi = split && (tl.expert >= E || mask == nullptr || mask[tl.expert] >= 2);
  if (hi != HI) return;
#define MOE_W4A8_TILE(M_)                                                                         \
  w4a8_tile<PASS, M_, WM>(smem, aq, as, perm, k, tl, slot, WM == 2 ? o.hi : o.lo,                 \
                          WM == 2 ? o.hi_s : o.lo_s, o.hi, o.hi_s, N, K, out_ld, out)
  if (nmf >= 4) MOE_W4A8_TILE(4);
  else if (nmf == 3) MOE_W4A8_TILE(3);
  else if (nmf == 2) MOE_W4A8_TILE(2);
  else MOE_W4A8_TILE(1);
#undef MOE_W4A8_TILE
}

// The quantised GEMV pass. With one-row tiles (decode of one token) every unit costs the
// same and, in the gate/up pass, reads the same staged token row: the grid then holds only
// as many workgroups as are resident at once (occupancy x compute units), each taking a
// contiguous range of units and quantising the token once, instead of a last round that
// leaves most compute units idle (576 units of 16 waves on 256 compute units: 47.6 ->
// 44.5 us for 8 experts of 4096 x 7168). With more rows per tile, units differ in cost
// and one workgroup per unit, scheduled as compute units free up, balances better
// (measured 30% slower at 4 tokens with the resident grid).
template <int KS, int RBW, int MAXNT, bool SWIGLU, bool SPLIT, bool QIN>
void launch_gemv(const int8_t* aq, const float* as, const void* raw, const int32_t* perm, int k,
                 const FfnItem* items, const int32_t* n_items, int max_items, const char* pool,
                 size_t stride, const tgemv::QuantOffsets& offs, const int32_t* mask, int E, int R,
                 int K, int out_ld, float* out, hipStream_t s) {
  constexpr int NW = KS < 4 ? 4 : KS;
  constexpr int rb_per_wg = NW / KS * RBW;
  constexpr int U = 2;
  const int upi = (R / 32 + rb_per_wg - 1) / rb_per_wg;
  const long long units = (long long)upi * max_items;
  if (units <= 0) return;
  const size_t lds = QIN ? (size_t)MAXNT * K : 0;  // the tile's int8 rows (K <= 8192)
  const auto kern = tgemv::int4_kernel<KS, RBW, NW, U, MAXNT, SWIGLU, SPLIT, QIN>;
  long long g = units;
  if constexpr (MAXNT == 1) {
    static std::atomic<long long> occ{-1};  // per instantiation
    const long long resident =
        resident_workgroups(reinterpret_cast<const void*>(kern), NW * 64, lds, occ);
    if (g > resident) g = resident;
  }
  if (g > tgemv::kGridCap) g = tgemv::kGridCap;
  hipLaunchKernelGGL(kern, dim3((unsigned)g), dim3(NW * 64), lds, s, aq, as, raw, perm, k, items,
                     n_items, pool, stride, offs, mask, E, R, K, out_ld, upi, out);
}

// One GEMV pass (first: gate/up with the SwiGLU epilogue; else: down). With
// split = true the items of split-precision experts pick their precision from
// mask; with QIN the workgroups quantise their activation rows from raw
// themselves, else they read aq / as (tgemv::int4_kernel).
template <int MAXNT, bool FIRST, bool SPLIT, bool QIN>
void launch_gemv_split(const tgemv::Split& sp, const int8_t* aq, const float* as, const void* raw,
                       const int32_t* perm, int k, const FfnItem* items, const int32_t* n_items,
                       int max_items, const char* pool, size_t stride,
                       const tgemv::QuantOffsets& offs, const int32_t* mask, int E, int R, int K,
                       int ld, float* out, hipStream_t s) {
#define MOE_W4_L(KS_, RBW_)                                                                       \
  launch_gemv<KS_, RBW_, MAXNT, FIRST, SPLIT, QIN>(aq, as, raw, perm, k, items, n_items,         \
                                                   max_items, pool, stride, offs, mask, E, R, K,  \
                                                   ld, out, s)
  if (sp.rbw == 2) {
    // 1024-thread groups hold 128 VGPRs: one-row tiles only
    if constexpr (MAXNT == 1) {
      if (sp.ks >= 16) {
        MOE_W4_L(16, 2);
        return;
      }
    }
    MOE_W4_L(8, 2);
    return;
  }
  switch (sp.ks) {
    case 1: MOE_W4_L(1, 4); break;
    case 2: MOE_W4_L(2, 4); break;
    case 4: MOE_W4_L(4, 4); break;
    default: MOE_W4_L(8, 4); break;
  }
#undef MOE_W4_L
}

void launch_gemv_any(bool first, bool split, int nt, const int8_t* aq, const float* as,
                     const void* raw, const int32_t* perm, int k, const FfnItem* items,
                     const int32_t* n_items,
                     int max_items, const char* pool, size_t stride, const SlotLayout& lay,
                     const int32_t* mask, int E, int H, int F, float* out, hipStream_t s) {
  const int R = first ? 2 * F : H, K = first ? H : F, ld = first ? F : H;
  const tgemv::QuantOffsets offs =
      first ? tgemv::QuantOffsets{lay.off_w13, lay.off_s13, lay.off_r13, lay.off_rs13}
            : tgemv::QuantOffsets{lay.off_w2, lay.off_s2, lay.off_h2, lay.off_hs2};
  const tgemv::Split sp = tgemv::choose_split_int4(R / 32 * max_items, K / 64);
#define MOE_W4_SPLIT(NT_, FIRST_, SPLIT_)                                                        \
  do {                                                                                           \
    if (raw)                                                                                     \
      launch_gemv_split<NT_, FIRST_, SPLIT_, true>(sp, aq, as, raw, perm, k, items, n_items,     \
                                                   max_items, pool, stride, offs, mask, E, R, K, \
                                                   ld, out, s);                                  \
    else                                                                                         \
      launch_gemv_split<NT_, FIRST_, SPLIT_, false>(sp, aq, as, raw, perm, k, items, n_items,    \
                                                    max_items, pool, stride, offs, mask, E, R,   \
                                                    K, ld, out, s);                              \
  } while (0)
#define MOE_W4_NT(NT_)                                     \
  do {                                                     \
    if (first) {                                           \
      if (split) MOE_W4_SPLIT(NT_, true, true);            \
      else MOE_W4_SPLIT(NT_, true, false);                 \
    } else {                                               \
      if (split) MOE_W4_SPLIT(NT_, false, true);           \
      else MOE_W4_SPLIT(NT_, false, false);                \
    }                                                      \
  } while (0)
  if (nt <= 1) MOE_W4_NT(1);
  else if (nt <= 2) MOE_W4_NT(2);
  else MOE_W4_NT(4);
#undef MOE_W4_NT
#undef MOE_W4_SPLIT
}

}  // namespace

// a6q as a stage of its own: per-row int8 codes of rows [rows, K] (the rule every
// int4 pass uses for the tokens and the SwiGLU intermediate).
extern "C" int moe_quantize_rows_int8(const void* in, int in_dtype, int rows, int K, int8_t* q,
                                      float* s, hipStream_t stream) {
  MOE_CHECK_ARG(rows >= 0 && K >= 8 && K % 8 == 0 && K <= 4 * 2048);
  MOE_CHECK_ARG(in_dtype == MOE_F32 || in_dtype == MOE_BF16);
  if (rows == 0) return MOE_OK;
  MOE_CHECK_ARG(in && q && s && ((uintptr_t)in % 16) == 0 && ((uintptr_t)q % 8) == 0);
  if (in_dtype == MOE_BF16)
    hipLaunchKernelGGL(quant_rows_kernel<MOE_BF16>, dim3((unsigned)rows), dim3(256), 0, stream, in,
                       K, nullptr, nullptr, nullptr, 0, 0, 0, q, s);
  else
    hipLaunchKernelGGL(quant_rows_kernel<MOE_F32>, dim3((unsigned)rows), dim3(256), 0, stream, in,
                       K, nullptr, nullptr, nullptr, 0, 0, 0, q, s);
  return moe_launch_status();
}

int ffn_int4(const void* x, const int32_t* perm, const int32_t* offsets, const int32_t* lut,
             const int32_t* group_mask, int n_shared, int shared_slot0, const char* pool,
             size_t stride, int num_slots, const SlotLayout& lay, int T, int H, int F, int E, int k,
             float* y, int32_t* err, char* ws, const FfnWorkspace& wl, hipStream_t s,
             bool planned, bool split) {
  int32_t* n_items = reinterpret_cast<int32_t*>(ws);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(ws + 4);
  FfnItem* items = reinterpret_cast<FfnItem*>(ws + wl.items);
  GemmTile* tiles = reinterpret_cast<GemmTile*>(ws + wl.tiles);
  float* hbuf = reinterpret_cast<float*>(ws + wl.h);
  int8_t* xq = reinterpret_cast<int8_t*>(ws + wl.xq);
  float* xs = reinterpret_cast<float*>(ws + wl.xs);
  int8_t* hq = reinterpret_cast<int8_t*>(ws + wl.hq);
  float* hs = reinterpret_cast<float*>(ws + wl.hs);
  if (H > 4 * 2048 || F > 4 * 2048) return MOE_EUNSUPPORTED;  // quant_rows covers 8192 values
  const long long tk = (long long)T * k;
  const long long rows = (long long)T * (k + n_shared);
  const int small_max =
      ffn_small_max(T, k, E, n_shared, split ? MOE_INT4G128_RESPLIT : MOE_INT4G128);
  // decode batches (not split-precision): groups of up to 32 rows on the MFMA GEMV, which
  // reads the rows quantised by quant_rows_kernel
  const int max_items = small_max == 0 ? 0 : (int)(tk < E ? tk : E) + n_shared;
  const int max_tiles = (T > small_max) ? wl.max_tiles : 0;
  if (max_tiles > 65535) return MOE_EUNSUPPORTED;
  if (!planned)
    launch_ffn_plan(offsets, lut, group_mask, E, n_shared, shared_slot0, num_slots, small_max,
                    items, n_items, tiles, n_tiles, err, reinterpret_cast<int32_t*>(ws + wl.sync), s);
  const bool skinny = !split && T >= 2 && small_max > kGemvMaxRows;
  // with no MFMA tile (and no MFMA GEMV) every row is quantised by the GEMV workgroups
  // that read it (a decode step then runs two weight passes and no separate quantisation)
  const bool fused = max_tiles == 0 && !skinny;
  if (!fused)
    hipLaunchKernelGGL(quant_rows_kernel<MOE_BF16>, dim3(T), dim3(256), 0, s, x, H, nullptr,
                       nullptr, nullptr, 0, 0, 0, xq, xs);
  const int nt = T < kGemvMaxRows ? T : kGemvMaxRows;
  // one token: both passes over even shares of the call's row blocks, in one launch when it fits
  if (T == 1 && !split && fused && max_items > 0 && decode_int4_fits(max_items, 2 * F, H, true) &&
      decode_int4_fits(max_items, H, F, false)) {
    int rc = launch_decode_int4_fused(x, items, n_items, max_items, pool, stride,
                                      lay.off_w13, lay.off_s13, lay.off_w2, lay.off_s2, H, F, hbuf,
                                      y, reinterpret_cast<int32_t*>(ws + wl.sync), err, s);
    if (rc != MOE_EUNSUPPORTED) return rc;
    rc = launch_decode_int4(true, x, items, n_items, max_items, pool, stride,
                                lay.off_w13, lay.off_s13, 2 * F, H, F, hbuf, s);
    if (rc == MOE_OK)
      rc = launch_decode_int4(false, hbuf, items, n_items, max_items, pool, stride,
                              lay.off_w2, lay.off_s2, H, F, H, y, s);
    if (rc != MOE_EUNSUPPORTED) return rc;
  }
  if (max_items > 0) {
    if (skinny)
      launch_skinny_w4a8(1, xq, xs, perm, k, items, n_items, max_items, pool, stride, lay.off_w13,
                         lay.off_s13, 2 * F, H, F, hbuf, s);
    else
      launch_gemv_any(true, split, nt, xq, xs, fused ? x : nullptr, perm, k, items, n_items,
                      max_items, pool, stride, lay, group_mask, E, H, F, hbuf, s);
  }
  const tgemv::QuantOffsets o13{lay.off_w13, lay.off_s13, lay.off_r13, lay.off_rs13};
  const tgemv::QuantOffsets o2{lay.off_w2, lay.off_s2, lay.off_h2, lay.off_hs2};
  const dim3 g13((2 * F + QBN - 1) / QBN, max_tiles), g2((H + QBN - 1) / QBN, max_tiles);
  if (max_tiles > 0) {
    hipLaunchKernelGGL((gemm_w4a8_kernel<1, false>), g13, dim3(512), 0, s, xq, xs, perm, k, tiles,
                       n_tiles, pool, stride, o13, group_mask, E, split ? 1 : 0, 2 * F, H, F, hbuf);
    if (split)
      hipLaunchKernelGGL((gemm_w4a8_kernel<1, true>), g13, dim3(512), 0, s, xq, xs, perm, k,
                         tiles, n_tiles, pool, stride, o13, group_mask, E, 1, 2 * F, H, F, hbuf);
  }
  if (!fused)
    hipLaunchKernelGGL(quant_rows_kernel<MOE_F32>, dim3((unsigned)rows), dim3(256), 0, s, hbuf, F,
                       offsets, lut, group_mask, E, n_shared, num_slots, hq, hs);
  if (max_items > 0) {
    if (skinny)
      launch_skinny_w4a8(2, hq, hs, perm, k, items, n_items, max_items, pool, stride, lay.off_w2,
                         lay.off_s2, H, F, H, y, s);
    else
      launch_gemv_any(false, split, nt, hq, hs, fused ? hbuf : nullptr, perm, k, items, n_items,
                      max_items, pool, stride, lay, group_mask, E, H, F, y, s);
  }
  if (max_tiles > 0) {
    hipLaunchKernelGGL((gemm_w4a8_kernel<2, false>), g2, dim3(512), 0, s, hq, hs, perm, k, tiles,
                       n_tiles, pool, stride, o2, group_mask, E, split ? 1 : 0, H, F, H, y);
    if (split)
      hipLaunchKernelGGL((gemm_w4a8_kernel<2, true>), g2, dim3(512), 0, s, hq, hs, perm, k,
                         tiles, n_tiles, pool, stride, o2, group_mask, E, 1, H, F, H, y);
  }
  return moe_launch_status();
}
