// Router logits, top-k selection and routing weights (moe_route).
//
// Gating as defined in "RapidMoE: Exploiting Cross-Asymmetry via Adaptive
// Residual Offloading for Large-Scale MoE Inference", Sec. 2.1: a linear
// projection of the token, softmax, and the k experts with the highest
// logits; the weights are normalised over the selected experts ("Communication-
// Aware Placement and Pruning for Efficient Mixture-of-Experts Inference",
// Sec. II-A, Eq. (1)).
//
// Kernels:
//   route_logits_mfma_kernel: bf16 tokens, many tokens and experts: the
//     logits as a dense contraction on v_mfma_f32_32x32x16_bf16, one
//     workgroup per 64 tokens x 64 experts. Each K step of 64 values copies
//     the tile's 64 token rows and 64 router rows (128 bytes each) into LDS
//     with asynchronous global -> LDS copies, 8 whole rows per instruction, in
//     a ring of 8 stages; wave w computes the 32 x 32 block w % 4 over half of
//     every step's K, and the two halves meet in LDS in a fixed order.
//   route_logits_kernel: one workgroup per (expert, tile of 8 tokens); its
//     256 threads split H into 8-element vectors (16-byte bf16 / 2x16-byte
//     fp32 loads), fp32 FMA, then a wave and a cross-wave reduction. A decode
//     step pulls w_router from HBM with E workgroups at once.
//   route_logits1_kernel: one token: one workgroup of 512 threads per expert,
//     every load of the router row and the token issued before the first FMA.
//   topk_softmax_kernel: one wave per token; lane l holds logits l, l+64, ...
//     Each of the k rounds takes the wave-wide (value desc, id asc) maximum
//     through xor shuffles; then softmax over the selected values.
#include <float.h>
#include <limits.h>

#include "common.h"
#include "ffn_internal.h"

namespace {

constexpr int kRouteTT = 8;   // tokens per workgroup
constexpr int kTopkMaxV = 16; // logits per lane (E <= 1024)
// The one-launch decode front end is used up to 4 tokens and 128 experts: measured against the
// separate logits, top-k and permutation kernels it is faster there and slower beyond (at 16
// tokens and 128 experts 45 us against 22 us; at 256 experts already from one token).
constexpr int kFrontMaxT = 4;
constexpr int kFrontMaxE = 128;

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

template <int FMT>
__global__ __launch_bounds__(256) void route_logits_kernel(const void* __restrict__ x,
                                                           const void* __restrict__ w,
                                                           const float* __restrict__ bias, int T,
                                                           int H, int E, float* __restrict__ logits) {
  __shared__ float red[4][kRouteTT];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * kRouteTT;
  const int nt = min(kRouteTT, T - t0);

  float acc[kRouteTT];
#pragma unroll
  for (int t = 0; t < kRouteTT; ++t) acc[t] = 0.f;

#pragma unroll 2
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float wv[8];
    load8<FMT>(w, (size_t)e * H + c, wv);
#pragma unroll
    for (int t = 0; t < kRouteTT; ++t) {
      if (t < nt) {
        float xv[8];
        load8<FMT>(x, (size_t)(t0 + t) * H + c, xv);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[t] = fmaf(wv[q], xv[q], acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouteTT; ++t) {
    const float v = wave_sum(acc[t]);
    if (lane == 0) red[wave][t] = v;
  }
  __syncthreads();
  if ((int)threadIdx.x < nt) {
    const int t = threadIdx.x;
    const float s = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
    logits[(size_t)(t0 + t) * E + e] = s + (bias ? bias[e] : 0.f);
  }
}

// One token: one workgroup of 512 threads per expert. Every thread issues all its NCH
// loads of 8-value chunks of the router row and of the token before its first FMA, so a
// logit costs one memory round trip rather than one per chunk. Chunks past H load a valid
// chunk again and leave the sum unchanged (a select, so no branch takes the loads apart
// from the sums).
constexpr int kLg1Threads = 512;
constexpr int kLg1MaxChunks = 4;  // H <= 512 * 8 * 4
template <int FMT, int NCH>
__global__ __launch_bounds__(kLg1Threads) void route_logits1_kernel(
    const void* __restrict__ x, const void* __restrict__ w, const float* __restrict__ bias, int H,
    int E, float* __restrict__ logits) {
  __shared__ float red[kLg1Threads / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x;
  // raw 16-byte words (bf16: one per chunk, fp32: two), unpacked only after every load is out
  constexpr int WPC = FMT == MOE_BF16 ? 1 : 2;
  u32x4 wr[NCH][WPC], xr[NCH][WPC];
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int c = ((int)threadIdx.x + u * kLg1Threads) * 8;
    const size_t cc = (size_t)(c < H ? c : H - 8);
    const char* wp = static_cast<const char*>(w) + ((size_t)e * H + cc) * (FMT == MOE_BF16 ? 2 : 4);
    const char* xp = static_cast<const char*>(x) + cc * (FMT == MOE_BF16 ? 2 : 4);
#pragma unroll
    for (int j = 0; j < WPC; ++j) {
      wr[u][j] = ld16(wp + 16 * j);
      xr[u][j] = ld16(xp + 16 * j);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every load out before the first use
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    float wv[8], xv[8];
    if constexpr (FMT == MOE_BF16) {
      const uint32_t a[4] = {wr[u][0].x, wr[u][0].y, wr[u][0].z, wr[u][0].w};
      const uint32_t b[4] = {xr[u][0].x, xr[u][0].y, xr[u][0].z, xr[u][0].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wv[2 * i] = bf16_lo(a[i]);
        wv[2 * i + 1] = bf16_hi(a[i]);
        xv[2 * i] = bf16_lo(b[i]);
        xv[2 * i + 1] = bf16_hi(b[i]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t a[4] = {wr[u][j].x, wr[u][j].y, wr[u][j].z, wr[u][j].w};
        const uint32_t b[4] = {xr[u][j].x, xr[u][j].y, xr[u][j].z, xr[u][j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wv[4 * j + i] = __uint_as_float(a[i]);
          xv[4 * j + i] = __uint_as_float(b[i]);
        }
      }
    }
    const bool in = ((int)threadIdx.x + u * kLg1Threads) * 8 < H;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float f = fmaf(wv[q], xv[q], acc);
      acc = in ? f : acc;
    }
  }
  const float v = wave_sum(acc);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kLg1Threads / 64; ++i) s += red[i];
    logits[e] = s + (bias ? bias[e] : 0.f);
  }
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;

// MFMA operand lanes (checked on gfx950): lane l holds row l % 32 and the 8
// K values 8 (l / 32) .. +7 of each 16-wide K step; accumulator r holds row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
constexpr int kLgRows = 64;    // tokens and experts of a tile
constexpr int kLgK = 64;       // K values of a stage (128 bytes a row)
constexpr int kLgStages = 8;  // 7 stages of copies in flight: the loop is bound by their latency
constexpr int kLgStageBytes = 2 * kLgRows * kLgK * 2;  // token rows, then router rows

// Asynchronous global -> LDS copy, 16 bytes per lane to lds + 16 lane (lds is
// the same for every lane of the wave), issued from inline assembly so that
// the compiler does not wait for every copy in flight before each LDS read it
// cannot prove disjoint from them. The kernel orders the copies with explicit
// waits on the vector-memory counter and barriers, and waits for all of them
// before it ends. m0 is listed as clobbered; the kernel holds no other m0 value.
__device__ __forceinline__ void lg_copy16(const void* g, void* lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(l), "v"(g) : "memory", "m0");
}

template <int N_>
__device__ __forceinline__ void lg_vm_wait() {
  // s_waitcnt with only the vector-memory counter limited (N_ < 64)
  __builtin_amdgcn_s_waitcnt((N_ & 15) | ((N_ >> 4) << 14) | (7 << 4) | (15 << 8));
}

__global__ __launch_bounds__(512) void route_logits_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const float* __restrict__ bias, int T, int H, int E, float* __restrict__ logits) {
  __shared__ __attribute__((aligned(1024))) char smem[kLgStages * kLgStageBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kLgRows, e0 = blockIdx.y * kLgRows;
  // copies: wave w takes rows 8 w .. 8 w + 7 of both operands, 8 lanes a row; row r's
  // 16-byte chunk c sits at position c ^ ((r / 2) % 8) of the row's 128 bytes, so the
  // operand reads of 16 consecutive lanes (16 consecutive rows, one chunk) cover all 16
  // groups of 16 bytes that the 64 LDS banks serve at once. Rows past the end read the
  // last row; their results are not stored.
  const int cr = 8 * wave + (lane >> 3);
  const int cc = (lane & 7) ^ ((cr >> 1) & 7);
  const uint16_t* a_src = x + (size_t)min(t0 + cr, T - 1) * H + 8 * cc;
  const uint16_t* b_src = w + (size_t)min(e0 + cr, E - 1) * H + 8 * cc;
  // compute: block (tm, te) of 32 tokens x 32 experts, K steps 2 kh and 2 kh + 1 of the 4
  const int tm = wave & 1, te = (wave >> 1) & 1, kh = wave >> 2;
  int roff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int r = lane & 31, c = 2 * (2 * kh + s) + (lane >> 5);
    roff[s] = r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
  }
  auto issue = [&](int kt, int buf) {
    char* st = smem + buf * kLgStageBytes;
    lg_copy16(a_src + kt * kLgK, st + wave * 1024);
    lg_copy16(b_src + kt * kLgK, st + kLgRows * 128 + wave * 1024);
  };
  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int nk = H / kLgK;
#pragma unroll
  for (int s = 0; s < kLgStages - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt % kLgStages;
    // copies issued after step kt: kLgStages - 2 stages of 2 until the last stages, then
    // wait for all
    if (kt + kLgStages - 2 < nk) lg_vm_wait<2 * (kLgStages - 2)>(); else lg_vm_wait<0>();
    __builtin_amdgcn_s_barrier();  // stage kt is in LDS; every wave is past step kt - 1
    if (kt + kLgStages - 1 < nk) issue(kt + kLgStages - 1, (kt + kLgStages - 1) % kLgStages);
    const char* A = smem + buf * kLgStageBytes + tm * 32 * 128;
    const char* Bm = smem + buf * kLgStageBytes + kLgRows * 128 + te * 32 * 128;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + roff[s]);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bm + roff[s]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done with the ring: its memory holds the upper K halves
  float* red = reinterpret_cast<float*>(smem) + (wave & 3) * (32 * 33);
  if (kh == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * 33 + (lane & 31)] = acc[r];
  }
  __syncthreads();
  if (kh == 0) {
    const int e = e0 + te * 32 + (lane & 31);
    const float be = (bias && e < E) ? bias[e] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int t = t0 + tm * 32 + i;
      const float v = acc[r] + red[i * 33 + (lane & 31)];
      if (t < T && e < E) logits[(size_t)t * E + e] = v + be;
    }
  }
}

// (value, id) order used for selection: larger value first, then smaller id.
__device__ __forceinline__ bool better(float v, int id, float bv, int bid) {
  return v > bv || (v == bv && id < bid);
}

// Top-k and routing weights of token t; executed by one whole wave. The
// outputs ([t*k + r]) may be global memory or LDS.
template <int NV>
__device__ void topk_token(const float* __restrict__ logits, int t, int E, int k, int renorm,
                           int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  float v[NV];
  uint32_t avail = 0;  // bit i: logit of expert lane + 64 i still selectable
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    v[i] = -INFINITY;
    if (e < E) {
      v[i] = logits[(size_t)t * E + e];
      avail |= 1u << i;
    }
  }
  float sel[NV];  // selected value r is held by lane r % 64 in sel[r / 64]
#pragma unroll
  for (int i = 0; i < NV; ++i) sel[i] = 0.f;
  float vmax = 0.f;

  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bid = INT_MAX;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if ((avail >> i) & 1u) {
        if (better(v[i], lane + 64 * i, bv, bid)) {
          bv = v[i];
          bid = lane + 64 * i;
        }
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oid = __shfl_xor(bid, m, 64);
      if (better(ov, oid, bv, bid)) {
        bv = ov;
        bid = oid;
      }
    }
    if (bid != INT_MAX && (bid & 63) == lane) avail &= ~(1u << (bid >> 6));
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (i == (r >> 6) && lane == (r & 63)) sel[i] = bv;
    if (r == 0) vmax = bv;
    if (lane == 0) ids[(size_t)t * k + r] = (bid == INT_MAX) ? -1 : bid;
  }

  float denom = 0.f;
  if (renorm) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < k) denom += expf(sel[i] - vmax);
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < E) denom += expf(v[i] - vmax);
  }
  denom = wave_sum(denom);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int r = lane + 64 * i;
    if (r < k) weights[(size_t)t * k + r] = expf(sel[i] - vmax) / denom;
  }
}

// NV logits per lane (E <= 64 NV): a launch at decode sizes runs from a cold
// instruction cache, so it holds only the code its E needs.
template <int NV>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, int renorm,
                                                           int32_t* __restrict__ ids,
                                                           float* __restrict__ weights) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token<NV>(logits, t, E, k, renorm, ids, weights);
}

// Second half of the decode front end, run by one workgroup (any size up to
// 1024 threads) once the logits of every token are visible at `lg`: top-k of
// every token (one wave per token), then a stable counting sort of the T*k
// assignments by expert. Every intermediate stays in LDS and the outputs are
// written once at the end: a barrier after a global store would wait for the
// store to complete.
struct FrontLds {
  int ids[1024];    // selected expert of assignment t*k + r
  float w[1024];    // its routing weight
  int cnt[1024];    // assignments per expert
  int off[1024];    // first position of each expert
  int perm[1024];   // assignment at each sorted position
  int wave[40];     // scan scratch
  float tmax[kFrontMaxT], tsum[kFrontMaxT];  // softmax max and sum of each token (scores)
};

// Softmax normaliser of token t (its max logit and the sum of exp(l - max)) for
// the routing scores; executed by one whole wave.
template <int NV>
__device__ void token_softmax_norm(const float* lg, int t, int E, float* tmax, float* tsum) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    if (e < E) m = fmaxf(m, lg[(size_t)t * E + e]);
  }
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    if (e < E) s += expf(lg[(size_t)t * E + e] - m);
  }
  s = wave_sum(s);
  if (lane == 0) {
    tmax[t] = m;
    tsum[t] = s;
  }
}

// Work list of the expert FFN written by the front end itself (see FrontPlan):
// the same items and tiles, in the same order, as the FFN's own plan kernel.
__device__ void front_plan(const FrontPlan& pl, int T, int E, int k, const FrontLds& L,
                           int* s_wave) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int G = E + pl.n_shared;
  const int per = (G + nthr - 1) / nthr;  // groups of this thread: [tid * per, +per)
  int n_it = 0, n_tl = 0;
  for (int g = tid * per; g < G && g < (tid + 1) * per; ++g) {
    const int rows = g < E ? L.cnt[g] : T;
    if (rows <= 0) continue;
    const int slot = g < E ? pl.lut[g] : pl.shared_slot0 + (g - E);
    if (slot < 0 || slot >= pl.num_slots) continue;
    if (rows <= pl.small_max) ++n_it; else n_tl += (rows + kGemmBM - 1) / kGemmBM;
  }
  int tot_it = 0, tot_tl = 0;
  int ip = block_exclusive_scan(n_it, s_wave, &tot_it);
  int tp = block_exclusive_scan(n_tl, s_wave, &tot_tl);
  for (int g = tid * per; g < G && g < (tid + 1) * per; ++g) {
    const int rows = g < E ? L.cnt[g] : T;
    if (rows <= 0) continue;
    const int begin = g < E ? L.off[g] : T * k + (g - E) * T;
    const int slot = g < E ? pl.lut[g] : pl.shared_slot0 + (g - E);
    if (slot < 0 || slot >= pl.num_slots) {
      atomicOr(pl.err, MOE_ERR_ABSENT);
      continue;
    }
    if (rows <= pl.small_max) {
      pl.items[ip++] = FfnItem{g, slot, begin, rows};
    } else {
      for (int r0 = 0; r0 < rows; r0 += kGemmBM)
        pl.tiles[tp++] = GemmTile{g, slot, begin + r0, min(kGemmBM, rows - r0)};
    }
  }
  if (tid == 0) {
    pl.n_items[0] = tot_it;
    pl.n_tiles[0] = tot_tl;
  }
  if (pl.sync)  // the one-token FFN launch's hand-off counters start at zero
    for (int i = tid; i < kStreamMaxItems; i += nthr) pl.sync[i] = 0;
}

template <int NV>
__device__ void front_select_and_sort(const float* lg, int T, int E, int k, int renorm,
                                      int32_t* __restrict__ ids, float* __restrict__ weights,
                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                      int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                      int32_t* __restrict__ distinct,
                                      int32_t* __restrict__ n_distinct, FrontLds& L, int* s_dist,
                                      const FrontPlan& pl) {
  const int tid = threadIdx.x, nthr = blockDim.x, wave = tid >> 6, nwaves = nthr >> 6;
  for (int t = wave; t < T; t += nwaves) {
    topk_token<NV>(lg, t, E, k, renorm, L.ids, L.w);
    if (pl.scores) token_softmax_norm<NV>(lg, t, E, L.tmax, L.tsum);
  }
  const int n = T * k;
  for (int i = tid; i < 1024; i += nthr) L.cnt[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += nthr) {
    const int ex = L.ids[i];
    if (ex >= 0 && ex < E) atomicAdd(&L.cnt[ex], 1);
  }
  __syncthreads();
  // exclusive scan of counts (4 experts per thread) and compaction of the routed set
  int c4[4], f4[4], csum = 0, fsum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ex = tid * 4 + j;
    c4[j] = (ex < E) ? L.cnt[ex] : 0;
    f4[j] = c4[j] > 0 ? 1 : 0;
    csum += c4[j];
    fsum += f4[j];
  }
  int total = 0, nd = 0;
  int cbase = block_exclusive_scan(csum, L.wave, &total);
  int fbase = block_exclusive_scan(fsum, L.wave, &nd);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ex = tid * 4 + j;
    if (ex < E) {
      L.off[ex] = cbase;
      if (f4[j]) s_dist[fbase] = ex;
    }
    cbase += c4[j];
    fbase += f4[j];
  }
  __syncthreads();
  // rank of assignment (t, j): tokens before t that picked the same expert
  for (int f = tid; f < n; f += nthr) {
    const int ex = L.ids[f];
    if (ex < 0 || ex >= E) continue;
    const int t = f / k;
    int rank = 0;
    for (int i = 0; i < t * k; ++i) rank += (L.ids[i] == ex) ? 1 : 0;
    L.perm[L.off[ex] + rank] = f;
  }
  __syncthreads();
  if (pl.lut) front_plan(pl, T, E, k, L, L.wave);  // its scans end with a barrier
  // outputs, no barrier after this point
  for (int i = tid; i < n; i += nthr) {
    ids[i] = L.ids[i];
    weights[i] = L.w[i];
    const int f = L.perm[i];
    perm[i] = f;
    inv[f] = i;
  }
  for (int ex = tid; ex < E; ex += nthr) {
    counts[ex] = L.cnt[ex];
    offsets[ex] = L.off[ex];
  }
  for (int i = tid; i < nd; i += nthr) distinct[i] = s_dist[i];
  if (tid == 0) {
    offsets[E] = total;
    n_distinct[0] = nd;
  }
  if (pl.scores) {  // routing scores: softmax probability averaged over the tokens
    for (int ex = tid; ex < E; ex += nthr) {
      float acc = 0.f;
      for (int t = 0; t < T; ++t) acc += expf(lg[(size_t)t * E + ex] - L.tmax[t]) / L.tsum[t];
      const float sc = acc / (float)T;
      pl.scores[ex] = sc;
      // split precision: the critical gate on the same float (RapidMoE Eqs. (3)-(4)):
      // 2 = high precision (score >= threshold), 1 = low precision
      if (pl.crit) pl.crit[ex] = sc >= pl.crit_threshold ? 2 : 1;
    }
  }
}

// The decode front end keeps the tokens in LDS (up to kFrontXBytes) so the
// weight loads of a lane are issued together, one memory round trip per
// kFrontU chunks, instead of one per loop iteration.
constexpr int kFrontU = 4;                     // 8-element chunks per lane in flight
constexpr size_t kFrontXBytes = 128 * 1024;    // tokens staged in LDS (T * H * element size)

// Copy the T token rows (T*H elements) into LDS, 16 bytes per thread per step.
__device__ __forceinline__ void stage_tokens(const void* __restrict__ x, size_t bytes,
                                             u32x4* __restrict__ s_x) {
  const u32x4* src = static_cast<const u32x4*>(x);
  const int nv = (int)(bytes / 16);
#pragma unroll 4
  for (int i = threadIdx.x; i < nv; i += blockDim.x) s_x[i] = src[i];
}

// acc[t] += w_chunk . x[t][c*8 .. c*8+7] for every token, x read from LDS
// (staged) or global memory.
template <int FMT, int MAXT>
__device__ __forceinline__ void dot_chunk(const float (&wv)[8], const void* __restrict__ x,
                                          const void* s_x, bool staged, int T, int H, int c,
                                          float (&acc)[MAXT]) {
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t < T) {
      float xv[8];
      load8<FMT>(staged ? s_x : x, (size_t)t * H + (size_t)c * 8, xv);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[t] = fmaf(wv[q], xv[q], acc[t]);
    }
  }
}

// Decode front end in one launch (T <= kFrontMaxT, T*k <= 1024) for routers
// too large for one workgroup: workgroup e computes the logits of expert e
// for every token (each lane loads kFrontU weight chunks at once); the last
// workgroup to finish (a device-scope counter, released and acquired with
// agent-scope fences) runs the selection and sort. The counter is left at
// zero for the next launch.
template <int FMT, int MAXT, int NV>
__global__ __launch_bounds__(256) void route_front_kernel(
    const void* __restrict__ x, const void* __restrict__ w,
    const float* __restrict__ bias, int T, int H, int E, int k, int renorm,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ weights,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ distinct, int32_t* __restrict__ n_distinct,
    unsigned* __restrict__ done, FrontPlan pl) {
  __shared__ u32x4 s_x[kFrontXBytes / 16];
  __shared__ float red[4][MAXT];
  __shared__ FrontLds L;
  __shared__ int s_dist[1024];
  __shared__ unsigned s_last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = blockIdx.x;
  constexpr int ES = FMT == MOE_BF16 ? 2 : 4;
  const size_t xbytes = (size_t)T * H * ES;
  const bool staged = xbytes <= kFrontXBytes;
  {
    const int nch = H / 8;
    float acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[t] = 0.f;
    for (int cb = 0; cb < nch; cb += 256 * kFrontU) {
      float wv[kFrontU][8];
#pragma unroll
      for (int u = 0; u < kFrontU; ++u) {
        const int c = cb + u * 256 + tid;
        if (c < nch) load8<FMT>(w, (size_t)e * H + (size_t)c * 8, wv[u]);
      }
      if (cb == 0 && staged) {
        stage_tokens(x, xbytes, s_x);
        __syncthreads();
      }
#pragma unroll
      for (int u = 0; u < kFrontU; ++u) {
        const int c = cb + u * 256 + tid;
        if (c < nch) dot_chunk<FMT, MAXT>(wv[u], x, s_x, staged, T, H, c, acc);
      }
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < T) {
        const float v = wave_sum(acc[t]);
        if (lane == 0) red[wave][t] = v;
      }
    }
    __syncthreads();
    if (tid < T) {
      const float sum = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
      logits[(size_t)tid * E + e] = sum + (bias ? bias[e] : 0.f);
    }
  }
  // publish this workgroup's logits, then count it
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(done, 1u) == gridDim.x - 1) ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // see every other workgroup's logits
  front_select_and_sort<NV>(logits, T, E, k, renorm, ids, weights, counts, offsets, perm, inv, distinct,
                        n_distinct, L, s_dist, pl);
  if (tid == 0) *done = 0u;
}

// Decode front end in one workgroup of 1024 threads, for small routers
// (E <= kSingleMaxE and E*H weights of at most kSingleMaxBytes): no
// device-scope hand-off at all. The E*H dot products are split into (expert,
// H slice) pairs, one wave per pair at a time (16/E slices per expert when
// E < 16); a pair's partial sums meet in LDS in slice order, then the same
// workgroup selects and sorts with the logits still in LDS.
constexpr int kSingleMaxE = 64;
constexpr size_t kSingleMaxBytes = 64 * 1024;

template <int FMT, int MAXT, int NV>
__global__ __launch_bounds__(1024) void route_front_single_kernel(
    const void* __restrict__ x, const void* __restrict__ w,
    const float* __restrict__ bias, int T, int H, int E, int k, int renorm,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ weights,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ distinct, int32_t* __restrict__ n_distinct,
    FrontPlan pl) {
  __shared__ u32x4 s_x[kFrontXBytes / 16];
  __shared__ float s_part[16 * kSingleMaxE];  // [pair][t]: pairs * T <= 1024; later the routed set
  __shared__ float s_lg[kFrontMaxT * kSingleMaxE];
  __shared__ FrontLds L;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int ES = FMT == MOE_BF16 ? 2 : 4;
  const size_t xbytes = (size_t)T * H * ES;
  const bool staged = xbytes <= kFrontXBytes;
  const int S = E < 16 ? 16 / E : 1;  // H slices per expert
  const int nch = H / 8;              // 8-element chunks of a row
  bool first = true;
  for (int p0 = 0; p0 < E * S; p0 += 16) {
    const int p = p0 + wave;
    const bool active = p < E * S;
    const int e = active ? p / S : 0, sl = active ? p - e * S : 0;
    const int c0 = sl * nch / S, c1 = active ? (sl + 1) * nch / S : 0;
    float acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[t] = 0.f;
    for (int cb = c0; cb < c1 || first; cb += 64 * kFrontU) {
      float wv[kFrontU][8];
#pragma unroll
      for (int u = 0; u < kFrontU; ++u) {
        const int c = cb + u * 64 + lane;
        if (c < c1) load8<FMT>(w, (size_t)e * H + (size_t)c * 8, wv[u]);
      }
      if (first) {  // every wave passes here exactly once, before its first dot product
        if (staged) stage_tokens(x, xbytes, s_x);
        __syncthreads();
        first = false;
      }
#pragma unroll
      for (int u = 0; u < kFrontU; ++u) {
        const int c = cb + u * 64 + lane;
        if (c < c1) dot_chunk<FMT, MAXT>(wv[u], x, s_x, staged, T, H, c, acc);
      }
    }
    if (active) {
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t < T) {
          const float v = wave_sum(acc[t]);
          if (lane == 0) s_part[p * T + t] = v;
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < T * E; i += 1024) {
    const int t = i / E, e = i - t * E;
    float sum = 0.f;
    for (int sl = 0; sl < S; ++sl) sum += s_part[(e * S + sl) * T + t];
    sum += bias ? bias[e] : 0.f;
    s_lg[i] = sum;
  }
  __syncthreads();
  // s_part is free from here on: it holds the routed set
  front_select_and_sort<NV>(s_lg, T, E, k, renorm, ids, weights, counts, offsets, perm, inv, distinct,
                        n_distinct, L, reinterpret_cast<int*>(s_part), pl);
  for (int i = tid; i < T * E; i += 1024) logits[i] = s_lg[i];
}

// Second half of the front end after a separate logits launch, for the token and
// expert counts the one-launch front end does not take (more than kFrontMaxT
// tokens or more than kFrontMaxE experts) while T <= kSelectMaxT and T*k <=
// kSelectMaxN: one workgroup of 1024 threads selects (one wave per token, all
// tokens at once), sorts and plans,
// replacing the top-k, count, rank and plan launches (each a few microseconds
// from a cold instruction cache at decode sizes). Its rank step compares each
// assignment with every earlier one, so the bound stays small.
constexpr int kSelectMaxT = 16;  // the workgroup's waves
constexpr int kSelectMaxN = 256;

template <int NV>
__global__ __launch_bounds__(1024) void select_sort_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm, int32_t* __restrict__ ids,
    float* __restrict__ weights, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ distinct,
    int32_t* __restrict__ n_distinct, FrontPlan pl) {
  __shared__ FrontLds L;
  __shared__ int s_dist[1024];
  front_select_and_sort<NV>(logits, T, E, k, renorm, ids, weights, counts, offsets, perm, inv,
                            distinct, n_distinct, L, s_dist, pl);
}

// Second half of the front end for one token, in one wave: top-k (topk_token), the
// routing scores, then every output written straight from registers. With one token each
// selected expert holds exactly one assignment, so the counting sort reduces to ranking
// the selected ids: the valid ones (finite logits) take sorted positions in id order, so
// offsets[e] = #{valid selected ids < e} and counts are 0/1, both read off the selection
// ballots; invalid assignments follow them in selection order. The FFN work list (when
// pl.lut is set) is the plan kernel's: the routed groups in id order, then the shared
// groups, each of one row, groups whose slot is out of range skipped and flagged.
constexpr int kDecodeSelectMaxK = 64;
// Order-preserving key of a logit (larger value, larger key); NaN and absent logits get 0,
// below every number (-inf included), as the (value desc, id asc) rule never prefers them.
__device__ __forceinline__ uint32_t logit_key(float f, bool present) {
  const uint32_t u = __float_as_uint(f);
  if (!present || f != f) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NV>
__global__ __launch_bounds__(64) void decode_select_kernel(
    const float* __restrict__ logits, int E, int k, int renorm, int32_t* __restrict__ ids,
    float* __restrict__ weights, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ distinct,
    int32_t* __restrict__ n_distinct, FrontPlan pl) {
  __shared__ uint32_t s_key[kDecodeSelectMaxK];  // candidates in id order: key, id, value,
  __shared__ int s_cid[kDecodeSelectMaxK];       // sorted position (-1: invalid)
  __shared__ float s_cv[kDecodeSelectMaxK];
  __shared__ int s_cpos[kDecodeSelectMaxK];
  __shared__ int s_ids[kDecodeSelectMaxK];  // selection order r: expert (or -1), value, position
  __shared__ float s_sel[kDecodeSelectMaxK];
  __shared__ int s_pos[kDecodeSelectMaxK];
  const int lane = threadIdx.x;
  float v[NV];
  uint32_t key[NV];
  int lutv[NV];  // slot-table entries, loaded with the logits
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? logits[e] : -INFINITY;
    lutv[i] = (pl.lut && e < E) ? pl.lut[e] : -1;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) key[i] = logit_key(v[i], lane + 64 * i < E);
  // the k-th largest key: the largest tau with #{key >= tau} >= k, bit by bit from the top
  uint32_t tau = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= k) tau = cand;
  }
  // selected: every key above tau, then keys equal to tau by ascending id up to k
  int n_gt = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) n_gt += __popcll(__ballot(key[i] > tau));
  const int need = k - n_gt;
  const bool as_item = 1 <= pl.small_max;
  // in id order: candidates, counts and offsets of the valid selected ids, and the work
  // list's routed groups (valid selected ids whose slot is in range)
  int eq_before = 0, base = 0, vbase = 0, tbase = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    const uint64_t meq = __ballot(key[i] == tau);
    const bool sel = key[i] > tau || (key[i] == tau && eq_before + popc_below(meq) < need);
    eq_before += __popcll(meq);
    const bool val = sel && key[i] != 0u;
    const uint64_t ms = __ballot(sel), mv = __ballot(val);
    const int vpos = vbase + popc_below(mv);  // #{valid selected ids < e}
    if (e < E) {
      counts[e] = val ? 1 : 0;
      offsets[e] = vpos;
    }
    if (sel) {
      const int p = base + popc_below(ms);
      s_key[p] = key[i];
      s_cid[p] = e;
      s_cv[p] = v[i];
      s_cpos[p] = val ? vpos : -1;
    }
    if (pl.lut) {
      const bool take = val && lutv[i] >= 0 && lutv[i] < pl.num_slots;
      if (val && !take) atomicOr(pl.err, MOE_ERR_ABSENT);
      const uint64_t mt = __ballot(take);
      if (take) {
        const int q = tbase + popc_below(mt);
        if (as_item) pl.items[q] = FfnItem{e, lutv[i], vpos, 1};
        else pl.tiles[q] = GemmTile{e, lutv[i], vpos, 1};
      }
      tbase += __popcll(mt);
    }
    base += __popcll(ms);
    vbase += __popcll(mv);
  }
  const int nvalid = vbase;
  __syncthreads();
  // selection order: (value desc, id asc), i.e. key desc, id asc
  if (lane < k) {
    const uint32_t mk = s_key[lane];
    const int mi = s_cid[lane];
    int r = 0;
    for (int q = 0; q < k; ++q) {
      const uint32_t qk = s_key[q];
      r += (qk > mk || (qk == mk && s_cid[q] < mi)) ? 1 : 0;
    }
    s_ids[r] = mk == 0u ? -1 : mi;
    s_sel[r] = s_cv[lane];
    s_pos[r] = s_cpos[lane];
  }
  __syncthreads();
  const float vmax = s_sel[0];
  const float sel = lane < k ? s_sel[lane] : 0.f;
  // exp(v - max) of every logit, for the weights over all E and for the scores
  float ex[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) ex[i] = lane + 64 * i < E ? expf(v[i] - vmax) : 0.f;
  // routing weights: softmax over the selected (renorm) or over all E, as topk_token forms it
  float denom = 0.f;
  if (renorm) {
    if (lane < k) denom += expf(sel - vmax);
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < E) denom += ex[i];
  }
  denom = wave_sum(denom);
  const float w_mine = lane < k ? expf(sel - vmax) / denom : 0.f;
  const int my = lane < k ? s_ids[lane] : -1;
  const bool valid = my >= 0;
  // sorted position: valid ids in ascending order, then the invalid assignments in order
  const int inval_before = popc_below(__ballot(lane < k && !valid));
  if (lane < k) {
    const int pos = valid ? s_pos[lane] : nvalid + inval_before;
    ids[lane] = my;
    weights[lane] = w_mine;
    perm[pos] = lane;
    inv[lane] = pos;
    if (valid) distinct[pos] = my;
  }
  if (lane == 0) {
    offsets[E] = nvalid;
    n_distinct[0] = nvalid;
  }
  if (pl.scores) {  // each expert's softmax probability (one token: the average is the value)
    // the normaliser as token_softmax_norm forms it (max of every logit = the first selected)
    float sm = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < E) sm += ex[i];
    sm = wave_sum(sm);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      if (e >= E) continue;
      float acc = 0.f;
      acc += ex[i] / sm;
      const float sc = acc / 1.f;
      pl.scores[e] = sc;
      if (pl.crit) pl.crit[e] = sc >= pl.crit_threshold ? 2 : 1;
    }
  }
  if (pl.lut) {
    // the shared groups E + s after the routed ones, lane s holding group E + s (row k + s)
    const int ns = pl.n_shared;
    const bool shared = lane < ns;
    const int slot = pl.shared_slot0 + lane;
    const bool take = shared && slot >= 0 && slot < pl.num_slots;
    if (shared && !take) atomicOr(pl.err, MOE_ERR_ABSENT);
    const uint64_t mt = __ballot(take);
    if (take) {
      const int q = tbase + popc_below(mt);
      if (as_item) pl.items[q] = FfnItem{E + lane, slot, k + lane, 1};
      else pl.tiles[q] = GemmTile{E + lane, slot, k + lane, 1};
    }
    if (lane == 0) {
      const int n_taken = tbase + __popcll(mt);
      pl.n_items[0] = as_item ? n_taken : 0;
      pl.n_tiles[0] = as_item ? 0 : n_taken;
    }
    if (pl.sync)  // the one-token FFN launch's hand-off counters start at zero
      for (int i = lane; i < kStreamMaxItems; i += 64) pl.sync[i] = 0;
  }
}

// Router logits of T > 0 tokens (arguments checked by the caller).
int launch_logits(const void* x, int x_dtype, const void* w_router, const float* bias, int T,
                  int H, int E, float* logits, hipStream_t stream) {
  dim3 g1(E, (T + kRouteTT - 1) / kRouteTT);
  if (g1.y > 65535u) return MOE_EUNSUPPORTED;
  if (T == 1 && H <= kLg1Threads * 8 * kLg1MaxChunks) {
    const int nch = (H + kLg1Threads * 8 - 1) / (kLg1Threads * 8);
#define MOE_LG1(FMT_, NCH_)                                                                    \
  hipLaunchKernelGGL((route_logits1_kernel<FMT_, NCH_>), dim3(E), dim3(kLg1Threads), 0, stream, x, \
                     w_router, bias, H, E, logits)
    if (x_dtype == MOE_BF16) {
      if (nch == 1) MOE_LG1(MOE_BF16, 1);
      else if (nch == 2) MOE_LG1(MOE_BF16, 2);
      else MOE_LG1(MOE_BF16, 4);
    } else {
      if (nch == 1) MOE_LG1(MOE_F32, 1);
      else if (nch == 2) MOE_LG1(MOE_F32, 2);
      else MOE_LG1(MOE_F32, 4);
    }
#undef MOE_LG1
  } else if (x_dtype == MOE_BF16 && T >= 64 && E >= 32 && H % kLgK == 0)
    hipLaunchKernelGGL(route_logits_mfma_kernel, dim3((T + kLgRows - 1) / kLgRows, (E + kLgRows - 1) / kLgRows),
                       dim3(512), 0, stream, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(w_router), bias, T, H, E, logits);
  else if (x_dtype == MOE_BF16)
    hipLaunchKernelGGL(route_logits_kernel<MOE_BF16>, g1, dim3(256), 0, stream, x, w_router, bias,
                       T, H, E, logits);
  else
    hipLaunchKernelGGL(route_logits_kernel<MOE_F32>, g1, dim3(256), 0, stream, x, w_router, bias,
                       T, H, E, logits);
  return MOE_OK;
}

}  // namespace

extern "C" int moe_route(const void* x, int x_dtype, const void* w_router, const float* bias,
                         int T, int H, int E, int k, int renorm, float* logits,
                         int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  MOE_CHECK_ARG(T >= 0 && H > 0 && H % 8 == 0);
  MOE_CHECK_ARG(k >= 1 && k <= E && E <= 64 * kTopkMaxV);
  MOE_CHECK_ARG(x_dtype == MOE_F32 || x_dtype == MOE_BF16);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(x && w_router && logits && topk_ids && topk_w);
  MOE_CHECK_ARG(((uintptr_t)x % 16) == 0 && ((uintptr_t)w_router % 16) == 0);

  int rc = launch_logits(x, x_dtype, w_router, bias, T, H, E, logits, stream);
  if (rc != MOE_OK) return rc;
#define MOE_TOPK(NV_)                                                                      \
  hipLaunchKernelGGL(topk_softmax_kernel<NV_>, dim3((T + 3) / 4), dim3(256), 0, stream, logits, \
                     T, E, k, renorm, topk_ids, topk_w)
  if (E <= 64) MOE_TOPK(1);
  else if (E <= 128) MOE_TOPK(2);
  else if (E <= 256) MOE_TOPK(4);
  else MOE_TOPK(kTopkMaxV);
#undef MOE_TOPK
  return moe_launch_status();
}

extern "C" int moe_route_permute(const void* x, int x_dtype, const void* w_router, const float* bias,
                                 int T, int H, int E, int k, int renorm, float* logits,
                                 int32_t* topk_ids, float* topk_w, int32_t* counts,
                                 int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* distinct,
                                 int32_t* n_distinct, uint32_t* sync_counter, hipStream_t stream) {
  return route_permute_plan(x, x_dtype, w_router, bias, T, H, E, k, renorm, logits, topk_ids, topk_w,
                            counts, offsets, perm, inv, distinct, n_distinct, sync_counter, nullptr,
                            nullptr, nullptr, stream);
}

int route_permute_plan(const void* x, int x_dtype, const void* w_router, const float* bias, int T,
                       int H, int E, int k, int renorm, float* logits, int32_t* topk_ids,
                       float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv, int32_t* distinct, int32_t* n_distinct,
                       uint32_t* sync_counter, const FrontPlan* plan, bool* planned,
                       bool* scored, hipStream_t stream) {
  if (planned) *planned = false;
  if (scored) *scored = false;
  MOE_CHECK_ARG(T >= 0 && H > 0 && H % 8 == 0);
  MOE_CHECK_ARG(k >= 1 && k <= E && E <= 64 * kTopkMaxV);
  MOE_CHECK_ARG(x_dtype == MOE_F32 || x_dtype == MOE_BF16);
  MOE_CHECK_ARG(counts && offsets && distinct && n_distinct && sync_counter);
  const bool front = T <= kFrontMaxT && E <= kFrontMaxE && T * k <= 1024;
  if (T == 0 || (!front && (T > kSelectMaxT || T * k > kSelectMaxN || E > 64 * kTopkMaxV))) {
    int rc = moe_route(x, x_dtype, w_router, bias, T, H, E, k, renorm, logits, topk_ids, topk_w,
                       stream);
    if (rc != MOE_OK) return rc;
    return moe_permute(topk_ids, T, k, E, counts, offsets, perm, inv, distinct, n_distinct, stream);
  }
  MOE_CHECK_ARG(x && w_router && logits && topk_ids && topk_w && perm && inv);
  MOE_CHECK_ARG(((uintptr_t)x % 16) == 0 && ((uintptr_t)w_router % 16) == 0);
  const size_t wbytes = (size_t)E * H * (x_dtype == MOE_BF16 ? 2 : 4);
  const bool single = E <= kSingleMaxE && wbytes <= kSingleMaxBytes;
  FrontPlan pl{};
  if (plan) {
    pl = *plan;
    if (pl.lut && E + pl.n_shared <= 1024) {
      if (planned) *planned = true;
    } else {
      pl.lut = nullptr;
    }
    if (pl.scores && scored) *scored = true;
  }
  if (T == 1 && k <= kDecodeSelectMaxK && k + (plan ? plan->n_shared : 0) <= 64) {
    // one token: the logits kernel, then one wave selects, ranks and plans
    int rc = launch_logits(x, x_dtype, w_router, bias, T, H, E, logits, stream);
    if (rc != MOE_OK) return rc;
#define MOE_DSELECT(NV_)                                                                          \
  hipLaunchKernelGGL(decode_select_kernel<NV_>, dim3(1), dim3(64), 0, stream, logits, E, k, renorm, \
                     topk_ids, topk_w, counts, offsets, perm, inv, distinct, n_distinct, pl)
    if (E <= 64) MOE_DSELECT(1);
    else if (E <= 128) MOE_DSELECT(2);
    else if (E <= 256) MOE_DSELECT(4);
    else MOE_DSELECT(kTopkMaxV);
#undef MOE_DSELECT
    return moe_launch_status();
  }
  if (!front) {  // logits, then one workgroup selects, sorts and plans
    if (T > kFrontMaxT) {  // its LDS holds the softmax normalisers of kFrontMaxT tokens
      pl.scores = nullptr;
      if (scored) *scored = false;
    }
    int rc = launch_logits(x, x_dtype, w_router, bias, T, H, E, logits, stream);
    if (rc != MOE_OK) return rc;
#define MOE_SELECT(NV_)                                                                          \
  hipLaunchKernelGGL(select_sort_kernel<NV_>, dim3(1), dim3(1024), 0, stream, logits, T, E, k, renorm, \
                     topk_ids, topk_w, counts, offsets, perm, inv, distinct, n_distinct, pl)
    if (E <= 64) MOE_SELECT(1);
    else if (E <= 128) MOE_SELECT(2);
    else if (E <= 256) MOE_SELECT(4);
    else MOE_SELECT(kTopkMaxV);
#undef MOE_SELECT
    return moe_launch_status();
  }
  // code specialised to the token count and logits per lane: the front end runs once per step,
  // from a cold instruction cache, so it should hold only the code the step needs
  const int maxt = T <= 1 ? 1 : kFrontMaxT;
  const int nv = E <= 64 ? 1 : 2;
#define MOE_FRONT(FMT_, MAXT_, NV_)                                                               \
  do {                                                                                           \
    if (single)                                                                                  \
      hipLaunchKernelGGL((route_front_single_kernel<FMT_, MAXT_, NV_>), dim3(1), dim3(1024), 0,  \
                         stream, x, w_router, bias, T, H, E, k, renorm, logits, topk_ids, topk_w, \
                         counts, offsets, perm, inv, distinct, n_distinct, pl);                  \
    else                                                                                         \
      hipLaunchKernelGGL((route_front_kernel<FMT_, MAXT_, NV_>), dim3(E), dim3(256), 0, stream, x, \
                         w_router, bias, T, H, E, k, renorm, logits, topk_ids, topk_w, counts,   \
                         offsets, perm, inv, distinct, n_distinct, sync_counter, pl);            \
  } while (0)
#define MOE_FRONT_NV(FMT_, MAXT_)                   \
  do {                                              \
    if (nv == 1) MOE_FRONT(FMT_, MAXT_, 1);         \
    else MOE_FRONT(FMT_, MAXT_, 2);                 \
  } while (0)
  if (x_dtype == MOE_BF16) {
    if (maxt == 1) MOE_FRONT_NV(MOE_BF16, 1);
    else MOE_FRONT_NV(MOE_BF16, kFrontMaxT);
  } else {
    if (maxt == 1) MOE_FRONT_NV(MOE_F32, 1);
    else MOE_FRONT_NV(MOE_F32, kFrontMaxT);
  }
#undef MOE_FRONT_NV
#undef MOE_FRONT
  return moe_launch_status();
}
