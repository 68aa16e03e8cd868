// One-token bf16 expert passes: every row block of the call in one even share per
// workgroup, both passes in one launch when they fit.
//
// The bf16 counterpart of the one-token int4 passes. With one token a pass is a GEMV per
// routed expert over its tile-major bf16 weights, read through the slot table (SeqMoE
// summary page): 1 KB chunks of 32 rows x 16 values, lane l holding row l % 32 and the
// values 8 (l / 32) .. +7 of the chunk. The call's row blocks, in (group, row block) order,
// are cut into one contiguous share per resident workgroup (equal to within one row
// block); wave j of the 16 takes the j-th sixteenth of the K chunks of every row block of
// the share and streams them with kDecP chunks in flight per lane; each wave keeps one
// partial per (row block, row) in LDS, and after one barrier each row block is summed over
// the waves in a fixed order and finished:
//   gate/up pass: activations = the token row (bf16, copied to LDS); h[n] = SiLU(g) * u of
//     rows 2n, 2n+1, rounded to bf16, as the GEMV passes store it;
//   down pass: activations = the h rows of the share's groups (bf16, copied to LDS);
//     y = the dot (fp32).
// Products and sums are fp32 (an FMA per weight). The one-launch form hands h over per
// group like the int4 form: device-scope stores of bf16 pairs, counted per group once
// they have completed; the down pass issues its first weight loads, waits for its
// groups' counts, then reads h with device-scope loads.
#include "common.h"
#include "decode_share.h"
#include "ffn_internal.h"
#include "tile_gemv.h"

namespace {

using namespace decode_share;

// h pairs (two bf16 in 32 bits) handed between the workgroups of one launch go through
// device-scope stores and loads, as the int4 form's fp32 h does.
__device__ __forceinline__ void store_h2(uint32_t* p, uint32_t v, bool shared) {
  if (shared) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
__device__ __forceinline__ u32x4 load_h16(const uint32_t* p, bool shared) {
  if (!shared) return ld16(p);
  u32x4 r;
  r.x = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  r.y = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  r.z = __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  r.w = __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return r;
}

// SWIGLU (gate/up pass): raw = the bf16 tokens (T = 1: row perm[p] / k is row 0 for every
// group, so the token loads wait for neither the work list nor perm),
// out = h (bf16, row p, column n of rows 2n, 2n+1). Otherwise (down pass): raw = h (bf16
// rows p), out = y (fp32). act: the workgroup's dynamic LDS, activation rows
// [SWIGLU ? 1 : n_items][K] bf16; red: [kDecNW][MAXRB][32] partials.
template <bool SWIGLU, int MAXRB>
__device__ __forceinline__ void bf16_pass(const void* __restrict__ raw,
                                          const FfnItem* __restrict__ items, int n_items,
                                          const char* __restrict__ pool, size_t stride,
                                          size_t off_w, int R, int K, int out_ld,
                                          void* __restrict__ out, uint16_t* act,
                                          float (*red)[MAXRB][32], const PassSync& sy) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rbi = R / 32, nkc = K / 16;
  const int total_rb = n_items * rbi;
  int b0, b1;
  share_of(total_rb, b0, b1);
  const int nrb = b1 - b0;  // <= MAXRB (the launch checks)
  // an empty share (more workgroups than row blocks) has nothing to load, wait for or count
  if (nrb == 0) return;
  // this wave's K slice of every row block of the share, as one stream of chunks walked by
  // two cursors (the loads kDecP chunks ahead of the sums); all cursor state is uniform
  const int c0 = nkc * wave / kDecNW, c1 = nkc * (wave + 1) / kDecNW;
  const int nq = nrb * (c1 - c0);  // > 0: every wave has a chunk of each block (K / 16 >= 16)
  const int kh = 8 * (lane >> 5);
  struct Cursor {
    int r, c, item;
    const char* base;  // the row block's first chunk, this lane's 16 bytes
  };
  auto at_block = [&](Cursor& u, int r) {
    const int b = b0 + r, item = b / rbi, rb = b - item * rbi;
    u.r = r;
    u.c = c0;
    u.item = item;
    u.base = pool + (size_t)items[item].slot * stride + off_w + (size_t)rb * nkc * 1024 + lane * 16;
  };
  // the next chunk; a load cursor past the share stays on its last chunk (loaded again, unused)
  auto advance = [&](Cursor& u) {
    if (u.c + 1 < c1) {
      ++u.c;
    } else if (u.r + 1 < nrb) {
      at_block(u, u.r + 1);
    }
  };
  float acc = 0.f;
  Cursor sum_at{}, load_at{};
  auto flush = [&](int r) {  // the row block's partial (both K halves of a row) into LDS
    const float v = acc + __shfl_xor(acc, 32, 64);
    if (lane < 32) red[wave][r][lane] = v;
    acc = 0.f;
  };
  auto consume = [&](const u32x4& w) {
    const u32x4 a =
        ld16(act + (SWIGLU ? 0 : (size_t)sum_at.item * K) + (size_t)sum_at.c * 16 + kh);
    acc = fmaf(bf16_lo(w.x), bf16_lo(a.x), acc);
    acc = fmaf(bf16_hi(w.x), bf16_hi(a.x), acc);
    acc = fmaf(bf16_lo(w.y), bf16_lo(a.y), acc);
    acc = fmaf(bf16_hi(w.y), bf16_hi(a.y), acc);
    acc = fmaf(bf16_lo(w.z), bf16_lo(a.z), acc);
    acc = fmaf(bf16_hi(w.z), bf16_hi(a.z), acc);
    acc = fmaf(bf16_lo(w.w), bf16_lo(a.w), acc);
    acc = fmaf(bf16_hi(w.w), bf16_hi(a.w), acc);
    if (sum_at.c + 1 == c1) flush(sum_at.r);  // uniform: the row block's slice is done
    advance(sum_at);
  };
  // Vector loads return in issue order: the token row goes out first (one 16-byte piece per
  // thread, K / 8 <= blockDim, an index past the end clamped to a valid one), then the first
  // kDecP weight chunks, which stay in flight while the copy into LDS waits for the row.
  const int npiece = K / 8;
  u32x4 tok{};
  if constexpr (SWIGLU) {
    const int pc = (int)threadIdx.x < npiece ? (int)threadIdx.x : npiece - 1;
    tok = ld16(static_cast<const uint16_t*>(raw) + (size_t)pc * 8);  // the one token
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 buf[kDecP];
  at_block(sum_at, 0);
  at_block(load_at, 0);
#pragma unroll
  for (int i = 0; i < kDecP; ++i) {
    buf[i] = ld16_stream(load_at.base + (size_t)load_at.c * 1024);
    advance(load_at);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SWIGLU) {
    if ((int)threadIdx.x < npiece) *reinterpret_cast<u32x4*>(act + (size_t)threadIdx.x * 8) = tok;
  } else {
    // one launch: the h rows this share reads are complete once every row block of their
    // groups is counted; then only the rows of the share's groups are copied
    if (sy.wait != nullptr) wait_groups(sy, b0 / rbi, (b1 - 1) / rbi);
    const int i0 = b0 / rbi, nrow = (b1 - 1) / rbi - i0 + 1;
    const int nv = nrow * npiece;
    const uint16_t* h = static_cast<const uint16_t*>(raw);
    for (int idx = threadIdx.x; idx < nv; idx += blockDim.x) {
      const int r = idx / npiece, pc = idx - r * npiece;
      const u32x4 v = load_h16(reinterpret_cast<const uint32_t*>(
                                   h + (size_t)items[i0 + r].row_begin * K + (size_t)pc * 8),
                               sy.wait != nullptr);
      *reinterpret_cast<u32x4*>(act + (size_t)(i0 + r) * K + (size_t)pc * 8) = v;
    }
  }
  __syncthreads();

  {
    int q0 = 0;
    for (; q0 + 2 * kDecP <= nq; q0 += kDecP) {
#pragma unroll
      for (int i = 0; i < kDecP; ++i) {
        consume(buf[i]);
        // the register's next load goes out after its value is used, so the loads of one
        // trip stay in flight across the back edge
        __builtin_amdgcn_sched_barrier(0);
        buf[i] = ld16_stream(load_at.base + (size_t)load_at.c * 1024);
        advance(load_at);
      }
    }
    // nq - q0 chunks left (fewer than 2 kDecP); the first min(kDecP, left) are loaded
#pragma unroll
    for (int i = 0; i < kDecP; ++i) {
      if (q0 + i < nq) {
        consume(buf[i]);
        if (q0 + kDecP + i < nq) {
          buf[i] = ld16_stream(load_at.base + (size_t)load_at.c * 1024);
          advance(load_at);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kDecP; ++i)
      if (q0 + kDecP + i < nq) consume(buf[i]);
  }
  __syncthreads();
  // each row block of the share: the 16 waves' partials in wave order, then the epilogue
  for (int r = wave; r < nrb; r += kDecNW) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kDecNW; ++w) v += red[w][r][lane & 31];
    const int b = b0 + r, item = b / rbi, rb = b - item * rbi;
    const FfnItem it = items[item];
    const int row = rb * 32 + (lane & 31);
    if constexpr (SWIGLU) {
      const float u = __shfl_xor(v, 1, 64);  // odd row = up of the same neuron
      const uint32_t hb = f32_to_bf16_rne(tgemv::silu(v) * u);  // valid on even lanes
      const uint32_t hn = __shfl_down(hb, 2, 64);               // neuron (row >> 1) + 1
      // lanes 0, 4, ..., 28: neurons 2m, 2m + 1 of the row block as one 32-bit pair
      if (lane < 32 && (lane & 3) == 0)
        store_h2(reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) +
                                             (size_t)it.row_begin * out_ld + (row >> 1)),
                 (hb & 0xFFFFu) | (hn << 16), sy.signal != nullptr);
    } else {
      if (lane < 32) static_cast<float*>(out)[(size_t)it.row_begin * out_ld + row] = v;
    }
  }
  if (sy.signal != nullptr) signal_groups(sy, b0, b1, rbi);
}

template <bool SWIGLU, int MAXRB>
__global__ __launch_bounds__(kDecNW * 64) __attribute__((amdgpu_waves_per_eu(4))) void
bf16_decode_kernel(const void* __restrict__ raw, const FfnItem* __restrict__ items,
                   const int32_t* __restrict__ n_items_p,
                   const char* __restrict__ pool, size_t stride, size_t off_w, int R, int K,
                   int out_ld, void* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t act[];
  __shared__ float red[kDecNW][MAXRB][32];
  bf16_pass<SWIGLU, MAXRB>(raw, items, n_items_p[0], pool, stride, off_w, R, K, out_ld,
                           out, act, red, PassSync{nullptr, nullptr, 0, nullptr, 0});
}

// Both passes of a one-token call in one launch (the grid resident at once): each workgroup
// runs its gate/up share, counts it per group, then its down share, whose first weight loads
// go out before it waits for the h rows.
template <int MAXRB>
__global__ __launch_bounds__(kDecNW * 64) __attribute__((amdgpu_waves_per_eu(4))) void
bf16_decode_fused_kernel(const void* __restrict__ x, const FfnItem* __restrict__ items,
                         const int32_t* __restrict__ n_items_p,
                         const char* __restrict__ pool, size_t stride, size_t off_w13,
                         size_t off_w2, int H, int F, uint16_t* __restrict__ hbuf,
                         float* __restrict__ y, int32_t* __restrict__ sync,
                         int32_t* __restrict__ err, int spin_cap) {
  extern __shared__ __attribute__((aligned(16))) uint16_t act[];
  __shared__ float red[kDecNW][MAXRB][32];
  const int n_items = n_items_p[0];
  bf16_pass<true, MAXRB>(x, items, n_items, pool, stride, off_w13, 2 * F, H, F, hbuf, act,
                         red, PassSync{sync, nullptr, 0, err, spin_cap});
  __syncthreads();  // the LDS of the first pass is free
  bf16_pass<false, MAXRB>(hbuf, items, n_items, pool, stride, off_w2, H, F, H, y, act,
                          red, PassSync{nullptr, sync, 2 * F / 32, err, spin_cap});
}

size_t bf16_decode_lds(bool swiglu, int max_items, int K) {
  return (size_t)(swiglu ? 1 : max_items) * K * 2;
}

}  // namespace

bool decode_bf16_fits(int max_items, int R, int K, bool swiglu) {
  if (max_items < 1 || max_items > kStreamMaxItems || R % 32 != 0 || K % 16 != 0 ||
      K / 16 < kDecNW || (swiglu && K / 8 > kDecNW * 64))
    return false;
  return bf16_decode_lds(swiglu, max_items, K) <= 96 * 1024;
}

int launch_decode_bf16(bool swiglu, const void* raw, const FfnItem* items, const int32_t* n_items,
                       int max_items,
                       const char* pool, size_t stride, size_t off_w, int R, int K, int out_ld,
                       void* out, hipStream_t s) {
  // the grid: the workgroups the compute units keep resident; every share has at most
  // ceil(blocks / grid) <= MAXRB row blocks
  const long long blocks = (long long)max_items * (R / 32);
  long long grid = (long long)decode_cus() * kDecWgPerCu;
  if (grid > blocks) grid = blocks;
  const long long per = (blocks + grid - 1) / grid;
  const size_t lds = bf16_decode_lds(swiglu, max_items, K);
#define MOE_BF16_DEC(SW_, MAXRB_)                                                              \
  hipLaunchKernelGGL((bf16_decode_kernel<SW_, MAXRB_>), dim3((unsigned)grid), dim3(kDecNW * 64), \
                     lds, s, raw, items, n_items, pool, stride, off_w, R, K, out_ld, out)
  if (per <= 8) {
    if (swiglu) MOE_BF16_DEC(true, 8);
    else MOE_BF16_DEC(false, 8);
  } else if (per <= 16) {
    if (swiglu) MOE_BF16_DEC(true, 16);
    else MOE_BF16_DEC(false, 16);
  } else {
    return MOE_EUNSUPPORTED;
  }
#undef MOE_BF16_DEC
  return moe_launch_status();
}

int launch_decode_bf16_fused(const void* x, const FfnItem* items,
                             const int32_t* n_items, int max_items, const char* pool,
                             size_t stride, size_t off_w13, size_t off_w2, int H, int F,
                             void* hbuf, float* y, int32_t* sync, int32_t* err, hipStream_t s) {
  if (!decode_bf16_fits(max_items, 2 * F, H, true) || !decode_bf16_fits(max_items, H, F, false))
    return MOE_EUNSUPPORTED;
  // kDecWgPerCu workgroups per compute unit, exactly as many as fit on one (16 waves of at
  // most 128 VGPRs; the LDS request admits no more), so the grid is resident at once and
  // every wait ends
  const long long b1 = (long long)max_items * (2 * F / 32), b2 = (long long)max_items * (H / 32);
  const long long grid = (long long)decode_cus() * kDecWgPerCu;
  const long long per = ((b1 > b2 ? b1 : b2) + grid - 1) / grid;
  const int maxrb = per <= 8 ? 8 : 16;
  const size_t l1 = bf16_decode_lds(true, max_items, H), l2 = bf16_decode_lds(false, max_items, F);
  const size_t stat = sizeof(float) * (size_t)kDecNW * maxrb * 32;
  const size_t lds = resident_lds(l1 > l2 ? l1 : l2, stat);
  if (lds == 0 || per > 16) return MOE_EUNSUPPORTED;
  uint16_t* h = static_cast<uint16_t*>(hbuf);
  if (per <= 8)
    hipLaunchKernelGGL((bf16_decode_fused_kernel<8>), dim3((unsigned)grid), dim3(kDecNW * 64), lds,
                       s, x, items, n_items, pool, stride, off_w13, off_w2, H, F, h, y,
                       sync, err, kSpinCap);
  else
    hipLaunchKernelGGL((bf16_decode_fused_kernel<16>), dim3((unsigned)grid), dim3(kDecNW * 64), lds,
                       s, x, items, n_items, pool, stride, off_w13, off_w2, H, F, h, y,
                       sync, err, kSpinCap);
  return moe_launch_status();
}
