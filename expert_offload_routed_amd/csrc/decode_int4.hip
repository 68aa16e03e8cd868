// One-token int4 expert passes: every row block of the call in one even share
// per workgroup.
//
// With one token a pass is a GEMV per routed expert over its tile-major int4
// weights (1 KB chunks of 32 rows x 64 codes; RapidMoE Eq. (7) through the
// slot table of the SeqMoE summary page). Work units of whole row-block pairs
// leave the pass with a ragged last round whenever their count is not a
// multiple of the resident workgroups (576 units on 256 workgroups: a third
// round on a quarter of them). Here the flat list of the call's row blocks,
// in (group, row block) order, is cut into one contiguous share per resident
// workgroup (equal to within one row block), and:
//   * wave j of the 16 takes the j-th sixteenth of the K chunks of every row
//     block of the share and streams them in one loop, kDecP chunks in flight
//     per lane, with no barrier until the share is done;
//   * the share's group scales (32 rows x K/128 bf16 per row block, contiguous
//     in the slot) are copied to LDS first, with the activation rows;
//   * each wave keeps one partial per (row block, row) in LDS; one barrier,
//     then each row block is summed over the 16 waves in a fixed order and
//     finished (activation scale, SwiGLU epilogue), so the result does not
//     depend on timing.
// Numerics are those of the int4 GEMV: per chunk the exact int32 dot of 16 q
// with the int8 row, times the group scale / 16, accumulated in fp32.
#include "common.h"
#include "decode_share.h"
#include "ffn_internal.h"
#include "tile_gemv.h"

namespace {

using namespace decode_share;

constexpr int kTokRegs = (8192 + 8 * kDecNW * 64 - 1) / (8 * kDecNW * 64);  // token row: K <= 8192

// SWIGLU (gate/up pass): one token row for every group (T = 1: row perm[p] / k of the bf16
// tokens is row 0 for every p, so its loads need neither the work list nor perm), out = h
// (fp32, row p, column n of rows 2n, 2n+1).
// Otherwise (down pass): row p of the fp32 h for each group; out = y (fp32).
// The workgroup's LDS of a pass: activation rows [SWIGLU ? 1 : n_items][K] int8, then the
// share's scales [MAXRB][32][K/128] bf16 (dynamic), and the fixed arrays below.
template <int MAXRB>
struct PassLds {
  int8_t* dyn;
  float* act_s;      // [kStreamMaxItems]
  float* wmax;       // [16]
  unsigned* row_max; // [kStreamMaxItems]
  float (*red)[MAXRB][32];  // [kDecNW]
};

// h handed between the workgroups of one launch goes through device-scope stores and loads
// (written through to, and read from, the level every XCD shares), so neither side needs an
// L2 writeback or invalidate; the counter is bumped only after the stores have completed.
__device__ __forceinline__ void store_h(float* p, float v, bool shared) {
  if (shared) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
__device__ __forceinline__ u32x4 load_h4(const float* p, bool shared) {
  if (!shared) return ld16(p);
  u32x4 r;
  r.x = __float_as_uint(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  r.y = __float_as_uint(__hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  r.z = __float_as_uint(__hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  r.w = __float_as_uint(__hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return r;
}

template <bool SWIGLU, int MAXRB>
__device__ __forceinline__ void decode_pass(
    const void* __restrict__ raw, const FfnItem* __restrict__ items, int n_items,
    const char* __restrict__ pool, size_t stride,
    size_t off_codes, size_t off_scales, int R, int K, int out_ld, float* __restrict__ out,
    const PassLds<MAXRB>& L, const PassSync& sy) {
  int8_t* lds = L.dyn;
  float* act_s = L.act_s;
  float* wmax = L.wmax;
  unsigned* row_max = L.row_max;
  float (*red)[MAXRB][32] = L.red;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rbi = R / 32, nkc = K / 64, G = K / 128;
  const int total_rb = n_items * rbi;
  int b0, b1;
  share_of(total_rb, b0, b1);
  const int nrb = b1 - b0;  // <= MAXRB (the launch checks)
  // an empty share (more workgroups than row blocks) has nothing to load, wait for or count
  if (nrb == 0) return;
  const size_t act_bytes = (size_t)(SWIGLU ? 1 : n_items) * K;
  int8_t* act_q = lds;
  uint16_t* sc_lds = reinterpret_cast<uint16_t*>(lds + ((act_bytes + 15) & ~(size_t)15));
  // this wave's K slice of every row block of the share, as one stream of chunks walked by
  // two cursors (the loads kDecP chunks ahead of the sums); all cursor state is uniform
  const int c0 = nkc * wave / kDecNW, c1 = nkc * (wave + 1) / kDecNW;
  const int nq = nrb * (c1 - c0);
  const int kh = 16 * (lane >> 5);
  struct Cursor {
    int r, c, item;
    const char* base;  // the row block's first chunk, this lane's 16 bytes
  };
  auto at_block = [&](Cursor& u, int r) {
    const int b = b0 + r, item = b / rbi, rb = b - item * rbi;
    u.r = r;
    u.c = c0;
    u.item = item;
    u.base = pool + (size_t)items[item].slot * stride + off_codes + (size_t)rb * nkc * 1024 + lane * 16;
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
  // the partial of row block r (after the K halves of a row meet) into LDS
  auto flush = [&](int r) {
    const float v = acc + __shfl_xor(acc, 32, 64);
    if (lane < 32) red[wave][r][lane] = v;
    acc = 0.f;
  };
  auto consume = [&](const u32x4& wv) {
    const int8_t* ap = act_q + (SWIGLU ? 0 : (size_t)sum_at.item * K) + (size_t)sum_at.c * 64 + kh;
    const u32x4 a0 = ld16(ap), a1 = ld16(ap + 32);
    const uint16_t sraw = sc_lds[((size_t)sum_at.r * 32 + (lane & 31)) * G + (sum_at.c >> 1)];
    acc = fmaf((float)tgemv::dot64_int4(wv, a0, a1), bf16_to_f32(sraw) * 0.0625f, acc);
    if (sum_at.c + 1 == c1) flush(sum_at.r);  // uniform: the row block's slice is done
    advance(sum_at);
  };
  // Vector loads return in issue order, so a wait for a value also waits for every load
  // issued before it. The loads the staging below needs (the share's scales, and the token
  // row of the gate/up pass) therefore go out first, then the first kDecP weight chunks,
  // which stay in flight while the staging waits for the earlier ones.
  // The share's scales: row block r's 64 G bytes, 16 bytes per thread, the first
  // kScaleRegs pieces of each thread held in registers until the staging.
  constexpr int kScaleRegs = 2;
  const int sbytes = 64 * G, per = sbytes / 16, nsc = nrb * per;
  auto scale_src = [&](int i, int& dst) {
    const int r = i / per, o = (i - r * per) * 16;
    const int b = b0 + r, item = b / rbi, rb = b - item * rbi;
    dst = r * sbytes + o;
    return pool + (size_t)items[item].slot * stride + off_scales + (size_t)rb * sbytes + o;
  };
  u32x4 sreg[kScaleRegs];
  int sdst[kScaleRegs];
  // These loads are issued by every lane (indexes past the end are clamped to valid ones,
  // whose values are not used), so the waits before their first use count only the loads
  // issued after them.
#pragma unroll
  for (int u = 0; u < kScaleRegs; ++u) {
    const int i = (int)threadIdx.x + u * (int)blockDim.x;
    sreg[u] = ld16(scale_src(i < nsc ? i : nsc - 1, sdst[u]));
  }
  // the token row (bf16; every group reads the same one): eight values per thread and register
  u32x4 tok[kTokRegs];
  if constexpr (SWIGLU) {
    const uint16_t* trow = static_cast<const uint16_t*>(raw);  // the one token
#pragma unroll
    for (int u = 0; u < kTokRegs; ++u) {
      const int e = ((int)threadIdx.x + u * (int)blockDim.x) * 8;
      tok[u] = ld16(trow + (e < K ? e : K - 8));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // nq > 0: a share has a row block and every wave a chunk of it (K / 64 >= 16 waves)
  u32x4 buf[kDecP];
  at_block(sum_at, 0);
  at_block(load_at, 0);
#pragma unroll
  for (int i = 0; i < kDecP; ++i) {
    buf[i] = ld16_stream(load_at.base + (size_t)load_at.c * 1024);
    advance(load_at);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < kScaleRegs; ++u) {
    const int i = (int)threadIdx.x + u * (int)blockDim.x;
    if (i < nsc) *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(sc_lds) + sdst[u]) = sreg[u];
  }
  for (int i = (int)threadIdx.x + kScaleRegs * (int)blockDim.x; i < nsc; i += blockDim.x) {
    int dst;
    const char* src = scale_src(i, dst);
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(sc_lds) + dst) = ld16(src);
  }
  // one launch: the h rows this share reads are complete once every row block of their
  // groups is counted (weights and scales above do not depend on them)
  if (sy.wait != nullptr) wait_groups(sy, b0 / rbi, (b1 - 1) / rbi);
  // the activation rows, quantised into LDS (same rule and codes as quant_rows_kernel)
  if constexpr (SWIGLU) {
    // the token row, held in registers (K <= 8 * kTokRegs * blockDim, which the launch checks): a
    // block-wide max, then the codes: s = max|v| / 127 (1 for a zero row),
    // q = clip(rint(v / s), -127, 127)
    {
      float v[kTokRegs][8];
      float amax = 0.f;
#pragma unroll
      for (int u = 0; u < kTokRegs; ++u) {
        const int e = ((int)threadIdx.x + u * (int)blockDim.x) * 8;
        if (e < K) {
          const uint32_t ww[4] = {tok[u].x, tok[u].y, tok[u].z, tok[u].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[u][2 * i] = __uint_as_float(ww[i] << 16);
            v[u][2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[u][i]));
        }
      }
      amax = wave_max(amax);
      if (lane == 0) wmax[wave] = amax;
      __syncthreads();
      float m = 0.f;
#pragma unroll
      for (int w = 0; w < kDecNW; ++w) m = fmaxf(m, wmax[w]);
      const float sc = (m == 0.f) ? 1.f : m / 127.f;
#pragma unroll
      for (int u = 0; u < kTokRegs; ++u) {
        const int e = ((int)threadIdx.x + u * (int)blockDim.x) * 8;
        if (e < K) {
          uint32_t w0 = 0, w1 = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float r = rintf(v[u][i] / sc);
            r = fminf(fmaxf(r, -127.f), 127.f);
            const uint32_t b = (uint32_t)((int)r & 0xFF);
            if (i < 4) w0 |= b << (8 * i); else w1 |= b << (8 * (i - 4));
          }
          *reinterpret_cast<uint2*>(act_q + e) = make_uint2(w0, w1);
        }
      }
      if (threadIdx.x == 0) act_s[0] = sc;
    }
  } else {
    // only the h rows of the share's groups (one or two for a large R): every thread loads
    // its float4s of those rows at once (a row-wide max through an LDS max over the float
    // bits, which order like the values for |v|), then quantises them from registers:
    // s = max|v| / 127 (1 for a zero row), q = clip(rint(v / s), -127, 127)
    const int i0 = b0 / rbi, nrow = (b1 - 1) / rbi - i0 + 1;
    const int q4 = K / 4, nv = nrow * q4;
    for (int r = threadIdx.x; r < nrow; r += blockDim.x) row_max[r] = 0u;
    __syncthreads();
    constexpr int NV = 4;  // float4 per thread held in registers
    const int nthr = blockDim.x;
    for (int base = 0; base < nv; base += NV * nthr) {
      u32x4 v[NV];
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int idx = base + u * nthr + (int)threadIdx.x;
        if (idx < nv) {
          const int r = idx / q4;
          v[u] = load_h4(static_cast<const float*>(raw) + (size_t)items[i0 + r].row_begin * K +
                         (size_t)(idx - r * q4) * 4, sy.wait != nullptr);
        }
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int idx = base + u * nthr + (int)threadIdx.x;
        if (idx < nv) {
          const float m = fmaxf(fmaxf(fabsf(__uint_as_float(v[u].x)), fabsf(__uint_as_float(v[u].y))),
                                fmaxf(fabsf(__uint_as_float(v[u].z)), fabsf(__uint_as_float(v[u].w))));
          atomicMax(&row_max[idx / q4], __float_as_uint(m));
        }
      }
      if (base + NV * nthr < nv) continue;  // more than one round: the codes read again below
      __syncthreads();
      for (int r = threadIdx.x; r < nrow; r += nthr) {
        const float amax = __uint_as_float(row_max[r]);
        act_s[i0 + r] = (amax == 0.f) ? 1.f : amax / 127.f;
      }
      if (base == 0) {  // one round: the values are still in registers
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          const int idx = u * nthr + (int)threadIdx.x;
          if (idx < nv) {
            const int r = idx / q4;
            const float amax = __uint_as_float(row_max[r]);
            const float sc = (amax == 0.f) ? 1.f : amax / 127.f;
            const float f[4] = {__uint_as_float(v[u].x), __uint_as_float(v[u].y),
                                __uint_as_float(v[u].z), __uint_as_float(v[u].w)};
            uint32_t word = 0;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              float rr = rintf(f[jj] / sc);
              rr = fminf(fmaxf(rr, -127.f), 127.f);
              word |= (uint32_t)((int)rr & 0xFF) << (8 * jj);
            }
            *reinterpret_cast<uint32_t*>(act_q + (size_t)(i0 + r) * K + (size_t)(idx - r * q4) * 4) = word;
          }
        }
      }
    }
    if (nv > NV * nthr) {
      // several rounds: the maxima are complete (the last round's barrier); quantise again
      for (int idx = threadIdx.x; idx < nv; idx += nthr) {
        const int r = idx / q4;
        const float amax = __uint_as_float(row_max[r]);
        const float sc = (amax == 0.f) ? 1.f : amax / 127.f;
        const u32x4 vv = load_h4(static_cast<const float*>(raw) + (size_t)items[i0 + r].row_begin * K +
                                 (size_t)(idx - r * q4) * 4, sy.wait != nullptr);
        const float f[4] = {__uint_as_float(vv.x), __uint_as_float(vv.y), __uint_as_float(vv.z),
                            __uint_as_float(vv.w)};
        uint32_t word = 0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float rr = rintf(f[jj] / sc);
          rr = fminf(fmaxf(rr, -127.f), 127.f);
          word |= (uint32_t)((int)rr & 0xFF) << (8 * jj);
        }
        *reinterpret_cast<uint32_t*>(act_q + (size_t)(i0 + r) * K + (size_t)(idx - r * q4) * 4) = word;
      }
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
    v *= act_s[SWIGLU ? 0 : item];
    const int row = rb * 32 + (lane & 31);
    if constexpr (SWIGLU) {
      const float u = __shfl_xor(v, 1, 64);  // odd row = up of the same neuron
      if (lane < 32 && (lane & 1) == 0)
        store_h(out + (size_t)it.row_begin * out_ld + (row >> 1), tgemv::silu(v) * u,
                sy.signal != nullptr);
    } else {
      if (lane < 32) out[(size_t)it.row_begin * out_ld + row] = v;
    }
  }
  if (sy.signal != nullptr) signal_groups(sy, b0, b1, rbi);
}

template <bool SWIGLU, int MAXRB>
__global__ __launch_bounds__(kDecNW * 64) __attribute__((amdgpu_waves_per_eu(4))) void int4_decode_kernel(
    const void* __restrict__ raw, const FfnItem* __restrict__ items,
    const int32_t* __restrict__ n_items_p,
    const char* __restrict__ pool, size_t stride, size_t off_codes, size_t off_scales, int R,
    int K, int out_ld, float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  __shared__ float act_s[kStreamMaxItems];
  __shared__ float wmax[16];
  __shared__ unsigned row_max[kStreamMaxItems];
  __shared__ float red[kDecNW][MAXRB][32];
  const PassLds<MAXRB> L{lds, act_s, wmax, row_max, red};
  decode_pass<SWIGLU, MAXRB>(raw, items, n_items_p[0], pool, stride, off_codes, off_scales,
                             R, K, out_ld, out, L, PassSync{nullptr, nullptr, 0, nullptr, 0});
}

// Both passes of a one-token call in one launch (one workgroup per compute unit, all
// resident): each workgroup runs its gate/up share, counts it per group, then its down
// share, whose weight loads and scale copies go out before it waits for the h rows.
template <int MAXRB>
__global__ __launch_bounds__(kDecNW * 64) __attribute__((amdgpu_waves_per_eu(4))) void
int4_decode_fused_kernel(
    const void* __restrict__ x, const FfnItem* __restrict__ items,
    const int32_t* __restrict__ n_items_p,
    const char* __restrict__ pool, size_t stride, size_t off_w13, size_t off_s13, size_t off_w2,
    size_t off_s2, int H, int F, float* __restrict__ hbuf, float* __restrict__ y,
    int32_t* __restrict__ sync, int32_t* __restrict__ err, int spin_cap) {
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  __shared__ float act_s[kStreamMaxItems];
  __shared__ float wmax[16];
  __shared__ unsigned row_max[kStreamMaxItems];
  __shared__ float red[kDecNW][MAXRB][32];
  const PassLds<MAXRB> L{lds, act_s, wmax, row_max, red};
  const int n_items = n_items_p[0];
  decode_pass<true, MAXRB>(x, items, n_items, pool, stride, off_w13, off_s13, 2 * F, H, F,
                           hbuf, L, PassSync{sync, nullptr, 0, err, spin_cap});
  __syncthreads();  // the LDS of the first pass is free
  decode_pass<false, MAXRB>(hbuf, items, n_items, pool, stride, off_w2, off_s2, H, F, H, y,
                            L, PassSync{nullptr, sync, 2 * F / 32, err, spin_cap});
}

template <bool SWIGLU, int MAXRB>
int launch_rb(const void* raw, const FfnItem* items,
              const int32_t* n_items, int max_items, const char* pool, size_t stride,
              size_t off_codes, size_t off_scales, int R, int K, int out_ld, float* out,
              hipStream_t s, long long grid, size_t lds) {
  hipLaunchKernelGGL((int4_decode_kernel<SWIGLU, MAXRB>), dim3((unsigned)grid), dim3(kDecNW * 64),
                     lds, s, raw, items, n_items, pool, stride, off_codes, off_scales, R,
                     K, out_ld, out);
  return moe_launch_status();
}

size_t decode_lds(bool swiglu, int max_items, int K, int maxrb) {
  const size_t act = (size_t)(swiglu ? 1 : max_items) * K;
  return ((act + 15) & ~(size_t)15) + (size_t)maxrb * 64 * (K / 128);
}

}  // namespace

bool decode_int4_fits(int max_items, int R, int K, bool swiglu) {
  if (max_items < 1 || max_items > kStreamMaxItems || R % 32 != 0 || K % 128 != 0 ||
      K / 64 < kDecNW || (swiglu && K > 8 * kTokRegs * kDecNW * 64))
    return false;
  return decode_lds(swiglu, max_items, K, 16) <= 96 * 1024;
}

int launch_decode_int4(bool swiglu, const void* raw, const FfnItem* items, const int32_t* n_items,
                       int max_items,
                       const char* pool, size_t stride, size_t off_codes, size_t off_scales, int R,
                       int K, int out_ld, float* out, hipStream_t s) {
  // the grid: the workgroups the compute units keep resident (16 waves of up to 128 VGPRs
  // per unit); every share has at most ceil(blocks / grid) <= MAXRB
  const int n = decode_cus();
  const long long blocks = (long long)max_items * (R / 32);
  long long grid = (long long)n * kDecWgPerCu;
  if (grid > blocks) grid = blocks;
  const long long per = (blocks + grid - 1) / grid;
  if (per <= 8)
    return swiglu ? launch_rb<true, 8>(raw, items, n_items, max_items, pool, stride,
                                       off_codes, off_scales, R, K, out_ld, out, s, grid,
                                       decode_lds(true, max_items, K, 8))
                  : launch_rb<false, 8>(raw, items, n_items, max_items, pool, stride,
                                        off_codes, off_scales, R, K, out_ld, out, s, grid,
                                        decode_lds(false, max_items, K, 8));
  if (per <= 16)
    return swiglu ? launch_rb<true, 16>(raw, items, n_items, max_items, pool, stride,
                                        off_codes, off_scales, R, K, out_ld, out, s, grid,
                                        decode_lds(true, max_items, K, 16))
                  : launch_rb<false, 16>(raw, items, n_items, max_items, pool, stride,
                                         off_codes, off_scales, R, K, out_ld, out, s, grid,
                                         decode_lds(false, max_items, K, 16));
  return MOE_EUNSUPPORTED;
}

int launch_decode_int4_fused(const void* x, const FfnItem* items,
                             const int32_t* n_items, int max_items, const char* pool,
                             size_t stride, size_t off_w13, size_t off_s13, size_t off_w2,
                             size_t off_s2, int H, int F, float* hbuf, float* y, int32_t* sync,
                             int32_t* err, hipStream_t s) {
  if (!decode_int4_fits(max_items, 2 * F, H, true) || !decode_int4_fits(max_items, H, F, false))
    return MOE_EUNSUPPORTED;
  const int n = decode_cus();
  // kDecWgPerCu workgroups per compute unit, exactly as many as fit on one (16 waves of at
  // most 128 VGPRs; the LDS request below admits no more), so the grid is resident at once
  // and every wait ends
  const long long b1 = (long long)max_items * (2 * F / 32), b2 = (long long)max_items * (H / 32);
  const long long grid = (long long)n * kDecWgPerCu;
  const long long per = ((b1 > b2 ? b1 : b2) + grid - 1) / grid;
  const int maxrb = per <= 8 ? 8 : 16;
  const size_t l1 = decode_lds(true, max_items, H, maxrb), l2 = decode_lds(false, max_items, F, maxrb);
  size_t lds = l1 > l2 ? l1 : l2;
  const size_t stat = sizeof(float) * (2 * kStreamMaxItems + 16 + (size_t)kDecNW * maxrb * 32);
  lds = resident_lds(lds, stat);
  if (lds == 0) return MOE_EUNSUPPORTED;
  if (per <= 8) {
    hipLaunchKernelGGL((int4_decode_fused_kernel<8>), dim3((unsigned)grid), dim3(kDecNW * 64), lds,
                       s, x, items, n_items, pool, stride, off_w13, off_s13, off_w2,
                       off_s2, H, F, hbuf, y, sync, err, kSpinCap);
    return moe_launch_status();
  }
  if (per <= 16) {
    hipLaunchKernelGGL((int4_decode_fused_kernel<16>), dim3((unsigned)grid), dim3(kDecNW * 64), lds,
                       s, x, items, n_items, pool, stride, off_w13, off_s13, off_w2,
                       off_s2, H, F, hbuf, y, sync, err, kSpinCap);
    return moe_launch_status();
  }
  return MOE_EUNSUPPORTED;
}
