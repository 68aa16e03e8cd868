// Grouped SwiGLU expert FFN over resident slots (moe_expert_ffn).
//
// Each routed expert group e (its rows [offsets[e], offsets[e+1]) of the
// permuted assignments) reads its weights through the slot table: slot =
// lut[e], weights at pool_base + slot * slot_stride (the fixed-base slot pool
// and expert_id -> slot_id table of the SeqMoE summary page, Mechanism). The
// expert is the SwiGLU FFN of "RapidMoE: Exploiting Cross-Asymmetry via
// Adaptive Residual Offloading for Large-Scale MoE Inference", Eq. (7):
// y = down(SiLU(gate x) * up x).
//
// Kernels (all enqueued on the caller's stream):
//   ffn_plan_kernel      one workgroup: compacts the selected, non-empty,
//                        resident groups into a work list in the workspace
//                        (ascending expert id) and flags absent experts.
//   ffn_w13_gemv_kernel  decode form of the first projection: each wave owns
//                        two neurons (their gate and up rows, interleaved in
//                        the slot) for one group and streams those rows once
//                        per tile of <= 8 tokens with 16-byte coalesced loads;
//                        fp32 FMA, wave reduction, SiLU(g) * u fused in the
//                        epilogue -> h [T*k, F] fp32 in the workspace.
//   ffn_w2_gemv_kernel   decode form of the down projection: each wave owns
//                        four output rows and streams them against h.
// The weights are read exactly once per token tile, so for decode groups
// (<= 8 rows) the passes are bound by HBM bandwidth on the weight bytes.
#include "common.h"
#include "ffn_internal.h"

namespace {

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

__device__ __forceinline__ float silu(float g) { return g / (1.f + expf(-g)); }

__global__ __launch_bounds__(1024) void ffn_plan_kernel(const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ lut,
                                                        const int32_t* __restrict__ mask, int E,
                                                        int num_slots,
                                                        FfnItem* __restrict__ items,
                                                        int32_t* __restrict__ n_items,
                                                        int32_t* __restrict__ err_word) {
  __shared__ int s_wave[16];
  const int e = threadIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int rows = 0, slot = -1, begin = 0;
  bool take = false;
  if (e < E) {
    begin = offsets[e];
    rows = offsets[e + 1] - begin;
    take = rows > 0 && (mask == nullptr || mask[e] != 0);
    if (take) {
      slot = lut[e];
      if (slot < 0 || slot >= num_slots) {
        atomicOr(err_word, MOE_ERR_ABSENT);
        take = false;
      }
    }
  }
  const uint64_t m = __ballot(take);
  if (lane == 0) s_wave[wave] = __popcll(m);
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += s_wave[w];
    total += s_wave[w];
  }
  if (take) {
    FfnItem it;
    it.expert = e;
    it.slot = slot;
    it.row_begin = begin;
    it.rows = rows;
    items[base + popc_below(m)] = it;
  }
  if (e == 0) n_items[0] = total;
}

// ------------------------------------------------------------ W13 (gate/up)
template <int WF, int XF, int NT>
__device__ __forceinline__ void w13_tile(const char* __restrict__ w13, const void* __restrict__ x,
                                         const int32_t* __restrict__ perm, int prow, int k, int H,
                                         int F, int n0, float* __restrict__ hbuf) {
  constexpr size_t esz = (WF == MOE_BF16) ? 2 : 4;
  const int lane = threadIdx.x & 63;
  int tok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) tok[t] = perm[prow + t] / k;
  float acc[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = 0.f;
  const size_t rowb = (size_t)H * esz;
  const char* r0 = w13 + (size_t)(2 * n0) * rowb;
  for (int c = lane * 8; c < H; c += 64 * 8) {
    float wv[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) load8<WF>(r0 + i * rowb, c, wv[i]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float xv[8];
      load8<XF>(x, (size_t)tok[t] * H + c, xv);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[i][t] = fmaf(wv[i][q], xv[q], acc[i][t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float g0 = wave_sum(acc[0][t]), u0 = wave_sum(acc[1][t]);
    const float g1 = wave_sum(acc[2][t]), u1 = wave_sum(acc[3][t]);
    if (lane == t) {
      float* hrow = hbuf + (size_t)(prow + t) * F;
      hrow[n0] = silu(g0) * u0;
      hrow[n0 + 1] = silu(g1) * u1;
    }
  }
}

template <int WF, int XF>
__global__ __launch_bounds__(256) void ffn_w13_gemv_kernel(const void* __restrict__ x,
                                                           const int32_t* __restrict__ perm, int k,
                                                           const FfnItem* __restrict__ items,
                                                           const int32_t* __restrict__ n_items,
                                                           const char* __restrict__ pool,
                                                           size_t stride, size_t off_w13, int H,
                                                           int F, float* __restrict__ hbuf) {
  if ((int)blockIdx.y >= n_items[0]) return;
  const FfnItem it = items[blockIdx.y];
  const int n0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 2;
  if (n0 >= F) return;
  const char* w13 = pool + (size_t)it.slot * stride + off_w13;
  int done = 0;
  for (; it.rows - done >= 8; done += 8)
    w13_tile<WF, XF, 8>(w13, x, perm, it.row_begin + done, k, H, F, n0, hbuf);
  const int p = it.row_begin + done;
  switch (it.rows - done) {
    case 1: w13_tile<WF, XF, 1>(w13, x, perm, p, k, H, F, n0, hbuf); break;
    case 2: w13_tile<WF, XF, 2>(w13, x, perm, p, k, H, F, n0, hbuf); break;
    case 3: w13_tile<WF, XF, 3>(w13, x, perm, p, k, H, F, n0, hbuf); break;
    case 4: w13_tile<WF, XF, 4>(w13, x, perm, p, k, H, F, n0, hbuf); break;
    case 5: w13_tile<WF, XF, 5>(w13, x, perm, p, k, H, F, n0, hbuf); break;
    case 6: w13_tile<WF, XF, 6>(w13, x, perm, p, k, H, F, n0, hbuf); break;
    case 7: w13_tile<WF, XF, 7>(w13, x, perm, p, k, H, F, n0, hbuf); break;
    default: break;
  }
}

// ---------------------------------------------------------------- W2 (down)
template <int WF, int NT>
__device__ __forceinline__ void w2_tile(const char* __restrict__ w2, const float* __restrict__ hbuf,
                                        int prow, int H, int F, int r0, float* __restrict__ y) {
  constexpr size_t esz = (WF == MOE_BF16) ? 2 : 4;
  const int lane = threadIdx.x & 63;
  float acc[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = 0.f;
  const size_t rowb = (size_t)F * esz;
  const char* rr = w2 + (size_t)r0 * rowb;
  for (int c = lane * 8; c < F; c += 64 * 8) {
    float wv[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) load8<WF>(rr + i * rowb, c, wv[i]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float hv[8];
      load8<MOE_F32>(hbuf, (size_t)(prow + t) * F + c, hv);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[i][t] = fmaf(wv[i][q], hv[q], acc[i][t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = wave_sum(acc[i][t]);
    if (lane == t) {
      float* yrow = y + (size_t)(prow + t) * H + r0;
#pragma unroll
      for (int i = 0; i < 4; ++i) yrow[i] = s[i];
    }
  }
}

template <int WF>
__global__ __launch_bounds__(256) void ffn_w2_gemv_kernel(const float* __restrict__ hbuf,
                                                          const FfnItem* __restrict__ items,
                                                          const int32_t* __restrict__ n_items,
                                                          const char* __restrict__ pool,
                                                          size_t stride, size_t off_w2, int H, int F,
                                                          float* __restrict__ y) {
  if ((int)blockIdx.y >= n_items[0]) return;
  const FfnItem it = items[blockIdx.y];
  const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4;
  if (r0 >= H) return;
  const char* w2 = pool + (size_t)it.slot * stride + off_w2;
  int done = 0;
  for (; it.rows - done >= 8; done += 8) w2_tile<WF, 8>(w2, hbuf, it.row_begin + done, H, F, r0, y);
  const int p = it.row_begin + done;
  switch (it.rows - done) {
    case 1: w2_tile<WF, 1>(w2, hbuf, p, H, F, r0, y); break;
    case 2: w2_tile<WF, 2>(w2, hbuf, p, H, F, r0, y); break;
    case 3: w2_tile<WF, 3>(w2, hbuf, p, H, F, r0, y); break;
    case 4: w2_tile<WF, 4>(w2, hbuf, p, H, F, r0, y); break;
    case 5: w2_tile<WF, 5>(w2, hbuf, p, H, F, r0, y); break;
    case 6: w2_tile<WF, 6>(w2, hbuf, p, H, F, r0, y); break;
    case 7: w2_tile<WF, 7>(w2, hbuf, p, H, F, r0, y); break;
    default: break;
  }
}

template <int WF, int XF>
void launch_dense(const void* x, const int32_t* perm, int k, const FfnItem* items,
                  const int32_t* n_items, const char* pool, size_t stride, const SlotLayout& lay,
                  int H, int F, int max_items, float* hbuf, float* y, hipStream_t s) {
  hipLaunchKernelGGL((ffn_w13_gemv_kernel<WF, XF>), dim3((F / 2 + 3) / 4, max_items), dim3(256), 0,
                     s, x, perm, k, items, n_items, pool, stride, lay.off_w13, H, F, hbuf);
  hipLaunchKernelGGL((ffn_w2_gemv_kernel<WF>), dim3((H / 4 + 3) / 4, max_items), dim3(256), 0, s,
                     hbuf, items, n_items, pool, stride, lay.off_w2, H, F, y);
}

}  // namespace

FfnWorkspace ffn_workspace_layout(int T, int H, int F, int E, int k, int w_dtype) {
  FfnWorkspace w{};
  const size_t rows = (size_t)T * k;
  size_t off = 256;  // n_items at offset 0
  w.items = off;
  off = align_up(off + (size_t)E * sizeof(FfnItem), 256);
  w.h = off;
  off = align_up(off + rows * F * sizeof(float), 256);
  if (w_dtype == MOE_INT4G128) {
    w.xq = off;
    off = align_up(off + (size_t)T * H, 256);
    w.xs = off;
    off = align_up(off + (size_t)T * sizeof(float), 256);
    w.hq = off;
    off = align_up(off + rows * F, 256);
    w.hs = off;
    off = align_up(off + rows * sizeof(float), 256);
  }
  w.total = off;
  return w;
}

extern "C" size_t moe_ffn_workspace_bytes(int T, int H, int F, int E, int k, int w_dtype) {
  if (T < 0 || H <= 0 || F <= 0 || E <= 0 || k <= 0) return 0;
  return ffn_workspace_layout(T, H, F, E, k, w_dtype).total;
}

extern "C" int moe_expert_ffn(const void* x, int x_dtype, const int32_t* perm,
                              const int32_t* offsets, const int32_t* lut,
                              const int32_t* group_mask, const void* pool_base, size_t slot_stride,
                              int num_slots, int w_dtype, int T, int H, int F, int E, int k, float* y_perm,
                              int32_t* err_word, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
  MOE_CHECK_ARG(T >= 0 && k >= 1 && k <= E && E <= 1024);
  MOE_CHECK_ARG(x_dtype == MOE_F32 || x_dtype == MOE_BF16);
  SlotLayout lay;
  if (slot_layout(H, F, w_dtype, &lay) != MOE_OK) return MOE_EINVAL;
  MOE_CHECK_ARG(slot_stride >= lay.slot_bytes && slot_stride % 256 == 0 && num_slots >= 1);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(x && perm && offsets && lut && pool_base && y_perm && err_word && workspace);
  MOE_CHECK_ARG(((uintptr_t)x % 16) == 0 && ((uintptr_t)pool_base % 256) == 0);
  const FfnWorkspace ws = ffn_workspace_layout(T, H, F, E, k, w_dtype);
  MOE_CHECK_ARG(ws_bytes >= ws.total && ((uintptr_t)workspace % 256) == 0);
  if (w_dtype == MOE_INT4G128) return MOE_EUNSUPPORTED;

  char* wsb = static_cast<char*>(workspace);
  int32_t* n_items = reinterpret_cast<int32_t*>(wsb);
  FfnItem* items = reinterpret_cast<FfnItem*>(wsb + ws.items);
  float* hbuf = reinterpret_cast<float*>(wsb + ws.h);
  const long long tk = (long long)T * k;
  const int max_items = (int)(tk < E ? tk : E);
  MOE_CHECK_ARG(max_items <= 65535);

  hipLaunchKernelGGL(ffn_plan_kernel, dim3(1), dim3(1024), 0, stream, offsets, lut, group_mask, E,
                     num_slots, items, n_items, err_word);
  const char* pool = static_cast<const char*>(pool_base);
  if (w_dtype == MOE_BF16 && x_dtype == MOE_BF16)
    launch_dense<MOE_BF16, MOE_BF16>(x, perm, k, items, n_items, pool, slot_stride, lay, H, F,
                                     max_items, hbuf, y_perm, stream);
  else if (w_dtype == MOE_BF16 && x_dtype == MOE_F32)
    launch_dense<MOE_BF16, MOE_F32>(x, perm, k, items, n_items, pool, slot_stride, lay, H, F,
                                    max_items, hbuf, y_perm, stream);
  else if (w_dtype == MOE_F32 && x_dtype == MOE_F32)
    launch_dense<MOE_F32, MOE_F32>(x, perm, k, items, n_items, pool, slot_stride, lay, H, F,
                                   max_items, hbuf, y_perm, stream);
  else
    launch_dense<MOE_F32, MOE_BF16>(x, perm, k, items, n_items, pool, slot_stride, lay, H, F,
                                    max_items, hbuf, y_perm, stream);
  return moe_launch_status();
}
