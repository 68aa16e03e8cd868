// Weighted scatter-combine of the routed experts' outputs (moe_combine).
//
// out[t] = sum_j w[t,j] * y_perm[inv[t*k+j]] + sum_s shared_y[s,t]: the
// weighted sum over the selected experts of "RapidMoE: Exploiting
// Cross-Asymmetry via Adaptive Residual Offloading for Large-Scale MoE
// Inference" (Sec. 2.1, Algorithm 1) and of "Communication-Aware Placement and
// Pruning for Efficient Mixture-of-Experts Inference" (Eq. (1)), plus the
// always-on shared experts with weight 1. Each thread owns 4 consecutive
// hidden values of one token and gathers the k rows in fixed j order (fp32,
// no atomics: bitwise deterministic). A zero weight skips its row.
#include "common.h"

namespace {

constexpr int kCombineBatch = 8;  // rows of a token whose loads are in flight together
constexpr int kSharedRegs = 2;    // shared-expert rows loaded ahead of the routed ones

template <int OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int T, int k,
                                                      int H, const float* __restrict__ shared,
                                                      int n_shared, void* __restrict__ out) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  // the shared experts' rows do not depend on the routing: the first kSharedRegs go out
  // before the routed rows (they are still added after them, in s order)
  u32x4 sv[kSharedRegs];
#pragma unroll
  for (int s = 0; s < kSharedRegs; ++s)
    if (s < n_shared) sv[s] = ld16(shared + ((size_t)s * T + t) * H + c);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  // kCombineBatch rows at a time: every row of the batch is loaded (an index past k reads row
  // k - 1 again, unused) before the first is summed, so a token costs one memory round trip
  // per batch rather than one per row; the sums keep the fixed j order
  for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
    u32x4 v[kCombineBatch];
    float wb[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int j = j0 + u < k ? j0 + u : k - 1;
      wb[u] = w[(size_t)t * k + j];
      v[u] = ld16(y + (size_t)inv[(size_t)t * k + j] * H + c);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the batch out before the first sum
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      // a row past k or of zero weight leaves the sums as they are (selects, not branches,
      // so that no load is moved behind one)
      const bool use = j0 + u < k && wb[u] != 0.f;
      const float f0 = fmaf(wb[u], __uint_as_float(v[u].x), a0);
      const float f1 = fmaf(wb[u], __uint_as_float(v[u].y), a1);
      const float f2 = fmaf(wb[u], __uint_as_float(v[u].z), a2);
      const float f3 = fmaf(wb[u], __uint_as_float(v[u].w), a3);
      a0 = use ? f0 : a0;
      a1 = use ? f1 : a1;
      a2 = use ? f2 : a2;
      a3 = use ? f3 : a3;
    }
  }
  auto add_shared = [&](const u32x4& v) {
    a0 += __uint_as_float(v.x);
    a1 += __uint_as_float(v.y);
    a2 += __uint_as_float(v.z);
    a3 += __uint_as_float(v.w);
  };
#pragma unroll
  for (int s = 0; s < kSharedRegs; ++s)
    if (s < n_shared) add_shared(sv[s]);
  for (int s = kSharedRegs; s < n_shared; ++s) add_shared(ld16(shared + ((size_t)s * T + t) * H + c));
  if constexpr (OUT == MOE_BF16) {
    uint16_t* o = static_cast<uint16_t*>(out) + (size_t)t * H + c;
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(a2) | ((uint32_t)f32_to_bf16_rne(a3) << 16);
    *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
  } else {
    float* o = static_cast<float*>(out) + (size_t)t * H + c;
    *reinterpret_cast<float4*>(o) = make_float4(a0, a1, a2, a3);
  }
}

}  // namespace

extern "C" int moe_combine(const float* y_perm, const int32_t* inv, const float* topk_w, int T,
                           int k, int H, const float* shared_y, int n_shared, void* out,
                           int out_dtype, hipStream_t stream) {
  MOE_CHECK_ARG(T >= 0 && k >= 1 && H > 0 && H % 4 == 0);
  MOE_CHECK_ARG(out_dtype == MOE_F32 || out_dtype == MOE_BF16);
  if (shared_y == nullptr) n_shared = 0;
  MOE_CHECK_ARG(n_shared >= 0);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(y_perm && inv && topk_w && out);
  MOE_CHECK_ARG(((uintptr_t)y_perm % 16) == 0 && ((uintptr_t)out % 16) == 0);
  MOE_CHECK_ARG(shared_y == nullptr || ((uintptr_t)shared_y % 16) == 0);
  MOE_CHECK_ARG(T <= 65535);
  const dim3 grid((H / 4 + 255) / 256, T);
  if (out_dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<MOE_BF16>, grid, dim3(256), 0, stream, y_perm, inv, topk_w,
                       T, k, H, shared_y, n_shared, out);
  else
    hipLaunchKernelGGL(combine_kernel<MOE_F32>, grid, dim3(256), 0, stream, y_perm, inv, topk_w, T,
                       k, H, shared_y, n_shared, out);
  return moe_launch_status();
}
