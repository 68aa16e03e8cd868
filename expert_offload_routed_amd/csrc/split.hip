// Step scores and the critical-expert split of split-precision experts.
//
// "RapidMoE: Exploiting Cross-Asymmetry via Adaptive Residual Offloading for
// Large-Scale MoE Inference" routes the experts of a step to two precisions
// (Algorithm 1): an expert whose gating score reaches the threshold of Eqs.
// (3)-(5), Theta * beta(l) * gamma(t), is critical and runs on its
// high-precision weights W^H; the others run on W^L. With several tokens the
// score of an expert is its router probability averaged over the tokens.
// moe_step_scores computes that score; moe_critical_split turns it into the
// group mask moe_expert_ffn reads for MOE_INT4G128_RESPLIT weights.
#include <math.h>

#include "common.h"
#include "ffn_internal.h"

namespace {

// Routing score of every expert at one step: its softmax probability over the
// step's tokens, averaged over the tokens (the score the eviction policies
// record). One workgroup of 16 waves; wave w takes tokens w, w + 16, ...;
// the per-wave partial sums meet in LDS in wave order.
constexpr int kScoreWaves = 16;
__global__ __launch_bounds__(kScoreWaves * 64) void step_scores_kernel(const float* __restrict__ logits,
                                                                      int T, int E, float* out) {
  __shared__ float part[kScoreWaves][1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kPer = 1024 / 64;  // experts per lane (E <= 1024)
  float acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
  for (int t = wave; t < T; t += kScoreWaves) {
    const float* row = logits + (size_t)t * E;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + 64 * i;
      if (e < E) m = fmaxf(m, row[e]);
    }
    m = wave_max(m);
    float v[kPer], sum = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? expf(row[e] - m) : 0.f;
      sum += v[i];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] += v[i] / sum;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) part[wave][lane + 64 * i] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kScoreWaves * 64) {
    float s = 0.f;
    for (int w = 0; w < kScoreWaves; ++w) s += part[w][e];
    out[e] = s / (float)T;
  }
}

__global__ __launch_bounds__(256) void critical_split_kernel(const float* __restrict__ scores, int E,
                                                             float threshold,
                                                             const int32_t* __restrict__ mask_in,
                                                             int n, int32_t* __restrict__ mask_out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int e = i % E;
  const bool on = mask_in == nullptr || mask_in[i] != 0;
  mask_out[i] = on ? (scores[e] >= threshold ? 2 : 1) : 0;
}

}  // namespace

void launch_step_scores(const float* logits, int T, int E, float* scores, hipStream_t s) {
  hipLaunchKernelGGL(step_scores_kernel, dim3(1), dim3(kScoreWaves * 64), 0, s, logits, T, E,
                     scores);
}

extern "C" int moe_step_scores(const float* logits, int T, int E, float* scores,
                               hipStream_t stream) {
  MOE_CHECK_ARG(T >= 1 && E >= 1 && E <= 1024 && logits && scores);
  launch_step_scores(logits, T, E, scores, stream);
  return moe_launch_status();
}

void launch_critical_split(const float* scores, int E, float threshold, const int32_t* mask_in,
                           int rows, int32_t* mask_out, hipStream_t s) {
  const int n = rows * E;
  hipLaunchKernelGGL(critical_split_kernel, dim3((n + 255) / 256), dim3(256), 0, s, scores, E,
                     threshold, mask_in, n, mask_out);
}

extern "C" int moe_critical_split(const float* scores, int E, float threshold,
                                  const int32_t* mask_in, int rows, int32_t* mask_out,
                                  hipStream_t stream) {
  MOE_CHECK_ARG(E >= 1 && rows >= 1 && scores && mask_out);
  MOE_CHECK_ARG((long long)rows * E <= INT32_MAX);
  launch_critical_split(scores, E, threshold, mask_in, rows, mask_out, stream);
  return moe_launch_status();
}
