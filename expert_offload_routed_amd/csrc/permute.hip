// Stable counting sort of the T*k routing assignments by expert (moe_permute).
//
// The expert kernel reads each expert's rows as one contiguous group, the
// layout the SeqMoE summary page (Mechanism) keeps fixed for the fused expert
// kernel. Integer work only; every output is deterministic.
//
//   permute_count_kernel (one workgroup of 1024 threads): LDS histogram of the
//     ids (integer atomics: the counts do not depend on their order), then a
//     block-wide exclusive scan for the offsets and a second scan that
//     compacts the experts with a non-zero count.
//   permute_rank_kernel (one wave per expert): a token picks an expert at most
//     once, so an expert's rows are the tokens that picked it in ascending
//     order. The wave walks the tokens 64 at a time; a ballot of "picked this
//     expert" and the popcount of the lanes below give each row its rank.
#include "common.h"

namespace {

__global__ __launch_bounds__(1024) void permute_count_kernel(const int32_t* __restrict__ ids, int n,
                                                             int E, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ distinct,
                                                             int32_t* __restrict__ n_distinct) {
  __shared__ int s_cnt[1024];
  __shared__ int s_wave[40];
  const int tid = threadIdx.x;
  s_cnt[tid] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  const int c = (tid < E) ? s_cnt[tid] : 0;
  int total = 0, nd = 0;
  const int off = block_exclusive_scan(c, s_wave, &total);
  const int pos = block_exclusive_scan(c > 0 ? 1 : 0, s_wave, &nd);
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = off;
    if (c > 0) distinct[pos] = tid;
  }
  if (tid == 0) {
    offsets[E] = total;
    n_distinct[0] = nd;
  }
}

__global__ __launch_bounds__(256) void permute_rank_kernel(const int32_t* __restrict__ ids, int T,
                                                           int k, int E,
                                                           const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  if (e >= E) return;
  const int cnt = counts[e];
  if (cnt == 0) return;
  int pos = offsets[e];
  const int end = pos + cnt;
  for (int t0 = 0; t0 < T && pos < end; t0 += 64) {
    const int t = t0 + lane;
    int jf = -1;
    if (t < T) {
      const int32_t* row = ids + (size_t)t * k;
      for (int j = 0; j < k; ++j)
        if (row[j] == e) jf = j;
    }
    const uint64_t m = __ballot(jf >= 0);
    if (jf >= 0) {
      const int p = pos + popc_below(m);
      const int f = t * k + jf;
      perm[p] = f;
      inv[f] = p;
    }
    pos += __popcll(m);
  }
}

}  // namespace

extern "C" int moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* distinct,
                           int32_t* n_distinct, hipStream_t stream) {
  MOE_CHECK_ARG(T >= 0 && k >= 1 && k <= E && E <= 1024);
  MOE_CHECK_ARG((long long)T * k < (1ll << 31));
  MOE_CHECK_ARG(counts && offsets && distinct && n_distinct);
  MOE_CHECK_ARG(T == 0 || (topk_ids && perm && inv));
  hipLaunchKernelGGL(permute_count_kernel, dim3(1), dim3(1024), 0, stream, topk_ids, T * k, E,
                     counts, offsets, distinct, n_distinct);
  if (T > 0)
    hipLaunchKernelGGL(permute_rank_kernel, dim3((E + 3) / 4), dim3(256), 0, stream, topk_ids, T,
                       k, E, counts, offsets, perm, inv);
  return moe_launch_status();
}
