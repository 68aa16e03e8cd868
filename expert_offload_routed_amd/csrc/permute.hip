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
//   permute_rank_kernel (one workgroup of 8 waves per expert): a token picks
//     an expert at most once, so an expert's rows are the tokens that picked
//     it in ascending order, which is the order of the flat index t * k + j of
//     the picks. The workgroup walks the flat ids in rounds of 8 x 64 x 64
//     entries, each wave a contiguous 4096 of them, 64 a load: first every
//     lane keeps one bit per load ("this entry is the expert") and the wave
//     counts them; after a barrier each wave starts at the expert's offset
//     plus the counts of the waves before it, and a ballot of the kept bits
//     and the popcount of the lanes below give each row its rank.
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
  for (int i0 = 0; i0 < n; i0 += 8 * 1024) {  // 8 loads in flight per thread
    int ev[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 1024 + tid;
      ev[u] = i < n ? ids[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (ev[u] >= 0 && ev[u] < E) atomicAdd(&s_cnt[ev[u]], 1);
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

constexpr int kRankWaves = 8;
constexpr int kRankLoads = 64;  // loads of 64 entries per wave and round (one bit each per lane)

__global__ __launch_bounds__(64 * kRankWaves) void permute_rank_kernel(
    const int32_t* __restrict__ ids, long long n, int E, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int s_n[kRankWaves];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x;
  const int cnt = counts[e];
  if (cnt == 0) return;  // the same for the whole workgroup
  int base = offsets[e];
  const int end = base + cnt;
  constexpr long long kRound = (long long)kRankWaves * kRankLoads * 64;
  for (long long r0 = 0; r0 < n; r0 += kRound) {
    const int32_t* blk = ids + r0;
    const int rem = (int)(n - r0 < kRound ? n - r0 : kRound);  // entries of this round
    const int l0 = wave * kRankLoads * 64 + lane;
    // loads of this wave that reach entries of the round (the same for all its lanes)
    const int first = wave * kRankLoads * 64;
    const int nl = rem <= first ? 0 : min(kRankLoads, (rem - first + 63) / 64);
    uint64_t mine = 0;  // bit i: entry r0 + l0 + 64 i is this expert
    for (int i0 = 0; i0 < nl; i0 += 16) {
      int v[16];  // 16 loads in flight (entries past the round's end read its last entry)
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int l = l0 + 64 * (i0 + u);
        v[u] = blk[l < rem ? l : rem - 1];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
        mine |= (uint64_t)(l0 + 64 * (i0 + u) < rem && v[u] == e) << (i0 + u);
    }
    const int cw = wave_sum_int(__popcll(mine));
    if (lane == 0) s_n[wave] = cw;
    __syncthreads();
    int pos = base, total = 0;
#pragma unroll
    for (int v = 0; v < kRankWaves; ++v) {
      const int c = s_n[v];
      pos += v < wave ? c : 0;
      total += c;
    }
    for (int i = 0; i < nl; ++i) {
      const bool hit = (mine >> i) & 1;
      const uint64_t m = __ballot(hit);
      if (hit) {
        const int p = pos + popc_below(m);
        const long long f = r0 + l0 + 64 * i;
        perm[p] = (int32_t)f;
        inv[f] = p;
      }
      pos += __popcll(m);
    }
    base += total;
    if (base >= end) break;  // every row of the expert is placed (the same for all waves)
    __syncthreads();         // s_n is rewritten by the next round
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
    hipLaunchKernelGGL(permute_rank_kernel, dim3(E), dim3(64 * kRankWaves), 0, stream, topk_ids,
                       (long long)T * k, E, counts, offsets, perm, inv);
  return moe_launch_status();
}
