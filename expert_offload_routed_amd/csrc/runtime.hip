// Layer runtime: one routed-expert MoE layer step over the slot cache, in C++.
//
// Order of a step (all on the caller's compute stream unless noted):
//   moe_route_permute (route + permute; one launch for decode batches), which
//   stores the distinct routed set straight into mapped pinned host memory ->
//   moe_plan_fills on the host tables -> one copy of the wave masks
//   -> moe_expert_ffn over the groups that are already resident, while the
//   misses are copied from the pinned host store on the fill stream and
//   committed with their tags -> moe_expert_ffn over each wave of filled
//   groups -> moe_combine. The shared experts sit in the n_shared slots after
//   the S routed ones and ride along as extra groups of the first expert FFN
//   call of the step (T rows each, placed after the T*k routed rows), so a
//   step plans and streams its weights once.
// The routed set is known only after the router ran (SeqMoE and HybriMoE
// summary pages, Problem), so a step whose layer may miss waits for that copy:
// the one host synchronisation of a step. When every expert of the layer is
// resident no residency decision can change, so the step does not wait: the
// routed set lands in a ring of pinned buffers and its LRU bookkeeping (clock
// and last use, with no fills) is replayed in step order before the next plan
// that needs the tables.
// Device orchestration (moe_ctx_set_orchestration): the GPU plans and fills by
// itself, so a step never waits for the host (SeqMoE summary page, Mechanism:
// the device owns the cache metadata and starts the miss copy from a kernel,
// out of the pinned, mapped host pool). One workgroup runs the same LRU plan on
// the device tables, keeping the slots in (last use, slot id) order; a copy
// kernel reads the missed experts from the mapped host store into their slots;
// the expert FFN and the combine follow on the same stream.
// The context allocates its pinned host staging and events once, at creation
// (the staging buffers' events on the first staging enable); every device buffer,
// the device planner's tables included, lives in the caller's workspace, and a
// step allocates nothing.
#include <limits.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <cmath>
#include <vector>

#include "common.h"
#include "ffn_internal.h"
#include "moe_runtime.h"

namespace {
constexpr int kRing = 64;  // deferred routed sets (and timing event pairs) in flight
constexpr int kDevMrsMaxW = 16;  // eviction-score window the device planner keeps state for
}

struct moe_layer_ctx {
  // configuration
  int t_max, H, F, E, k, L, S, x_dtype, w_dtype, n_shared;
  char* pool;
  size_t stride;
  int32_t* lut;
  int32_t* owner;
  uint64_t* tags;
  const char* host_store;
  std::vector<int32_t> blob_of;
  int32_t* err;
  hipStream_t cs, fs;
  // device buffers (inside the caller's workspace)
  float* logits;
  int32_t* ids;
  float* topw;
  int32_t *counts, *offsets, *perm, *inv, *dist;  // dist: distinct[E] then n_distinct
  uint32_t* sync;  // counter of the one-launch decode front end
  float* y_perm;
  char* ws;
  size_t ws_bytes;
  int32_t* masks;
  float* scores;  // [E] routing scores of the latest step (split precision)
  int32_t* crit;  // [E] group precision of a fully resident step (split precision)
  int sh_T;  // T the shared groups' rows (perm and offsets tails) were written for
  // host state
  int32_t* ring_h;  // pinned [kRing][2E+1]: per step the routed set [E], its size, and the
                    // experts' routing scores [E] (float), written by the device
  int32_t* ring_d;  // device address of ring_h
  hipEvent_t ring_ev[kRing];
  int ring_layer[kRing];
  int ring_head, ring_count;  // deferred entries: ring_head .. ring_head + count - 1
  int ring_next;              // next ring entry to use
  int32_t* masks_h;    // pinned [(E+2)*E]
  int32_t* sh_rows_h;  // pinned [t_max*n_shared + n_shared]: tails of perm and offsets
  std::vector<int32_t> lut_h, owner_h, resident;  // resident[l]: experts of layer l in the pool
  std::vector<int64_t> last_use;
  int64_t clock;
  // eviction policy (moe_ctx_set_policy): LRU unless set
  int policy, window;
  double params[5];
  std::vector<double> pol_state;
  int last_ring;  // ring entry of the latest step
  // split-precision experts (moe_ctx_set_split): thresholds per layer
  int split;
  std::vector<float> split_th;
  // prefill full-layer staging (moe_ctx_set_staging): two buffers of E slots each
  int stage;               // 0: off; 1: steps with T >= the layer's threshold are staged
  int stage_thr;           // token threshold; -1: floor(resident slots of the layer / k)
  int stage_slot0;         // first staging slot: buffer b holds expert e in slot0 + b*E + e
  int32_t* d_stage_lut;    // [2E] device: those slots, one expert->slot row per buffer
  bool stage_ready;        // the table is written and the events exist
  int buf_layer[2];        // layer each buffer holds (or is loading); -1: none
  int buf_last;            // buffer of the latest staged step
  hipEvent_t ev_ready[2];  // the buffer's load finished (fill stream)
  hipEvent_t ev_free[2];   // the last compute that read the buffer finished (compute stream)
  int64_t stage_steps, stage_copies;
  int next_hint;           // layer of the next step (moe_ctx_forward_steps); -1: layer + 1
  // device orchestration (moe_ctx_set_orchestration)
  int orch;                 // 0: plans on the host; 1: plans and fills on the device
  bool orch_ready;          // d_blob is written (the tables below live in the workspace)
  const char* store_dev;    // device address of the pinned host store
  int32_t* d_order;         // [S] slots by (last use, slot id)
  int64_t* d_last_use;      // [S]
  int64_t* d_clock;         // [1]
  int32_t* d_blob;          // [L*E] weight set of each layer-expert
  int32_t* d_fills;         // [2E] (expert, slot) of the step's fills
  int32_t* d_nfills;        // [1]
  int64_t* d_counters;      // [4] as totals, since the last handoff to the host
  double* d_pol;            // eviction-score state of the device planner (host layout)
  uint64_t next_tag;
  std::vector<int32_t> wave_of, is_hit, fill_e, fill_s, fill_w;
  std::vector<uint64_t> fill_tag;  // tag of each fill of the step
  hipEvent_t ev_fill, ev_compute;
  int64_t totals[4];  // over completed plans: distinct, hits, fills, waves
  // miss prefetch (moe_ctx_set_prefetch): the next step's layer and router (given by
  // moe_ctx_forward_steps), the overlap window and bandwidth, the speculative routing
  int prefetch;
  double pf_window_us, pf_bw_gbs;
  const void* next_wr;
  const float* next_bias;
  float* spec_logits;  // device [t_max*E]
  int32_t* spec_ids;   // device [t_max*k]
  float* spec_w;       // device [t_max*k]
  float* spec_scores;  // device [E]
  int32_t* spec_h;     // pinned [t_max*k] predicted ids, then [E] predicted scores (float)
  hipEvent_t ev_pf_before;             // compute before the current step's expert FFN
  std::vector<char> pf_pending;        // [L*E] prefetched, not yet planned by its layer
  std::vector<int32_t> pf_e, pf_s;     // the latest prefetch's experts and slots
  std::vector<uint64_t> pf_tag;
  int64_t pf_issued, pf_used;
  // timing of the expert FFN calls of a step: one event pair per step, collected lazily
  int timing;
  hipEvent_t tev0[kRing], tev1[kRing];
  int t_head, t_count;
  double ffn_ms;
  long ffn_calls;
};

namespace {

// Device work buffers of a context, carved from the caller's workspace.
struct CtxLayout {
  size_t sync, logits, ids, topw, counts, offsets, perm, inv, dist, y_perm, ws, masks, scores, crit,
      total;
  size_t ws_bytes;
  // device orchestration's tables and staging's slot table (used only once switched on)
  size_t order, last_use, clock, blob, fills, nfills, counters, stage_lut, pol;
  // the prefetch's speculative routing of the next layer
  size_t spec_logits, spec_ids, spec_w, spec_scores;
};

CtxLayout ctx_layout(int t_max, int H, int F, int E, int k, int L, int S, int w_dtype,
                     int n_shared) {
  CtxLayout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + (bytes ? bytes : 1), 256);
    return at;
  };
  const size_t tk = (size_t)t_max * k;
  const size_t rows = (size_t)t_max * (k + n_shared);  // routed rows, then shared rows
  l.sync = take(4);
  l.logits = take((size_t)t_max * E * 4);
  l.ids = take(tk * 4);
  l.topw = take(tk * 4);
  l.counts = take((size_t)E * 4);
  l.offsets = take((size_t)(E + n_shared + 1) * 4);
  l.perm = take(rows * 4);
  l.inv = take(tk * 4);
  l.dist = take((size_t)(E + 1) * 4);
  l.y_perm = take(rows * H * 4);
  l.ws_bytes = ffn_workspace_layout(t_max, H, F, E, k, w_dtype, n_shared).total;
  l.ws = take(l.ws_bytes);
  l.masks = take((size_t)(E + 2) * E * 4);
  l.scores = take((size_t)E * 4);
  l.crit = take((size_t)E * 4);
  l.order = take((size_t)S * 4);
  l.last_use = take((size_t)S * 8);
  l.clock = take(8);
  l.blob = take((size_t)L * E * 4);
  l.fills = take(2 * (size_t)E * 4);
  l.nfills = take(4);
  l.counters = take(4 * 8);
  l.stage_lut = take(2 * (size_t)E * 4);
  // the eviction-score state in the host layout (moe_policy_state_doubles), W <= kDevMrsMaxW:
  // per layer [observed steps, ring of W vectors, keep scores], and for the routing-history
  // score three more vectors (ema, latest score, step of the last selection) before keep
  l.pol = take((size_t)L * (1 + (size_t)kDevMrsMaxW * E + 4 * (size_t)E) * sizeof(double));
  l.spec_logits = take((size_t)t_max * E * 4);
  l.spec_ids = take(tk * 4);
  l.spec_w = take(tk * 4);
  l.spec_scores = take((size_t)E * 4);
  l.total = off;
  return l;
}

__global__ void commit_after_fill_kernel(int32_t* lut, int32_t idx, int32_t* owner, int32_t slot,
                                         const uint64_t* tags, uint64_t tag, int32_t* err_word) {
  if (threadIdx.x != 0) return;
  if (tags[slot] != tag) {
    atomicOr(err_word, MOE_ERR_STALE_TAG);
    return;
  }
  const int32_t old = owner[slot];
  if (old >= 0 && lut[old] == slot) lut[old] = -1;
  lut[idx] = slot;
  owner[slot] = idx;
}


// LRU plan of one layer call on the device: the rule of moe_plan_fills for a
// routed set that fits the pool (n_distinct <= S, one wave). Victims are the
// empty slots by id, then the slots of `order` (kept sorted by (last use, slot
// id)) that hold no hit; the slots used by the call move, by id, to the end of
// the order. Thread t owns slots / order positions 4t .. 4t+3.
constexpr int kDevPlanMaxS = 4096;
// With pol (the eviction-score state: Minus Recent Score or routing-history, per doubles per
// layer, the keep scores its last E) the slots holding no hit are taken by (owner's keep
// score, last use, slot id) instead, the order of moe_plan_fills_policy: a bitonic sort of the
// slots in LDS by that order when a step misses (none when it does not).
__global__ __launch_bounds__(1024) void device_plan_kernel(
    int layer, int E, int S, const int32_t* __restrict__ routed /* [E] then the count */,
    int32_t* lut, int32_t* owner, int64_t* last_use, int64_t* clock, int32_t* order,
    int32_t* fills, int32_t* n_fills, int64_t* counters, const double* __restrict__ pol,
    long per) {
  __shared__ uint32_t s_kept[kDevPlanMaxS / 32], s_used[kDevPlanMaxS / 32];
  __shared__ int s_miss[1024], s_vict[1024], s_wave[40];
  __shared__ int s_order[kDevPlanMaxS];
  __shared__ double s_keep[kDevPlanMaxS];   // Minus Recent Score: candidates' keep scores,
  __shared__ int64_t s_lu[kDevPlanMaxS];    // their last uses
  __shared__ uint32_t s_cand[kDevPlanMaxS / 32];
  const int tid = threadIdx.x;
  const int nd = routed[E];
  const int64_t now = clock[0] + 1;
  int32_t* row = lut + (size_t)layer * E;
  for (int i = tid; i < kDevPlanMaxS / 32; i += blockDim.x) s_kept[i] = s_used[i] = s_cand[i] = 0u;
  __syncthreads();
  int is_hit = 0, is_miss = 0, ex = -1;
  if (tid < nd) {
    ex = routed[tid];
    const int sl = row[ex];
    if (sl >= 0) {
      is_hit = 1;
      atomicOr(&s_kept[sl >> 5], 1u << (sl & 31));
      atomicOr(&s_used[sl >> 5], 1u << (sl & 31));
    } else {
      is_miss = 1;
    }
  }
  int nmiss = 0, nhit = 0;
  const int mpos = block_exclusive_scan(is_miss, s_wave, &nmiss);  // ends with a barrier
  (void)block_exclusive_scan(is_hit, s_wave, &nhit);
  if (is_miss) s_miss[mpos] = ex;
  // victims: empty slots by id
  int sl4[4], cnt = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sl = tid * 4 + j;
    sl4[j] = (sl < S && owner[sl] < 0) ? 1 : 0;
    cnt += sl4[j];
  }
  int nempty = 0;
  int pos = block_exclusive_scan(cnt, s_wave, &nempty);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (sl4[j]) {
      if (pos < nmiss) s_vict[pos] = tid * 4 + j;
      ++pos;
    }
  // then the slots holding no hit, in LRU order (or the policy's)
  int o4[4], ok4[4];
  cnt = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = tid * 4 + j;
    o4[j] = idx < S ? order[idx] : -1;
    ok4[j] = (o4[j] >= 0 && owner[o4[j]] >= 0 && !((s_kept[o4[j] >> 5] >> (o4[j] & 31)) & 1u)) ? 1 : 0;
    cnt += ok4[j];
  }
  int nre = 0;
  pos = nempty + block_exclusive_scan(cnt, s_wave, &nre);
  if (pol == nullptr) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (ok4[j]) {
        if (pos < nmiss) s_vict[pos] = o4[j];
        ++pos;
      }
  } else if (nmiss > nempty) {  // uniform: the candidates' keep scores and last uses into LDS
    for (int sl = tid; sl < S; sl += blockDim.x) {
      const int32_t o = owner[sl];
      const bool cand = o >= 0 && !((s_kept[sl >> 5] >> (sl & 31)) & 1u);
      double kv = 0.0;
      if (cand) {
        const double* st = pol + (size_t)(o / E) * per;
        if (st[0] != 0.0) kv = st[per - E + o % E];  // a layer never observed keeps 0
      }
      s_keep[sl] = kv;
      s_lu[sl] = last_use[sl];
      if (cand) atomicOr(&s_cand[sl >> 5], 1u << (sl & 31));
    }
    __syncthreads();
    // a bitonic sort of the slot ids (padded to a power of two) by that order, candidates
    // first; the first nmiss - nempty of them are the victims, in order
    int n2 = 1;
    while (n2 < S) n2 <<= 1;
    for (int i = tid; i < n2; i += blockDim.x) s_order[i] = i;
    __syncthreads();
    auto before = [&](int a, int b) {  // slot a strictly before slot b
      const bool ca = a < S && ((s_cand[a >> 5] >> (a & 31)) & 1u);
      const bool cb = b < S && ((s_cand[b >> 5] >> (b & 31)) & 1u);
      if (ca != cb) return ca;
      if (!ca) return a < b;
      if (s_keep[a] != s_keep[b]) return s_keep[a] < s_keep[b];
      if (s_lu[a] != s_lu[b]) return s_lu[a] < s_lu[b];
      return a < b;
    };
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int q = tid; q < n2 / 2; q += blockDim.x) {
          const int lo = 2 * q - (q & (stride - 1)), hi = lo + stride;
          const int a = s_order[lo], b = s_order[hi];
          if ((lo & size) == 0 ? before(b, a) : before(a, b)) {
            s_order[lo] = b;
            s_order[hi] = a;
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < nmiss - nempty; i += blockDim.x) s_vict[nempty + i] = s_order[i];
  }
  __syncthreads();
  // fills: miss i -> victim i (n_distinct <= S leaves enough victims)
  if (tid < nmiss) {
    const int sl = s_vict[tid], me = s_miss[tid];
    const int32_t old = owner[sl];
    if (old >= 0) lut[old] = -1;
    row[me] = sl;
    owner[sl] = layer * E + me;
    fills[2 * tid] = me;
    fills[2 * tid + 1] = sl;
    atomicOr(&s_used[sl >> 5], 1u << (sl & 31));
  }
  __syncthreads();
  // new order: the unused slots as they were, then the used slots by id
  int keep4[4];
  cnt = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    keep4[j] = (o4[j] >= 0 && !((s_used[o4[j] >> 5] >> (o4[j] & 31)) & 1u)) ? 1 : 0;
    cnt += keep4[j];
  }
  int nkeep = 0;
  pos = block_exclusive_scan(cnt, s_wave, &nkeep);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (keep4[j]) s_order[pos++] = o4[j];
  int u4[4];
  cnt = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sl = tid * 4 + j;
    u4[j] = (sl < S && ((s_used[sl >> 5] >> (sl & 31)) & 1u)) ? 1 : 0;
    cnt += u4[j];
  }
  int nused = 0;
  pos = nkeep + block_exclusive_scan(cnt, s_wave, &nused);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (u4[j]) {
      s_order[pos++] = tid * 4 + j;
      last_use[tid * 4 + j] = now;
    }
  __syncthreads();
  for (int i = tid; i < S; i += blockDim.x) order[i] = s_order[i];
  if (tid == 0) {
    clock[0] = now;
    n_fills[0] = nmiss;
    counters[0] += nd;
    counters[1] += nhit;
    counters[2] += nmiss;
    counters[3] += nd > 0 ? 1 : 0;
  }
}

#pragma clang fp contract(off)
// Minus Recent Score on the device (HybriMoE summary page, Mechanism), the arithmetic of
// moe_policy_observe: the layer's routing scores of this step go into its ring of the last
// W steps; then every expert's keep score is the sum of its ring entries, oldest to
// newest, minus the newest (fp64, no contraction). state: per layer [observed steps, ring
// W x E, keep E]. One workgroup, E <= blockDim.
__global__ __launch_bounds__(1024) void device_mrs_observe_kernel(double* state, int layer, int E,
                                                                  int W,
                                                                  const float* __restrict__ scores) {
  double* st = state + (size_t)layer * (1 + (size_t)W * E + E);
  const long n = (long)st[0];  // steps observed before this one
  double* ring = st + 1;
  double* keep = st + 1 + (size_t)W * E;
  const int e = threadIdx.x;
  if (e < E) {
    ring[(size_t)(n % W) * E + e] = (double)scores[e];
    const long n1 = n + 1, m = n1 < W ? n1 : W;
    double total = 0.0;
    for (long i = n1 - m; i < n1; ++i) total += ring[(size_t)(i % W) * E + e];
    keep[e] = total - ring[(size_t)((n1 - 1) % W) * E + e];
  }
  __syncthreads();  // every thread has read the count
  if (threadIdx.x == 0) st[0] = (double)(n + 1);
}

// Routing-history score on the device (MoE-CORE summary page, Mechanism), the arithmetic of
// moe_policy_observe: this step's selections (0/1 per expert, from the routed set) go into
// the layer's ring of the last W steps; the moving average, latest routing score and step of
// the last selection are updated; then every expert's keep score is w0 * count / max count +
// w1 * ema / max ema + w2 * score / max score + w3 * (1 - age / max age), each term 0 (the
// last 1) when its maximum over the layer is 0, summed in that order (fp64, no
// contraction). state: per layer [observed steps, ring W x E, ema E, score E, last E, keep E].
// One workgroup of 1024 threads, E <= 1024.
__global__ __launch_bounds__(1024) void device_history_observe_kernel(
    double* state, int layer, int E, int W, const float* __restrict__ scores,
    const int32_t* __restrict__ routed /* [E] then the count */, double w0, double w1, double w2,
    double w3, double lam) {
  __shared__ double s_max[4][16];
  double* st = state + (size_t)layer * (1 + (size_t)W * E + 4 * (size_t)E);
  const long n = (long)st[0];  // steps observed before this one
  double* ring = st + 1;
  double* row = ring + (size_t)(n % W) * E;
  double* ema = ring + (size_t)W * E;
  double* score = ema + E;
  double* last = score + E;
  double* keep = last + E;
  const int e = threadIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (e < E) row[e] = 0.0;
  __syncthreads();
  if (e < routed[E]) row[routed[e]] = 1.0;
  __syncthreads();
  const long n1 = n + 1, m = n1 < W ? n1 : W;
  double f[4] = {0.0, 0.0, 0.0, 0.0};  // count, ema, score, age (0 past E)
  if (e < E) {
    const double sel = row[e];
    ema[e] = lam * ema[e] + (1.0 - lam) * sel;
    score[e] = (double)scores[e];
    if (sel != 0.0) last[e] = (double)n1;
    for (long i = n1 - m; i < n1; ++i) f[0] += ring[(size_t)(i % W) * E + e];
    f[1] = ema[e];
    f[2] = score[e];
    f[3] = (double)n1 - last[e];
  }
  // each feature's maximum over the layer (from 0, like the host's; exact in any order)
  double mx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    double v = f[j];
    for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
    if (lane == 0) s_max[j][wave] = v;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    double v = 0.0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) v = fmax(v, s_max[j][i]);
    mx[j] = v;
  }
  if (e < E) {
    const double n_cnt = mx[0] > 0.0 ? f[0] / mx[0] : 0.0;
    const double n_ema = mx[1] > 0.0 ? f[1] / mx[1] : 0.0;
    const double n_score = mx[2] > 0.0 ? f[2] / mx[2] : 0.0;
    const double fresh = mx[3] > 0.0 ? 1.0 - f[3] / mx[3] : 1.0;
    double total = w0 * n_cnt;
    total += w1 * n_ema;
    total += w2 * n_score;
    total += w3 * fresh;
    keep[e] = total;
  }
  __syncthreads();  // every thread has read the count
  if (threadIdx.x == 0) st[0] = (double)n1;
}
#pragma clang fp contract(on)

// Copy the step's fills from the mapped host store into their slots (16 bytes
// per lane, every workgroup striding over each expert's bytes in turn).
__global__ __launch_bounds__(256) void device_fill_kernel(const char* __restrict__ store,
                                                          const int32_t* __restrict__ blob_of,
                                                          int layer, int E, char* pool,
                                                          size_t stride,
                                                          const int32_t* __restrict__ fills,
                                                          const int32_t* __restrict__ n_fills) {
  const int nf = n_fills[0];
  const size_t per = stride / 16;
  const size_t g = blockIdx.x * (size_t)blockDim.x + threadIdx.x, gs = (size_t)gridDim.x * blockDim.x;
  for (int f = 0; f < nf; ++f) {
    const u32x4* src = reinterpret_cast<const u32x4*>(store + (size_t)blob_of[(size_t)layer * E + fills[2 * f]] * stride);
    u32x4* dst = reinterpret_cast<u32x4*>(pool + (size_t)fills[2 * f + 1] * stride);
    for (size_t j = g; j < per; j += gs) dst[j] = src[j];
  }
}

__global__ void write_tag_kernel(uint64_t* tags, int slot, uint64_t tag) {
  if (threadIdx.x == 0) tags[slot] = tag;
}

void destroy(moe_layer_ctx* c) {
  if (!c) return;
  void* host[] = {c->ring_h, c->masks_h, c->sh_rows_h, c->spec_h};
  for (void* p : host)
    if (p) (void)hipHostFree(p);
  for (int i = 0; i < kRing; ++i) {
    if (c->ring_ev[i]) (void)hipEventDestroy(c->ring_ev[i]);
    if (c->tev0[i]) (void)hipEventDestroy(c->tev0[i]);
    if (c->tev1[i]) (void)hipEventDestroy(c->tev1[i]);
  }
  for (int b = 0; b < 2; ++b) {
    if (c->ev_ready[b]) (void)hipEventDestroy(c->ev_ready[b]);
    if (c->ev_free[b]) (void)hipEventDestroy(c->ev_free[b]);
  }
  if (c->ev_fill) (void)hipEventDestroy(c->ev_fill);
  if (c->ev_compute) (void)hipEventDestroy(c->ev_compute);
  if (c->ev_pf_before) (void)hipEventDestroy(c->ev_pf_before);
  delete c;
}

void recount_resident(moe_layer_ctx* c) {
  for (int l = 0; l < c->L; ++l) {
    int n = 0;
    for (int e = 0; e < c->E; ++e) n += c->lut_h[(size_t)l * c->E + e] >= 0;
    c->resident[l] = n;
  }
}

// Copy one expert into a slot on the fill stream, write its tag back, and
// commit it on the compute stream once the copy is done.
// The copy half of a fill, on the fill stream: the expert's bytes into the slot, then its
// tag (returned in *tag).
int fill_copy(moe_layer_ctx* c, int slot, int layer, int expert, uint64_t* tag) {
  const int idx = layer * c->E + expert;
  *tag = c->next_tag++;
  const size_t off = (size_t)c->blob_of[idx] * c->stride;
  hipError_t e = hipSuccess;
  if (c->store_dev) {  // the store is mapped: a copy kernel (the stride is a multiple of 256)
    const int rc = launch_host_copy(c->pool + (size_t)slot * c->stride, c->store_dev + off,
                                    c->stride, c->fs);
    if (rc != MOE_OK) return rc;
  } else {
    e = hipMemcpyAsync(c->pool + (size_t)slot * c->stride, c->host_store + off, c->stride,
                       hipMemcpyHostToDevice, c->fs);
  }
  if (e != hipSuccess) return moe_hip_status(e);
  hipLaunchKernelGGL(write_tag_kernel, dim3(1), dim3(64), 0, c->fs, c->tags, slot, *tag);
  return moe_launch_status();
}

// The compute stream waits for the fill stream's copies so far.
int compute_after_fills(moe_layer_ctx* c) {
  if (c->fs == c->cs) return MOE_OK;
  hipError_t e = hipEventRecord(c->ev_fill, c->fs);
  if (e == hipSuccess) e = hipStreamWaitEvent(c->cs, c->ev_fill, 0);
  return moe_hip_status(e);
}

// The commit half, on the compute stream after the copy: the table entry and the owner,
// once the slot's tag is still this fill's.
int fill_commit(moe_layer_ctx* c, int slot, int layer, int expert, uint64_t tag) {
  hipLaunchKernelGGL(commit_after_fill_kernel, dim3(1), dim3(64), 0, c->cs, c->lut,
                     layer * c->E + expert, c->owner, slot, c->tags, tag, c->err);
  return moe_launch_status();
}

// Make the fill stream wait for everything enqueued so far on the compute stream.
int fills_after_compute(moe_layer_ctx* c) {
  if (c->fs == c->cs) return MOE_OK;
  hipError_t e = hipEventRecord(c->ev_compute, c->cs);
  if (e == hipSuccess) e = hipStreamWaitEvent(c->fs, c->ev_compute, 0);
  return moe_hip_status(e);
}

// Host plan of one routed set under the context's eviction policy (moves the
// host tables), with counters; entry = the step's ring entry (routed set, its
// size, then the routing scores).
int run_plan(moe_layer_ctx* c, int layer, const int32_t* entry, int32_t* n_fills,
             int32_t* n_waves) {
  const int* distinct = entry;
  const int nd = entry[c->E];
  const float* scores = reinterpret_cast<const float*>(entry + c->E + 1);
  int rc = moe_policy_observe(c->policy, c->pol_state.data(), c->L, c->E, c->window, layer, scores,
                              distinct, nd, c->params);
  if (rc != MOE_OK) return rc;
  rc = moe_plan_fills_policy(c->policy, c->pol_state.data(), c->window, c->params, c->lut_h.data(),
                             c->owner_h.data(), c->last_use.data(), &c->clock, c->S, c->L, c->E,
                             layer, distinct, nd, c->wave_of.data(), c->is_hit.data(),
                             c->fill_e.data(), c->fill_s.data(), c->fill_w.data(), n_fills, n_waves);
  if (rc != MOE_OK) return rc;
  int hits = 0;
  for (int i = 0; i < nd; ++i) hits += c->is_hit[distinct[i]];
  // prefetched experts of this layer: used when routed now; pending no longer either way
  char* pend = c->pf_pending.data() + (size_t)layer * c->E;
  for (int i = 0; i < nd; ++i) c->pf_used += pend[distinct[i]];
  memset(pend, 0, c->E);
  c->totals[0] += nd;
  c->totals[1] += hits;
  c->totals[2] += *n_fills;
  c->totals[3] += *n_waves;
  if (*n_fills) recount_resident(c);
  return MOE_OK;
}

// Replay the bookkeeping of deferred steps, oldest first.
int drain(moe_layer_ctx* c) {
  while (c->ring_count > 0) {
    const int r = c->ring_head;
    const hipError_t e = hipEventSynchronize(c->ring_ev[r]);
    if (e != hipSuccess) return moe_hip_status(e);
    const int32_t* d = c->ring_h + (size_t)r * (2 * c->E + 1);
    int32_t nf = 0, nw = 0;
    const int rc = run_plan(c, c->ring_layer[r], d, &nf, &nw);
    if (rc != MOE_OK) return rc;
    c->ring_head = (c->ring_head + 1) % kRing;
    c->ring_count -= 1;
  }
  return MOE_OK;
}

// Fold finished timing pairs into the total; all = every pending pair.
void collect_timing(moe_layer_ctx* c, bool all) {
  while (c->t_count > 0 && (all || c->t_count >= kRing - 1)) {
    const int r = c->t_head;
    float ms = 0.f;
    if (hipEventSynchronize(c->tev1[r]) == hipSuccess &&
        hipEventElapsedTime(&ms, c->tev0[r], c->tev1[r]) == hipSuccess) {
      c->ffn_ms += ms;
      c->ffn_calls += 1;
    } else {
      (void)hipGetLastError();
    }
    c->t_head = (c->t_head + 1) % kRing;
    c->t_count -= 1;
  }
}

// Hand the residency state from the device planner back to the host tables.
int sync_from_device(moe_layer_ctx* c) {
  hipError_t e = hipStreamSynchronize(c->cs);
  if (e != hipSuccess) return moe_hip_status(e);
  int64_t cnt[4];
  if ((e = hipMemcpy(c->lut_h.data(), c->lut, c->lut_h.size() * sizeof(int32_t), hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(c->owner_h.data(), c->owner, c->owner_h.size() * sizeof(int32_t), hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(c->last_use.data(), c->d_last_use, c->last_use.size() * sizeof(int64_t), hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(&c->clock, c->d_clock, sizeof(int64_t), hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(cnt, c->d_counters, sizeof(cnt), hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemset(c->d_counters, 0, sizeof(cnt))) != hipSuccess)
    return moe_hip_status(e);
  if (c->policy != MOE_POLICY_LRU &&
      (e = hipMemcpy(c->pol_state.data(), c->d_pol, c->pol_state.size() * sizeof(double),
                     hipMemcpyDeviceToHost)) != hipSuccess)
    return moe_hip_status(e);
  for (int i = 0; i < 4; ++i) c->totals[i] += cnt[i];
  recount_resident(c);
  return MOE_OK;
}

// Hand the host tables' LRU state, and under an eviction score the policy state, to the
// device planner (the device tables themselves are already current once the stream runs).
int push_to_device(moe_layer_ctx* c) {
  std::vector<int32_t> order(c->S);
  for (int s = 0; s < c->S; ++s) order[s] = s;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return c->last_use[a] < c->last_use[b]; });
  hipError_t e = hipStreamSynchronize(c->cs);
  if (e == hipSuccess) e = hipMemcpy(c->d_order, order.data(), c->S * sizeof(int32_t), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(c->d_last_use, c->last_use.data(), c->S * sizeof(int64_t), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(c->d_clock, &c->clock, sizeof(int64_t), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemset(c->d_counters, 0, 4 * sizeof(int64_t));
  if (e == hipSuccess && c->policy != MOE_POLICY_LRU)
    e = hipMemcpy(c->d_pol, c->pol_state.data(), c->pol_state.size() * sizeof(double),
                  hipMemcpyHostToDevice);
  return moe_hip_status(e);
}

}  // namespace

extern "C" size_t moe_ctx_workspace_bytes(int t_max, int H, int F, int E, int k, int L, int S,
                                          int w_dtype, int n_shared) {
  if (t_max < 1 || H <= 0 || F <= 0 || E < 1 || k < 1 || L < 1 || S < 1 || n_shared < 0) return 0;
  return ctx_layout(t_max, H, F, E, k, L, S, w_dtype, n_shared).total;
}

extern "C" int moe_ctx_create(moe_layer_ctx** out, int t_max, int H, int F, int E, int k, int L,
                              int S, int x_dtype, int w_dtype, int n_shared, void* pool_base,
                              size_t slot_stride, int32_t* lut, int32_t* owner,
                              uint64_t* slot_tags, const void* host_store,
                              const int32_t* blob_of, const void* shared_pool, int32_t* err_word,
                              void* workspace, size_t ws_bytes, hipStream_t compute_stream,
                              hipStream_t fill_stream) {
  MOE_CHECK_ARG(out && t_max >= 1 && k >= 1 && k <= E && E <= 1024 && L >= 1 && S >= 1);
  MOE_CHECK_ARG(x_dtype == MOE_F32 || x_dtype == MOE_BF16);
  MOE_CHECK_ARG(n_shared >= 0 && E + n_shared <= 1024);
  MOE_CHECK_ARG(pool_base && lut && owner && slot_tags && host_store && blob_of && err_word);
  SlotLayout lay;
  if (slot_layout(H, F, w_dtype, &lay) != MOE_OK) return MOE_EINVAL;
  MOE_CHECK_ARG(slot_stride >= lay.slot_bytes && slot_stride % 256 == 0);
  // the shared experts are the n_shared slots right after the S routed slots
  MOE_CHECK_ARG(n_shared == 0 ||
                shared_pool == static_cast<const char*>(pool_base) + (size_t)S * slot_stride);
  const CtxLayout cl = ctx_layout(t_max, H, F, E, k, L, S, w_dtype, n_shared);
  MOE_CHECK_ARG(workspace && ws_bytes >= cl.total && ((uintptr_t)workspace % 256) == 0);
  *out = nullptr;
  moe_layer_ctx* c = new (std::nothrow) moe_layer_ctx();
  if (!c) return MOE_EHIP;
  c->t_max = t_max; c->H = H; c->F = F; c->E = E; c->k = k; c->L = L; c->S = S;
  c->x_dtype = x_dtype; c->w_dtype = w_dtype; c->n_shared = n_shared;
  c->pool = static_cast<char*>(pool_base);
  c->stride = slot_stride;
  c->lut = lut; c->owner = owner; c->tags = slot_tags;
  c->host_store = static_cast<const char*>(host_store);
  c->blob_of.assign(blob_of, blob_of + (size_t)L * E);
  c->err = err_word;
  c->cs = compute_stream;
  c->fs = fill_stream;
  c->lut_h.assign((size_t)L * E, -1);
  c->owner_h.assign(S, -1);
  c->resident.assign(L, 0);
  c->last_use.assign(S, 0);
  c->clock = 0;
  c->policy = MOE_POLICY_LRU;
  c->window = 1;
  for (double& v : c->params) v = 0.0;
  c->last_ring = -1;
  c->split = 0;
  c->stage = 0;
  c->stage_thr = -1;
  c->stage_slot0 = S + n_shared;
  c->buf_layer[0] = c->buf_layer[1] = -1;
  c->buf_last = -1;
  c->ev_ready[0] = c->ev_ready[1] = c->ev_free[0] = c->ev_free[1] = nullptr;
  c->stage_steps = c->stage_copies = 0;
  c->next_hint = -1;
  c->orch = 0;
  c->store_dev = nullptr;
  {  // fills read a store the device can map through a copy kernel
    void* dev = nullptr;
    if (hipHostGetDevicePointer(&dev, const_cast<void*>(host_store), 0) == hipSuccess && dev)
      c->store_dev = static_cast<const char*>(dev);
    else
      (void)hipGetLastError();
  }
  c->orch_ready = false;
  c->next_tag = 1;
  c->wave_of.resize(E); c->is_hit.resize(E);
  c->fill_e.resize(E); c->fill_s.resize(E); c->fill_w.resize(E);
  c->sh_T = -1;
  char* wb = static_cast<char*>(workspace);
  c->sync = reinterpret_cast<uint32_t*>(wb + cl.sync);
  c->logits = reinterpret_cast<float*>(wb + cl.logits);
  c->ids = reinterpret_cast<int32_t*>(wb + cl.ids);
  c->topw = reinterpret_cast<float*>(wb + cl.topw);
  c->counts = reinterpret_cast<int32_t*>(wb + cl.counts);
  c->offsets = reinterpret_cast<int32_t*>(wb + cl.offsets);
  c->perm = reinterpret_cast<int32_t*>(wb + cl.perm);
  c->inv = reinterpret_cast<int32_t*>(wb + cl.inv);
  c->dist = reinterpret_cast<int32_t*>(wb + cl.dist);
  c->y_perm = reinterpret_cast<float*>(wb + cl.y_perm);
  c->ws = wb + cl.ws;
  c->ws_bytes = cl.ws_bytes;
  c->masks = reinterpret_cast<int32_t*>(wb + cl.masks);
  c->scores = reinterpret_cast<float*>(wb + cl.scores);
  c->crit = reinterpret_cast<int32_t*>(wb + cl.crit);
  c->d_order = reinterpret_cast<int32_t*>(wb + cl.order);
  c->d_last_use = reinterpret_cast<int64_t*>(wb + cl.last_use);
  c->d_clock = reinterpret_cast<int64_t*>(wb + cl.clock);
  c->d_blob = reinterpret_cast<int32_t*>(wb + cl.blob);
  c->d_fills = reinterpret_cast<int32_t*>(wb + cl.fills);
  c->d_nfills = reinterpret_cast<int32_t*>(wb + cl.nfills);
  c->d_counters = reinterpret_cast<int64_t*>(wb + cl.counters);
  c->d_pol = reinterpret_cast<double*>(wb + cl.pol);
  c->d_stage_lut = reinterpret_cast<int32_t*>(wb + cl.stage_lut);
  c->stage_ready = false;
  c->spec_logits = reinterpret_cast<float*>(wb + cl.spec_logits);
  c->spec_ids = reinterpret_cast<int32_t*>(wb + cl.spec_ids);
  c->spec_w = reinterpret_cast<float*>(wb + cl.spec_w);
  c->spec_scores = reinterpret_cast<float*>(wb + cl.spec_scores);
  c->prefetch = 0;
  c->pf_window_us = c->pf_bw_gbs = 0.0;
  c->next_wr = nullptr;
  c->next_bias = nullptr;
  c->pf_pending.assign((size_t)L * E, 0);
  c->pf_issued = c->pf_used = 0;
  int bad = 0;
  // coherent, mapped: the permutation kernel stores the routed set straight into it
  bad |= hipHostMalloc(reinterpret_cast<void**>(&c->ring_h),
                       (size_t)kRing * (2 * E + 1) * sizeof(int32_t),
                       hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess;
  if (!bad) bad |= hipHostGetDevicePointer(reinterpret_cast<void**>(&c->ring_d), c->ring_h, 0) !=
                   hipSuccess;
  bad |= hipHostMalloc(reinterpret_cast<void**>(&c->masks_h),
                       (size_t)(E + 2) * E * sizeof(int32_t)) != hipSuccess;
  bad |= hipHostMalloc(reinterpret_cast<void**>(&c->sh_rows_h),
                       ((size_t)t_max * n_shared + n_shared + 1) * sizeof(int32_t)) != hipSuccess;
  bad |= hipHostMalloc(reinterpret_cast<void**>(&c->spec_h),
                       ((size_t)t_max * k + E) * sizeof(int32_t)) != hipSuccess;
  bad |= hipEventCreateWithFlags(&c->ev_pf_before, hipEventDisableTiming) != hipSuccess;
  bad |= hipEventCreateWithFlags(&c->ev_fill, hipEventDisableTiming) != hipSuccess;
  bad |= hipEventCreateWithFlags(&c->ev_compute, hipEventDisableTiming) != hipSuccess;
  for (int i = 0; i < kRing; ++i) {
    bad |= hipEventCreateWithFlags(&c->ring_ev[i], hipEventDisableTiming) != hipSuccess;
    bad |= hipEventCreate(&c->tev0[i]) != hipSuccess;
    bad |= hipEventCreate(&c->tev1[i]) != hipSuccess;
  }
  if (bad) {
    (void)hipGetLastError();
    destroy(c);
    return MOE_EHIP;
  }
  if (hipMemset(c->sync, 0, sizeof(uint32_t)) != hipSuccess) {
    (void)hipGetLastError();
    destroy(c);
    return MOE_EHIP;
  }
  *out = c;
  return MOE_OK;
}

extern "C" int moe_ctx_destroy(moe_layer_ctx* ctx) {
  if (!ctx) return MOE_EINVAL;
  (void)hipStreamSynchronize(ctx->cs);
  if (ctx->fs != ctx->cs) (void)hipStreamSynchronize(ctx->fs);
  destroy(ctx);
  return MOE_OK;
}

extern "C" int moe_ctx_place(moe_layer_ctx* c, int slot, int layer, int expert) {
  MOE_CHECK_ARG(c && slot >= 0 && slot < c->S && layer >= 0 && layer < c->L && expert >= 0 &&
                expert < c->E);
  int rc = c->orch ? sync_from_device(c) : drain(c);
  if (rc != MOE_OK) return rc;
  MOE_CHECK_ARG(c->lut_h[(size_t)layer * c->E + expert] < 0);
  // the copy must not overtake kernels that may still read the slot
  if ((rc = fills_after_compute(c)) != MOE_OK) return rc;
  uint64_t tag = 0;
  if ((rc = fill_copy(c, slot, layer, expert, &tag)) != MOE_OK ||
      (rc = compute_after_fills(c)) != MOE_OK || (rc = fill_commit(c, slot, layer, expert, tag)) != MOE_OK)
    return rc;
  const int idx = layer * c->E + expert;
  const int32_t old = c->owner_h[slot];
  if (old >= 0 && c->lut_h[old] == slot) c->lut_h[old] = -1;
  c->lut_h[idx] = slot;
  c->owner_h[slot] = idx;
  recount_resident(c);
  return c->orch ? push_to_device(c) : MOE_OK;
}

extern "C" int moe_ctx_read_tables(moe_layer_ctx* c, int32_t* lut_out, int32_t* owner_out,
                                   int64_t* last_use_out, int64_t* clock_out) {
  MOE_CHECK_ARG(c);
  const int rc = c->orch ? sync_from_device(c) : drain(c);
  if (rc != MOE_OK) return rc;
  if (lut_out) memcpy(lut_out, c->lut_h.data(), c->lut_h.size() * sizeof(int32_t));
  if (owner_out) memcpy(owner_out, c->owner_h.data(), c->owner_h.size() * sizeof(int32_t));
  if (last_use_out) memcpy(last_use_out, c->last_use.data(), c->last_use.size() * sizeof(int64_t));
  if (clock_out) *clock_out = c->clock;
  return MOE_OK;
}

extern "C" int moe_ctx_counters(moe_layer_ctx* c, int64_t* out4) {
  MOE_CHECK_ARG(c && out4);
  const int rc = c->orch ? sync_from_device(c) : drain(c);
  if (rc != MOE_OK) return rc;
  for (int i = 0; i < 4; ++i) out4[i] = c->totals[i];
  return MOE_OK;
}

extern "C" int moe_ctx_set_prefetch(moe_layer_ctx* c, int enable, double t_remain_us,
                                    double t_attn_us, double t_launch_us, double bw_gbs) {
  MOE_CHECK_ARG(c && (enable == 0 || enable == 1));
  if (!enable) {
    c->prefetch = 0;
    return MOE_OK;
  }
  MOE_CHECK_ARG(std::isfinite(t_remain_us) && std::isfinite(t_attn_us) &&
                std::isfinite(t_launch_us) && std::isfinite(bw_gbs) && bw_gbs > 0.0);
  c->pf_window_us = t_remain_us + t_attn_us - t_launch_us;
  c->pf_bw_gbs = bw_gbs;
  c->prefetch = 1;
  return MOE_OK;
}

extern "C" int moe_ctx_prefetch_counters(moe_layer_ctx* c, int64_t* out) {
  MOE_CHECK_ARG(c && out);
  const int rc = c->orch ? sync_from_device(c) : drain(c);
  if (rc != MOE_OK) return rc;
  out[0] = c->pf_issued;
  out[1] = c->pf_used;
  return MOE_OK;
}

extern "C" int moe_ctx_set_timing(moe_layer_ctx* c, int enable) {
  MOE_CHECK_ARG(c);
  collect_timing(c, true);
  c->timing = enable;
  c->ffn_ms = 0.0;
  c->ffn_calls = 0;
  return MOE_OK;
}

extern "C" int moe_ctx_ffn_time(moe_layer_ctx* c, double* total_ms, long* steps) {
  MOE_CHECK_ARG(c && total_ms && steps);
  collect_timing(c, true);
  *total_ms = c->ffn_ms;
  *steps = c->ffn_calls;
  return MOE_OK;
}

extern "C" int moe_ctx_set_policy(moe_layer_ctx* c, int policy, int window, const double* params) {
  MOE_CHECK_ARG(c);
  // the device planner runs LRU and both eviction scores (window up to kDevMrsMaxW)
  MOE_CHECK_ARG(!c->orch || policy == MOE_POLICY_LRU || (window >= 1 && window <= kDevMrsMaxW));
  size_t n = 0;
  if (policy != MOE_POLICY_LRU) {
    n = moe_policy_state_doubles(policy, c->L, c->E, window);
    MOE_CHECK_ARG(n > 0);
  }
  if (policy == MOE_POLICY_HISTORY) {
    MOE_CHECK_ARG(params);
    for (int i = 0; i < 4; ++i) MOE_CHECK_ARG(params[i] >= 0.0);
    MOE_CHECK_ARG(params[4] >= 0.0 && params[4] <= 1.0);
  }
  const int rc = drain(c);  // steps so far are booked under the previous policy
  if (rc != MOE_OK) return rc;
  c->policy = policy;
  c->window = policy == MOE_POLICY_LRU ? 1 : window;
  for (int i = 0; i < 5; ++i) c->params[i] = (policy == MOE_POLICY_HISTORY) ? params[i] : 0.0;
  c->pol_state.assign(n, 0.0);
  if (c->orch && policy != MOE_POLICY_LRU) {  // the device planner's state starts empty too
    hipError_t e = hipStreamSynchronize(c->cs);
    if (e == hipSuccess) e = hipMemset(c->d_pol, 0, n * sizeof(double));
    return moe_hip_status(e);
  }
  return MOE_OK;
}

extern "C" int moe_ctx_set_split(moe_layer_ctx* c, int enable, float theta, const float* beta,
                                 float gamma) {
  MOE_CHECK_ARG(c && (enable == 0 || enable == 1));
  MOE_CHECK_ARG(!enable || c->w_dtype == MOE_INT4G128_RESPLIT);
  if (enable) {
    MOE_CHECK_ARG(std::isfinite(theta) && std::isfinite(gamma));
    c->split_th.assign(c->L, 0.f);
    for (int l = 0; l < c->L; ++l) {
      const double b = beta ? (double)beta[l] : 1.0;
      MOE_CHECK_ARG(std::isfinite(b));
      c->split_th[l] = (float)((double)theta * b * (double)gamma);
    }
  }
  // steps already enqueued keep the setting they were enqueued with
  c->split = enable;
  return MOE_OK;
}

extern "C" int moe_ctx_step_scores(moe_layer_ctx* c, float* scores) {
  MOE_CHECK_ARG(c && scores);
  if (c->split || c->orch) {  // the scores of the latest step stay on the device
    hipError_t e = hipStreamSynchronize(c->cs);
    if (e == hipSuccess) e = hipMemcpy(scores, c->scores, (size_t)c->E * sizeof(float),
                                       hipMemcpyDeviceToHost);
    return e == hipSuccess ? MOE_OK : moe_hip_status(e);
  }
  MOE_CHECK_ARG(c->policy != MOE_POLICY_LRU && c->last_ring >= 0);
  const hipError_t e = hipEventSynchronize(c->ring_ev[c->last_ring]);
  if (e != hipSuccess) return moe_hip_status(e);
  memcpy(scores, c->ring_h + (size_t)c->last_ring * (2 * c->E + 1) + c->E + 1,
         (size_t)c->E * sizeof(float));
  return MOE_OK;
}

extern "C" int moe_ctx_set_orchestration(moe_layer_ctx* c, int mode) {
  MOE_CHECK_ARG(c && (mode == MOE_ORCH_HOST || mode == MOE_ORCH_DEVICE));
  if (mode == c->orch) return MOE_OK;
  if (mode == MOE_ORCH_HOST) {
    const int rc = sync_from_device(c);
    if (rc != MOE_OK) return rc;
    c->orch = 0;
    return MOE_OK;
  }
  MOE_CHECK_ARG(c->S <= kDevPlanMaxS && !c->stage);
  MOE_CHECK_ARG(c->policy == MOE_POLICY_LRU || c->window <= kDevMrsMaxW);
  void* dev = nullptr;
  if (hipHostGetDevicePointer(&dev, const_cast<void*>(static_cast<const void*>(c->host_store)), 0) !=
          hipSuccess ||
      !dev) {
    (void)hipGetLastError();
    return MOE_EINVAL;  // the host store must be pinned memory the device can read
  }
  c->store_dev = static_cast<const char*>(dev);
  int rc = drain(c);
  if (rc != MOE_OK) return rc;
  if (!c->orch_ready) {  // the weight set table, in the caller's workspace
    const hipError_t e = hipMemcpy(c->d_blob, c->blob_of.data(),
                                   c->blob_of.size() * sizeof(int32_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) return moe_hip_status(e);
    c->orch_ready = true;
  }
  if ((rc = push_to_device(c)) != MOE_OK) return rc;
  c->orch = 1;
  return MOE_OK;
}

// One layer step planned and filled by the device (T*k <= S): no host wait.
int forward_device(moe_layer_ctx* c, int layer, const void* x, int T, const void* w_router,
                   const float* bias, void* out, int out_dtype) {
  const int E = c->E, k = c->k, H = c->H, F = c->F, nsh = c->n_shared;
  const int nslots = c->S + nsh;
  const bool scored_pol = c->policy != MOE_POLICY_LRU;  // an eviction score
  FrontPlan fp{};
  fp.scores = c->scores;  // split precision (with the critical gate) and the eviction scores
  if (c->split) {
    fp.crit = c->crit;
    fp.crit_threshold = c->split_th[layer];
  }
  bool scored = false;
  int rc = route_permute_plan(x, c->x_dtype, w_router, bias, T, H, E, k, 1, c->logits, c->ids,
                              c->topw, c->counts, c->offsets, c->perm, c->inv, c->dist, c->dist + E,
                              c->sync, (c->split || scored_pol) ? &fp : nullptr, nullptr, &scored,
                              c->cs);
  if (rc != MOE_OK) return rc;
  if ((c->split || scored_pol) && !scored) {  // more tokens than the front end scores: separate launches
    launch_step_scores(c->logits, T, E, c->scores, c->cs);
    if (c->split) launch_critical_split(c->scores, E, c->split_th[layer], nullptr, 1, c->crit, c->cs);
  }
  // the step's scores join the layer's history before the plan reads it (as on the host)
  if (c->policy == MOE_POLICY_MRS)
    hipLaunchKernelGGL(device_mrs_observe_kernel, dim3(1), dim3(1024), 0, c->cs, c->d_pol, layer,
                       E, c->window, c->scores);
  else if (c->policy == MOE_POLICY_HISTORY)
    hipLaunchKernelGGL(device_history_observe_kernel, dim3(1), dim3(1024), 0, c->cs, c->d_pol,
                       layer, E, c->window, c->scores, c->dist, c->params[0], c->params[1],
                       c->params[2], c->params[3], c->params[4]);
  const long per = scored_pol ? (long)moe_policy_state_doubles(c->policy, 1, E, c->window) : 0;
  hipLaunchKernelGGL(device_plan_kernel, dim3(1), dim3(1024), 0, c->cs, layer, E, c->S, c->dist,
                     c->lut, c->owner, c->d_last_use, c->d_clock, c->d_order, c->d_fills,
                     c->d_nfills, c->d_counters, scored_pol ? c->d_pol : nullptr, per);
  hipLaunchKernelGGL(device_fill_kernel, dim3(128), dim3(256), 0, c->cs, c->store_dev, c->d_blob,
                     layer, E, c->pool, c->stride, c->d_fills, c->d_nfills);
  if ((rc = moe_launch_status()) != MOE_OK) return rc;
  const bool timing = c->timing != 0;
  hipError_t e;
  if (timing) {
    collect_timing(c, false);
    const int tr = (c->t_head + c->t_count) % kRing;
    if ((e = hipEventRecord(c->tev0[tr], c->cs)) != hipSuccess) return moe_hip_status(e);
  }
  if ((rc = expert_ffn(x, c->x_dtype, c->perm, c->offsets, c->lut + (size_t)layer * E,
                       c->split ? c->crit : nullptr, nsh, c->S, c->pool, c->stride, nslots,
                       c->w_dtype, T, H, F, E, k, c->y_perm, c->err, c->ws, c->ws_bytes,
                       c->cs)) != MOE_OK)
    return rc;
  if (timing) {
    const int tr = (c->t_head + c->t_count) % kRing;
    if ((e = hipEventRecord(c->tev1[tr], c->cs)) != hipSuccess) return moe_hip_status(e);
    c->t_count += 1;
  }
  const float* shared_y = nsh ? c->y_perm + (size_t)T * k * H : nullptr;
  return moe_combine(c->y_perm, c->inv, c->topw, T, k, H, shared_y, c->n_shared, out, out_dtype, c->cs);
}

// ------------------------------------------------------ full-layer staging --
extern "C" int moe_ctx_set_staging(moe_layer_ctx* c, int enable, int threshold, int pool_slots) {
  MOE_CHECK_ARG(c && (enable == 0 || enable == 1) && threshold >= -1);
  if (!enable) {
    c->stage = 0;
    return MOE_OK;
  }
  MOE_CHECK_ARG(!c->orch);  // staged steps are planned on the host
  MOE_CHECK_ARG((long long)pool_slots >= (long long)c->stage_slot0 + 2LL * c->E);
  hipError_t e = hipSuccess;
  if (!c->stage_ready) {  // the buffers' slot table, in the caller's workspace
    std::vector<int32_t> h(2 * (size_t)c->E);
    for (int i = 0; i < 2 * c->E; ++i) h[i] = c->stage_slot0 + i;
    e = hipMemcpy(c->d_stage_lut, h.data(), h.size() * sizeof(int32_t), hipMemcpyHostToDevice);
    for (int b = 0; b < 2 && e == hipSuccess; ++b) {
      e = hipEventCreateWithFlags(&c->ev_ready[b], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_free[b], hipEventDisableTiming);
      // nothing has read or is loading either buffer yet
      if (e == hipSuccess) e = hipEventRecord(c->ev_free[b], c->cs);
      if (e == hipSuccess) e = hipEventRecord(c->ev_ready[b], c->cs);
    }
    if (e != hipSuccess) return moe_hip_status(e);
    c->stage_ready = true;
  }
  c->stage = 1;
  c->stage_thr = threshold;
  return MOE_OK;
}

extern "C" int moe_ctx_stage_counters(moe_layer_ctx* c, int64_t* out) {
  MOE_CHECK_ARG(c && out);
  out[0] = c->stage_steps;
  out[1] = c->stage_copies;
  return MOE_OK;
}

namespace {

// Load every routed expert of `layer` into staging buffer b on the fill stream, once the
// compute that last read the buffer has finished; consecutive weight sets go in one copy.
int stage_load(moe_layer_ctx* c, int b, int layer) {
  hipError_t e = hipStreamWaitEvent(c->fs, c->ev_free[b], 0);
  const int E = c->E;
  for (int e0 = 0; e0 < E && e == hipSuccess;) {
    const int32_t blob0 = c->blob_of[(size_t)layer * E + e0];
    int n = 1;
    while (e0 + n < E && c->blob_of[(size_t)layer * E + e0 + n] == blob0 + n) ++n;
    char* dst = c->pool + (size_t)(c->stage_slot0 + b * E + e0) * c->stride;
    if (c->store_dev) {
      if (launch_host_copy(dst, c->store_dev + (size_t)blob0 * c->stride, (size_t)n * c->stride,
                           c->fs) != MOE_OK)
        e = hipErrorLaunchFailure;
    } else {
      e = hipMemcpyAsync(dst, c->host_store + (size_t)blob0 * c->stride, (size_t)n * c->stride,
                         hipMemcpyHostToDevice, c->fs);
    }
    e0 += n;
  }
  if (e == hipSuccess) e = hipEventRecord(c->ev_ready[b], c->fs);
  if (e != hipSuccess) return moe_hip_status(e);
  c->buf_layer[b] = layer;
  c->stage_copies += E;
  return MOE_OK;
}

// One staged step (MoE-CORE summary page, Mechanism): every routed expert of the layer
// runs from a staging buffer holding the whole layer; the other buffer then starts
// loading the next layer. The decode cache and its tables are not touched.
int forward_staged(moe_layer_ctx* c, int layer, const void* x, int T, const void* w_router,
                   const float* bias, void* out, int out_dtype) {
  const int E = c->E, k = c->k, H = c->H, F = c->F, nsh = c->n_shared;
  FrontPlan fp{};
  fp.scores = c->split ? c->scores : nullptr;
  if (c->split) {
    fp.crit = c->crit;
    fp.crit_threshold = c->split_th[layer];
  }
  bool scored = false;
  int rc = route_permute_plan(x, c->x_dtype, w_router, bias, T, H, E, k, 1, c->logits, c->ids,
                              c->topw, c->counts, c->offsets, c->perm, c->inv, c->dist, c->dist + E,
                              c->sync, fp.scores ? &fp : nullptr, nullptr, &scored, c->cs);
  if (rc != MOE_OK) return rc;
  if (c->split && !scored) {
    launch_step_scores(c->logits, T, E, c->scores, c->cs);
    launch_critical_split(c->scores, E, c->split_th[layer], nullptr, 1, c->crit, c->cs);
  }
  // the buffer holding the layer, else the one the latest staged step did not read
  int b = c->buf_layer[0] == layer ? 0 : c->buf_layer[1] == layer ? 1 : (c->buf_last == 0 ? 1 : 0);
  if (c->buf_layer[b] != layer && (rc = stage_load(c, b, layer)) != MOE_OK) return rc;
  hipError_t e = hipStreamWaitEvent(c->cs, c->ev_ready[b], 0);
  if (e != hipSuccess) return moe_hip_status(e);
  const bool timing = c->timing != 0;
  if (timing) {
    collect_timing(c, false);
    const int tr = (c->t_head + c->t_count) % kRing;
    if ((e = hipEventRecord(c->tev0[tr], c->cs)) != hipSuccess) return moe_hip_status(e);
  }
  if ((rc = expert_ffn(x, c->x_dtype, c->perm, c->offsets, c->d_stage_lut + (size_t)b * E,
                       c->split ? c->crit : nullptr, nsh, c->S, c->pool, c->stride,
                       c->stage_slot0 + 2 * E, c->w_dtype, T, H, F, E, k, c->y_perm, c->err, c->ws,
                       c->ws_bytes, c->cs)) != MOE_OK)
    return rc;
  if (timing) {
    const int tr = (c->t_head + c->t_count) % kRing;
    if ((e = hipEventRecord(c->tev1[tr], c->cs)) != hipSuccess) return moe_hip_status(e);
    c->t_count += 1;
  }
  if ((e = hipEventRecord(c->ev_free[b], c->cs)) != hipSuccess) return moe_hip_status(e);
  c->buf_last = b;
  c->stage_steps += 1;
  // prefetch: the other buffer loads the next layer while this one computes
  const int nl = c->next_hint >= 0 ? c->next_hint : (layer + 1) % c->L;
  if (nl < c->L && nl != layer && c->buf_layer[1 - b] != nl &&
      (rc = stage_load(c, 1 - b, nl)) != MOE_OK)
    return rc;
  const float* shared_y = nsh ? c->y_perm + (size_t)T * k * H : nullptr;
  return moe_combine(c->y_perm, c->inv, c->topw, T, k, H, shared_y, c->n_shared, out, out_dtype,
                     c->cs);
}

// Plan the prefetch of layer nl from the speculative routing of this step (after its own
// plan, which the deferred bookkeeping replays first) and start the copies on the fill
// stream once the compute enqueued before this step's expert FFN has finished.
int plan_and_copy_prefetch(moe_layer_ctx* c, int nl, int T, int32_t* n_pf) {
  const int E = c->E, k = c->k;
  *n_pf = 0;
  int rc = drain(c);  // replays this step's deferred plan too; waits for the speculative copies
  if (rc != MOE_OK) return rc;
  hipError_t e = hipEventSynchronize(c->ev_pf_before);
  if (e != hipSuccess) return moe_hip_status(e);
  c->pf_e.resize(E);
  c->pf_s.resize(E);
  c->pf_tag.resize(E);
  const float* pscores = reinterpret_cast<const float*>(c->spec_h + (size_t)T * k);
  rc = moe_plan_prefetch(c->policy, c->pol_state.data(), c->window, c->params, c->lut_h.data(),
                         c->owner_h.data(), c->last_use.data(), &c->clock, c->S, c->L, E, nl,
                         c->spec_h, T * k, pscores, c->pf_window_us, c->pf_bw_gbs, c->stride,
                         c->pf_e.data(), c->pf_s.data(), n_pf);
  if (rc != MOE_OK || *n_pf == 0) return rc;
  recount_resident(c);
  if (c->fs != c->cs && (e = hipStreamWaitEvent(c->fs, c->ev_pf_before, 0)) != hipSuccess)
    return moe_hip_status(e);
  for (int i = 0; i < *n_pf; ++i) {
    const int idx = nl * E + c->pf_e[i];
    c->pf_tag[i] = c->next_tag++;
    rc = slot_prefetch(c->pool, c->stride, c->pf_s[i],
                       c->host_store + (size_t)c->blob_of[idx] * c->stride, c->stride, c->tags,
                       c->pf_tag[i], c->fs);
    if (rc != MOE_OK) return rc;
    c->pf_pending[idx] = 1;
  }
  c->pf_issued += *n_pf;
  return MOE_OK;
}

int commit_prefetch(moe_layer_ctx* c, int nl, int n_pf) {
  hipError_t e;
  if (c->fs != c->cs) {
    if ((e = hipEventRecord(c->ev_fill, c->fs)) != hipSuccess) return moe_hip_status(e);
    if ((e = hipStreamWaitEvent(c->cs, c->ev_fill, 0)) != hipSuccess) return moe_hip_status(e);
  }
  for (int i = 0; i < n_pf; ++i)
    hipLaunchKernelGGL(commit_after_fill_kernel, dim3(1), dim3(64), 0, c->cs, c->lut,
                       nl * c->E + c->pf_e[i], c->owner, c->pf_s[i], c->tags, c->pf_tag[i],
                       c->err);
  return moe_launch_status();
}

}  // namespace

extern "C" int moe_layer_forward(moe_layer_ctx* c, int layer, const void* x, int T,
                                 const void* w_router, const float* bias, void* out, int out_dtype,
                                 int32_t* stats) {
  MOE_CHECK_ARG(c && layer >= 0 && layer < c->L && T >= 0 && T <= c->t_max);
  MOE_CHECK_ARG(out_dtype == MOE_F32 || out_dtype == MOE_BF16);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(x && w_router && out);
  const int E = c->E, k = c->k, H = c->H, F = c->F, nsh = c->n_shared;
  int rc;
  hipError_t e;
  if (nsh && c->sh_T != T) {
    // rows of the shared groups: group E + s holds rows T*k + s*T + t with
    // perm value t*k (token t); offsets[E + 1 + s] = T*k + (s + 1)*T. The
    // pinned staging is rewritten only once the stream drained its last copy.
    if ((e = hipStreamSynchronize(c->cs)) != hipSuccess) return moe_hip_status(e);
    int32_t* h = c->sh_rows_h;
    for (int sh = 0; sh < nsh; ++sh)
      for (int t = 0; t < T; ++t) h[(size_t)sh * T + t] = t * k;
    for (int sh = 0; sh < nsh; ++sh) h[(size_t)T * nsh + sh] = T * k + (sh + 1) * T;
    if ((e = hipMemcpyAsync(c->perm + (size_t)T * k, h, (size_t)T * nsh * sizeof(int32_t),
                            hipMemcpyHostToDevice, c->cs)) != hipSuccess ||
        (e = hipMemcpyAsync(c->offsets + E + 1, h + (size_t)T * nsh, nsh * sizeof(int32_t),
                            hipMemcpyHostToDevice, c->cs)) != hipSuccess)
      return moe_hip_status(e);
    c->sh_T = T;
  }
  // staged: a layer not wholly resident, at or above the token threshold
  if (c->stage && c->resident[layer] < E &&
      T >= (c->stage_thr >= 0 ? c->stage_thr : c->resident[layer] / k)) {
    if (stats) stats[0] = stats[1] = stats[2] = stats[3] = -1;
    return forward_staged(c, layer, x, T, w_router, bias, out, out_dtype);
  }
  if (c->orch) {
    if (T * k > c->S) return MOE_EUNSUPPORTED;  // more routed experts than slots: plan on the host
    if (stats) stats[0] = stats[1] = stats[2] = stats[3] = -1;
    return forward_device(c, layer, x, T, w_router, bias, out, out_dtype);
  }
  const int nslots = c->S + nsh;
  // the routed set is written by the device into the next ring entry (pinned host memory)
  if (c->ring_count == kRing && (rc = drain(c)) != MOE_OK) return rc;
  const int r = c->ring_next;
  int32_t* dh = c->ring_h + (size_t)r * (2 * E + 1);
  int32_t* dd = c->ring_d + (size_t)r * (2 * E + 1);
  const bool all_resident = c->resident[layer] == E;
  const int32_t* lut_row = c->lut + (size_t)layer * E;
  // a fully resident layer's FFN work list comes from the front end itself, and so do the
  // routing scores an eviction policy records (next to the routed set)
  FrontPlan fp{};
  bool planned = false, scored = false;
  const bool want_scores = c->policy != MOE_POLICY_LRU;  // recorded next to the routed set
  float* ring_scores = reinterpret_cast<float*>(dd + E + 1);
  // split precision: the scores stay on the device and decide each group's precision; the
  // front end's FFN work list is not used (high-precision groups are items at any size)
  if (c->split) fp.scores = c->scores;
  else if (want_scores) fp.scores = ring_scores;
  // a wholly resident layer takes each group's precision straight from the front end
  if (c->split && all_resident) {
    fp.crit = c->crit;
    fp.crit_threshold = c->split_th[layer];
  }
  const bool front_plan = all_resident && c->w_dtype != MOE_INT4G128_RESPLIT;
  if (front_plan) {
    const FfnWorkspace wl = ffn_workspace_layout(T, H, F, E, k, c->w_dtype, nsh);
    fp.lut = lut_row;
    fp.num_slots = nslots;
    fp.n_shared = nsh;
    fp.shared_slot0 = c->S;
    fp.small_max = c->w_dtype == MOE_F32 ? INT_MAX : ffn_small_max(T, k, E, nsh, c->w_dtype);
    fp.items = reinterpret_cast<FfnItem*>(c->ws + wl.items);
    fp.n_items = reinterpret_cast<int32_t*>(c->ws);
    fp.tiles = reinterpret_cast<GemmTile*>(c->ws + wl.tiles);
    fp.n_tiles = reinterpret_cast<int32_t*>(c->ws + 4);
    fp.err = c->err;
    fp.sync = reinterpret_cast<int32_t*>(c->ws + wl.sync);
  }
  if ((rc = route_permute_plan(x, c->x_dtype, w_router, bias, T, H, E, k, 1, c->logits, c->ids,
                               c->topw, c->counts, c->offsets, c->perm, c->inv, dd, dd + E, c->sync,
                               (front_plan || fp.scores) ? &fp : nullptr, &planned, &scored,
                               c->cs)) != MOE_OK)
    return rc;
  if (fp.scores && !scored) {  // the front end did not write them (more tokens)
    launch_step_scores(c->logits, T, E, fp.scores, c->cs);
    if ((rc = moe_launch_status()) != MOE_OK) return rc;
  }
  if (c->split && want_scores &&
      (e = hipMemcpyAsync(dh + E + 1, c->scores, (size_t)E * sizeof(float),
                          hipMemcpyDeviceToHost, c->cs)) != hipSuccess)
    return moe_hip_status(e);
  if ((e = hipEventRecord(c->ring_ev[r], c->cs)) != hipSuccess) return moe_hip_status(e);
  // miss prefetch: the next step's router on this step's tokens predicts its routed set
  // (MoE-CORE summary page, Mechanism); enqueued after the routed set's event, so the host
  // plans this step while the prediction runs, and reads it once the FFN is enqueued
  const int nl = c->next_hint;
  const bool pf = c->prefetch && nl >= 0 && c->next_wr && c->resident[nl] < E;
  if (pf) {
    if ((rc = moe_route(x, c->x_dtype, c->next_wr, c->next_bias, T, H, E, k, 1, c->spec_logits,
                        c->spec_ids, c->spec_w, c->cs)) != MOE_OK)
      return rc;
    launch_step_scores(c->spec_logits, T, E, c->spec_scores, c->cs);
    if ((e = hipMemcpyAsync(c->spec_h, c->spec_ids, (size_t)T * k * sizeof(int32_t),
                            hipMemcpyDeviceToHost, c->cs)) != hipSuccess ||
        (e = hipMemcpyAsync(c->spec_h + (size_t)T * k, c->spec_scores, (size_t)E * sizeof(float),
                            hipMemcpyDeviceToHost, c->cs)) != hipSuccess ||
        (e = hipEventRecord(c->ev_pf_before, c->cs)) != hipSuccess)
      return moe_hip_status(e);
  }
  c->ring_next = (r + 1) % kRing;
  c->last_ring = r;

  int32_t n_fills = 0, n_waves = 0, nd = -1, hits = -1;
  const bool timing = c->timing != 0;
  if (timing) {
    collect_timing(c, false);
    const int tr = (c->t_head + c->t_count) % kRing;
    if ((e = hipEventRecord(c->tev0[tr], c->cs)) != hipSuccess) return moe_hip_status(e);
  }
  if (all_resident) {
    // no miss is possible: defer the bookkeeping, run every routed group
    c->ring_layer[r] = layer;
    c->ring_count += 1;
    if (c->split && !scored)  // the front end did not write the scores (and gate)
      launch_critical_split(c->scores, E, c->split_th[layer], nullptr, 1, c->crit, c->cs);
    if ((rc = expert_ffn(x, c->x_dtype, c->perm, c->offsets, lut_row, c->split ? c->crit : nullptr,
                         nsh, c->S, c->pool, c->stride, nslots, c->w_dtype, T, H, F, E, k,
                         c->y_perm, c->err, c->ws, c->ws_bytes, c->cs, planned)) != MOE_OK)
      return rc;
  } else {
    if ((rc = drain(c)) != MOE_OK) return rc;  // earlier steps first: their entries precede r
    c->ring_head = c->ring_next;                 // entry r is consumed here, not deferred
    if ((e = hipEventSynchronize(c->ring_ev[r])) != hipSuccess) return moe_hip_status(e);
    nd = dh[E];
    if ((rc = run_plan(c, layer, dh, &n_fills, &n_waves)) != MOE_OK) return rc;
    // masks: row 0 = resident groups, row 1 + w = groups filled in wave w
    const int rows = n_waves + 1;
    memset(c->masks_h, 0, (size_t)rows * E * sizeof(int32_t));
    hits = 0;
    for (int i = 0; i < nd; ++i) {
      const int ex = dh[i];
      if (c->is_hit[ex]) {
        c->masks_h[ex] = 1;
        ++hits;
      } else {
        c->masks_h[(size_t)(1 + c->wave_of[ex]) * E + ex] = 1;
      }
    }
    // wave 0 fills only overwrite slots no resident group of this step reads: their copies
    // go out first (behind the compute stream's work so far), before the rest is enqueued
    c->fill_tag.resize((size_t)n_fills);
    int fi = 0;
    if (n_fills && (rc = fills_after_compute(c)) != MOE_OK) return rc;
    for (; fi < n_fills && c->fill_w[fi] == 0; ++fi)
      if ((rc = fill_copy(c, c->fill_s[fi], layer, c->fill_e[fi], &c->fill_tag[fi])) != MOE_OK)
        return rc;
    if ((e = hipMemcpyAsync(c->masks, c->masks_h, (size_t)rows * E * sizeof(int32_t),
                            hipMemcpyHostToDevice, c->cs)) != hipSuccess)
      return moe_hip_status(e);
    // split precision: each selected group takes its precision from the step's scores
    if (c->split)
      launch_critical_split(c->scores, E, c->split_th[layer], c->masks, rows, c->masks, c->cs);
    if (hits || nsh) {  // resident groups, and the shared experts
      if ((rc = expert_ffn(x, c->x_dtype, c->perm, c->offsets, lut_row, c->masks, nsh, c->S,
                           c->pool, c->stride, nslots, c->w_dtype, T, H, F, E, k, c->y_perm,
                           c->err, c->ws, c->ws_bytes, c->cs)) != MOE_OK)
        return rc;
    }
    int fc = 0;  // fills committed
    for (int w = 0; w < n_waves; ++w) {
      if (w > 0) {  // a later wave's copies wait for the compute that read its slots
        if ((rc = fills_after_compute(c)) != MOE_OK) return rc;
        for (; fi < n_fills && c->fill_w[fi] == w; ++fi)
          if ((rc = fill_copy(c, c->fill_s[fi], layer, c->fill_e[fi], &c->fill_tag[fi])) != MOE_OK)
            return rc;
      }
      if (fc == fi) continue;  // no fill in this wave
      if ((rc = compute_after_fills(c)) != MOE_OK) return rc;
      for (; fc < fi; ++fc)
        if ((rc = fill_commit(c, c->fill_s[fc], layer, c->fill_e[fc], c->fill_tag[fc])) != MOE_OK)
          return rc;
      if ((rc = expert_ffn(x, c->x_dtype, c->perm, c->offsets, lut_row,
                           c->masks + (size_t)(1 + w) * E, 0, 0, c->pool, c->stride, nslots,
                           c->w_dtype, T, H, F, E, k, c->y_perm, c->err, c->ws, c->ws_bytes,
                           c->cs)) != MOE_OK)
        return rc;
    }
  }
  if (timing) {
    const int tr = (c->t_head + c->t_count) % kRing;
    if ((e = hipEventRecord(c->tev1[tr], c->cs)) != hipSuccess) return moe_hip_status(e);
    c->t_count += 1;
  }
  // the prefetch copies start behind this step's fills and overlap its expert FFN (the slots
  // they take were not used by this step, only by compute enqueued before it)
  int32_t n_pf = 0;
  if (pf && (rc = plan_and_copy_prefetch(c, nl, T, &n_pf)) != MOE_OK) return rc;
  const float* shared_y = nsh ? c->y_perm + (size_t)T * k * H : nullptr;
  if ((rc = moe_combine(c->y_perm, c->inv, c->topw, T, k, H, shared_y, c->n_shared, out, out_dtype,
                        c->cs)) != MOE_OK)
    return rc;
  // the compute stream commits each prefetched expert once its copy has landed
  if (n_pf && (rc = commit_prefetch(c, nl, n_pf)) != MOE_OK) return rc;
  if (stats) {
    stats[0] = nd;
    stats[1] = hits;
    stats[2] = n_fills;
    stats[3] = n_waves;
  }
  return MOE_OK;
}

extern "C" int moe_ctx_forward_steps(moe_layer_ctx* c, int n, const int32_t* layers,
                                     const void* const* xs, int T, const void* const* w_routers,
                                     const float* const* biases, void* const* outs,
                                     int out_dtype) {
  MOE_CHECK_ARG(c && n >= 0 && (n == 0 || (layers && xs && w_routers && biases && outs)));
  for (int i = 0; i < n; ++i) {
    // the staging prefetch and the miss prefetch follow the given order
    c->next_hint = i + 1 < n ? layers[i + 1] : -1;
    c->next_wr = i + 1 < n ? w_routers[i + 1] : nullptr;
    c->next_bias = i + 1 < n ? biases[i + 1] : nullptr;
    const int rc = moe_layer_forward(c, layers[i], xs[i], T, w_routers[i], biases[i], outs[i],
                                     out_dtype, nullptr);
    c->next_hint = -1;
    c->next_wr = nullptr;
    c->next_bias = nullptr;
    if (rc != MOE_OK) return rc;
  }
  return MOE_OK;
}

extern "C" int moe_ctx_outputs(const moe_layer_ctx* c, float** logits, int32_t** ids,
                               float** topk_w, int32_t** perm, int32_t** offsets,
                               int32_t** inv) {
  MOE_CHECK_ARG(c);
  if (logits) *logits = c->logits;
  if (ids) *ids = c->ids;
  if (topk_w) *topk_w = c->topw;
  if (perm) *perm = c->perm;
  if (offsets) *offsets = c->offsets;
  if (inv) *inv = c->inv;
  return MOE_OK;
}
