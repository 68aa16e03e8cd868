/*
 * moe_runtime.h - one routed-expert MoE layer step over the slot cache, run
 * by the library (host orchestration in C++ over the entry points of
 * moe_offload.h).
 *
 * A step follows the pages' problem statement: the routed experts are known
 * only after the router runs, the expert kernel must see one fixed slot
 * layout, and misses are copied from a pinned host pool on a separate stream
 * while resident experts compute (SeqMoE summary page, Mechanism; HybriMoE
 * summary page, Mechanism: misses = routed set minus cached set). The step
 * synchronises with the host once, to read the distinct routed set for the
 * residency plan (moe_plan_fills).
 *
 * Ownership: the caller owns the slot pool, the device tables, the pinned
 * host store, the shared-expert pool, the error word, the device workspace
 * (moe_ctx_workspace_bytes) and both streams; the context allocates no device
 * memory, only a few KB of pinned host staging and its events, once, in
 * moe_ctx_create (and four events on the first staging enable), and frees them in
 * moe_ctx_destroy. A context is used by one host thread at a
 * time. Status codes as in moe_offload.h.
 */
#ifndef MOE_RUNTIME_H
#define MOE_RUNTIME_H

#include "moe_offload.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_layer_ctx moe_layer_ctx;

/* moe_ctx_workspace_bytes: device workspace a context of these sizes needs (0 on
 * bad sizes): the step's buffers, the expert FFN's workspace, and the tables of
 * device orchestration (O(S + L*E)) and of full-layer staging (O(E)), so that the
 * context allocates no device memory. L layers, S routed slots. */
size_t moe_ctx_workspace_bytes(int t_max, int H, int F, int E, int k, int L, int S, int w_dtype,
                               int n_shared);

/* moe_ctx_create: context for a stack of L layers sharing one slot pool.
 *   t_max       largest token count of a step
 *   H, F, E, k  hidden size, expert FFN size, routed experts per layer, top-k
 *   S           routed slots in the pool (pool_base + s * slot_stride, s < S)
 *   x_dtype     MOE_F32 or MOE_BF16 (tokens and router weights)
 *   w_dtype     expert weight format (MOE_F32, MOE_BF16, MOE_INT4G128)
 *   n_shared    always-on shared experts (0 = none); their packed weights sit
 *               in the n_shared slots that follow the S routed slots:
 *               shared_pool must equal pool_base + S * slot_stride (EINVAL
 *               otherwise). They are computed as extra groups of the step's
 *               first expert FFN call (one plan, one weight pass for all).
 *   lut         [L*E] int32 device table (expert -> slot, -1 = absent)
 *   owner       [S] int32 device: lut index held by each slot, -1 = empty
 *   slot_tags   [S] uint64 device
 *   host_store  pinned host memory: weight set b at host_store + b*slot_stride
 *   blob_of     host [L*E]: weight set of (layer, expert) (copied at creation)
 *   err_word    [1] int32 device (MOE_ERR_* bits)
 *   workspace   device, 256-byte aligned, ws_bytes >= moe_ctx_workspace_bytes()
 * The device tables must start empty (-1); moe_ctx_place fills the initial
 * residents. */
int moe_ctx_create(moe_layer_ctx** ctx, int t_max, int H, int F, int E, int k, int L, int S,
                   int x_dtype, int w_dtype, int n_shared, void* pool_base, size_t slot_stride,
                   int32_t* lut, int32_t* owner, uint64_t* slot_tags, const void* host_store,
                   const int32_t* blob_of, const void* shared_pool, int32_t* err_word,
                   void* workspace, size_t ws_bytes, hipStream_t compute_stream,
                   hipStream_t fill_stream);

/* moe_ctx_destroy: wait for both streams, free the context's buffers. */
int moe_ctx_destroy(moe_layer_ctx* ctx);

/* moe_ctx_place: copy (layer, expert) into an empty or reusable slot before
 * the first step (initial residency); the expert must not be resident. */
int moe_ctx_place(moe_layer_ctx* ctx, int slot, int layer, int expert);

/* moe_layer_forward: one step of layer `layer` on T tokens (T <= t_max).
 *   x         [T,H] device, x_dtype
 *   w_router  [E,H] device, x_dtype; bias [E] fp32 device or NULL
 *   out       [T,H] device in out_dtype (MOE_F32 or MOE_BF16)
 *   stats     host int32[4] or NULL: distinct routed experts, hits, fills, waves
 *             of this step; -1 for the first two when the layer was fully
 *             resident (the step did not wait for its routed set; the
 *             counters of moe_ctx_counters include it once it completed)
 * Returns after enqueuing the step. A layer with a non-resident expert waits
 * for its routed set (the residency plan needs it); a fully resident layer
 * does not wait, and its LRU bookkeeping is replayed, in step order, before
 * the next plan, moe_ctx_read_tables or moe_ctx_counters. */
int moe_layer_forward(moe_layer_ctx* ctx, int layer, const void* x, int T, const void* w_router,
                      const float* bias, void* out, int out_dtype, int32_t* stats);

/* moe_ctx_forward_steps: n layer steps in order, exactly as n calls of
 * moe_layer_forward (stats NULL) would run them; host arrays of length n hold
 * each step's layer and device pointers (bias entries may be NULL). One call
 * for a whole stack step keeps the host ahead of the GPU. Stops at the first
 * step that fails and returns its status. */
int moe_ctx_forward_steps(moe_layer_ctx* ctx, int n, const int32_t* layers, const void* const* xs,
                          int T, const void* const* w_routers, const float* const* biases,
                          void* const* outs, int out_dtype);

/* moe_ctx_read_tables: host copies of the tables as the plan left them
 * (lut [L*E], owner [S], last_use [S], clock [1]); any pointer may be NULL.
 * Waits for the routed sets of earlier steps whose bookkeeping was deferred. */
int moe_ctx_read_tables(moe_layer_ctx* ctx, int32_t* lut, int32_t* owner, int64_t* last_use,
                        int64_t* clock);

/* moe_ctx_counters: totals over all steps so far (waits like
 * moe_ctx_read_tables): out[0] distinct routed experts, out[1] hits,
 * out[2] fills, out[3] fill waves. */
int moe_ctx_counters(moe_layer_ctx* ctx, int64_t* out);

/* moe_ctx_outputs: device buffers of the last step, inside the workspace
 * (logits [T,E], topk ids and weights [T,k], perm, offsets [E+1], inv); any
 * pointer may be NULL. */
int moe_ctx_outputs(const moe_layer_ctx* ctx, float** logits, int32_t** ids, float** topk_w,
                    int32_t** perm, int32_t** offsets, int32_t** inv);

/* moe_ctx_set_policy: eviction policy of the context's residency plans
 * (MOE_POLICY_LRU, MOE_POLICY_MRS or MOE_POLICY_HISTORY, include/moe_offload.h;
 * window and params as for moe_policy_observe, params NULL unless HISTORY).
 * Steps already enqueued are booked under the previous policy first; the
 * policy's history starts empty. With a policy other than LRU every step also
 * computes the experts' routing scores (softmax over each token's logits,
 * averaged over the step's tokens) into its pinned staging, and each plan
 * records them (moe_policy_observe) before choosing victims
 * (moe_plan_fills_policy). Allocates the policy state (host) here, not per
 * step. Under device orchestration any policy with window <= 16 (the
 * device history is cleared). MOE_EINVAL on bad arguments. */
int moe_ctx_set_policy(moe_layer_ctx* ctx, int policy, int window, const double* params);

/* moe_ctx_step_scores: the routing scores [E] (host floats) of the latest
 * step, waiting for that step's router; MOE_EINVAL under LRU without split
 * precision, or before any step. */
int moe_ctx_step_scores(moe_layer_ctx* ctx, float* scores);

/* moe_ctx_set_split: split-precision routing for a context over
 * MOE_INT4G128_RESPLIT experts (RapidMoE Algorithm 1 with the threshold of
 * Eqs. (3)-(5)). With enable = 1 every step computes the experts' routing
 * scores (moe_step_scores) and runs routed expert e of layer l on its
 * high-precision weights W^H when score[e] >= theta * beta[l] * gamma (the
 * product in double, rounded to float; beta NULL = 1 for every layer), else on
 * W^L (moe_critical_split); shared experts always run on W^H. gamma is the
 * phase factor, 1 for prefill and alpha for decode: call again to switch
 * phase. With enable = 0 (the default) every group runs on W^H. Applies to
 * steps enqueued from now on. MOE_EINVAL unless the context's weights are
 * MOE_INT4G128_RESPLIT (enable = 1) or the constants are finite. */
int moe_ctx_set_split(moe_layer_ctx* ctx, int enable, float theta, const float* beta,
                      float gamma);

/* moe_ctx_set_staging: prefill full-layer staging (MoE-CORE summary page,
 * Mechanism). Two staging buffers, each holding every routed expert of one
 * layer, live in the pool after the routed and shared slots: buffer b holds
 * expert e in slot S + n_shared + b*E + e (the pool allocation must hold
 * pool_slots >= S + n_shared + 2E slots; the caller owns it). With enable = 1
 * a step of layer l whose layer is not wholly resident and whose token count
 * T >= threshold (threshold = -1: floor(K_l / k), K_l = the decode cache's
 * slots holding layer l's experts) runs every routed expert from the buffer
 * holding layer l, loading it first (one copy per run of consecutive weight
 * sets, on the fill stream, after the compute that last read the buffer);
 * once the step's compute is enqueued the other buffer starts loading the
 * next layer (l + 1 mod L, or the next layer given to moe_ctx_forward_steps).
 * A buffer that already holds the layer is not reloaded. Staged steps leave
 * the decode cache (tables, recency, policy history, counters) untouched;
 * their stats are -1. Not with device orchestration (MOE_EINVAL). The first
 * enable writes the buffers' [2E] slot table into the workspace and creates four
 * events. */
int moe_ctx_set_staging(moe_layer_ctx* ctx, int enable, int threshold, int pool_slots);

/* moe_ctx_stage_counters: out[0] staged steps, out[1] experts copied into the
 * staging buffers, since creation. */
int moe_ctx_stage_counters(moe_layer_ctx* ctx, int64_t* out);

/* moe_ctx_set_prefetch: miss prefetch (MoE-CORE summary page, Mechanism).
 * Within moe_ctx_forward_steps, a step whose next step's layer is not wholly
 * resident also evaluates the next step's router on its own tokens (before the
 * next step's real input exists) and prefetches the top predicted experts that
 * are not resident: moe_plan_prefetch after the step's own plan, with window
 * t_remain_us + t_attn_us - t_launch_us (the caller's estimates of the
 * remaining compute of this layer, the attention of the next one, and the
 * launch overhead, in microseconds) and bw_gbs the host-to-device bandwidth.
 * Each copy (slot_prefetch) starts on the fill stream behind the step's own
 * fills, as soon as the compute enqueued before this step's expert FFN has
 * finished, so it overlaps that FFN; the compute stream commits it by tag at
 * the end of the step, before the next step. Host orchestration only (steps
 * under device orchestration or full-layer staging do not prefetch), and a
 * step waits for the host to read the prediction. enable = 0 switches it off;
 * MOE_EINVAL for non-finite times or a bandwidth <= 0. */
int moe_ctx_set_prefetch(moe_layer_ctx* ctx, int enable, double t_remain_us, double t_attn_us,
                         double t_launch_us, double bw_gbs);

/* moe_ctx_prefetch_counters: out[0] experts prefetched, out[1] prefetched
 * experts that their layer's next step routed, since creation. */
int moe_ctx_prefetch_counters(moe_layer_ctx* ctx, int64_t* out);

/* moe_ctx_set_orchestration: where the residency plan runs.
 *   MOE_ORCH_HOST (default): the host plans each step that may miss, after
 *     reading the routed set, and the fills are copies on the fill stream (a copy
 *     kernel reading the mapped pinned store, else a copy-engine transfer).
 *   MOE_ORCH_DEVICE: the GPU plans and fills by itself and a step never waits
 *     for the host (SeqMoE summary page, Mechanism: the device owns the cache
 *     metadata and starts the miss copy from a kernel out of the pinned,
 *     mapped host pool). One workgroup runs the plan of moe_plan_fills (LRU)
 *     or moe_plan_fills_policy (Minus Recent Score or the routing-history
 *     score, window <= 16, its history recorded on the device as
 *     moe_policy_observe does, with the same arithmetic) on the device tables
 *     (identical tables and fills); a kernel then copies the missed experts
 *     from the host store (which must be hipHostMalloc memory the device can
 *     map) into their slots; the expert FFN and the combine follow on the
 *     compute stream. Needs S <= 4096 and a window <= 16; a step
 *     with T*k > S returns MOE_EUNSUPPORTED (switch back to the host to run
 *     it). The per-step stats of moe_layer_forward are -1 in this mode; the
 *     totals of moe_ctx_counters and the tables of moe_ctx_read_tables are
 *     read back from the device (a stream synchronisation).
 * Switching hands the tables over (host -> device: the slots' LRU order and
 * clock, and the policy's history; device -> host: everything). The device planner's state sits in
 * the workspace; the first switch to the device writes its weight set table
 * there. */
#define MOE_ORCH_HOST 0
#define MOE_ORCH_DEVICE 1
int moe_ctx_set_orchestration(moe_layer_ctx* ctx, int mode);

/* moe_ctx_set_timing: when enabled, each step records HIP events on the
 * compute stream around its expert FFN calls (the routed groups, including
 * any fill waves, then the shared experts); moe_ctx_ffn_time
 * returns the summed milliseconds and the number of timed steps (resetting
 * happens on moe_ctx_set_timing). */
int moe_ctx_set_timing(moe_layer_ctx* ctx, int enable);
int moe_ctx_ffn_time(moe_layer_ctx* ctx, double* total_ms, long* steps);

#ifdef __cplusplus
}
#endif
#endif /* MOE_RUNTIME_H */
