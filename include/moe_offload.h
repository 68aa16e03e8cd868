/*
 * moe_offload.h - C ABI of the routed-expert MoE layer over a device-resident
 * expert slot cache, for AMD Instinct MI355X (gfx950).
 *
 * The layer, as the source pages define it:
 *   - gating: a linear projection of the token, softmax, and the top-k experts
 *     by logit ("RapidMoE: Exploiting Cross-Asymmetry via Adaptive Residual
 *     Offloading for Large-Scale MoE Inference", Sec. 2.1);
 *   - output: the sum over the selected experts of the normalised routing
 *     weight times the expert's output ("Communication-Aware Placement and
 *     Pruning for Efficient Mixture-of-Experts Inference", Sec. II-A, Eq. (1);
 *     RapidMoE Algorithm 1);
 *   - expert: a SwiGLU FFN, down(SiLU(gate x) * up x) (RapidMoE Eq. (7));
 *   - residency: one pool of expert slots at a fixed base address, shared by
 *     every MoE layer, and a table that rewrites expert_id to slot_id so the
 *     expert kernel always sees the same layout; misses are copied from a
 *     pinned host pool, and a per-slot monotonically increasing tag decides
 *     whether a copied expert may be committed (SeqMoE summary page,
 *     Mechanism); only routed experts are cached, shared experts stay
 *     resident (SeqMoE and HybriMoE summary pages, Mechanism).
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless the comment says "host".
 *   - The caller owns all memory passed in; the library keeps no pointer after
 *     the call returns (except that enqueued work reads/writes them later).
 *   - Calls only enqueue work on the given stream(s) and return; they never
 *     synchronise the device, except the host-only helpers.
 *   - Return value: MOE_OK (0), MOE_EINVAL (-1) invalid argument (nothing was
 *     enqueued), MOE_EUNSUPPORTED (-2) dtype/shape this build does not
 *     support, MOE_EHIP (-3) a HIP runtime error (the HIP error is consumed).
 *   - Faults found on the device are OR-ed into a caller-owned int32 error
 *     word (MOE_ERR_* bits); kernels never trap.
 *   - No mutable global state: calls on different streams may run
 *     concurrently as long as their buffers do not overlap.
 *   - Row-major layouts; T tokens, H hidden size, F expert FFN size, E routed
 *     experts per layer, k experts per token, S pool slots, L layers.
 */
#ifndef MOE_OFFLOAD_H
#define MOE_OFFLOAD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element formats */
enum {
  MOE_F32 = 0,      /* IEEE binary32 */
  MOE_BF16 = 1,     /* bfloat16 (upper half of binary32, round-to-nearest-even) */
  MOE_INT4G128 = 2,  /* expert weights only: signed 4-bit codes, one bf16 scale per
                        128 consecutive input values of an output row; with these
                        weights the activations are quantised per row to int8 */
  MOE_INT4G128_RESPLIT = 3  /* expert weights only: split precision (RapidMoE Sec. 4.4,
                        Algorithm 3): the MOE_INT4G128 weights W^Q of gate/up and
                        W^L of down, then the residual W^R = int4(W - W^Q) of gate/up
                        and down at 8 bits (W^H); see moe_slot_layout */
};

/* status codes */
enum { MOE_OK = 0, MOE_EINVAL = -1, MOE_EUNSUPPORTED = -2, MOE_EHIP = -3 };

/* device error-word bits */
#define MOE_ERR_ABSENT 1    /* a routed expert had no slot (table entry -1); its rows were skipped */
#define MOE_ERR_STALE_TAG 2 /* a commit found another tag in the slot; table left unchanged */
#define MOE_ERR_SYNC 4      /* a one-token expert FFN launch waited past its limit for h rows of
                               other workgroups (not all resident at once); its y is invalid */

/* ------------------------------------------------------------------ gating -
 * moe_route: router logits, top-k selection and routing weights.
 *   logits[t,e] = sum_h x[t,h] * w_router[e,h] + bias[e]        (fp32 accumulate)
 *   topk_ids[t,:] = the k experts with the largest logits, ordered by
 *                   (logit descending, expert id ascending)
 *   topk_w[t,j]   = softmax(logits[t,:])[ids[t,j]], divided by the sum over
 *                   the k selected when renorm != 0
 * (RapidMoE Sec. 2.1; CAP Eq. (1).) Selection is on the logits; the bias is
 * part of the logit.
 *   x         [T,H] in x_dtype (MOE_F32 or MOE_BF16)
 *   w_router  [E,H] in x_dtype; row e is expert e's projection vector
 *   bias      [E] fp32, may be NULL (no bias)
 *   logits    [T,E] fp32 out (required: it is the hand-off between the
 *             projection and the selection kernels)
 *   topk_ids  [T,k] int32 out; topk_w [T,k] fp32 out
 * Requires 1 <= k <= E <= 1024, H % 8 == 0, T >= 0 (T == 0 is a no-op).
 */
int moe_route(const void* x, int x_dtype, const void* w_router, const float* bias,
              int T, int H, int E, int k, int renorm,
              float* logits, int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* ------------------------------------------------------------- permutation -
 * moe_permute: counting sort of the T*k assignments by expert, stable in token
 * order, so each expert's rows form one contiguous block (the grouped layout
 * the expert kernel reads; SeqMoE Mechanism: the expert kernel sees a fixed,
 * contiguous layout).
 *   topk_ids   [T,k] int32, each row k distinct ids in [0,E)
 *   counts     [E] int32 out: assignments per expert
 *   offsets    [E+1] int32 out: exclusive prefix sum of counts
 *   perm       [T*k] int32 out: sorted position -> flat assignment t*k+j
 *   inv        [T*k] int32 out: flat assignment -> sorted position
 *   distinct   [E] int32 out: experts with count > 0, ascending (first n_distinct valid)
 *   n_distinct [1] int32 out
 * Requires 1 <= k <= E <= 1024, T*k < 2^31. Ids outside [0,E) are not
 * counted and leave their perm/inv entries unwritten.
 */
int moe_permute(const int32_t* topk_ids, int T, int k, int E,
                int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                int32_t* distinct, int32_t* n_distinct, hipStream_t stream);

/* moe_route_permute: moe_route followed by moe_permute (same arguments and
 * outputs). For decode batches (T <= 16 and T*k <= 1024) both run in one
 * launch: the workgroups that compute the logits count themselves on
 * sync_counter and the last one selects and sorts; otherwise the two calls
 * are made in turn.
 *   sync_counter  [1] uint32 device; zero before the first call, and every
 *                 call leaves it zero (calls sharing it must not overlap)
 */
int moe_route_permute(const void* x, int x_dtype, const void* w_router, const float* bias,
                      int T, int H, int E, int k, int renorm,
                      float* logits, int32_t* topk_ids, float* topk_w,
                      int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                      int32_t* distinct, int32_t* n_distinct, uint32_t* sync_counter,
                      hipStream_t stream);

/* ------------------------------------------------------------- slot layout -
 * The byte layout of one expert inside a slot (and inside the pinned host
 * store, which holds the same bytes so a fill is one contiguous copy). The
 * slot pool is one allocation: slot s starts at pool_base + s * slot_stride
 * (the fixed-base [num_slots, dim0, dim1] pool of the SeqMoE page).
 * Two matrices: W13 [2F, H] (row 2n = gate row n, row 2n+1 = up row n) at
 * off_w13 and W2 [H, F] (down projection) at off_w2, each in a layout that
 * depends on the format:
 *   MOE_F32:      row-major.
 *   MOE_BF16:     tile-major: element (r, c) of W [R, K] is bf16 number c % 8
 *                 of the 16 bytes of lane (r % 32) + 32 ((c % 16) / 8) in the
 *                 1 KB chunk (r / 32) * (K / 16) + c / 16. A chunk is the
 *                 operand fragment of one 32x32x16 bf16 MFMA, and the chunks
 *                 of a 32-row block are consecutive (R % 32 == 0).
 *   MOE_INT4G128: tile-major: chunk (r / 32) * (K / 64) + c / 64 of 1 KB;
 *                 lane (r % 32) + 32 ((c % 32) / 16) holds 16 bytes; bytes
 *                 [8h, 8h + 8) hold the 16 codes of the 32-wide k step
 *                 h = (c % 64) / 32; each 4-byte word covers 8 consecutive
 *                 codes c0..c7 with byte i = c_i (low nibble) | c_{i+4} (high
 *                 nibble). Scales: s13 at off_s13, [2F, H/128] bf16 row-major
 *                 (rows as W13); s2 at off_s2, [H, F/128].
 *   MOE_INT4G128_RESPLIT: the four MOE_INT4G128 sections at the same offsets
 *                 (so a slot of this format is also a MOE_INT4G128 slot, read
 *                 at the low precision), then the residual of W13 as int4 in
 *                 the same layout at off_r13 with scales [2F, H/128] at
 *                 off_rs13, and W2 at 8 bits at off_h2: signed bytes,
 *                 tile-major, chunk (r / 32) * (K / 32) + c / 32 of 1 KB, lane
 *                 (r % 32) + 32 ((c % 32) / 16), byte c % 16 of its 16; scales
 *                 [H, F/128] bf16 at off_hs2 (moe_slot_layout_resplit).
 * Every section starts on a 256-byte boundary; slot_bytes is a multiple of 4096.
 * Returns MOE_EINVAL for a bad format or sizes (H, F multiples of 16; H of 32
 * for bf16; both of 128 for int4).
 */
int moe_slot_layout(int H, int F, int w_dtype, size_t* slot_bytes,
                    size_t* off_w13, size_t* off_w2, size_t* off_s13, size_t* off_s2);

/* The four extra sections of a MOE_INT4G128_RESPLIT slot (see above). */
int moe_slot_layout_resplit(int H, int F, size_t* off_r13, size_t* off_rs13, size_t* off_h2,
                            size_t* off_hs2);

/* moe_pack_expert_host (host only, not on the hot path): write one expert in
 * the slot layout into dst (host, slot_bytes). Inputs are host arrays in
 * nn.Linear orientation: gate, up [F,H], down [H,F] as fp32/bf16 values, or
 * for int4 packed codes gate, up [F,H/2], down [H,F/2] bytes plus bf16 scales
 * gate_s, up_s [F,H/128], down_s [H,F/128] (NULL for dense formats). */
int moe_pack_expert_host(const void* gate, const void* up, const void* down,
                         const void* gate_s, const void* up_s, const void* down_s,
                         int H, int F, int w_dtype, void* dst);

/* moe_quantize_resplit_host (host only, not on the hot path): quantise one
 * expert from float32 weights gate, up [F,H] and down [H,F] (nn.Linear
 * orientation) into a MOE_INT4G128_RESPLIT slot at dst (slot_bytes), following
 * RapidMoE Algorithm 3 with b_q = b_r = 4:
 *   quant_b(w), per row and group of 128 inputs: s = bf16(max|w| / (2^(b-1)-1))
 *     (float32 division, round to nearest even), q = clip(rint(w / s),
 *     -2^(b-1), 2^(b-1)-1) with the division in float32, q = 0 where s = 0;
 *   gate, up:  W^Q = quant_4(W),  W^R = quant_4(W - q s)  (float32 residual);
 *   down:      W^L = quant_4(W),  W^H = quant_8(W).
 * Returns MOE_EINVAL for bad sizes (H, F multiples of 128). */
int moe_quantize_resplit_host(const float* gate, const float* up, const float* down, int H, int F,
                              void* dst);

/* moe_critical_split: the precision of every expert group at one step
 * (RapidMoE Eq. (4) with Algorithm 1): an expert is critical when its routing
 * score is at least threshold, the score being its router probability
 * averaged over the step's tokens (the mean of the softmax of each token's
 * logits, moe_step_scores) and threshold = Theta * beta(l) * gamma(t) (Eqs.
 * (3), (5)), computed by the caller. For r in [0, rows), e in [0, E):
 *   mask_out[r*E + e] = 0                            if mask_in && mask_in[r*E + e] == 0
 *                       2 if scores[e] >= threshold  (critical: W^H)
 *                       1 otherwise                  (W^L)
 * i.e. a moe_expert_ffn group mask for MOE_INT4G128_RESPLIT weights. scores
 * [E] float32, mask_in (NULL: every group) and mask_out [rows, E] int32, all
 * device; mask_out may equal mask_in. The comparison is float32. Enqueued on
 * stream. */
int moe_critical_split(const float* scores, int E, float threshold, const int32_t* mask_in,
                       int rows, int32_t* mask_out, hipStream_t stream);

/* moe_step_scores: the router probabilities of every expert averaged over the
 * step's T tokens, from the logits [T,E] (float32) of moe_route; scores [E]
 * float32 out (device). Enqueued on stream. */
int moe_step_scores(const float* logits, int T, int E, float* scores, hipStream_t stream);

/* --------------------------------------------------------------- expert FFN -
 * moe_ffn_workspace_bytes: device workspace moe_expert_ffn needs for these
 * sizes (work list, SwiGLU intermediate, int8 activations).
 */
size_t moe_ffn_workspace_bytes(int T, int H, int F, int E, int k, int w_dtype);

/* moe_ffn_workspace_offsets: where moe_expert_ffn keeps its intermediates
 * inside the workspace, as byte offsets (0 where the weight format has none):
 *   offs[0] h  [T*k, F] fp32: SwiGLU intermediate of sorted position p (row p)
 *   offs[1] xq [T, H] int8 and offs[2] xs [T] fp32: int8 codes and row scales
 *           of the tokens (MOE_INT4G128 weights)
 *   offs[3] hq [T*k, F] int8 and offs[4] hs [T*k] fp32: the same for h
 * With MOE_INT4G128 weights xq/xs/hq/hs are written by calls that run MFMA
 * tiles or the MFMA GEMV (T >= 2); a one-token call quantises inside the GEMV
 * workgroups' LDS and leaves them unwritten, and h holds fp32 values only for
 * rows of computed groups. Host-only; offs is a host array of 5 entries.
 * Returns MOE_EINVAL for bad sizes or formats. */
int moe_ffn_workspace_offsets(int T, int H, int F, int E, int k, int w_dtype, size_t* offs);

/* moe_quantize_rows_int8: the int8 activation rows that int4 weights meet
 * (the int4 workload's W4A8 definition: per-row symmetric int8), as a stage
 * of its own. For each row r of in [rows, K]:
 *   s[r] = max_c |in[r,c]| / 127 (IEEE fp32 division), or 1 for a zero row
 *   q[r,c] = clip(rint(in[r,c] / s[r]), -127, 127)   (round to nearest even)
 * the rule moe_expert_ffn applies to the tokens and to the SwiGLU
 * intermediate before each int4 projection.
 *   in   [rows, K] in in_dtype (MOE_F32 or MOE_BF16), 16-byte aligned
 *   q    [rows, K] int8 out; s [rows] fp32 out
 * Requires K % 8 == 0, 8 <= K <= 8192; rows == 0 is a no-op. Enqueued on
 * stream. */
int moe_quantize_rows_int8(const void* in, int in_dtype, int rows, int K, int8_t* q, float* s,
                           hipStream_t stream);

/* moe_expert_ffn: grouped SwiGLU FFN of every routed expert group, reading the
 * expert's weights through the slot table (SeqMoE Mechanism; RapidMoE Eq. (7)):
 *   for each expert e with offsets[e] < offsets[e+1] and group_mask[e] != 0:
 *     slot = lut[e]; W = pool_base + slot * slot_stride (moe_slot_layout)
 *     for each sorted position p in [offsets[e], offsets[e+1]):
 *       x_p = x[perm[p] / k]
 *       y_perm[p] = down(SiLU(gate x_p) * up x_p)            (fp32)
 *   x         [T,H] tokens in x_dtype (MOE_F32 or MOE_BF16)
 *   perm, offsets from moe_permute
 *   lut       [E] int32: this layer's row of the expert->slot table (-1 = absent)
 *   group_mask [E] int32 or NULL (NULL = every routed expert); lets a caller
 *             run resident experts while misses are still being copied
 *   pool_base, slot_stride, num_slots: the slot pool; w_dtype the weight format
 *   y_perm    [T*k,H] fp32 out: rows of skipped groups are left untouched
 *   err_word  [1] int32: MOE_ERR_ABSENT is OR-ed in when a selected group's
 *             lut entry is -1 or not below num_slots (that group is skipped);
 *             MOE_ERR_SYNC when the one-token int4 launch (both passes in one
 *             launch, one workgroup per compute unit) could not hand h over
 *             between its workgroups within its wait limit, as when another
 *             kernel holds compute units meanwhile (y_perm is then invalid)
 *   workspace device buffer of ws_bytes >= moe_ffn_workspace_bytes(...)
 * With MOE_INT4G128_RESPLIT, group_mask[e] picks the precision of routed
 * group e (RapidMoE Algorithm 1): 0 skips it, 1 runs it on W^L (the
 * MOE_INT4G128 sections), 2 on W^H (gate, up = W^Q + W^R, each int4 x int8
 * group product scaled and summed in fp32; down on its 8-bit codes); a NULL
 * mask runs every group on W^H. W^H groups always take the GEMV path (token
 * tiles of up to 4 rows; decode batch sizes), W^L groups the MOE_INT4G128
 * paths.
 * With MOE_INT4G128 the tokens and the SwiGLU intermediate are quantised per
 * row to int8 (scale = max|row| / 127, IEEE fp32 division, round to nearest
 * even) before the int4 x int8 products (int32 accumulation per 128 values,
 * scaled by the group scales in fp32).
 */
int moe_expert_ffn(const void* x, int x_dtype, const int32_t* perm, const int32_t* offsets,
                   const int32_t* lut, const int32_t* group_mask,
                   const void* pool_base, size_t slot_stride, int num_slots, int w_dtype,
                   int T, int H, int F, int E, int k,
                   float* y_perm, int32_t* err_word, void* workspace, size_t ws_bytes,
                   hipStream_t stream);

/* moe_expert_ffn_noalloc: moe_expert_ffn without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * kernels and results as moe_expert_ffn with n_shared = 0; the workspace is a
 * static device array of moe_noalloc_scratch_bytes() bytes (32 MB) inside the
 * library, one copy per GPU, held until the process ends. The call allocates
 * nothing; its first call on a device looks up that device's copy of the array
 * (a host-side query, no allocation). Sizes whose moe_ffn_workspace_bytes
 * exceed the array return MOE_EINVAL (decode batches fit: e.g. 32 tokens of
 * the 7168 x 2048 int4 expert shape need about 6 MB). Every call on a GPU
 * shares that GPU's array: calls whose execution overlaps on one GPU (other
 * streams, other threads) race and must not be issued; calls in order on one
 * stream are safe. The array keeps the last call's contents; each call writes
 * or clears everything it reads. */
int moe_expert_ffn_noalloc(const void* x, int x_dtype, const int32_t* perm,
                           const int32_t* offsets, const int32_t* lut,
                           const int32_t* group_mask, const void* pool_base, size_t slot_stride,
                           int num_slots, int w_dtype, int T, int H, int F, int E, int k,
                           float* y_perm, int32_t* err_word, hipStream_t stream);

/* moe_noalloc_scratch_bytes: size of the static array moe_expert_ffn_noalloc
 * uses as its workspace (host-only query). */
size_t moe_noalloc_scratch_bytes(void);

/* ------------------------------------------------------------------ combine -
 * moe_combine: weighted sum of the routed experts' outputs (RapidMoE Sec. 2.1,
 * Algorithm 1; CAP Eq. (1)) plus the always-on shared experts (weight 1):
 *   out[t,:] = sum_{j<k, topk_w[t,j] != 0} topk_w[t,j] * y_perm[inv[t*k+j],:]
 *            + sum_{s<n_shared} shared_y[s,t,:]
 * accumulated in fp32 in this fixed order (deterministic; a zero weight
 * skips its term, so a NaN in an unused row cannot reach the output).
 *   shared_y  [n_shared,T,H] fp32 or NULL (n_shared ignored when NULL)
 *   out       [T,H] in out_dtype (MOE_F32, or MOE_BF16 rounded to nearest even)
 */
int moe_combine(const float* y_perm, const int32_t* inv, const float* topk_w,
                int T, int k, int H, const float* shared_y, int n_shared,
                void* out, int out_dtype, hipStream_t stream);

/* ---------------------------------------------------------------- slot fill -
 * slot_fill: copy one expert from the pinned host store into a slot and
 * commit it into the table (SeqMoE Mechanism: pinned host pool, copy on a
 * separate stream, commit only when the slot's tag matches):
 *   fill_stream:    copy bytes host_src -> pool_base + slot*slot_stride;
 *                   then slot_tags[slot] = tag (the tag written back by this copy)
 *   compute_stream: waits for the copy, then commits:
 *                   if slot_tags[slot] == tag:
 *                      old = owner[slot]; if old >= 0 and lut[old] == slot: lut[old] = -1
 *                      lut[lut_index] = slot; owner[slot] = lut_index
 *                   else: table unchanged, MOE_ERR_STALE_TAG OR-ed into err_word
 *   host_src   host pointer into page-locked memory (hipHostMalloc or torch
 *              pin_memory); pageable memory is rejected with MOE_EINVAL
 *   lut        the whole table [L*E] int32; lut_index = layer*E + expert
 *   owner      [S] int32: lut index held by each slot, -1 = empty
 *   slot_tags  [S] uint64 (device)
 * The copy is ordered after earlier work on fill_stream only: the caller must
 * make fill_stream wait for any kernel that may still read this slot.
 * fill_stream may equal compute_stream.
 */
int slot_fill(void* pool_base, size_t slot_stride, int32_t slot,
              const void* host_src, size_t bytes,
              int32_t* lut, int32_t lut_index, int32_t* owner,
              uint64_t* slot_tags, uint64_t tag, int32_t* err_word,
              hipStream_t fill_stream, hipStream_t compute_stream);

/* slot_prefetch: the copy half of slot_fill, for a copy started before the
 * expert is known to be needed (MoE-CORE summary page, Mechanism: the next
 * layer's experts are predicted and copied ahead; SeqMoE summary page,
 * Mechanism: a per-slot tag is the only synchronisation between a copy and
 * its use):
 *   fill_stream: copy bytes host_src -> pool_base + slot*slot_stride;
 *                then slot_tags[slot] = tag
 * The table is not touched: the caller commits later with slot_commit(tag),
 * on the stream that will read the slot, after waiting for fill_stream. A
 * later fill of the same slot with a newer tag makes that commit a refused,
 * stale one (MOE_ERR_STALE_TAG), so a prefetch that lost its slot can never
 * point the table at another expert's bytes. host_src must be page-locked
 * (MOE_EINVAL otherwise). Arguments as in slot_fill. */
int slot_prefetch(void* pool_base, size_t slot_stride, int32_t slot, const void* host_src,
                  size_t bytes, uint64_t* slot_tags, uint64_t tag, hipStream_t fill_stream);

/* slot_commit: the commit step of slot_fill alone, on one stream, for a copy
 * whose tag was written back by other means (e.g. a prefetcher). Same rule
 * and same error bit as above. */
int slot_commit(int32_t* lut, int32_t lut_index, int32_t* owner, int32_t slot,
                const uint64_t* slot_tags, uint64_t tag, int32_t* err_word,
                hipStream_t stream);

/* ------------------------------------------------------- residency (host) -
 * moe_plan_fills (host only): least-recently-used residency plan for one
 * layer call. The pages name misses as the routed set minus the cached set
 * and LRU as the baseline replacement (HybriMoE summary page, Mechanism) but
 * give no hot-path victim rule; this is the plain one:
 *   U = distinct[0..n_distinct) (ascending), hits = U with lut[layer*E+e] >= 0,
 *   misses = the rest (ascending). Victims: empty slots (ascending id), then
 *   slots not holding a hit, by (last_use, slot id) ascending.
 *   |misses| <= |victims|: one wave, misses[i] -> victims[i].
 *   else: wave 0 = hits + the first S-|hits| misses (into the victims); each
 *   later wave takes up to S more misses into slots 0,1,2,...
 *   clock[0] += 1 once per call; every slot used gets last_use = clock.
 * State (host arrays, updated in place to the state after the last wave):
 *   lut [L*E] int32, owner [S] int32 (lut index or -1), last_use [S] int64,
 *   clock [1] int64.
 * Outputs (host): wave_of [E] int32 = wave in which expert e is computed, -1
 *   if not routed; is_hit [E] int32 = 1 for hits; fill_expert, fill_slot,
 *   fill_wave [n_distinct] int32 and n_fills; n_waves.
 * Returns MOE_EINVAL for bad sizes or ids (state untouched).
 */
int moe_plan_fills(int32_t* lut, int32_t* owner, int64_t* last_use, int64_t* clock,
                   int S, int L, int E, int layer,
                   const int32_t* distinct, int n_distinct,
                   int32_t* wave_of, int32_t* is_hit,
                   int32_t* fill_expert, int32_t* fill_slot, int32_t* fill_wave,
                   int32_t* n_fills, int32_t* n_waves);

/* ------------------------------------------------- miss prefetch (host) -
 * moe_prefetch_count: how many experts a prefetch copy can hide (MoE-CORE
 * summary page, Mechanism): floor(window_us * bw_gbs * 1000 / expert_bytes)
 * in float64, where window_us = remaining compute of the current layer plus
 * the attention of the next, minus the launch overhead (microseconds) and
 * bw_gbs the host-to-device bandwidth (GB/s); capped by free_slots; 0 when
 * the window or the bandwidth is not positive. */
int moe_prefetch_count(double window_us, double bw_gbs, size_t expert_bytes, int free_slots);

/* moe_plan_prefetch (host only): after the current step's plan, choose the
 * experts of the next step's layer `layer` to copy ahead. The next layer's
 * router evaluated on the current hidden state predicted the routed ids
 * pred_ids [n_pred] and the routing scores pred_scores [E] (softmax
 * probability averaged over the tokens). Candidates: the predicted experts not
 * resident in `layer`, by score descending, ties to the lower id. Free slots:
 * empty slots by id, then slots whose last use is before *clock (the current
 * step did not use them) and that hold no predicted expert of `layer`, in the
 * victim order of moe_plan_fills_policy. The first moe_prefetch_count(window,
 * bw, expert_bytes, free) candidates (at most all) take the free slots in
 * order: the tables move as for a fill, and the slot's last use becomes
 * *clock. Outputs fill_expert/fill_slot [n_fills] (E entries suffice). The
 * caller copies them (slot_prefetch) and commits each with slot_commit.
 * Arguments otherwise as moe_plan_fills_policy; MOE_EINVAL for bad sizes, ids
 * or parameters. */
int moe_plan_prefetch(int policy, const double* state, int window, const double* params,
                      int32_t* lut, int32_t* owner, int64_t* last_use, const int64_t* clock,
                      int S, int L, int E, int layer, const int32_t* pred_ids, int n_pred,
                      const float* pred_scores, double window_us, double bw_gbs,
                      size_t expert_bytes, int32_t* fill_expert, int32_t* fill_slot,
                      int32_t* n_fills);

/* ----------------------------------------------- eviction policies (host) -
 * Which cached expert to evict when a miss needs a slot. LRU is the plan of
 * moe_plan_fills. Two scores from the pages replace its victim order:
 *   MOE_POLICY_MRS: Minus Recent Score (HybriMoE summary page, Mechanism): the
 *     expert's routing scores over the last `window` steps of its layer (the
 *     current one included), summed oldest to newest, minus the newest one.
 *   MOE_POLICY_HISTORY: routing-history score (MoE-CORE summary page,
 *     Mechanism): params = {w_cnt, w_ema, w_score, w_fresh, lambda}, weights
 *     >= 0, 0 <= lambda <= 1. Features of expert e of a layer: cnt = times
 *     selected in the last `window` steps; ema <- lambda*ema + (1-lambda)*[selected]
 *     every step (from 0); score = its latest routing score; age = steps since
 *     its last selection (the step count if never). Each of cnt, ema, score is
 *     divided by its maximum over the layer's E experts (0 if that maximum is
 *     0); fresh = 1 - age / max age (1 if max age is 0). keep = w_cnt*cnt +
 *     w_ema*ema + w_score*score + w_fresh*fresh, summed in that order.
 * A routing score is the expert's softmax probability averaged over the
 * step's tokens (float). All policy arithmetic is float64 in the order given,
 * without contraction.
 */
#define MOE_POLICY_LRU 0
#define MOE_POLICY_MRS 1
#define MOE_POLICY_HISTORY 2

/* Doubles of policy state for L layers of E experts (0 for LRU or bad sizes).
 * The caller zero-fills it once; the layout is internal. */
size_t moe_policy_state_doubles(int policy, int L, int E, int window);

/* Record one step of `layer` into the policy state: scores [E] (host floats,
 * the step's routing scores) and the routed set distinct[0..n_distinct). A
 * no-op for LRU (state, scores may be NULL). Call it once per layer step,
 * before moe_plan_fills_policy for that step. Returns MOE_EINVAL for bad
 * sizes, ids or parameters (state untouched). */
int moe_policy_observe(int policy, double* state, int L, int E, int window, int layer,
                       const float* scores, const int32_t* distinct, int n_distinct,
                       const double* params);

/* moe_plan_fills with the slots not holding a hit ordered by (owner's keep
 * score under `policy`, last use, slot id) ascending: the lowest score is
 * evicted first; empty slots still come first. Policy LRU gives exactly
 * moe_plan_fills. state/window/params as for moe_policy_observe (not
 * modified); the other arguments, state updates and errors as
 * moe_plan_fills. */
int moe_plan_fills_policy(int policy, const double* state, int window, const double* params,
                          int32_t* lut, int32_t* owner, int64_t* last_use, int64_t* clock,
                          int S, int L, int E, int layer,
                          const int32_t* distinct, int n_distinct,
                          int32_t* wave_of, int32_t* is_hit,
                          int32_t* fill_expert, int32_t* fill_slot, int32_t* fill_wave,
                          int32_t* n_fills, int32_t* n_waves);

/* Library version string and the gfx target it was built for (host). */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_OFFLOAD_H */
