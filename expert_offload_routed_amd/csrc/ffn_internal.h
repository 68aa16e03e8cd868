// Internal layouts shared by the host code of the FFN and slot sources.
#pragma once

#include <atomic>

#include <stddef.h>
#include <stdint.h>

// One routed expert group of the permuted assignments.
struct FfnItem {
  int32_t expert;
  int32_t slot;
  int32_t row_begin;  // first sorted position of the group
  int32_t rows;       // assignments in the group
};

// One M-tile of a large group for the MFMA GEMM path.
struct GemmTile {
  int32_t expert;
  int32_t slot;
  int32_t row_begin;  // first sorted position of the tile
  int32_t rows;       // rows in the tile (<= kGemmBM)
};

constexpr int kGemmBM = 128;     // rows of an MFMA M-tile
constexpr int kGemvMaxRows = 4;  // groups up to this many rows take the GEMV path
// bf16 or int4 with two or more tokens: groups up to this many rows take the MFMA GEMV
// (skinny.hip)
constexpr int kSkinnyMaxRows = 32;
constexpr int kSkinnyGridCap = 16384;  // workgroups of a skinny pass (they loop over units)

// Byte layout of one expert inside a slot (see moe_slot_layout).
struct SlotLayout {
  size_t slot_bytes, off_w13, off_w2, off_s13, off_s2;
  size_t off_r13, off_rs13, off_h2, off_hs2;  // MOE_INT4G128_RESPLIT only (else 0)
};

// Sections of the moe_expert_ffn workspace (byte offsets).
struct FfnWorkspace {
  size_t sync;  // kStreamMaxItems int32 counters, zeroed by whichever kernel writes the work list
  size_t items, tiles, h, xq, xs, hq, hs, total;
  int max_tiles;
};

// One-token int4 passes over even shares of row blocks (decode_int4.hip)
constexpr int kStreamMaxItems = 64;  // groups of a one-token call they take
bool decode_int4_fits(int max_items, int R, int K, bool swiglu);
// Both one-token int4 passes in one launch, handing h over through the sync counters
// (zero at launch); MOE_EUNSUPPORTED when the call does not fit it.
int launch_decode_int4_fused(const void* x, const FfnItem* items, const int32_t* n_items,
                             int max_items, const char* pool,
                             size_t stride, size_t off_w13, size_t off_s13, size_t off_w2,
                             size_t off_s2, int H, int F, float* hbuf, float* y, int32_t* sync,
                             int32_t* err, hipStream_t s);

// The bf16 counterparts (decode_bf16.hip): h is bf16 (rows of F values), y fp32.
bool decode_bf16_fits(int max_items, int R, int K, bool swiglu);
int launch_decode_bf16_fused(const void* x, const FfnItem* items, const int32_t* n_items,
                             int max_items, const char* pool,
                             size_t stride, size_t off_w13, size_t off_w2, int H, int F,
                             void* hbuf, float* y, int32_t* sync, int32_t* err, hipStream_t s);
int launch_decode_bf16(bool swiglu, const void* raw, const FfnItem* items,
                       const int32_t* n_items, int max_items,
                       const char* pool, size_t stride, size_t off_w, int R, int K, int out_ld,
                       void* out, hipStream_t s);

static inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Copy of `bytes` (a multiple of 16, both addresses 16-byte aligned) from pinned host memory,
// read through its device address src_dev, to device memory dst: a copy kernel on `stream`
// (slots.hip). MOE_EINVAL when the sizes or alignments do not fit it.
int launch_host_copy(void* dst, const void* src_dev, size_t bytes, hipStream_t stream);

int slot_layout(int H, int F, int w_dtype, SlotLayout* out);

#include <hip/hip_runtime.h>
// The FFN work list: groups of <= small_max rows as FfnItem, the others cut
// into kGemmBM-row GemmTile (see ffn_plan_kernel in ffn.hip).
void launch_ffn_plan(const int32_t* offsets, const int32_t* lut, const int32_t* mask, int E,
                     int n_shared, int shared_slot0, int num_slots, int small_max, FfnItem* items,
                     int32_t* n_items, GemmTile* tiles, int32_t* n_tiles, int32_t* err_word,
                     int32_t* sync, hipStream_t s);
// One one-token int4 pass over the work list's items: the call's row blocks in one even
// share per workgroup (pass 1 with the SwiGLU epilogue from the bf16 tokens; pass 2 from
// the fp32 h rows). MOE_EUNSUPPORTED when a share would exceed 16 row blocks.
int launch_decode_int4(bool swiglu, const void* raw, const FfnItem* items,
                       const int32_t* n_items, int max_items,
                       const char* pool, size_t stride, size_t off_codes, size_t off_scales, int R,
                       int K, int out_ld, float* out, hipStream_t s);
// Workgroups of kernel `kern` resident at once on the current device (occupancy with
// `threads` threads and `lds` bytes of dynamic LDS, times the compute units). `cache`,
// one per kernel instantiation, keeps the occupancy for the last LDS size.
long long resident_workgroups(const void* kern, int threads, size_t lds,
                              std::atomic<long long>& cache);
// Largest group that takes the GEMV path (0: every group takes the MFMA tiles).
int ffn_small_max(int T, int k, int E, int n_shared, int w_dtype);
// One bf16 pass over the work list's items on MFMA (groups of up to kSkinnyMaxRows rows):
// pass 1 reads tokens act[perm[p] / k] and writes h = SiLU(gate) * up (bf16), pass 2
// reads h rows p and writes y (fp32); weights at slot + off, [R, K] tile-major.
void launch_skinny_bf16(int pass, const void* act, const int32_t* perm, int k,
                        const FfnItem* items, const int32_t* n_items, int max_items,
                        const char* pool, size_t stride, size_t off, int R, int K, int out_ld,
                        void* out, hipStream_t s);
// The same over int4 weights (codes at off_codes, group scales at off_scales) with int8 rows
// aq and their scales as (pass 1: tokens perm[p] / k, pass 2: h rows p); out is fp32 (pass 1:
// h = SiLU(gate) * up, pass 2: y).
void launch_skinny_w4a8(int pass, const int8_t* aq, const float* as, const int32_t* perm, int k,
                        const FfnItem* items, const int32_t* n_items, int max_items,
                        const char* pool, size_t stride, size_t off_codes, size_t off_scales,
                        int R, int K, int out_ld, float* out, hipStream_t s);
void launch_gemm_bf16(int pass, const void* act, const int32_t* perm, int k, const GemmTile* tiles,
                      const int32_t* n_tiles, int max_tiles, const char* pool, size_t stride,
                      size_t off, int N, int K, int out_ld, void* out, hipStream_t s);
// Workspace of a call over T tokens with E routed experts (k per token) and
// n_shared shared experts carried as extra groups.
FfnWorkspace ffn_workspace_layout(int T, int H, int F, int E, int k, int w_dtype, int n_shared);
// Expert FFN work list for the decode front end to write: routed groups
// through `lut` (E entries) and n_shared shared groups (T rows each after the
// T*k routed rows, slots shared_slot0 + s), groups of <= small_max rows as
// items, the others as kGemmBM-row tiles, into the FFN workspace's lists.
struct FrontPlan {
  float* scores;  // when set: each expert's softmax probability averaged over the tokens [E]
  int32_t* crit;  // when set with scores: group precision [E], 2 if scores[e] >= crit_threshold
                  // (split-precision experts at high precision), else 1
  float crit_threshold;
  const int32_t* lut;  // when set: write the FFN work list below
  int num_slots, n_shared, shared_slot0, small_max;
  FfnItem* items;
  int32_t* n_items;
  GemmTile* tiles;
  int32_t* n_tiles;
  int32_t* err;
  int32_t* sync;  // when set with lut: the FFN's kStreamMaxItems hand-off counters, zeroed
};
// moe_route_permute that, on its one-launch path, also writes the expert FFN's
// work list described by *plan when plan->lut is set (*planned = true; otherwise
// the FFN plans) and the routing scores when plan->scores is set (*scored =
// true; otherwise the caller computes them).
int route_permute_plan(const void* x, int x_dtype, const void* w_router, const float* bias, int T,
                       int H, int E, int k, int renorm, float* logits, int32_t* topk_ids,
                       float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv, int32_t* distinct, int32_t* n_distinct,
                       uint32_t* sync_counter, const FrontPlan* plan, bool* planned,
                       bool* scored, hipStream_t stream);
// moe_expert_ffn with the shared experts as groups E .. E+n_shared-1: offsets
// has E + n_shared + 1 entries, group E + s holds T rows (perm value t * k for
// token t) and reads slot shared_slot0 + s; group_mask applies to routed groups.
int expert_ffn(const void* x, int x_dtype, const int32_t* perm, const int32_t* offsets,
               const int32_t* lut, const int32_t* group_mask, int n_shared, int shared_slot0,
               const void* pool_base, size_t slot_stride, int num_slots, int w_dtype, int T, int H,
               int F, int E, int k, float* y_perm, int32_t* err_word, void* workspace,
               size_t ws_bytes, hipStream_t stream, bool planned = false);
// The routing score of every expert at one step (moe_step_scores) on stream s.
void launch_step_scores(const float* logits, int T, int E, float* scores, hipStream_t s);
// moe_critical_split on stream s (arguments checked by the caller).
void launch_critical_split(const float* scores, int E, float threshold, const int32_t* mask_in,
                           int rows, int32_t* mask_out, hipStream_t s);
