// Internal layouts shared by the host code of the FFN and slot sources.
#pragma once

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

// Byte layout of one expert inside a slot (see moe_slot_layout).
struct SlotLayout {
  size_t slot_bytes, off_w13, off_w2, off_s13, off_s2;
};

// Sections of the moe_expert_ffn workspace (byte offsets).
struct FfnWorkspace {
  size_t items, tiles, h, xq, xs, xg, hq, hs, hg, total;
  int max_tiles;
};

static inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int slot_layout(int H, int F, int w_dtype, SlotLayout* out);

#include <hip/hip_runtime.h>
// The FFN work list: groups of <= small_max rows as FfnItem, the others cut
// into kGemmBM-row GemmTile (see ffn_plan_kernel in ffn.hip).
void launch_ffn_plan(const int32_t* offsets, const int32_t* lut, const int32_t* mask, int E,
                     int num_slots, int small_max, FfnItem* items, int32_t* n_items,
                     GemmTile* tiles, int32_t* n_tiles, int32_t* err_word, hipStream_t s);
void launch_gemm_bf16(int pass, const void* act, const int32_t* perm, int k, const GemmTile* tiles,
                      const int32_t* n_tiles, int max_tiles, const char* pool, size_t stride,
                      size_t off, int N, int K, int out_ld, void* out, hipStream_t s);
FfnWorkspace ffn_workspace_layout(int T, int H, int F, int E, int k, int w_dtype);
