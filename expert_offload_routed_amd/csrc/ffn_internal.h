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

// Byte layout of one expert inside a slot (see moe_slot_layout).
struct SlotLayout {
  size_t slot_bytes, off_w13, off_w2, off_s13, off_s2;
};

// Sections of the moe_expert_ffn workspace (byte offsets).
struct FfnWorkspace {
  size_t items, h, xq, xs, hq, hs, total;
};

static inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int slot_layout(int H, int F, int w_dtype, SlotLayout* out);
FfnWorkspace ffn_workspace_layout(int T, int H, int F, int E, int k, int w_dtype);
