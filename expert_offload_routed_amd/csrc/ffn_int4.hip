// int4 group-128 weights with int8 per-row activations (moe_expert_ffn, MOE_INT4G128).
#include "common.h"
#include "ffn_internal.h"

int ffn_int4(const void* x, const int32_t* perm, const int32_t* offsets, const int32_t* lut,
             const int32_t* group_mask, const char* pool, size_t stride, int num_slots,
             const SlotLayout& lay, int T, int H, int F, int E, int k, float* y, int32_t* err,
             char* ws, const FfnWorkspace& wl, hipStream_t s) {
  return MOE_EUNSUPPORTED;
}
