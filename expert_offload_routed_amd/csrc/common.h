// Device helpers shared by the kernels of libmoe_offload (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_offload.h"

#define MOE_WAVE 64

// ----------------------------------------------------------- status plumbing
#define MOE_CHECK_ARG(cond)      \
  do {                           \
    if (!(cond)) return MOE_EINVAL; \
  } while (0)

static inline int moe_hip_status(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MOE_EHIP;
  }
  return MOE_OK;
}

// Check that the launches just enqueued were accepted.
static inline int moe_launch_status() { return moe_hip_status(hipGetLastError()); }

// --------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, MOE_WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, MOE_WAVE));
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, MOE_WAVE);
  return v;
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Lanes below this one whose bit is set in a 64-bit wave mask.
__device__ __forceinline__ int popc_below(uint64_t mask) {
  const uint32_t l = __lane_id();
  const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
  return __popcll(mask & below);
}

// One 16-byte vector of weights or activations.
struct __attribute__((aligned(16))) u32x4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

// Non-temporal 16-byte load for weights that are streamed once.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p));
  u32x4 r;
  r.x = v.x;
  r.y = v.y;
  r.z = v.z;
  r.w = v.w;
  return r;
}

// ------------------------------------------------------------------- scans
// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive scan over a workgroup of up to 1024 threads (s_wave: >= 33 ints of
// LDS); returns this thread's exclusive prefix and the total in *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nwaves = (blockDim.x + 63) >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = (lane < nwaves) ? s_wave[lane] : 0;
    const int winc = wave_inclusive_scan(w);
    if (lane < 16) s_wave[16 + lane] = winc - w;
    if (lane == 15) s_wave[32] = winc;
  }
  __syncthreads();
  const int r = s_wave[16 + wave] + inc - v;
  *total = s_wave[32];
  __syncthreads();
  return r;
}
