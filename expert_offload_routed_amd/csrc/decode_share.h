// Pieces shared by the one-token expert passes over even shares of row blocks
// (decode_int4.hip, decode_bf16.hip): the workgroup shape, the cross-workgroup hand-off
// of the one-launch form, and the launch sizing that keeps that form's grid resident.
#pragma once

#include <atomic>

#include "common.h"

namespace decode_share {

constexpr int kDecNW = 16;                 // waves per workgroup
constexpr int kDecWgPerCu = 16 / kDecNW;  // workgroups resident per compute unit
constexpr int kDecP = 8;                   // weight chunks in flight per lane

// Cross-workgroup hand-off of the one-launch form (both passes in one kernel): the gate/up
// pass writes h with device-scope stores and, once they have completed, adds per group the
// row blocks it finished to signal[group]; the down pass waits, before it reads h (with
// device-scope loads), until wait[group] holds all 2F/32 row blocks of each group its share
// reads. A wait that passes spin_cap polls (workgroups not all resident) gives up and flags
// MOE_ERR_SYNC instead of hanging.
struct PassSync {
  int32_t* signal;
  const int32_t* wait;
  int wait_target;
  int32_t* err;
  int spin_cap;
};

// The share of row blocks [b0, b1) of this workgroup among the call's total_rb.
__device__ __forceinline__ void share_of(int total_rb, int& b0, int& b1) {
  b0 = (int)((long long)total_rb * blockIdx.x / gridDim.x);
  b1 = (int)((long long)total_rb * (blockIdx.x + 1) / gridDim.x);
}

// Down pass of the one-launch form: thread 0 polls the counts of groups g0..g1, then the
// workgroup meets (the h rows are read after this).
__device__ __forceinline__ void wait_groups(const PassSync& sy, int g0, int g1) {
  if (threadIdx.x == 0) {
    bool late = false;
    for (int g = g0; g <= g1; ++g) {
      int spins = 0;
      while (__hip_atomic_load(sy.wait + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
             sy.wait_target) {
        if (++spins > sy.spin_cap) {
          late = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (late) atomicOr(sy.err, MOE_ERR_SYNC);
  }
  __syncthreads();
}

// Gate/up pass of the one-launch form: every wave's device-scope h stores of the share have
// completed (vector-memory counter at zero) before the barrier, and the per-group counts of
// the share's row blocks [b0, b1) go out after it.
__device__ __forceinline__ void signal_groups(const PassSync& sy, int b0, int b1, int rbi) {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int g = b0 / rbi; g <= (b1 - 1) / rbi; ++g) {
      const int lo = g * rbi > b0 ? g * rbi : b0, hi = (g + 1) * rbi < b1 ? (g + 1) * rbi : b1;
      __hip_atomic_fetch_add(sy.signal + g, hi - lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// compute units of the current device (queried once)
inline int decode_cus() {
  static std::atomic<int> cus{0};
  int n = cus.load(std::memory_order_relaxed);
  if (n <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus.store(n, std::memory_order_relaxed);
  }
  return n;
}

// Dynamic LDS of a one-launch kernel with `stat` bytes of static LDS: 160 KB per unit, a
// workgroup's total above 160 / (kDecWgPerCu + 1) KB keeps one more off the unit, at most
// 160 / kDecWgPerCu KB lets kDecWgPerCu share it. 0 when `need` does not fit.
inline size_t resident_lds(size_t need, size_t stat) {
  const size_t lo = 160 * 1024 / (kDecWgPerCu + 1) + 1024, hi = 160 * 1024 / kDecWgPerCu - 512;
  size_t lds = need;
  if (lds + stat < lo) lds = lo - stat;
  return lds + stat > hi ? 0 : lds;
}

constexpr int kSpinCap = 1 << 16;  // polls before a wait gives up (about 0.1 s; a normal wait is a few)

}  // namespace decode_share
