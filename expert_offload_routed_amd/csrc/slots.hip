// Slot pool layout, host packing, tagged slot fills and the host LRU plan.
//
// The SeqMoE summary page (Mechanism) gives the residency design: one pool of
// slots at a fixed base address shared by every MoE layer, a table rewriting
// expert_id to slot_id so the expert kernel's layout never changes, misses
// copied from a pinned host pool on a separate stream, and a monotonically
// increasing per-slot tag that the copy writes back; a copied expert is
// committed into the table only when the written-back tag equals the tag the
// commit expects, so a superseded copy never lands in the table.
//
// The HybriMoE summary page (Mechanism) defines misses as the routed set minus
// the cached set and uses LRU as the baseline replacement; moe_plan_fills is
// that baseline made precise (the pages give no hot-path victim rule).
#include <string.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "common.h"
#include "ffn_internal.h"

#ifndef MOE_VERSION_STRING
#define MOE_VERSION_STRING "moe_offload 0.1 gfx950"
#endif

// ------------------------------------------------------------------ layout --
int slot_layout(int H, int F, int w_dtype, SlotLayout* out) {
  if (H <= 0 || F <= 0 || H % 16 != 0 || F % 16 != 0) return MOE_EINVAL;
  SlotLayout l{};
  if (w_dtype == MOE_BF16 && H % 32 != 0) return MOE_EINVAL;  // 32-row tiles of W2
  if (w_dtype == MOE_F32 || w_dtype == MOE_BF16) {
    const size_t es = (w_dtype == MOE_F32) ? 4 : 2;
    l.off_w13 = 0;
    l.off_w2 = align_up((size_t)2 * F * H * es, 256);
    l.off_s13 = l.off_s2 = 0;
    l.slot_bytes = align_up(l.off_w2 + (size_t)H * F * es, 4096);
  } else if (w_dtype == MOE_INT4G128 || w_dtype == MOE_INT4G128_RESPLIT) {
    if (H % 128 != 0 || F % 128 != 0) return MOE_EINVAL;
    l.off_w13 = 0;
    l.off_w2 = align_up((size_t)2 * F * (H / 2), 256);
    l.off_s13 = align_up(l.off_w2 + (size_t)H * (F / 2), 256);
    l.off_s2 = align_up(l.off_s13 + (size_t)2 * F * (H / 128) * 2, 256);
    size_t end = l.off_s2 + (size_t)H * (F / 128) * 2;
    if (w_dtype == MOE_INT4G128_RESPLIT) {
      l.off_r13 = align_up(end, 256);                                 // int4 residual of W13
      l.off_rs13 = align_up(l.off_r13 + (size_t)2 * F * (H / 2), 256);  // its scales
      l.off_h2 = align_up(l.off_rs13 + (size_t)2 * F * (H / 128) * 2, 256);  // W2 at 8 bits
      l.off_hs2 = align_up(l.off_h2 + (size_t)H * F, 256);                // its scales
      end = l.off_hs2 + (size_t)H * (F / 128) * 2;
    }
    l.slot_bytes = align_up(end, 4096);
  } else {
    return MOE_EINVAL;
  }
  *out = l;
  return MOE_OK;
}

extern "C" int moe_slot_layout(int H, int F, int w_dtype, size_t* slot_bytes, size_t* off_w13,
                               size_t* off_w2, size_t* off_s13, size_t* off_s2) {
  SlotLayout l;
  const int rc = slot_layout(H, F, w_dtype, &l);
  if (rc != MOE_OK) return rc;
  if (slot_bytes) *slot_bytes = l.slot_bytes;
  if (off_w13) *off_w13 = l.off_w13;
  if (off_w2) *off_w2 = l.off_w2;
  if (off_s13) *off_s13 = l.off_s13;
  if (off_s2) *off_s2 = l.off_s2;
  return MOE_OK;
}

extern "C" int moe_slot_layout_resplit(int H, int F, size_t* off_r13, size_t* off_rs13,
                                       size_t* off_h2, size_t* off_hs2) {
  SlotLayout l;
  const int rc = slot_layout(H, F, MOE_INT4G128_RESPLIT, &l);
  if (rc != MOE_OK) return rc;
  if (off_r13) *off_r13 = l.off_r13;
  if (off_rs13) *off_rs13 = l.off_rs13;
  if (off_h2) *off_h2 = l.off_h2;
  if (off_hs2) *off_hs2 = l.off_hs2;
  return MOE_OK;
}

namespace {

// Tile-major bf16: element (r, c) of W [R, K] in 1 KB chunk (r / 32) * (K / 16) + c / 16,
// lane (r % 32) + 32 ((c % 16) / 8), element c % 8 of the lane's 16 bytes.
void pack_tiles_bf16(char* dst, const char* src_rows[], int R, int K) {
  const int nks = K / 16;
  for (int rb = 0; rb < R / 32; ++rb)
    for (int ks = 0; ks < nks; ++ks)
      for (int lane = 0; lane < 64; ++lane) {
        const int r = rb * 32 + (lane & 31);
        const int c = ks * 16 + 8 * (lane >> 5);
        memcpy(dst + ((size_t)(rb * nks + ks) * 64 + lane) * 16, src_rows[r] + (size_t)c * 2, 16);
      }
}

// Signed 4-bit code c of a row in the logical format (even index in the low nibble).
inline uint8_t code_at(const uint8_t* row, int c) { return (row[c >> 1] >> ((c & 1) * 4)) & 0xF; }

// Tile-major int4: chunk (r / 32) * (K / 64) + c / 64 of 1 KB; lane (r % 32) + 32 ((c % 32) / 16)
// holds 16 bytes: bytes [8 h, 8 h + 8) for the 16 codes of k-step half h = (c % 64) / 32; in each
// 4-byte word of 8 consecutive codes, byte i = code i (low nibble) | code i + 4 (high nibble).
void pack_tiles_int4(char* dst, const uint8_t* src_rows[], int R, int K) {
  const int nkc = K / 64;
  for (int rb = 0; rb < R / 32; ++rb)
    for (int kc = 0; kc < nkc; ++kc)
      for (int lane = 0; lane < 64; ++lane) {
        const uint8_t* row = src_rows[rb * 32 + (lane & 31)];
        uint8_t* out = reinterpret_cast<uint8_t*>(dst) + ((size_t)(rb * nkc + kc) * 64 + lane) * 16;
        for (int h = 0; h < 2; ++h)
          for (int w = 0; w < 2; ++w) {
            const int c0 = kc * 64 + h * 32 + 16 * (lane >> 5) + w * 8;
            for (int i = 0; i < 4; ++i)
              out[h * 8 + w * 4 + i] =
                  (uint8_t)(code_at(row, c0 + i) | (code_at(row, c0 + i + 4) << 4));
          }
      }
}

// Tile-major int8: chunk (r / 32) * (K / 32) + c / 32 of 1 KB; lane (r % 32) + 32 ((c % 32) / 16)
// holds the 16 consecutive codes c..c+15 of its row, one byte each.
void pack_tiles_int8(char* dst, const int8_t* const src_rows[], int R, int K) {
  const int nkc = K / 32;
  for (int rb = 0; rb < R / 32; ++rb)
    for (int kc = 0; kc < nkc; ++kc)
      for (int lane = 0; lane < 64; ++lane) {
        const int8_t* row = src_rows[rb * 32 + (lane & 31)];
        memcpy(dst + ((size_t)(rb * nkc + kc) * 64 + lane) * 16, row + kc * 32 + 16 * (lane >> 5),
               16);
      }
}

}  // namespace

extern "C" int moe_pack_expert_host(const void* gate, const void* up, const void* down,
                                    const void* gate_s, const void* up_s, const void* down_s,
                                    int H, int F, int w_dtype, void* dst) {
  SlotLayout l;
  if (slot_layout(H, F, w_dtype, &l) != MOE_OK) return MOE_EINVAL;
  MOE_CHECK_ARG(gate && up && down && dst);
  char* d = static_cast<char*>(dst);
  memset(d, 0, l.slot_bytes);
  const char* g = static_cast<const char*>(gate);
  const char* u = static_cast<const char*>(up);
  const char* dn = static_cast<const char*>(down);
  if (w_dtype == MOE_F32) {  // row-major, gate and up rows interleaved
    const size_t rb13 = (size_t)H * 4, rb2 = (size_t)F * 4;
    for (int n = 0; n < F; ++n) {
      memcpy(d + l.off_w13 + (size_t)(2 * n) * rb13, g + (size_t)n * rb13, rb13);
      memcpy(d + l.off_w13 + (size_t)(2 * n + 1) * rb13, u + (size_t)n * rb13, rb13);
    }
    memcpy(d + l.off_w2, dn, (size_t)H * rb2);
    return MOE_OK;
  }
  // rows of W13 in interleaved order (2n = gate n, 2n + 1 = up n) and of W2
  const size_t rb13 = (w_dtype == MOE_BF16) ? (size_t)H * 2 : (size_t)H / 2;
  const size_t rb2 = (w_dtype == MOE_BF16) ? (size_t)F * 2 : (size_t)F / 2;
  std::vector<const char*> r13(2 * F), r2(H);
  for (int n = 0; n < F; ++n) {
    r13[2 * n] = g + (size_t)n * rb13;
    r13[2 * n + 1] = u + (size_t)n * rb13;
  }
  for (int r = 0; r < H; ++r) r2[r] = dn + (size_t)r * rb2;
  if (w_dtype == MOE_BF16) {
    pack_tiles_bf16(d + l.off_w13, r13.data(), 2 * F, H);
    pack_tiles_bf16(d + l.off_w2, r2.data(), H, F);
    return MOE_OK;
  }
  MOE_CHECK_ARG(gate_s && up_s && down_s);
  pack_tiles_int4(d + l.off_w13, reinterpret_cast<const uint8_t**>(r13.data()), 2 * F, H);
  pack_tiles_int4(d + l.off_w2, reinterpret_cast<const uint8_t**>(r2.data()), H, F);
  // scales stay row-major: [2F, H/128] (gate/up interleaved) and [H, F/128]
  const size_t sb13 = (size_t)(H / 128) * 2, sb2 = (size_t)(F / 128) * 2;
  const char* gs = static_cast<const char*>(gate_s);
  const char* us = static_cast<const char*>(up_s);
  for (int n = 0; n < F; ++n) {
    memcpy(d + l.off_s13 + (size_t)(2 * n) * sb13, gs + (size_t)n * sb13, sb13);
    memcpy(d + l.off_s13 + (size_t)(2 * n + 1) * sb13, us + (size_t)n * sb13, sb13);
  }
  memcpy(d + l.off_s2, down_s, (size_t)H * sb2);
  return MOE_OK;
}

// ------------------------------------------------- split-precision experts --
// RapidMoE Algorithm 3 (RESplit) with b_q = b_r = 4: the float32 decisions
// (the group maximum over 2^(b-1)-1, the code rint(w / s)) are taken exactly
// as IEEE float32 operations, so contraction into fused multiply-adds is off.
#pragma clang fp contract(off)
namespace {

uint16_t bf16_bits_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

float bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// Symmetric b-bit quantisation of one row of K values in groups of 128: codes
// q[K] (int8) and the bf16 scale of each group s[K / 128].
void quantize_row_g128(const float* w, int K, int bits, int8_t* q, uint16_t* s) {
  const float qmax = (float)((1 << (bits - 1)) - 1);
  const float qlo = -(float)(1 << (bits - 1));
  for (int g = 0; g < K / 128; ++g) {
    float m = 0.f;
    for (int c = 0; c < 128; ++c) m = std::max(m, std::fabs(w[g * 128 + c]));
    const uint16_t sb = bf16_bits_rne(m / qmax);
    const float sv = bf16_value(sb);
    s[g] = sb;
    for (int c = 0; c < 128; ++c) {
      float v = 0.f;
      if (sv != 0.f) v = std::min(std::max(std::rint(w[g * 128 + c] / sv), qlo), qmax);
      q[g * 128 + c] = (int8_t)v;
    }
  }
}

// int4 codes of a row (int8 values in [-8, 7]) as nibbles, even index in the low nibble.
void nibbles_of(const int8_t* q, int K, uint8_t* out) {
  for (int c = 0; c < K; c += 2)
    out[c / 2] = (uint8_t)((q[c] & 0xF) | ((q[c + 1] & 0xF) << 4));
}

}  // namespace

extern "C" int moe_quantize_resplit_host(const float* gate, const float* up, const float* down,
                                         int H, int F, void* dst) {
  SlotLayout l;
  if (slot_layout(H, F, MOE_INT4G128_RESPLIT, &l) != MOE_OK) return MOE_EINVAL;
  MOE_CHECK_ARG(gate && up && down && dst);
  char* d = static_cast<char*>(dst);
  memset(d, 0, l.slot_bytes);
  // W13 rows interleaved (2n = gate n, 2n + 1 = up n): W^Q codes and the residual's codes
  std::vector<uint8_t> nq((size_t)2 * F * (H / 2)), nr((size_t)2 * F * (H / 2));
  std::vector<uint16_t> sq((size_t)2 * F * (H / 128)), sr((size_t)2 * F * (H / 128));
  std::vector<int8_t> q(H), rq(H);
  std::vector<float> res(H);
  for (int n = 0; n < F; ++n)
    for (int j = 0; j < 2; ++j) {
      const float* w = (j == 0 ? gate : up) + (size_t)n * H;
      const size_t row = (size_t)2 * n + j;
      uint16_t* s_row = sq.data() + row * (H / 128);
      quantize_row_g128(w, H, 4, q.data(), s_row);
      for (int c = 0; c < H; ++c) res[c] = w[c] - (float)q[c] * bf16_value(s_row[c / 128]);
      quantize_row_g128(res.data(), H, 4, rq.data(), sr.data() + row * (H / 128));
      nibbles_of(q.data(), H, nq.data() + row * (H / 2));
      nibbles_of(rq.data(), H, nr.data() + row * (H / 2));
    }
  // W2 [H, F]: W^L at 4 bits, W^H at 8 bits
  std::vector<uint8_t> nl((size_t)H * (F / 2));
  std::vector<int8_t> qh((size_t)H * F), ql(F);
  std::vector<uint16_t> sl((size_t)H * (F / 128)), sh((size_t)H * (F / 128));
  for (int r = 0; r < H; ++r) {
    const float* w = down + (size_t)r * F;
    quantize_row_g128(w, F, 4, ql.data(), sl.data() + (size_t)r * (F / 128));
    nibbles_of(ql.data(), F, nl.data() + (size_t)r * (F / 2));
    quantize_row_g128(w, F, 8, qh.data() + (size_t)r * F, sh.data() + (size_t)r * (F / 128));
  }
  std::vector<const uint8_t*> r13(2 * F), rr13(2 * F), r2(H);
  std::vector<const int8_t*> h2(H);
  for (int i = 0; i < 2 * F; ++i) {
    r13[i] = nq.data() + (size_t)i * (H / 2);
    rr13[i] = nr.data() + (size_t)i * (H / 2);
  }
  for (int r = 0; r < H; ++r) {
    r2[r] = nl.data() + (size_t)r * (F / 2);
    h2[r] = qh.data() + (size_t)r * F;
  }
  pack_tiles_int4(d + l.off_w13, r13.data(), 2 * F, H);
  pack_tiles_int4(d + l.off_w2, r2.data(), H, F);
  pack_tiles_int4(d + l.off_r13, rr13.data(), 2 * F, H);
  pack_tiles_int8(d + l.off_h2, h2.data(), H, F);
  memcpy(d + l.off_s13, sq.data(), sq.size() * 2);
  memcpy(d + l.off_s2, sl.data(), sl.size() * 2);
  memcpy(d + l.off_rs13, sr.data(), sr.size() * 2);
  memcpy(d + l.off_hs2, sh.data(), sh.size() * 2);
  return MOE_OK;
}
#pragma clang fp contract(on)

// -------------------------------------------------------- tags and commits --
namespace {

// Host -> device copy of a fill, 16 bytes per lane, the grid striding over them, reading
// pinned host memory through its device mapping. A copy kernel rather than a copy-engine
// transfer keeps a fill and the kernels queued after it on one queue: measured on the
// one-token fill path, the copy-engine transfer left about 0.1-0.3 ms between its end and
// the next kernel of its stream, the kernel none (both move 56 GB/s).
__global__ __launch_bounds__(256) void host_copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, size_t n16) {
  const size_t g = blockIdx.x * (size_t)blockDim.x + threadIdx.x, gs = (size_t)gridDim.x * blockDim.x;
  for (size_t j = g; j < n16; j += gs) dst[j] = src[j];
}
constexpr int kHostCopyBlocks = 128;

__global__ void tag_writeback_kernel(uint64_t* tags, int slot, uint64_t tag) {
  if (threadIdx.x == 0) tags[slot] = tag;
}

__global__ void slot_commit_kernel(int32_t* lut, int32_t idx, int32_t* owner, int32_t slot,
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

}  // namespace

int launch_host_copy(void* dst, const void* src_dev, size_t bytes, hipStream_t stream) {
  if (bytes % 16 != 0 || (uintptr_t)dst % 16 != 0 || (uintptr_t)src_dev % 16 != 0)
    return MOE_EINVAL;
  if (bytes == 0) return MOE_OK;
  hipLaunchKernelGGL(host_copy_kernel, dim3(kHostCopyBlocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src_dev), static_cast<u32x4*>(dst), bytes / 16);
  return moe_launch_status();
}

namespace {
// the copy of a fill: the kernel when the pinned source is mapped at its own address (as
// pinned allocations are) and 16-byte aligned, else a copy-engine transfer
int copy_fill(char* dst, const void* host_src, const hipPointerAttribute_t& attr, size_t bytes,
              hipStream_t stream) {
  if (attr.devicePointer == host_src && bytes % 16 == 0 && (uintptr_t)host_src % 16 == 0 &&
      (uintptr_t)dst % 16 == 0)
    return launch_host_copy(dst, host_src, bytes, stream);
  return moe_hip_status(hipMemcpyAsync(dst, host_src, bytes, hipMemcpyHostToDevice, stream));
}
}  // namespace

extern "C" int slot_commit(int32_t* lut, int32_t lut_index, int32_t* owner, int32_t slot,
                           const uint64_t* slot_tags, uint64_t tag, int32_t* err_word,
                           hipStream_t stream) {
  MOE_CHECK_ARG(lut && owner && slot_tags && err_word && slot >= 0 && lut_index >= 0);
  hipLaunchKernelGGL(slot_commit_kernel, dim3(1), dim3(64), 0, stream, lut, lut_index, owner, slot,
                     slot_tags, tag, err_word);
  return moe_launch_status();
}

extern "C" int slot_fill(void* pool_base, size_t slot_stride, int32_t slot, const void* host_src,
                         size_t bytes, int32_t* lut, int32_t lut_index, int32_t* owner,
                         uint64_t* slot_tags, uint64_t tag, int32_t* err_word,
                         hipStream_t fill_stream, hipStream_t compute_stream) {
  MOE_CHECK_ARG(pool_base && host_src && lut && owner && slot_tags && err_word);
  MOE_CHECK_ARG(slot >= 0 && lut_index >= 0 && bytes <= slot_stride);
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host_src) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_EINVAL;  // not memory the runtime knows: pageable host memory
  }
  if (attr.type != hipMemoryTypeHost) return MOE_EINVAL;

  char* dst = static_cast<char*>(pool_base) + (size_t)slot * slot_stride;
  int rc = copy_fill(dst, host_src, attr, bytes, fill_stream);
  if (rc != MOE_OK) return rc;
  hipError_t e;
  hipLaunchKernelGGL(tag_writeback_kernel, dim3(1), dim3(64), 0, fill_stream, slot_tags, slot, tag);
  if (fill_stream != compute_stream) {
    hipEvent_t ev;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return moe_hip_status(e);
    e = hipEventRecord(ev, fill_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(compute_stream, ev, 0);
    (void)hipEventDestroy(ev);
    if (e != hipSuccess) return moe_hip_status(e);
  }
  hipLaunchKernelGGL(slot_commit_kernel, dim3(1), dim3(64), 0, compute_stream, lut, lut_index,
                     owner, slot, slot_tags, tag, err_word);
  return moe_launch_status();
}

extern "C" int slot_prefetch(void* pool_base, size_t slot_stride, int32_t slot,
                             const void* host_src, size_t bytes, uint64_t* slot_tags,
                             uint64_t tag, hipStream_t fill_stream) {
  MOE_CHECK_ARG(pool_base && host_src && slot_tags && slot >= 0 && bytes <= slot_stride);
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host_src) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_EINVAL;  // not memory the runtime knows: pageable host memory
  }
  if (attr.type != hipMemoryTypeHost) return MOE_EINVAL;
  char* dst = static_cast<char*>(pool_base) + (size_t)slot * slot_stride;
  const int rc = copy_fill(dst, host_src, attr, bytes, fill_stream);
  if (rc != MOE_OK) return rc;
  hipLaunchKernelGGL(tag_writeback_kernel, dim3(1), dim3(64), 0, fill_stream, slot_tags, slot, tag);
  return moe_launch_status();
}

// ------------------------------------------------------- host LRU planning --
// ------------------------------------------------------- eviction scores --
// Host state of an eviction policy, per layer (doubles):
//   MRS:     [observed steps, ring of the last W score vectors (W x E), keep (E)]
//   HISTORY: [observed steps, ring of the last W selection vectors (W x E, 0/1),
//             ema (E), latest score (E), step of the last selection (E, 0 = never),
//             keep (E)]
// A layer's state changes only when it is observed, so its keep scores are
// computed then and read by every later plan until its next step.
// All arithmetic is float64 in a fixed order without contraction, so the
// victim order is reproducible bit for bit.
namespace {

size_t policy_layer_doubles(int policy, int E, int W) {
  if (policy == MOE_POLICY_MRS) return 1 + (size_t)W * E + E;
  if (policy == MOE_POLICY_HISTORY) return 1 + (size_t)W * E + 4 * (size_t)E;
  return 0;
}

// keep scores of a layer (the last E doubles of its state)
inline double* keep_of(double* st, int policy, int E, int W) {
  return st + policy_layer_doubles(policy, E, W) - E;
}
inline const double* keep_of(const double* st, int policy, int E, int W) {
  return st + policy_layer_doubles(policy, E, W) - E;
}

#pragma clang fp contract(off)

// Minus Recent Score (HybriMoE summary page, Mechanism): the expert's routing
// scores over the last W steps of its layer, summed oldest to newest, minus the
// newest one.
double mrs_keep(const double* st, int E, int W, int e) {
  const long n = (long)st[0];
  if (n == 0) return 0.0;
  const long m = n < W ? n : W;
  const double* ring = st + 1;
  double total = 0.0;
  for (long i = n - m; i < n; ++i) total += ring[(size_t)(i % W) * E + e];
  return total - ring[(size_t)((n - 1) % W) * E + e];
}

// Routing-history score (MoE-CORE summary page, Mechanism): window count, EMA
// of selections, latest score and freshness (1 - age / max age), each divided
// by its maximum over the layer, weighted by w[0..3].
struct HistoryNorm {
  double m_cnt, m_ema, m_score, m_age;
};

double history_count(const double* st, int E, int W, int e) {
  const long n = (long)st[0];
  const long m = n < W ? n : W;
  const double* ring = st + 1;
  double c = 0.0;
  for (long i = n - m; i < n; ++i) c += ring[(size_t)(i % W) * E + e];
  return c;
}

HistoryNorm history_norm(const double* st, int E, int W) {
  const double* ema = st + 1 + (size_t)W * E;
  const double* score = ema + E;
  const double* last = score + E;
  HistoryNorm h{0.0, 0.0, 0.0, 0.0};
  for (int e = 0; e < E; ++e) {
    h.m_cnt = std::max(h.m_cnt, history_count(st, E, W, e));
    h.m_ema = std::max(h.m_ema, ema[e]);
    h.m_score = std::max(h.m_score, score[e]);
    h.m_age = std::max(h.m_age, st[0] - last[e]);
  }
  return h;
}

double history_keep(const double* st, int E, int W, const double* w, const HistoryNorm& h, int e) {
  const double* ema = st + 1 + (size_t)W * E;
  const double* score = ema + E;
  const double* last = score + E;
  const double cnt = history_count(st, E, W, e);
  const double age = st[0] - last[e];
  const double n_cnt = h.m_cnt > 0.0 ? cnt / h.m_cnt : 0.0;
  const double n_ema = h.m_ema > 0.0 ? ema[e] / h.m_ema : 0.0;
  const double n_score = h.m_score > 0.0 ? score[e] / h.m_score : 0.0;
  const double fresh = h.m_age > 0.0 ? 1.0 - age / h.m_age : 1.0;
  double total = w[0] * n_cnt;
  total += w[1] * n_ema;
  total += w[2] * n_score;
  total += w[3] * fresh;
  return total;
}

#pragma clang fp contract(on)

bool policy_args_ok(int policy, const double* state, int W, const double* params) {
  if (policy == MOE_POLICY_LRU) return true;
  if (policy != MOE_POLICY_MRS && policy != MOE_POLICY_HISTORY) return false;
  if (!state || W < 1) return false;
  if (policy == MOE_POLICY_HISTORY) {
    if (!params) return false;
    for (int i = 0; i < 4; ++i)
      if (!(params[i] >= 0.0)) return false;
    if (!(params[4] >= 0.0 && params[4] <= 1.0)) return false;
  }
  return true;
}

// The plan of moe_plan_fills with the reusable slots ordered by keep[slot]
// first when keep is given.
int plan_fills(int32_t* lut, int32_t* owner, int64_t* last_use, int64_t* clock, int S, int L,
               int E, int layer, const int32_t* distinct, int n_distinct, int32_t* wave_of,
               int32_t* is_hit, int32_t* fill_expert, int32_t* fill_slot, int32_t* fill_wave,
               int32_t* n_fills, int32_t* n_waves, int policy, const double* state, int W,
               const double* params) {
  MOE_CHECK_ARG(lut && owner && last_use && clock && wave_of && is_hit && n_fills && n_waves);
  MOE_CHECK_ARG(S >= 1 && L >= 1 && E >= 1 && layer >= 0 && layer < L);
  MOE_CHECK_ARG(n_distinct >= 0 && n_distinct <= E);
  MOE_CHECK_ARG(n_distinct == 0 || (distinct && fill_expert && fill_slot && fill_wave));
  MOE_CHECK_ARG(policy_args_ok(policy, state, W, params));
  // The routed set must be strictly ascending ids in range.
  for (int i = 0; i < n_distinct; ++i) {
    if (distinct[i] < 0 || distinct[i] >= E) return MOE_EINVAL;
    if (i > 0 && distinct[i] <= distinct[i - 1]) return MOE_EINVAL;
  }
  int32_t* row = lut + (size_t)layer * E;
  for (int e = 0; e < E; ++e) {
    wave_of[e] = -1;
    is_hit[e] = 0;
  }
  std::vector<int> hits, misses;
  std::vector<char> kept(S, 0);
  for (int i = 0; i < n_distinct; ++i) {
    const int e = distinct[i];
    if (row[e] >= 0) {
      hits.push_back(e);
      kept[row[e]] = 1;
      is_hit[e] = 1;
    } else {
      misses.push_back(e);
    }
  }
  // Victims (only when something misses): empty slots by id, then the other
  // slots by (owner's keep score, last use, id); only as many as the misses
  // need are ordered.
  std::vector<int> victims, used;
  if (!misses.empty()) {
    for (int s = 0; s < S; ++s)
      if (owner[s] < 0) victims.push_back(s);
    std::vector<int> reuse;
    for (int s = 0; s < S; ++s)
      if (owner[s] >= 0 && !kept[s]) reuse.push_back(s);
    const size_t need = misses.size() > victims.size() ? misses.size() - victims.size() : 0;
    std::vector<double> keep;
    if (policy != MOE_POLICY_LRU && need > 0) {
      keep.assign(S, 0.0);
      const size_t per = policy_layer_doubles(policy, E, W);
      for (int s : reuse) {
        const int l = owner[s] / E, e = owner[s] % E;
        const double* st = state + (size_t)l * per;
        if (st[0] != 0.0)
          keep[s] = keep_of(st, policy, E, W)[e];
        else  // a layer never observed has no cached scores yet
          keep[s] = policy == MOE_POLICY_MRS ? 0.0 : history_keep(st, E, W, params, HistoryNorm{0.0, 0.0, 0.0, 0.0}, e);
      }
    }
    auto first = [&](int a, int b) {
      if (!keep.empty() && keep[a] != keep[b]) return keep[a] < keep[b];
      return last_use[a] < last_use[b] || (last_use[a] == last_use[b] && a < b);
    };
    const size_t take = need < reuse.size() ? need : reuse.size();
    std::partial_sort(reuse.begin(), reuse.begin() + take, reuse.end(), first);
    victims.insert(victims.end(), reuse.begin(), reuse.begin() + take);
  }

  *clock += 1;
  int nf = 0, nw = 1;
  auto assign = [&](int e, int s, int wave) {
    const int32_t old = owner[s];
    if (old >= 0) lut[old] = -1;
    row[e] = s;
    owner[s] = layer * E + e;
    fill_expert[nf] = e;
    fill_slot[nf] = s;
    fill_wave[nf] = wave;
    ++nf;
    wave_of[e] = wave;
    used.push_back(s);
  };
  for (int e : hits) {
    wave_of[e] = 0;
    used.push_back(row[e]);
  }
  if (misses.size() <= victims.size()) {
    for (size_t i = 0; i < misses.size(); ++i) assign(misses[i], victims[i], 0);
  } else {
    const size_t first_n = victims.size();
    for (size_t i = 0; i < first_n; ++i) assign(misses[i], victims[i], 0);
    int wave = 1;
    for (size_t i = first_n; i < misses.size(); i += S, ++wave) {
      for (size_t j = i; j < misses.size() && j < i + S; ++j) assign(misses[j], (int)(j - i), wave);
      nw = wave + 1;
    }
  }
  for (int s : used) last_use[s] = *clock;
  *n_fills = nf;
  *n_waves = (n_distinct == 0) ? 0 : nw;
  return MOE_OK;
}

}  // namespace

extern "C" int moe_plan_fills(int32_t* lut, int32_t* owner, int64_t* last_use, int64_t* clock,
                              int S, int L, int E, int layer, const int32_t* distinct,
                              int n_distinct, int32_t* wave_of, int32_t* is_hit,
                              int32_t* fill_expert, int32_t* fill_slot, int32_t* fill_wave,
                              int32_t* n_fills, int32_t* n_waves) {
  return plan_fills(lut, owner, last_use, clock, S, L, E, layer, distinct, n_distinct, wave_of,
                    is_hit, fill_expert, fill_slot, fill_wave, n_fills, n_waves, MOE_POLICY_LRU,
                    nullptr, 0, nullptr);
}

extern "C" int moe_plan_fills_policy(int policy, const double* state, int window,
                                     const double* params, int32_t* lut, int32_t* owner,
                                     int64_t* last_use, int64_t* clock, int S, int L, int E,
                                     int layer, const int32_t* distinct, int n_distinct,
                                     int32_t* wave_of, int32_t* is_hit, int32_t* fill_expert,
                                     int32_t* fill_slot, int32_t* fill_wave, int32_t* n_fills,
                                     int32_t* n_waves) {
  return plan_fills(lut, owner, last_use, clock, S, L, E, layer, distinct, n_distinct, wave_of,
                    is_hit, fill_expert, fill_slot, fill_wave, n_fills, n_waves, policy, state,
                    window, params);
}

extern "C" int moe_prefetch_count(double window_us, double bw_gbs, size_t expert_bytes,
                                  int free_slots) {
  if (!(window_us > 0.0) || expert_bytes == 0 || free_slots <= 0 || !(bw_gbs > 0.0)) return 0;
  const double n = std::floor(window_us * bw_gbs * 1000.0 / (double)expert_bytes);
  return n < (double)free_slots ? (int)n : free_slots;
}

extern "C" int moe_plan_prefetch(int policy, const double* state, int window,
                                 const double* params, int32_t* lut, int32_t* owner,
                                 int64_t* last_use, const int64_t* clock, int S, int L, int E,
                                 int layer, const int32_t* pred_ids, int n_pred,
                                 const float* pred_scores, double window_us, double bw_gbs,
                                 size_t expert_bytes, int32_t* fill_expert, int32_t* fill_slot,
                                 int32_t* n_fills) {
  MOE_CHECK_ARG(lut && owner && last_use && clock && n_fills && pred_scores);
  MOE_CHECK_ARG(S >= 1 && L >= 1 && E >= 1 && layer >= 0 && layer < L && n_pred >= 0);
  MOE_CHECK_ARG(n_pred == 0 || (pred_ids && fill_expert && fill_slot));
  MOE_CHECK_ARG(policy_args_ok(policy, state, window, params));
  *n_fills = 0;
  std::vector<char> pred(E, 0);
  for (int i = 0; i < n_pred; ++i) {
    if (pred_ids[i] < 0 || pred_ids[i] >= E) return MOE_EINVAL;
    pred[pred_ids[i]] = 1;
  }
  int32_t* row = lut + (size_t)layer * E;
  std::vector<int> cand;
  for (int e = 0; e < E; ++e)
    if (pred[e] && row[e] < 0) cand.push_back(e);
  std::stable_sort(cand.begin(), cand.end(),
                   [&](int a, int b) { return pred_scores[a] > pred_scores[b]; });
  if (cand.empty()) return MOE_OK;
  // free slots: empty ones by id, then those the current step did not use and that hold no
  // predicted expert of this layer, in the victim order of the policy
  std::vector<int> freeslots, reuse;
  for (int s = 0; s < S; ++s) {
    if (owner[s] < 0) {
      freeslots.push_back(s);
    } else if (last_use[s] < *clock) {
      const int l = owner[s] / E, e = owner[s] % E;
      if (!(l == layer && pred[e])) reuse.push_back(s);
    }
  }
  std::vector<double> keep;
  if (policy != MOE_POLICY_LRU && !reuse.empty()) {
    keep.assign(S, 0.0);
    const size_t per = policy_layer_doubles(policy, E, window);
    for (int s : reuse) {
      const int l = owner[s] / E, e = owner[s] % E;
      const double* st = state + (size_t)l * per;
      if (st[0] != 0.0)
        keep[s] = keep_of(st, policy, E, window)[e];
      else
        keep[s] = policy == MOE_POLICY_MRS
                      ? 0.0
                      : history_keep(st, E, window, params, HistoryNorm{0.0, 0.0, 0.0, 0.0}, e);
    }
  }
  std::sort(reuse.begin(), reuse.end(), [&](int a, int b) {
    if (!keep.empty() && keep[a] != keep[b]) return keep[a] < keep[b];
    return last_use[a] < last_use[b] || (last_use[a] == last_use[b] && a < b);
  });
  freeslots.insert(freeslots.end(), reuse.begin(), reuse.end());
  int n = moe_prefetch_count(window_us, bw_gbs, expert_bytes, (int)freeslots.size());
  if (n > (int)cand.size()) n = (int)cand.size();
  for (int i = 0; i < n; ++i) {
    const int e = cand[i], s = freeslots[i];
    const int32_t old = owner[s];
    if (old >= 0) lut[old] = -1;
    row[e] = s;
    owner[s] = layer * E + e;
    last_use[s] = *clock;
    fill_expert[i] = e;
    fill_slot[i] = s;
  }
  *n_fills = n;
  return MOE_OK;
}

extern "C" size_t moe_policy_state_doubles(int policy, int L, int E, int window) {
  if (L < 1 || E < 1 || window < 1) return 0;
  return (size_t)L * policy_layer_doubles(policy, E, window);
}

#pragma clang fp contract(off)
extern "C" int moe_policy_observe(int policy, double* state, int L, int E, int window, int layer,
                                  const float* scores, const int32_t* distinct, int n_distinct,
                                  const double* params) {
  MOE_CHECK_ARG(L >= 1 && E >= 1 && layer >= 0 && layer < L);
  MOE_CHECK_ARG(policy_args_ok(policy, state, window, params));
  MOE_CHECK_ARG(n_distinct >= 0 && n_distinct <= E && (n_distinct == 0 || distinct));
  if (policy == MOE_POLICY_LRU) return MOE_OK;
  MOE_CHECK_ARG(scores);
  for (int i = 0; i < n_distinct; ++i)
    if (distinct[i] < 0 || distinct[i] >= E) return MOE_EINVAL;
  const int W = window;
  double* st = state + (size_t)layer * policy_layer_doubles(policy, E, W);
  const long n = (long)st[0];  // steps observed before this one
  double* ring = st + 1 + (size_t)(n % W) * E;
  if (policy == MOE_POLICY_MRS) {
    for (int e = 0; e < E; ++e) ring[e] = (double)scores[e];
  } else {
    double* ema = st + 1 + (size_t)W * E;
    double* score = ema + E;
    double* last = score + E;
    for (int e = 0; e < E; ++e) ring[e] = 0.0;
    for (int i = 0; i < n_distinct; ++i) ring[distinct[i]] = 1.0;
    const double lam = params[4];
    for (int e = 0; e < E; ++e) {
      ema[e] = lam * ema[e] + (1.0 - lam) * ring[e];
      score[e] = (double)scores[e];
      if (ring[e] != 0.0) last[e] = (double)(n + 1);
    }
  }
  st[0] = (double)(n + 1);
  double* keep = keep_of(st, policy, E, W);
  if (policy == MOE_POLICY_MRS) {
    for (int e = 0; e < E; ++e) keep[e] = mrs_keep(st, E, W, e);
  } else {
    const HistoryNorm h = history_norm(st, E, W);
    for (int e = 0; e < E; ++e) keep[e] = history_keep(st, E, W, params, h, e);
  }
  return MOE_OK;
}
#pragma clang fp contract(on)

extern "C" const char* moe_version(void) { return MOE_VERSION_STRING; }
