// Grouped SwiGLU expert FFN over resident slots (moe_expert_ffn).
//
// Each routed expert group e (its rows [offsets[e], offsets[e+1]) of the
// permuted assignments) reads its weights through the slot table: slot =
// lut[e], weights at pool_base + slot * slot_stride (the fixed-base slot pool
// and expert_id -> slot_id table of the SeqMoE summary page, Mechanism). The
// expert is the SwiGLU FFN of "RapidMoE: Exploiting Cross-Asymmetry via
// Adaptive Residual Offloading for Large-Scale MoE Inference", Eq. (7):
// y = down(SiLU(gate x) * up x).
//
// Kernels (all on the caller's stream):
//   ffn_plan_kernel  one workgroup: selected, non-empty, resident groups go to
//                    the GEMV list (<= small_max rows) or are cut into
//                    kGemmBM-row MFMA tiles; absent experts set MOE_ERR_ABSENT.
//                    Inside the library a call may also carry the shared
//                    experts as groups E .. E+n_shared-1 (T rows each, slots
//                    shared_slot0 + s), so one plan and one pair of weight
//                    passes cover the routed and the shared experts.
//   GEMV passes      decode groups: tile-major bf16 weights (tile_gemv.h),
//                    every load a contiguous 1 KB chunk, split-K over the
//                    waves of a workgroup; row-major fp32 weights
//                    (ffn_gemv.h). Weights are streamed once per token tile
//                    with non-temporal 16-byte loads; HBM-bound.
//   GEMM passes      (gemm.hip) groups with more rows: bf16 MFMA tiles.
// The SwiGLU intermediate h lives in the workspace: bf16 with bf16 weights
// (the A operand of the second MFMA pass), fp32 with fp32 weights.
#include <limits.h>

#include <mutex>

#include "common.h"
#include "ffn_gemv.h"
#include "ffn_internal.h"
#include "tile_gemv.h"

namespace {

constexpr int kGemvGridCap = 8192;  // workgroups of a GEMV pass (they loop over work units)

__global__ __launch_bounds__(1024) void ffn_plan_kernel(
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ lut,
    const int32_t* __restrict__ mask, int E, int n_shared, int shared_slot0, int num_slots,
    int small_max, FfnItem* __restrict__ items, int32_t* __restrict__ n_items,
    GemmTile* __restrict__ tiles, int32_t* __restrict__ n_tiles, int32_t* __restrict__ err_word,
    int32_t* __restrict__ sync) {
  __shared__ int s_wave[40];
  const int e = threadIdx.x;
  if (e < kStreamMaxItems) sync[e] = 0;  // the one-token FFN launch's hand-off counters
  int rows = 0, slot = -1, begin = 0;
  bool take = false;
  if (e < E + n_shared) {
    begin = offsets[e];
    rows = offsets[e + 1] - begin;
    const bool routed = e < E;
    take = rows > 0 && (!routed || mask == nullptr || mask[e] != 0);
    if (take) {
      slot = routed ? lut[e] : shared_slot0 + (e - E);
      if (slot < 0 || slot >= num_slots) {
        atomicOr(err_word, MOE_ERR_ABSENT);
        take = false;
      }
    }
  }
  const bool small = take && rows <= small_max;
  const int ntile = (take && !small) ? (rows + kGemmBM - 1) / kGemmBM : 0;
  int total_items = 0, total_tiles = 0;
  const int ipos = block_exclusive_scan(small ? 1 : 0, s_wave, &total_items);
  const int tpos = block_exclusive_scan(ntile, s_wave, &total_tiles);
  if (small) items[ipos] = FfnItem{e, slot, begin, rows};
  for (int i = 0; i < ntile; ++i) {
    const int r0 = i * kGemmBM;
    tiles[tpos + i] = GemmTile{e, slot, begin + r0, min(kGemmBM, rows - r0)};
  }
  if (e == 0) {
    n_items[0] = total_items;
    n_tiles[0] = total_tiles;
  }
}

template <int WF, int AF, int OF, int RPW, int KS, int U, int MAXNT, bool SWIGLU>
void launch_pass(const void* act, const int32_t* perm, int k, const FfnItem* items,
                 const int32_t* n_items, int max_items, const char* pool, size_t stride,
                 size_t off, int rows, int K, int out_ld, void* out, hipStream_t s) {
  const unsigned rb = gemv::row_blocks<RPW, KS>(rows);
  const long long units = (long long)rb * max_items;
  const unsigned grid = (unsigned)(units < kGemvGridCap ? units : kGemvGridCap);
  if (grid == 0) return;
  hipLaunchKernelGGL((gemv::pass_kernel<WF, AF, OF, RPW, KS, U, MAXNT, SWIGLU, true>), dim3(grid),
                     dim3(256), 0, s, act, perm, k, items, n_items, pool, stride, off, rows, K,
                     out_ld, (int)rb, out);
}

// One tile-major bf16 GEMV pass: KS waves per RBW row blocks.
template <int KS, int RBW, int MAXNT, bool SWIGLU, int AF, int OF>
void launch_tile_pass(const void* act, const int32_t* perm, int k, const FfnItem* items,
                      const int32_t* n_items, int max_items, const char* pool, size_t stride,
                      size_t off, int R, int K, int out_ld, void* out, hipStream_t s) {
  constexpr int NW = KS < 4 ? 4 : KS;
  constexpr int rb_per_wg = NW / KS * RBW;
  const int upi = (R / 32 + rb_per_wg - 1) / rb_per_wg;
  const long long units = (long long)upi * max_items;
  const unsigned grid = (unsigned)(units < tgemv::kGridCap ? units : tgemv::kGridCap);
  if (grid == 0) return;
  constexpr int U = (KS == 16 && MAXNT >= 4) ? 2 : 4;  // stay within 128 VGPRs at 1024 threads
  hipLaunchKernelGGL((tgemv::bf16_kernel<AF, OF, KS, RBW, NW, U, MAXNT, SWIGLU>), dim3(grid),
                     dim3(NW * 64), 0, s, act, perm, k, items, n_items, pool, stride, off, R, K,
                     out_ld, upi, out);
}

template <int RBW, int MAXNT, bool SWIGLU, int AF, int OF>
void launch_tile_ks(int ks, const void* act, const int32_t* perm, int k, const FfnItem* items,
                    const int32_t* n_items, int max_items, const char* pool, size_t stride,
                    size_t off, int R, int K, int out_ld, void* out, hipStream_t s) {
#define MOE_TILE_KS(KS_)                                                                         \
  launch_tile_pass<KS_, RBW, MAXNT, SWIGLU, AF, OF>(act, perm, k, items, n_items, max_items, pool, \
                                                    stride, off, R, K, out_ld, out, s)
  switch (ks) {
    case 1: MOE_TILE_KS(1); break;
    case 2: MOE_TILE_KS(2); break;
    case 4: MOE_TILE_KS(4); break;
    case 8: MOE_TILE_KS(8); break;
    default:
      if constexpr (RBW == 1) MOE_TILE_KS(16);  // 1024-thread groups: 128 VGPRs, RBW = 1 only
      else MOE_TILE_KS(8);
      break;
  }
#undef MOE_TILE_KS
}

template <int MAXNT, bool SWIGLU, int AF, int OF>
void launch_tile_any(const void* act, const int32_t* perm, int k, const FfnItem* items,
                     const int32_t* n_items, int max_items, const char* pool, size_t stride,
                     size_t off, int R, int K, int out_ld, void* out, hipStream_t s) {
  const tgemv::Split sp = tgemv::choose_split_bf16(R / 32 * max_items, K / 16, MAXNT);
  if (sp.rbw == 1)
    launch_tile_ks<1, MAXNT, SWIGLU, AF, OF>(sp.ks, act, perm, k, items, n_items, max_items, pool,
                                             stride, off, R, K, out_ld, out, s);
  else
    launch_tile_ks<2, MAXNT, SWIGLU, AF, OF>(sp.ks, act, perm, k, items, n_items, max_items, pool,
                                             stride, off, R, K, out_ld, out, s);
}

// bf16 tokens and weights: small groups on the tile-major GEMV (one token) or the MFMA
// GEMV (decode batches, skinny.hip), MFMA tiles for the rest.
template <int MAXNT>
void launch_bf16(const void* x, const int32_t* perm, int k, const FfnItem* items,
                 const int32_t* n_items, int max_items, const GemmTile* tiles,
                 const int32_t* n_tiles, int max_tiles, const char* pool, size_t stride,
                 const SlotLayout& lay, int H, int F, void* hbuf, float* y, hipStream_t s) {
  if constexpr (MAXNT == 1)
    launch_tile_any<MAXNT, true, MOE_BF16, MOE_BF16>(x, perm, k, items, n_items, max_items, pool,
                                                     stride, lay.off_w13, 2 * F, H, F, hbuf, s);
  else
    launch_skinny_bf16(1, x, perm, k, items, n_items, max_items, pool, stride, lay.off_w13, 2 * F,
                       H, F, hbuf, s);
  if (max_tiles > 0)
    launch_gemm_bf16(1, x, perm, k, tiles, n_tiles, max_tiles, pool, stride, lay.off_w13, 2 * F, H,
                     F, hbuf, s);
  if constexpr (MAXNT == 1)
    launch_tile_any<MAXNT, false, MOE_BF16, MOE_F32>(hbuf, perm, k, items, n_items, max_items,
                                                     pool, stride, lay.off_w2, H, F, H, y, s);
  else
    launch_skinny_bf16(2, hbuf, perm, k, items, n_items, max_items, pool, stride, lay.off_w2, H, F,
                       H, y, s);
  if (max_tiles > 0)
    launch_gemm_bf16(2, hbuf, perm, k, tiles, n_tiles, max_tiles, pool, stride, lay.off_w2, H, F, H,
                     y, s);
}

// fp32 tokens and weights: GEMV for every group (token tiles of up to 8 rows).
template <int MAXNT>
void launch_f32(const void* x, const int32_t* perm, int k, const FfnItem* items,
                const int32_t* n_items, int max_items, const char* pool, size_t stride,
                const SlotLayout& lay, int H, int F, void* hbuf, float* y, hipStream_t s) {
  launch_pass<MOE_F32, MOE_F32, MOE_F32, 4, 2, 1, MAXNT, true>(
      x, perm, k, items, n_items, max_items, pool, stride, lay.off_w13, 2 * F, H, F, hbuf, s);
  launch_pass<MOE_F32, MOE_F32, MOE_F32, 4, 4, 1, MAXNT, false>(
      hbuf, perm, k, items, n_items, max_items, pool, stride, lay.off_w2, H, F, H, y, s);
}

}  // namespace

long long resident_workgroups(const void* kern, int threads, size_t lds,
                              std::atomic<long long>& cache) {
  static std::atomic<int> cus[64];  // compute units per device
  int dev = 0, n = 256;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    n = cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
      if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          n <= 0)
        n = 256;
      cus[dev].store(n, std::memory_order_relaxed);
    }
  }
  long long o = cache.load(std::memory_order_relaxed);  // (lds << 8) | workgroups per CU
  if (o < 0 || (size_t)(o >> 8) != lds) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, threads, lds) != hipSuccess ||
        nb < 1)
      nb = 1;
    o = ((long long)lds << 8) | (nb > 255 ? 255 : nb);
    cache.store(o, std::memory_order_relaxed);
  }
  return (o & 0xFF) * (long long)n;
}

void launch_ffn_plan(const int32_t* offsets, const int32_t* lut, const int32_t* mask, int E,
                     int n_shared, int shared_slot0, int num_slots, int small_max, FfnItem* items,
                     int32_t* n_items, GemmTile* tiles, int32_t* n_tiles, int32_t* err_word,
                     int32_t* sync, hipStream_t s) {
  hipLaunchKernelGGL(ffn_plan_kernel, dim3(1), dim3(1024), 0, s, offsets, lut, mask, E, n_shared,
                     shared_slot0, num_slots, small_max, items, n_items, tiles, n_tiles, err_word,
                     sync);
}

int ffn_small_max(int T, int k, int E, int n_shared, int w_dtype) {
  // with many rows per group on average, every group takes the MFMA tiles and
  // the GEMV passes are not launched at all
  const long long rows = (long long)T * (k + n_shared);
  if (rows > 16LL * (E + n_shared)) return 0;
  // decode batches of bf16 or int4 (not split-precision) experts: groups of up to 32 rows
  // on the MFMA GEMV; one token: the GEMV
  return ((w_dtype == MOE_BF16 || w_dtype == MOE_INT4G128) && T >= 2) ? kSkinnyMaxRows
                                                                       : kGemvMaxRows;
}

FfnWorkspace ffn_workspace_layout(int T, int H, int F, int E, int k, int w_dtype, int n_shared) {
  FfnWorkspace w{};
  const size_t rows = (size_t)T * (k + n_shared);
  const size_t groups = (size_t)E + n_shared;
  // upper bound on MFMA tiles: sum over groups of ceil(rows / BM) <= rows / BM + groups
  w.max_tiles = (int)(rows / kGemmBM + (rows < groups ? rows : groups) + 1);
  size_t off = 256;  // n_items at offset 0, n_tiles at offset 4
  w.sync = off;
  off = align_up(off + kStreamMaxItems * sizeof(int32_t), 256);
  w.items = off;
  off = align_up(off + groups * sizeof(FfnItem), 256);
  w.tiles = off;
  off = align_up(off + (size_t)w.max_tiles * sizeof(GemmTile), 256);
  w.h = off;
  off = align_up(off + rows * F * sizeof(float), 256);
  if (w_dtype == MOE_INT4G128 || w_dtype == MOE_INT4G128_RESPLIT) {
    // int8 rows and their fp32 scales
    w.xq = off;
    off = align_up(off + (size_t)T * H, 256);
    w.xs = off;
    off = align_up(off + (size_t)T * sizeof(float), 256);
    w.hq = off;
    off = align_up(off + rows * F, 256);
    w.hs = off;
    off = align_up(off + rows * sizeof(float), 256);
  }
  w.total = off;
  return w;
}

extern "C" size_t moe_ffn_workspace_bytes(int T, int H, int F, int E, int k, int w_dtype) {
  if (T < 0 || H <= 0 || F <= 0 || E <= 0 || k <= 0) return 0;
  return ffn_workspace_layout(T, H, F, E, k, w_dtype, 0).total;
}

extern "C" int moe_ffn_workspace_offsets(int T, int H, int F, int E, int k, int w_dtype,
                                         size_t* offs) {
  MOE_CHECK_ARG(T >= 0 && H > 0 && F > 0 && E > 0 && k > 0 && offs);
  MOE_CHECK_ARG(w_dtype >= MOE_F32 && w_dtype <= MOE_INT4G128_RESPLIT);
  const FfnWorkspace w = ffn_workspace_layout(T, H, F, E, k, w_dtype, 0);
  offs[0] = w.h;
  offs[1] = w.xq;
  offs[2] = w.xs;
  offs[3] = w.hq;
  offs[4] = w.hs;
  return MOE_OK;
}

int ffn_int4(const void* x, const int32_t* perm, const int32_t* offsets, const int32_t* lut,
             const int32_t* group_mask, int n_shared, int shared_slot0, const char* pool,
             size_t stride, int num_slots, const SlotLayout& lay, int T, int H, int F, int E, int k,
             float* y, int32_t* err, char* ws, const FfnWorkspace& wl, hipStream_t s, bool planned,
             bool split);

extern "C" int moe_expert_ffn(const void* x, int x_dtype, const int32_t* perm,
                              const int32_t* offsets, const int32_t* lut,
                              const int32_t* group_mask, const void* pool_base, size_t slot_stride,
                              int num_slots, int w_dtype, int T, int H, int F, int E, int k,
                              float* y_perm, int32_t* err_word, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
  return expert_ffn(x, x_dtype, perm, offsets, lut, group_mask, 0, 0, pool_base, slot_stride,
                    num_slots, w_dtype, T, H, F, E, k, y_perm, err_word, workspace, ws_bytes,
                    stream);
}

// ----------------------------------------------- allocation-free variant --
// moe_expert_ffn_noalloc keeps its workspace in this array. In host code the name
// is only a stand-in for the device symbol: every host use goes through the address
// hipGetSymbolAddress returns on the device (one copy per GPU, looked up once per
// device on its first call there).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return moe_hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOE_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" size_t moe_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int moe_expert_ffn_noalloc(const void* x, int x_dtype, const int32_t* perm,
                                      const int32_t* offsets, const int32_t* lut,
                                      const int32_t* group_mask, const void* pool_base,
                                      size_t slot_stride, int num_slots, int w_dtype, int T,
                                      int H, int F, int E, int k, float* y_perm,
                                      int32_t* err_word, hipStream_t stream) {
  MOE_CHECK_ARG(T >= 0 && H > 0 && F > 0 && k >= 1 && k <= E && E <= 1024);
  if (T == 0) return MOE_OK;
  const FfnWorkspace w = ffn_workspace_layout(T, H, F, E, k, w_dtype, 0);
  if (w.total > kNoAllocScratchBytes) return MOE_EINVAL;  // beyond the static scratch
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != MOE_OK) return rc;
  return expert_ffn(x, x_dtype, perm, offsets, lut, group_mask, 0, 0, pool_base, slot_stride,
                    num_slots, w_dtype, T, H, F, E, k, y_perm, err_word, ws,
                    kNoAllocScratchBytes, stream);
}

int expert_ffn(const void* x, int x_dtype, const int32_t* perm, const int32_t* offsets,
               const int32_t* lut, const int32_t* group_mask, int n_shared, int shared_slot0,
               const void* pool_base, size_t slot_stride, int num_slots, int w_dtype, int T, int H,
               int F, int E, int k, float* y_perm, int32_t* err_word, void* workspace,
               size_t ws_bytes, hipStream_t stream, bool planned) {
  MOE_CHECK_ARG(T >= 0 && k >= 1 && k <= E && n_shared >= 0 && E + n_shared <= 1024);
  MOE_CHECK_ARG(x_dtype == MOE_F32 || x_dtype == MOE_BF16);
  SlotLayout lay;
  if (slot_layout(H, F, w_dtype, &lay) != MOE_OK) return MOE_EINVAL;
  MOE_CHECK_ARG(slot_stride >= lay.slot_bytes && slot_stride % 256 == 0 && num_slots >= 1);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(x && perm && offsets && lut && pool_base && y_perm && err_word && workspace);
  MOE_CHECK_ARG(((uintptr_t)x % 16) == 0 && ((uintptr_t)pool_base % 256) == 0);
  MOE_CHECK_ARG(((uintptr_t)y_perm % 16) == 0);
  const FfnWorkspace ws = ffn_workspace_layout(T, H, F, E, k, w_dtype, n_shared);
  MOE_CHECK_ARG(ws_bytes >= ws.total && ((uintptr_t)workspace % 256) == 0);
  // supported pairs: fp32 tokens with fp32 weights; bf16 tokens with bf16 or int4 weights
  if (w_dtype == MOE_F32 && x_dtype != MOE_F32) return MOE_EUNSUPPORTED;
  if (w_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (w_dtype == MOE_BF16 && (H % 64 != 0 || F % 64 != 0)) return MOE_EUNSUPPORTED;

  char* wsb = static_cast<char*>(workspace);
  if (w_dtype == MOE_INT4G128 || w_dtype == MOE_INT4G128_RESPLIT)
    return ffn_int4(x, perm, offsets, lut, group_mask, n_shared, shared_slot0,
                    static_cast<const char*>(pool_base), slot_stride, num_slots, lay, T, H, F, E, k,
                    y_perm, err_word, wsb, ws, stream, planned, w_dtype == MOE_INT4G128_RESPLIT);

  int32_t* n_items = reinterpret_cast<int32_t*>(wsb);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(wsb + 4);
  FfnItem* items = reinterpret_cast<FfnItem*>(wsb + ws.items);
  GemmTile* tiles = reinterpret_cast<GemmTile*>(wsb + ws.tiles);
  void* hbuf = wsb + ws.h;
  const long long tk = (long long)T * k;
  const bool bf16 = (w_dtype == MOE_BF16);
  // a group holds at most T rows (a token picks an expert once)
  const int small_max = bf16 ? ffn_small_max(T, k, E, n_shared, w_dtype) : INT_MAX;
  const int max_items = small_max == 0 ? 0 : (int)(tk < E ? tk : E) + n_shared;
  const int max_tiles = (bf16 && T > small_max) ? ws.max_tiles : 0;
  MOE_CHECK_ARG(max_tiles <= 65535);

  if (!planned)
    launch_ffn_plan(offsets, lut, group_mask, E, n_shared, shared_slot0, num_slots, small_max,
                    items, n_items, tiles, n_tiles, err_word,
                    reinterpret_cast<int32_t*>(wsb + ws.sync), stream);
  const char* pool = static_cast<const char*>(pool_base);
  if (bf16) {
    // one token: both passes over even shares of the call's row blocks, in one launch when
    // it fits
    if (T == 1 && max_items > 0 && max_tiles == 0 && decode_bf16_fits(max_items, 2 * F, H, true) &&
        decode_bf16_fits(max_items, H, F, false)) {
      int rc = launch_decode_bf16_fused(x, items, n_items, max_items, pool, slot_stride,
                                        lay.off_w13, lay.off_w2, H, F, hbuf, y_perm,
                                        reinterpret_cast<int32_t*>(wsb + ws.sync), err_word,
                                        stream);
      if (rc == MOE_EUNSUPPORTED) {
        rc = launch_decode_bf16(true, x, items, n_items, max_items, pool, slot_stride,
                                lay.off_w13, 2 * F, H, F, hbuf, stream);
        if (rc == MOE_OK)
          rc = launch_decode_bf16(false, hbuf, items, n_items, max_items, pool,
                                  slot_stride, lay.off_w2, H, F, H, y_perm, stream);
      }
      if (rc != MOE_EUNSUPPORTED) return rc;
    }
    if (T <= 1)
      launch_bf16<1>(x, perm, k, items, n_items, max_items, tiles, n_tiles, max_tiles, pool,
                     slot_stride, lay, H, F, hbuf, y_perm, stream);
    else
      launch_bf16<kSkinnyMaxRows>(x, perm, k, items, n_items, max_items, tiles, n_tiles,
                                  max_tiles, pool, slot_stride, lay, H, F, hbuf, y_perm, stream);
  } else {
    if (T <= 1)
      launch_f32<1>(x, perm, k, items, n_items, max_items, pool, slot_stride, lay, H, F, hbuf,
                    y_perm, stream);
    else if (T <= 2)
      launch_f32<2>(x, perm, k, items, n_items, max_items, pool, slot_stride, lay, H, F, hbuf,
                    y_perm, stream);
    else if (T <= 4)
      launch_f32<4>(x, perm, k, items, n_items, max_items, pool, slot_stride, lay, H, F, hbuf,
                    y_perm, stream);
    else
      launch_f32<8>(x, perm, k, items, n_items, max_items, pool, slot_stride, lay, H, F, hbuf,
                    y_perm, stream);
  }
  return moe_launch_status();
}
