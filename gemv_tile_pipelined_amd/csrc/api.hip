// api.hip -- the C ABI of include/gemvtile.h: argument checks, the per-device
// compute-unit cache, and kernel launches on the caller's stream.
//
// Every argument check happens before the first HIP call, so invalid calls are
// reported the same way on a machine without a GPU.  Nothing here allocates
// device memory, synchronises, or keeps a pointer past the call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/gemvtile.h"
#include "kernels.hpp"
#include "tile_order.hpp"

namespace {

// Largest M or N: tile origins and row indices are 32-bit in the kernels, and
// a whole tile past the last row must still be addressable.
constexpr int64_t kMaxRows = (int64_t{1} << 31) - 512;
// Largest K of the GEMM: a 256-row panel of A or B (256 * K * 2 bytes) must
// stay below 2^31 bytes, the range of one buffer descriptor's 32-bit offsets.
constexpr int64_t kMaxGemmK = 4194296;
// Largest K of the GEMV (chunk indices are 32-bit).
constexpr int64_t kMaxGemvK = (int64_t{1} << 31) - 8;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

// Compute units of the current device, cached per device.
int current_cu_count(int *out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GEMVTILE_ERR_DEVICE;
  if (dev >= 0 && dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *out = cached;
      return GEMVTILE_OK;
    }
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return GEMVTILE_ERR_DEVICE;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  *out = cus;
  return GEMVTILE_OK;
}

int check_gemm(const void *A, const void *B, const void *D, int64_t M, int64_t N, int64_t K, bool *noop) {
  *noop = false;
  if (M < 0 || N < 0 || K < 0) return GEMVTILE_ERR_INVALID_ARG;
  if (M == 0 || N == 0) {
    *noop = true;
    return GEMVTILE_OK;
  }
  if (D == nullptr) return GEMVTILE_ERR_INVALID_ARG;
  if (K > 0 && (A == nullptr || B == nullptr)) return GEMVTILE_ERR_INVALID_ARG;
  if (M > kMaxRows || N > kMaxRows) return GEMVTILE_ERR_UNSUPPORTED;
  if (K % 8 != 0 || K > kMaxGemmK) return GEMVTILE_ERR_UNSUPPORTED;
  if (misaligned(D, 2)) return GEMVTILE_ERR_UNSUPPORTED;
  if (K > 0 && (misaligned(A, 16) || misaligned(B, 16))) return GEMVTILE_ERR_UNSUPPORTED;
  return GEMVTILE_OK;
}

int check_gemv(const void *x, const void *W, const void *y, int64_t N, int64_t K, bool *noop) {
  *noop = false;
  if (N < 0 || K < 0) return GEMVTILE_ERR_INVALID_ARG;
  if (N == 0) {
    *noop = true;
    return GEMVTILE_OK;
  }
  if (y == nullptr) return GEMVTILE_ERR_INVALID_ARG;
  if (K > 0 && (x == nullptr || W == nullptr)) return GEMVTILE_ERR_INVALID_ARG;
  if (N > kMaxRows) return GEMVTILE_ERR_UNSUPPORTED;
  if (K % 8 != 0 || K > kMaxGemvK) return GEMVTILE_ERR_UNSUPPORTED;
  if (misaligned(y, 2)) return GEMVTILE_ERR_UNSUPPORTED;
  if (K > 0 && (misaligned(x, 16) || misaligned(W, 16))) return GEMVTILE_ERR_UNSUPPORTED;
  return GEMVTILE_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? GEMVTILE_OK : GEMVTILE_ERR_LAUNCH; }

// The kernel family and index of a gemvtile_gemm_f16_variant number.
enum class Family { kTiled, kSkinny, kWs, kInvalid };
struct VariantRef {
  Family family;
  int index;
};
VariantRef classify_variant(int variant) {
  if (gt::gemm_variant_exists(variant)) return {Family::kTiled, variant};
  if (variant >= gt::kSkinnyVariantBase && gt::skinny_variant_exists(variant - gt::kSkinnyVariantBase))
    return {Family::kSkinny, variant - gt::kSkinnyVariantBase};
  if (variant >= gt::kGemmWsVariantBase && variant < gt::kGemmWsVariantBase + gt::kGemmWsVariants)
    return {Family::kWs, variant - gt::kGemmWsVariantBase};
  return {Family::kInvalid, 0};
}

// dtype: gt::kF16 or gt::kBF16.  bf16 runs the default kernels only
// (variant 0).
int run_gemm(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *stream, int variant,
             int dtype = gt::kF16) {
  bool noop = false;
  int st = check_gemm(A, B, D, M, N, K, &noop);
  if (st != GEMVTILE_OK || noop) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // +0 is the all-zero pattern in both formats.
  if (K == 0) return to_status(gt::launch_fill_zero_f16(D, M * N, s));
  const bool skinny = M <= gt::kSkinnyMaxRows || N <= gt::kSkinnyMaxRows;
  const VariantRef v = classify_variant(variant);
  if (v.family == Family::kInvalid) return GEMVTILE_ERR_INVALID_ARG;
  // the skinny kernel as gemm_f16 launches it (skinny 0) and the small-side
  // split (skinny 60) also take 17..64 rows on the smaller side
  const bool skinny_wide = (M < N ? M : N) <= gt::kSkinnyWideRows;
  if (v.family == Family::kSkinny && !skinny && !((v.index == 0 || v.index == 60) && skinny_wide))
    return GEMVTILE_ERR_UNSUPPORTED;
  int cus = 0;
  st = current_cu_count(&cus);
  if (st != GEMVTILE_OK) return st;
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  // Forced launch shapes of the skinny and wave-specialised families (f16
  // only); the skinny ones apply to skinny shapes only.
  if (v.family == Family::kSkinny)
    return to_status(gt::launch_gemm_skinny_f16(v.index, A, B, D, m, n, k, cus, s));
  if (v.family == Family::kWs) return to_status(gt::launch_gemm_ws_f16(v.index, A, B, D, m, n, k, cus, s));
  if (variant == 0 && (M == 1 || N == 1)) {
    // One row on a side is the batch-1 product y = x·Wᵀ: M == 1 is
    // D[0][n] = A[0]·B[n] (x = A, W = B); N == 1 is D[m][0] = A[m]·B[0]
    // (x = B, W = A), whose [M,1] output is a contiguous vector.
    const void *x = M == 1 ? A : B;
    const void *W = M == 1 ? B : A;
    const int rows = M == 1 ? n : m;
    return to_status(dtype == gt::kBF16 ? gt::launch_gemv_bf16(x, W, D, rows, k, cus, s)
                                        : gt::launch_gemv_f16(0, x, W, D, rows, k, cus, s));
  }
  // Variant 0 sends shapes with at most 16 rows on one side, and those with
  // 17..64 on the smaller side (skinny_wide_route), to the skinny kernel.
  if (variant == 0 && (skinny || gt::skinny_wide_route(M, N)))
    return to_status(dtype == gt::kBF16 ? gt::launch_gemm_skinny_bf16(A, B, D, m, n, k, cus, s)
                                        : gt::launch_gemm_skinny_f16(0, A, B, D, m, n, k, cus, s));
  return to_status(dtype == gt::kBF16 ? gt::launch_gemm_bf16(A, B, D, m, n, k, cus, s)
                                      : gt::launch_gemm_f16(variant, A, B, D, m, n, k, cus, s));
}

int run_gemv(const void *x, const void *W, void *y, int64_t N, int64_t K, void *stream, int variant,
             int dtype = gt::kF16) {
  bool noop = false;
  int st = check_gemv(x, W, y, N, K, &noop);
  if (st != GEMVTILE_OK || noop) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) return to_status(gt::launch_fill_zero_f16(y, N, s));
  int cus = 0;
  st = current_cu_count(&cus);
  if (st != GEMVTILE_OK) return st;
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  if (dtype == gt::kBF16) return to_status(gt::launch_gemv_bf16(x, W, y, n, k, cus, s));
  return to_status(gt::launch_gemv_f16(variant, x, W, y, n, k, cus, s));
}

}  // namespace

extern "C" {

int gemm_f16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *stream) {
  return run_gemm(A, B, D, M, N, K, stream, 0);
}

}  // extern "C"

namespace {
// gemm_bias_f16 / gemm_bias_bf16: the GEMM checks, then the activation code
// and the bias pointer (element aligned, may be NULL), before any HIP call.
int run_gemm_bias(const void *A, const void *B, const void *bias, void *D, int64_t M, int64_t N, int64_t K, int act,
                  void *stream, int dtype) {
  if (act != GEMVTILE_ACT_NONE && act != GEMVTILE_ACT_RELU) return GEMVTILE_ERR_INVALID_ARG;
  bool noop = false;
  int st = check_gemm(A, B, D, M, N, K, &noop);
  if (st != GEMVTILE_OK || noop) return st;
  if (bias != nullptr && misaligned(bias, 2)) return GEMVTILE_ERR_UNSUPPORTED;
  int cus = 0;
  st = current_cu_count(&cus);
  if (st != GEMVTILE_OK) return st;
  return to_status(gt::launch_gemm_bias(dtype, A, B, bias, act == GEMVTILE_ACT_RELU ? 1 : 0, D, static_cast<int>(M),
                                        static_cast<int>(N), static_cast<int>(K), cus, static_cast<hipStream_t>(stream)));
}
}  // namespace

extern "C" {

int gemm_bias_f16(const void *A, const void *B, const void *bias, void *D, int64_t M, int64_t N, int64_t K, int act,
                  void *stream) {
  return run_gemm_bias(A, B, bias, D, M, N, K, act, stream, gt::kF16);
}

int gemm_bias_bf16(const void *A, const void *B, const void *bias, void *D, int64_t M, int64_t N, int64_t K, int act,
                   void *stream) {
  return run_gemm_bias(A, B, bias, D, M, N, K, act, stream, gt::kBF16);
}

}  // extern "C"

namespace {
// Split K applies to shapes of the tiled kernel and of the skinny kernel
// (2..16 rows on a side), not to the GEMV's (one row on a side); elsewhere
// gemm_splitk_* is the plain GEMM.
int splitk_splits(int64_t M, int64_t N, int64_t K, int cus) {
  if (M == 1 || N == 1) return 1;
  if (M <= gt::kSkinnyMaxRows || N <= gt::kSkinnyMaxRows)
    return gt::skinny_splitk_splits(M <= gt::kSkinnyMaxRows ? N : M, K, cus);
  return gt::gemm_splitk_splits(M, N, K, cus);
}

// ws == nullptr with ws_bytes == -1: use the static scratch of
// gemm_splitk_f16_noalloc instead of a caller's workspace.
int run_gemm_splitk(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *ws,
                    int64_t ws_bytes, void *stream, int dtype) {
  const bool use_static = ws == nullptr && ws_bytes == -1;
  if (ws_bytes < 0 && !use_static) return GEMVTILE_ERR_INVALID_ARG;
  bool noop = false;
  int st = check_gemm(A, B, D, M, N, K, &noop);
  if (st != GEMVTILE_OK || noop) return st;
  int cus = 0;
  st = current_cu_count(&cus);
  if (st != GEMVTILE_OK) return st;
  const int splits = K == 0 ? 1 : splitk_splits(M, N, K, cus);
  if (splits == 1) return run_gemm(A, B, D, M, N, K, stream, 0, dtype);
  const int64_t need = static_cast<int64_t>(splits) * M * N * 4;
  if (use_static) {
    if (need > gt::kNoAllocScratchBytes) return GEMVTILE_ERR_SCRATCH;
    if (gt::noalloc_scratch(&ws) != hipSuccess) return GEMVTILE_ERR_DEVICE;
  } else {
    if (ws == nullptr || ws_bytes < need) return GEMVTILE_ERR_INVALID_ARG;
    if (misaligned(ws, 16)) return GEMVTILE_ERR_UNSUPPORTED;
  }
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M <= gt::kSkinnyMaxRows || N <= gt::kSkinnyMaxRows)
    return to_status(gt::launch_gemm_skinny_splitk(dtype, A, B, D, m, n, k, ws, splits, s));
  return to_status(gt::launch_gemm_splitk(dtype, A, B, D, m, n, k, ws, splits, cus, s));
}
}  // namespace

extern "C" {

int gemm_splitk_f16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *workspace,
                    int64_t workspace_bytes, void *stream) {
  return run_gemm_splitk(A, B, D, M, N, K, workspace, workspace_bytes, stream, gt::kF16);
}

int gemm_splitk_bf16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *workspace,
                     int64_t workspace_bytes, void *stream) {
  return run_gemm_splitk(A, B, D, M, N, K, workspace, workspace_bytes, stream, gt::kBF16);
}

int gemm_splitk_f16_noalloc(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *stream) {
  return run_gemm_splitk(A, B, D, M, N, K, nullptr, -1, stream, gt::kF16);
}

int64_t gemvtile_gemm_splitk_workspace(int64_t M, int64_t N, int64_t K, int64_t num_cus) {
  if (M <= 0 || N <= 0 || K <= 0 || num_cus <= 0 || num_cus > (int64_t{1} << 20)) return 0;
  const int splits = splitk_splits(M, N, K, static_cast<int>(num_cus));
  return splits > 1 ? static_cast<int64_t>(splits) * M * N * 4 : 0;
}

int gemvtile_gemm_splitk_splits(int64_t M, int64_t N, int64_t K, int64_t num_cus) {
  if (M <= 0 || N <= 0 || K <= 0 || num_cus <= 0 || num_cus > (int64_t{1} << 20)) return 1;
  return splitk_splits(M, N, K, static_cast<int>(num_cus));
}

int gemv_f16(const void *x, const void *W, void *y, int64_t N, int64_t K, void *stream) {
  return run_gemv(x, W, y, N, K, stream, 0);
}

int gemm_bf16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *stream) {
  return run_gemm(A, B, D, M, N, K, stream, 0, gt::kBF16);
}

int gemv_bf16(const void *x, const void *W, void *y, int64_t N, int64_t K, void *stream) {
  return run_gemv(x, W, y, N, K, stream, 0, gt::kBF16);
}

int gemvtile_gemm_f16_variant(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *stream,
                              int variant) {
  if (classify_variant(variant).family == Family::kInvalid)
    return GEMVTILE_ERR_INVALID_ARG;
  return run_gemm(A, B, D, M, N, K, stream, variant);
}

int gemvtile_gemm_f16_timed(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *stream,
                            uint64_t *stamps, int64_t stamps_len) {
  bool noop = false;
  int st = check_gemm(A, B, D, M, N, K, &noop);
  if (st != GEMVTILE_OK) return st;
  if (noop || K == 0 || M <= gt::kSkinnyMaxRows || N <= gt::kSkinnyMaxRows) return GEMVTILE_ERR_UNSUPPORTED;
  int cus = 0;
  st = current_cu_count(&cus);
  if (st != GEMVTILE_OK) return st;
  const int64_t tiles = ((M + gt::kGemmBM - 1) / gt::kGemmBM) * ((N + gt::kGemmBN - 1) / gt::kGemmBN);
  const int64_t grid = tiles < cus ? tiles : cus;
  if (stamps == nullptr || stamps_len < 8 * grid || misaligned(stamps, 8)) return GEMVTILE_ERR_INVALID_ARG;
  return to_status(gt::launch_gemm_f16_timed(A, B, D, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), cus,
                                             stamps, static_cast<hipStream_t>(stream)));
}

int gemvtile_gemv_f16_variant(const void *x, const void *W, void *y, int64_t N, int64_t K, void *stream,
                              int variant) {
  if (!gt::gemv_variant_exists(variant)) return GEMVTILE_ERR_INVALID_ARG;
  return run_gemv(x, W, y, N, K, stream, variant);
}

const char *gemvtile_status_string(int status) {
  switch (status) {
    case GEMVTILE_OK: return "ok";
    case GEMVTILE_ERR_INVALID_ARG: return "invalid argument (NULL pointer with a nonzero extent, or a negative size)";
    case GEMVTILE_ERR_UNSUPPORTED: return "unsupported (K % 8 != 0, misaligned pointer, or a size beyond the limits)";
    case GEMVTILE_ERR_LAUNCH: return "kernel launch failed";
    case GEMVTILE_ERR_DEVICE: return "HIP device query failed";
    case GEMVTILE_ERR_SCRATCH:
      return "gemm_splitk_f16_noalloc: the split-K partial sums of this shape exceed its static scratch (16 MiB); "
             "use gemm_splitk_f16 with a workspace";
    default: return "unknown status";
  }
}

int gemvtile_tile_coord(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t group_m, int64_t *tm, int64_t *tn) {
  if (tm == nullptr || tn == nullptr || tiles_m <= 0 || tiles_n <= 0 || group_m <= 0) return GEMVTILE_ERR_INVALID_ARG;
  if (t < 0 || t >= tiles_m * tiles_n) return GEMVTILE_ERR_INVALID_ARG;
  const gt::TileCoord c = gt::tile_of(t, tiles_m, tiles_n, group_m);
  *tm = c.tm;
  *tn = c.tn;
  return GEMVTILE_OK;
}

int64_t gemvtile_ring_trace(int variant, int64_t ktu, int32_t *events, int64_t cap, int *info) {
  if (ktu < 1 || ktu > (int64_t{1} << 20) || cap < 0 || (events == nullptr && cap > 0)) return -1;
  int dummy[8];
  return gt::ring_trace(variant, static_cast<int>(ktu), events, cap, info != nullptr ? info : dummy);
}

int64_t gemvtile_xcd_logical_id(int64_t w, int64_t grid) {
  if (grid <= 0 || w < 0 || w >= grid) return -1;
  return gt::xcd_logical_id(w, grid);
}

void gemvtile_gemm_config(int *bm, int *bn, int *bk, int *stages, int *threads, int *group_m) {
  if (bm) *bm = gt::kGemmBM;
  if (bn) *bn = gt::kGemmBN;
  if (bk) *bk = gt::kGemmBK;
  if (stages) *stages = gt::kGemmStages;
  if (threads) *threads = gt::kGemmThreads;
  if (group_m) *group_m = gt::kGemmGroupM;
}

int gemvtile_device_caps(int *num_cus, int *clock_khz, int *mem_clock_khz, int *mem_bus_bits) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GEMVTILE_ERR_DEVICE;
  const struct {
    int *out;
    hipDeviceAttribute_t attr;
  } q[] = {{num_cus, hipDeviceAttributeMultiprocessorCount},
           {clock_khz, hipDeviceAttributeClockRate},
           {mem_clock_khz, hipDeviceAttributeMemoryClockRate},
           {mem_bus_bits, hipDeviceAttributeMemoryBusWidth}};
  for (const auto &e : q) {
    if (e.out == nullptr) continue;
    if (hipDeviceGetAttribute(e.out, e.attr, dev) != hipSuccess) return GEMVTILE_ERR_DEVICE;
  }
  return GEMVTILE_OK;
}

int64_t gemvtile_gemv_grid(int64_t N, int64_t K, int64_t num_cus) {
  if (N <= 0 || K < 0 || num_cus <= 0 || num_cus > (int64_t{1} << 20)) return 0;
  return gt::gemv_default_grid(N, K, static_cast<int>(num_cus));
}

int64_t gemvtile_gemm_grid(int64_t M, int64_t N, int64_t K, int64_t num_cus) {
  if (M <= 0 || N <= 0 || K < 0 || num_cus <= 0) return 0;
  // One row on a side: the GEMV kernel over the other side's rows.
  if (M == 1 || N == 1) return gemvtile_gemv_grid(M == 1 ? N : M, K, num_cus);
  // Skinny shapes (at most 16 rows on a side, or 17..64 on the smaller
  // side, skinny_wide_route): one workgroup per 32, 16, 8, 4, 2 or
  // 1 rows of the other side, times the small side's 16-row blocks when it
  // is split.
  if (num_cus > (int64_t{1} << 20)) return 0;
  const int cus = static_cast<int>(num_cus);
  if (M <= gt::kSkinnyMaxRows || N <= gt::kSkinnyMaxRows || gt::skinny_wide_route(M, N)) {
    const int64_t R = M <= gt::kSkinnyMaxRows ? N : N <= gt::kSkinnyMaxRows ? M : (M <= N ? N : M);
    const int64_t S = M <= gt::kSkinnyMaxRows ? M : N <= gt::kSkinnyMaxRows ? N : (M <= N ? M : N);
    if (gt::skinny_qsplit(R, S, cus)) {
      const int64_t rows = gt::skinny_qsplit_rows(R, S, cus);
      return (R + rows - 1) / rows * ((S + 15) / 16);
    }
    const int64_t rows = gt::skinny_default_rows(R, cus);
    return (R + rows - 1) / rows;
  }
  const gt::GemmTileShape &t = gt::kGemmTileShapes[gt::gemm_default_tile(M, N, cus)];
  const int64_t tiles = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
  return tiles < num_cus ? tiles : num_cus;
}

int gemvtile_gemm_tile(int64_t M, int64_t N, int64_t num_cus, int *bm, int *bn, int *stages) {
  if (M <= 0 || N <= 0 || num_cus <= 0 || num_cus > (int64_t{1} << 20)) return GEMVTILE_ERR_INVALID_ARG;
  const gt::GemmTileShape &t = gt::kGemmTileShapes[gt::gemm_default_tile(M, N, static_cast<int>(num_cus))];
  if (bm) *bm = t.bm;
  if (bn) *bn = t.bn;
  if (stages) *stages = t.stages;
  return GEMVTILE_OK;
}

}  // extern "C"
