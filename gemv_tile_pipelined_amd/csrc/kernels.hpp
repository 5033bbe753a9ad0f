// kernels.hpp -- launchers the C ABI layer calls, and the shape of the
// default GEMM kernel.  All launchers enqueue on `stream` and return the HIP
// error of the launch; they do no argument checking of their own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gt {

// Element formats of operands and results.
constexpr int kF16 = 0;   // IEEE binary16
constexpr int kBF16 = 1;  // bfloat16 (1 sign, 8 exponent, 7 fraction bits)

// Default GEMM kernel: 256x256 output tiles, K tiles of 64, a two-stage LDS
// ring, 256 threads (4 waves), grouped tile order 8 tile rows high.
constexpr int kGemmBM = 256;
constexpr int kGemmBN = 256;
constexpr int kGemmBK = 64;
constexpr int kGemmStages = 2;
constexpr int kGemmThreads = 256;
constexpr int kGemmGroupM = 8;
// gemvtile_gemm_f16_variant numbers of the tiled kernel: 0 (the default)
// and the ablations of gemm.hip.  Numbers of ablations that were measured and
// not kept stay unused.
constexpr int kGemmVariants = 33;
inline bool gemm_variant_exists(int v) { return (v >= 0 && v <= 3) || v == 10 || (v >= 20 && v <= 28) || v == 30 || v == 31 || v == 32; }

// Output tile of the tiled GEMM.  The 256x256 default needs about one tile
// per CU to fill the chip; outputs that give fewer take smaller tiles, each
// with a deeper ring so that its shorter K tiles still cover the load
// latency (2 stages at 256x256, 3 at 256x128 and 128x256, 4 at 128x128 and
// 128x64).
enum GemmTile { kTile256x256 = 0, kTile256x128 = 1, kTile128x256 = 2, kTile128x128 = 3, kTile128x64 = 4 };
constexpr int kGemmTiles = 5;
struct GemmTileShape {
  int bm, bn, stages;
  // Work rate relative to 256x256 when every CU has tiles to spare, in
  // percent (measured at 8192^3: 256x128 and 128x256 run at about 0.9 of the
  // 256x256 rate, 128x128 at about 0.76; 128x64 at 0.69-0.79 of the 128x128
  // rate at 1024-4096 x 1024 x 4096-14336).
  int rate_pct;
};
constexpr GemmTileShape kGemmTileShapes[kGemmTiles] = {
    {256, 256, 2, 100}, {256, 128, 3, 90}, {128, 256, 3, 90}, {128, 128, 4, 76}, {128, 64, 4, 55}};
// Split K (below) picks among the first kGemmSplitKTiles tiles only: its
// constants were measured with them.
constexpr int kGemmSplitKTiles = 4;
// The tile for an M x N output on num_cus CUs: the one with the least
// estimated time, i.e. waves of tiles over the CUs times tile area over rate;
// ties go to the larger tile (the lower enum value).  `tiles` limits the
// choice to the first entries of kGemmTileShapes.
inline GemmTile gemm_default_tile(int64_t M, int64_t N, int num_cus, int tiles = kGemmTiles) {
  int best = kTile256x256;
  int64_t best_cost = -1;
  for (int t = 0; t < tiles; ++t) {
    const GemmTileShape &s = kGemmTileShapes[t];
    const int64_t tiles = ((M + s.bm - 1) / s.bm) * ((N + s.bn - 1) / s.bn);
    const int64_t waves = (tiles + num_cus - 1) / num_cus;
    // waves * bm * bn / (rate_pct / 100), scaled to stay integral
    const int64_t cost = waves * s.bm * s.bn * 100 / s.rate_pct;
    if (best_cost < 0 || cost < best_cost) {
      best = t;
      best_cost = cost;
    }
  }
  return static_cast<GemmTile>(best);
}

// Split K (gemm_splitk_*): when the output's tiles (of the tile
// gemm_default_tile picks) cannot give every CU one, each tile's K tiles of
// 64 are cut into `splits` slices, so that tiles x splits units fill the CUs.
// Every slice keeps at least kSplitKMinTiles K tiles and none is empty.  The
// split is taken only when the K tiles it takes off the K loop,
// KT (1 - 1/splits), reach kSplitKMinSaved plus one K tile for every
// kSplitKOutputsPerTile partial sums it stores and reads back (splits M N):
// a K tile of the 128x128 tile takes about 0.35 us, a few microseconds go to
// the reduction's launch and the partial kernel's start, and the partial
// sums cost about 0.35 us per 2 MB written and read.  The constants come
// from timing every admissible slice count on outputs of 128..2048 x
// 128..4096 with K = 1024..14336 on an MI355X: there the rule never chose a
// split slower than the unsplit GEMM, and its choice was within 2.9 us of
// the fastest.  Returns 1 (no split) otherwise.
constexpr int kSplitKMinTiles = 10;
constexpr int kSplitKMinSaved = 12;
constexpr int kSplitKOutputsPerTile = 1 << 18;
inline int gemm_splitk_splits(int64_t M, int64_t N, int64_t K, int num_cus) {
  const GemmTileShape &s = kGemmTileShapes[gemm_default_tile(M, N, num_cus, kGemmSplitKTiles)];
  const int64_t tiles = ((M + s.bm - 1) / s.bm) * ((N + s.bn - 1) / s.bn);
  const int64_t kt = (K + 63) / 64;
  if (tiles >= num_cus || kt < 2 * kSplitKMinTiles) return 1;
  int64_t splits = num_cus / tiles;
  if (splits > kt / kSplitKMinTiles) splits = kt / kSplitKMinTiles;
  if (splits < 2) return 1;
  const int64_t per = (kt + splits - 1) / splits;
  splits = (kt + per - 1) / per;  // drop slices that would be empty
  const double saved = static_cast<double>(kt) * static_cast<double>(splits - 1) / static_cast<double>(splits);
  const double cost = kSplitKMinSaved + static_cast<double>(splits) * static_cast<double>(M) * static_cast<double>(N) /
                                            static_cast<double>(kSplitKOutputsPerTile);
  return saved >= cost ? static_cast<int>(splits) : 1;
}
// gemvtile_gemv_f16_variant numbers of the GEMV kernel's launch shapes.
inline bool gemv_variant_exists(int v) {
  return v == 0 || (v >= 6 && v <= 12) || v == 20 || v == 21 || v == 28 || v == 29 || (v >= 37 && v <= 41);
}
// GEMMs with at most this many rows on one side (M or N) take the skinny
// kernel (skinny.hip).
constexpr int kSkinnyMaxRows = 16;
// gemm_f16 / gemm_bf16 also send shapes whose smaller side has 17..64 rows
// to the skinny kernel (two or four 16-row blocks of the small operand per
// MFMA step, or the small side split into 16-row blocks over the grid): the
// tiled kernel's 128-row tiles would leave most of each tile idle there.
constexpr int kSkinnyWideRows = 64;
// The default's choice for such shapes (S = 17..64 rows on the smaller side,
// R on the larger): the skinny kernel whatever R.  Measured on MI355X
// against the tiled kernel past the R where 128x128 tiles fill the CUs, it
// was 5-27 % faster (64x16384x4096 39.9 -> 29.7 us, 24x24576x4096 47.0 ->
// 34.2 us, 64x12288x14336 123.8 -> 93.0 us, 64x65536x4096 122.7 -> 116.4
// us), with 32 large-side rows per workgroup in K tiles of 256.
inline bool skinny_wide_route(int64_t M, int64_t N) {
  const int64_t S = M < N ? M : N;
  return S > kSkinnyMaxRows && S <= kSkinnyWideRows;
}
// gemvtile_gemm_f16_variant numbers each kernel family from a fixed base:
// tiled GEMM 0.., skinny kSkinnyVariantBase + (0, 4, 12, 30, 47),
// wave-specialised kGemmWsVariantBase...  Numbers of launch shapes measured
// and not kept stay unused.
constexpr int kSkinnyVariantBase = 100;
constexpr int kGemmWsVariantBase = 200;
inline bool skinny_variant_exists(int v) {
  return v == 0 || v == 4 || v == 12 || v == 30 || v == 47 || v == 52 || v == 60;
}
// Wave-specialised (producer / consumer) GEMM launch shapes (gemm_ws.hip).
constexpr int kGemmWsVariants = 2;
static_assert(kGemmVariants <= kSkinnyVariantBase && kSkinnyVariantBase + 61 <= kGemmWsVariantBase,
              "variant families must not overlap");

// The default GEMV launch for an N x K matrix on a device with num_cus
// compute units: 8 waves per workgroup, each wave on `rows_per_wave` rows and
// one of `ksplit` slices of K.  Rows of kGemvSplitMinK or more elements take
// 2 rows per workgroup (K split 8 ways) whenever that gives every CU a
// workgroup: the many small workgroups finish closer together than 16-row
// ones (2-5 % faster from K = 8192 up; level at K = 6144, 2-3 % slower at
// K = 4096).  Shorter rows take 16 rows per workgroup while that still gives
// every CU a workgroup; below that the waves split K 2, 4 or 8 ways (8, 4 or
// 2 rows per workgroup).  Below 2 rows per CU a workgroup takes one row in 8
// slices.
//
// W is read with non-temporal loads when it holds kGemvStreamMinElems
// elements or more (64 MiB of fp16), with cached loads below that: with cold
// W every launch measured faster that way below 64 MiB (4096x4096: 7.2 ->
// 6.7 us; 2048x8192: 7.3 -> 6.8 us; 512x4096: 3.5 -> 3.0 us), and slower
// from 64 MiB up (8192x4096: 11.9 -> 12.8 us; 4096x14336: 19.6 -> 21.5 us).
struct GemvLaunch {
  int rows_per_wave;
  int ksplit;
  bool nontemporal;
};
constexpr int kGemvWaves = 8;
constexpr int64_t kGemvSplitMinK = 8192;
constexpr int64_t kGemvStreamMinElems = int64_t{1} << 25;
inline GemvLaunch gemv_default_launch(int64_t N, int64_t K, int num_cus) {
  const int64_t c = num_cus;
  const bool nt = N * K >= kGemvStreamMinElems;
  if (K >= kGemvSplitMinK && N >= 2 * c) return {2, 8, nt};
  if (N >= 16 * c) return {2, 1, nt};
  if (N >= 8 * c) return {2, 2, nt};
  if (N >= 4 * c) return {2, 4, nt};
  if (N >= 2 * c) return {2, 8, nt};
  return {1, 8, nt};
}
inline int64_t gemv_default_grid(int64_t N, int64_t K, int num_cus) {
  const GemvLaunch l = gemv_default_launch(N, K, num_cus);
  const int64_t rows = static_cast<int64_t>(l.rows_per_wave) * kGemvWaves / l.ksplit;
  return (N + rows - 1) / rows;
}

// At 16 P rows per workgroup the default skinny launch streams P with
// non-temporal loads (and K tiles of 256 in a 6-stage ring) only for K of
// at least kSkinnyStreamMinK elements:
// below 8192 cached loads measured faster (8x4096x4096: 8.8 -> 7.4 us;
// 8x4096x6144: 10.5 -> 9.4 us); from 8192 up the non-temporal form is the
// faster (8x4096x14336: 20.0 us against 23.2 us cached; 8x4096x28672: 36.5
// against 42.0 us).  Launches of 16 or 8 P rows per workgroup start each
// workgroup's K walk at kSkinnyRotateXcd's K tile (skinny.hip).
constexpr int kSkinnyStreamMinK = 8192;
constexpr int kSkinnyRotateXcd = 2;

// P rows per workgroup of the default skinny launch for R rows of the large
// operand.  From 32 rows per CU up: 32, 48 or 64, whichever gives a CU the
// fewest rows over whole rounds of workgroups (ties to the larger: fewer
// re-reads of the small side), in K tiles of 256 (32 rows) or 128 (48, 64)
// so that a ring of 3 or 4 stages still fits the LDS; each workgroup then
// stages the small side once per 32-64 P rows instead of 16 (64x8192x8192
// 40.4 -> 27.7 us, 24x8192x4096 16.0 -> 12.4 us, 16x8192x8192 24.4 -> 21.8
// us; 64x12288x14336 at 48 rows 98.3 -> 71.9 us, 64x16384x4096 at 64 rows
// 30.0 -> 25.9 us).  Below that, the largest of 16, 8, 4, 2 with
// R >= rows * num_cus, else 1.
inline int skinny_default_rows(int64_t R, int num_cus) {
  if (R >= int64_t{32} * num_cus) {
    int best = 32;
    int64_t best_rows = ((R + 31) / 32 + num_cus - 1) / num_cus * 32;
    for (int rows = 48; rows <= 64; rows += 16) {
      const int64_t per_cu = ((R + rows - 1) / rows + num_cus - 1) / num_cus * rows;
      if (per_cu <= best_rows) {
        best = rows;
        best_rows = per_cu;
      }
    }
    return best;
  }
  for (int rows = 16; rows > 1; rows >>= 1)
    if (R >= static_cast<int64_t>(rows) * num_cus) return rows;
  return 1;
}
// 17..64 small-side rows against few large-side rows: the small side is
// split into ceil(S / 16) blocks of 16 rows along the grid's y dimension,
// each workgroup staging one block (the launches of the S <= 16 case), when
// the staged form above would take fewer than 8 P rows per workgroup, or 8
// with at most 32 small-side rows.  Each workgroup then re-reads 16 Q rows
// per P row block instead of all S, and P is read ceil(S / 16) times, from
// the caches after the first (64x1024x14336 31.0 -> 17.5 us, 48x1500x4104
// 20.1 -> 11.6 us, 20x2048x4096 7.8 -> 6.2 us; at 16 P rows per workgroup,
// or 8 with 64 small-side rows, it measured 13-125 % slower).
inline bool skinny_qsplit(int64_t R, int64_t S, int num_cus) {
  if (S <= kSkinnyMaxRows || S > kSkinnyWideRows) return false;
  const int pr = skinny_default_rows(R, num_cus);
  return pr < 8 || (pr == 8 && S <= 32);
}
// P rows per workgroup of the split launch: the most of 16, 8, 4, 2 that
// still gives every CU a workgroup (counting the ceil(S / 16) small-side
// blocks), else 1.
inline int skinny_qsplit_rows(int64_t R, int64_t S, int num_cus) {
  const int64_t qb = (S + 15) / 16;
  for (int rows = 16; rows > 1; rows >>= 1)
    if ((R + rows - 1) / rows * qb >= num_cus) return rows;
  return 1;
}

// Split K on the skinny kernel (gemm_splitk_*, with R rows on the large side
// and 2..16 on the small one): while ceil(R / 16) blocks of 16 rows leave
// CUs idle, each block's K tiles of 512 are cut into `splits` slices of at
// least kSkinnySplitMinTiles tiles, so that blocks x splits workgroups fill
// the CUs; every slice is non-empty.  The unsplit kernel instead takes
// fewer rows per workgroup, which re-reads the small operand from the
// caches once per workgroup; it is fast at short K, and the split's second
// launch costs about 2 us, so the split is taken only for KT >=
// kSkinnySplitBaseTiles + kSkinnySplitFillTiles * blocks / num_cus K tiles
// (longer K the more CUs the blocks already fill).  The constants come from
// kernel-trace timings of every admissible slice count on 2, 8 and 16 small
// rows, 64..3072 large rows and K = 1024..14336 on an MI355X: there the rule
// was never slower than no split and within 0.1 us of the fastest choice.
// Returns 1 (no split) otherwise.
constexpr int kSkinnySplitMinTiles = 2;
constexpr int kSkinnySplitBaseTiles = 8;
constexpr int kSkinnySplitFillTiles = 64;
inline int skinny_splitk_splits(int64_t R, int64_t K, int num_cus) {
  const int64_t blocks = (R + 15) / 16;
  const int64_t kt = (K + 511) / 512;
  if (blocks >= num_cus || kt < 2 * kSkinnySplitMinTiles) return 1;
  if (kt * num_cus < static_cast<int64_t>(kSkinnySplitBaseTiles) * num_cus + kSkinnySplitFillTiles * blocks) return 1;
  int64_t splits = num_cus / blocks;
  if (splits > kt / kSkinnySplitMinTiles) splits = kt / kSkinnySplitMinTiles;
  if (splits < 2) return 1;
  const int64_t per = (kt + splits - 1) / splits;
  return static_cast<int>((kt + per - 1) / per);  // drop slices that would be empty
}

// The static scratch of gemm_splitk_f16_noalloc (FP32 partial sums,
// [splits][M][N]) and the device address of the current device's copy of it.
constexpr int64_t kNoAllocScratchBytes = int64_t{16} << 20;
hipError_t noalloc_scratch(void **ptr);

// s_waitcnt immediate for "lgkmcnt(0)" alone on gfx9-family targets
// (vmcnt field [3:0]|[15:14] = 63, expcnt [6:4] = 7, lgkmcnt [11:8] = 0).
// Issued through the builtin so the compiler knows the LDS reads are done.
constexpr unsigned kWaitLgkm0 = 0xC07F;

// The K-loop schedule of tiled GEMM variant `variant` (a
// gemvtile_gemm_f16_variant number whose kernel has a multi-stage ring) over
// ktu K tiles, as the host-side trace of the ring walker (ring.hpp): up to
// `cap` events of five int32 each are written to `events` (which may be
// NULL); returns the number of events, or -1 for a variant without a ring.
// info[0..7] receive the kernel's loads per wave per K tile, operand reads
// and MFMAs per wave per K step, K steps per K tile, ring stages, bm, bn and
// whether it runs the early-free schedule (1) or not (0).
int64_t ring_trace(int variant, int ktu, int32_t *events, int64_t cap, int *info);
// The 256x256 tiled kernel of gemm_f16 with per-workgroup timestamps
// (kEpiTimed in gemm_kernel.hpp) written to stamps[8 * workgroup ...].
hipError_t launch_gemm_f16_timed(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                                 uint64_t *stamps, hipStream_t stream);
hipError_t launch_gemm_f16(int variant, const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                           hipStream_t stream);
hipError_t launch_gemm_skinny_f16(int variant, const void *A, const void *B, void *D, int M, int N, int K,
                                  int num_cus, hipStream_t stream);
hipError_t launch_gemv_f16(int variant, const void *x, const void *W, void *y, int N, int K, int num_cus,
                           hipStream_t stream);
hipError_t launch_gemm_ws_f16(int variant, const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                              hipStream_t stream);
hipError_t launch_fill_zero_f16(void *p, int64_t count, hipStream_t stream);
// bf16 operands and results: the default launch shape of each kernel.
// D = act(A·Bᵀ + bias) on the tiled kernel (the tile gemm_default_tile
// picks, whatever the shape), dtype kF16 or kBF16; bias [N] or NULL, relu 0
// or 1.  K == 0 fills D with act(bias).
hipError_t launch_gemm_bias(int dtype, const void *A, const void *B, const void *bias, int relu, void *D, int M, int N,
                            int K, int num_cus, hipStream_t stream);
// Split-K GEMM on the tiled kernel: `splits` K slices write FP32 partial
// sums to ws [splits][M][N], then a reduction adds them in slice order and
// rounds into D.  dtype kF16 or kBF16.
hipError_t launch_gemm_splitk(int dtype, const void *A, const void *B, void *D, int M, int N, int K, void *ws,
                              int splits, int num_cus, hipStream_t stream);
// The same for shapes with 2..16 rows on one side, on the skinny kernel
// (16 rows of the large side per workgroup, `splits` workgroups per block
// of rows).
hipError_t launch_gemm_skinny_splitk(int dtype, const void *A, const void *B, void *D, int M, int N, int K, void *ws,
                                     int splits, hipStream_t stream);
// D[i] = round(ws[0][i] + ... + ws[splits-1][i]) for i < count, in slice order.
hipError_t launch_splitk_reduce(int dtype, const float *ws, void *D, int64_t count, int splits, hipStream_t stream);
hipError_t launch_gemm_bf16(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                            hipStream_t stream);
hipError_t launch_gemm_skinny_bf16(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                                   hipStream_t stream);
hipError_t launch_gemv_bf16(const void *x, const void *W, void *y, int N, int K, int num_cus, hipStream_t stream);

}  // namespace gt
