/*
 * gemvtile.h -- C ABI of the MI355X (gfx950) FP16 / BF16 GEMM and GEMV library.
 *
 * Every entry point takes plain pointers and sizes; no C++ or framework type
 * crosses this boundary.  All matrices are dense and row-major.  "fp16" means
 * IEEE 754 binary16; "bf16" means bfloat16 (1 sign bit, 8 exponent bits with
 * bias 127, 7 fraction bits: the upper half of a binary32).  Device pointers are HIP device (or managed) pointers on
 * the device that is current for the calling host thread.
 *
 * Ownership: the caller allocates and frees every buffer.  The library keeps
 * no pointer after a call returns and allocates no device memory on these
 * paths (no hidden workspace).
 *
 * Streams: every compute call is stream-ordered and asynchronous.  It
 * enqueues its kernel on `stream` (a hipStream_t; NULL is the default stream)
 * and returns at once; the result is ready when that stream reaches the
 * point of the call.  Errors found before the launch are returned without any
 * HIP call being made, so they are reported identically on a machine with no
 * GPU.
 *
 * Aliasing: D (or y) must not overlap A, B (or x, W); doing so is undefined.
 * Thread safety: calls from several host threads are safe; the library's only
 * mutable state is a per-device cache of the compute-unit count.
 */
#ifndef GEMVTILE_H
#define GEMVTILE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum gemvtile_status {
    GEMVTILE_OK = 0,
    GEMVTILE_ERR_INVALID_ARG = 1, /* NULL pointer with a nonzero extent, negative size */
    GEMVTILE_ERR_UNSUPPORTED = 2, /* K % 8 != 0, misaligned pointer, size beyond the limits below */
    GEMVTILE_ERR_LAUNCH = 3,      /* the HIP launch failed (no gfx950 device, bad stream, ...) */
    GEMVTILE_ERR_DEVICE = 4,      /* a HIP runtime query failed */
    GEMVTILE_ERR_SCRATCH = 5      /* gemm_splitk_f16_noalloc: partial sums beyond its static scratch */
};

/*
 * gemm_f16 -- D = A · Bᵀ with FP32 accumulation and one final rounding of each
 * output to fp16, round-to-nearest, ties to even.
 *
 *   D[m,n] = fp16_rne( sum_{k<K} A[m,k] * B[n,k] )   for m < M, n < N
 *
 * Defined by "使用 TMA 为 GEMM 建立 Pipeline" (TVM TIRx GEMM chapter), step 4
 * full kernel: A is (M,K), B is (N,K), D is (M,N), fp16 in and out with the
 * accumulator in FP32; the same layout is the Croqtile tutorial's ch. 7
 * pipelined matmul (lhs [M,K], rhs [N,K]) and the SM120 walk-through
 * "TensorCore_GEMM_with_TMA" §2.2 entrance, whose epilogue rounds with `_rn`.
 *
 *   A  device pointer, [M,K] fp16, row-major (leading dimension K), 16-byte aligned
 *   B  device pointer, [N,K] fp16, row-major (leading dimension K), 16-byte aligned
 *   D  device pointer, [M,N] fp16, row-major (leading dimension N), 2-byte aligned;
 *      only the M·N elements are written
 *   M, N, K  sizes; 0 <= M, N <= 2^31 - 512; 0 <= K <= 4,194,296 and K % 8 == 0
 *   stream   hipStream_t or NULL
 *
 * M == 0 or N == 0: returns GEMVTILE_OK and touches nothing (pointers may be NULL).
 * K == 0: D is filled with +0 (the empty sum); A and B may be NULL.
 * M, N need not be multiples of any tile size: edge tiles read zeros beyond
 * the matrix and write only inside it.  The summation order within FP32 is
 * unspecified (several results are correct up to rounding).
 * Otherwise the tiled kernel runs with 256x256 output tiles, or with
 * 256x128, 128x256, 128x128 or 128x64 ones when the output has too few 256x256
 * tiles to keep every compute unit busy (gemvtile_gemm_tile gives the choice);
 * it writes D with non-temporal stores, so D is not left in the caches.
 * When the smaller side has at most 64 rows -- a decode batch against a
 * weight matrix --, the call runs a bandwidth-bound kernel that streams the
 * larger operand once instead of the tiled one (32, 48 or 64 rows of it per
 * workgroup when it gives every compute unit 32, else 16, 8, 4, 2 or 1;
 * with 17..64 rows on the smaller side and few on the larger, the smaller
 * side is split into 16-row blocks over the workgroups instead), and when
 * M == 1 or N == 1 the GEMV kernel of gemv_f16; results are deterministic
 * either way.
 * Returns a gemvtile_status.
 */
int gemm_f16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * gemv_f16 -- y = x · Wᵀ (the batch-1 decode product), FP32 accumulation,
 * one fp16 rounding (nearest, ties to even) per output.
 *
 *   y[n] = fp16_rne( sum_{k<K} x[k] * W[n,k] )   for n < N
 *
 * Defined by "Learning TileLang with GEMV", §01 GEMV: the matrix is (N,K)
 * row-major as nn.Linear stores its weight, all kernels accumulate in FP32.
 *
 *   x  device pointer, [K] fp16, 16-byte aligned
 *   W  device pointer, [N,K] fp16, row-major (leading dimension K), 16-byte aligned
 *   y  device pointer, [N] fp16, 2-byte aligned
 *   N, K  sizes; 0 <= N <= 2^31 - 1; 0 <= K <= 2^31 - 8 and K % 8 == 0
 *   stream hipStream_t or NULL
 *
 * N == 0: returns GEMVTILE_OK and touches nothing.  K == 0: y is filled with +0.
 * When N is too small to give every compute unit a workgroup of 16 rows, or
 * when K >= 8192, the waves of a workgroup also split K (§5.2
 * block_split_k's reason: enough blocks in flight); the slices' FP32 partial
 * sums are added in LDS in a fixed order (gemvtile_gemv_grid gives the
 * workgroup count).  The row sums
 * are deterministic: no atomics, no split across workgroups, no workspace.
 * Returns a gemvtile_status.
 */
int gemv_f16(const void *x, const void *W, void *y, int64_t N, int64_t K, void *stream);

/*
 * gemm_bf16 / gemv_bf16 -- gemm_f16 and gemv_f16 with bf16 operands and
 * results: the same contract (layouts, sizes and their limits, alignment,
 * degenerate shapes, streams, errors, determinism), FP32 accumulation, and
 * one rounding of each output to bf16, round-to-nearest, ties to even.
 *
 *   D[m,n] = bf16_rne( sum_k A[m,k] * B[n,k] )     y[n] = bf16_rne( sum_k x[k] * W[n,k] )
 *
 * bf16 in and out with FP32 accumulators is the element type of the SM120
 * walk-through "TensorCore_GEMM_with_TMA" (§2.2 entrance: nv_bfloat16 A, B,
 * C; §2.3 kernel: FP32 accumulators rounded with __float22bfloat162_rn).
 * Shapes route as for fp16 (M or N == 1: the GEMV kernel; M or N <= 16, or
 * 17..64 rows on the smaller side as gemm_f16 describes: the skinny kernel;
 * otherwise the tiled
 * kernel), each in its default launch shape.
 */
int gemm_bf16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *stream);
int gemv_bf16(const void *x, const void *W, void *y, int64_t N, int64_t K, void *stream);

/* Activation codes of the fused epilogue. */
enum gemvtile_act {
    GEMVTILE_ACT_NONE = 0, /* identity */
    GEMVTILE_ACT_RELU = 1  /* v < 0 -> +0, else v (a NaN stays NaN) */
};

/*
 * gemm_bias_f16 / gemm_bias_bf16 -- the GEMM with a fused epilogue: a bias
 * added to every row and an activation, before the one rounding.
 *
 *   D[m,n] = rne( act( sum_{k<K} A[m,k] * B[n,k] + bias[n] ) )
 *
 * The pages' kernels end their epilogue at the rounded store and define no
 * bias or activation; this is the plain definition of the usual fused
 * epilogue, in the same element format as gemm_f16 (fp16) or gemm_bf16
 * (bf16).  The sum is accumulated in FP32, bias[n] is added in FP32, the
 * activation is applied, and the result is rounded once (nearest, ties to
 * even).
 *
 *   A, B, D, M, N, K, stream  as for gemm_f16 / gemm_bf16 (same layouts,
 *            limits, alignment and degenerate shapes)
 *   bias   device pointer to N elements of the operand format, 2-byte
 *          aligned, or NULL for no bias
 *   act    GEMVTILE_ACT_NONE or GEMVTILE_ACT_RELU
 *
 * K == 0: D[m,n] = act(bias[n]) (+0 with no bias).  Every shape runs the
 * tiled kernel with the tile gemvtile_gemm_tile gives (the skinny and GEMV
 * kernels have no fused epilogue), so outputs with 16 rows or fewer on a
 * side are slower here than through gemm_f16.  An unknown act returns
 * GEMVTILE_ERR_INVALID_ARG, a misaligned bias GEMVTILE_ERR_UNSUPPORTED, both
 * before any HIP call.  Returns a gemvtile_status.
 */
int gemm_bias_f16(const void *A, const void *B, const void *bias, void *D, int64_t M, int64_t N, int64_t K, int act,
                  void *stream);
int gemm_bias_bf16(const void *A, const void *B, const void *bias, void *D, int64_t M, int64_t N, int64_t K, int act,
                   void *stream);

/*
 * gemm_splitk_f16 / gemm_splitk_bf16 -- gemm_f16 / gemm_bf16 with K split
 * across workgroups, for outputs too small to keep every compute unit busy
 * even with 128x128 tiles (a 1024x1024 output has 64 of them), and for
 * decode-batch shapes with 2..16 rows on one side whose other side has too
 * few blocks of 16 rows (8 x 1024 has 64).  Same contract and result
 * definition as gemm_f16 / gemm_bf16.
 *
 * The pages split K over blocks for the GEMV ("Learning TileLang with GEMV",
 * §5.2 block_split_k) and add the partial sums with FP32 atomics into a
 * zeroed output.  Here each (tile, K slice) workgroup unit stores its FP32
 * partial sums to `workspace`, [splits][M][N] floats, and a second kernel
 * adds the slices in slice order and rounds once: no atomics, no zeroing,
 * and every output is deterministic (the summation order depends only on
 * the shape and the device's compute-unit count).
 *
 *   workspace        device memory, 16-byte aligned, owned by the caller; its
 *                    contents on entry do not matter and are overwritten
 *   workspace_bytes  its size; at least gemvtile_gemm_splitk_workspace(M, N,
 *                    K, #CUs) for the current device
 *
 * Shapes that do not split (their tiles or row blocks already fill the CUs,
 * K too short for the split to pay, or one row on a side) run exactly as
 * gemm_f16 / gemm_bf16 and do not touch the workspace, which may then be
 * NULL.  A workspace that is too small
 * or NULL when needed returns GEMVTILE_ERR_INVALID_ARG, a misaligned one
 * GEMVTILE_ERR_UNSUPPORTED; these checks follow the (cached) compute-unit
 * query and precede any launch.  Calls that share a workspace must be
 * ordered on one stream.  Returns a gemvtile_status.
 */
int gemm_splitk_f16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *workspace,
                    int64_t workspace_bytes, void *stream);
int gemm_splitk_bf16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *workspace,
                     int64_t workspace_bytes, void *stream);

/*
 * gemm_splitk_f16_noalloc -- gemm_splitk_f16 for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): no workspace argument, and no
 * allocation of any kind on the call path.  Same result, rounding and
 * determinism as gemm_splitk_f16 (the same kernels, in the same order).
 *
 * The FP32 partial sums go to a static device array of 16 MiB
 * (splits * M * N * 4 bytes are needed, see gemvtile_gemm_splitk_workspace)
 * that the library holds on each device it runs on until the process ends.
 * Shapes split only while their tiles (128x128 whenever they split) leave
 * compute units idle, and tiles * splits <= #CUs, so on parts with up to
 * 256 compute units every shape fits; a shape that needs more (on a larger
 * part) returns GEMVTILE_ERR_SCRATCH before any launch (use
 * gemm_splitk_f16 with a workspace then).  Shapes that do not split run
 * exactly as gemm_f16 and need none.  Every partial sum the reduction reads
 * is written by the same call, so the array needs no clearing; it keeps the
 * last call's contents.  All calls on one device share its one array:
 * calls that overlap on one GPU (on different streams, or from different
 * host threads without ordering) race and give undefined results; order
 * them on one stream.  Returns a gemvtile_status.
 */
int gemm_splitk_f16_noalloc(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * gemvtile_gemm_splitk_splits / gemvtile_gemm_splitk_workspace -- the number
 * of K slices gemm_splitk_* uses for an M x N x K product on `num_cus`
 * compute units, and the workspace bytes it needs (splits * M * N * 4, or 0
 * when it does not split).  With T tiles of the tile gemvtile_gemm_tile
 * picks and KT = ceil(K / 64) K tiles: no split when T >= num_cus or
 * KT < 20; otherwise
 * splits = min(floor(num_cus / T), floor(KT / 10)), each slice ceil(KT /
 * splits) K tiles, minus slices left empty; 1 (0 bytes) below 2, and 1 unless
 * the K loop gets shorter by KT (splits - 1) / splits >= 12 + splits M N /
 * 2^18 K tiles (evaluated in double precision): a fixed cost, and one for
 * the partial sums' traffic.  With 2..16 rows on one side (the skinny
 * kernel), with B = ceil(R / 16) blocks of the other side's R rows and KT =
 * ceil(K / 512): no split when B >= num_cus, KT < 4 or KT num_cus < 8
 * num_cus + 64 B; otherwise splits = min(floor(num_cus / B), floor(KT / 2)),
 * each slice ceil(KT / splits) K tiles, minus slices left empty.  One row
 * on a side (the GEMV) never splits.  Host-only arithmetic; 1 and 0 for
 * sizes <= 0 or num_cus out of (0, 2^20].
 */
int gemvtile_gemm_splitk_splits(int64_t M, int64_t N, int64_t K, int64_t num_cus);
int64_t gemvtile_gemm_splitk_workspace(int64_t M, int64_t N, int64_t K, int64_t num_cus);

/* A static, human-readable name for a status code (never NULL). */
const char *gemvtile_status_string(int status);

/*
 * gemvtile_tile_coord -- the grouped tile order the persistent GEMM walks
 * (host-callable, no GPU needed).  Tile index t in [0, tiles_m*tiles_n) maps
 * to the output tile (*tm, *tn); consecutive t run down `group_m` tile rows of
 * one tile column, then move to the next column; the last group may be
 * shorter.  This is the threadblock swizzle of "TensorCore_GEMM_with_TMA"
 * §2.3 kernel (GROUP_M = 8), which the TVM chapter's step 6 persistent
 * scheduler (l2_group_size = 8) also uses for L2 locality.
 * Returns GEMVTILE_ERR_INVALID_ARG for t out of range, non-positive sizes or
 * NULL outputs.
 */
int gemvtile_tile_coord(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t group_m, int64_t *tm, int64_t *tn);

/*
 * gemvtile_gemm_config -- the compile-time shape of the 256x256 tiled GEMM
 * kernel that gemm_f16 launches on large outputs: output tile BM x BN, K
 * tile BK, LDS ring depth, threads per workgroup and the grouped-order
 * height.  Any output pointer may be NULL.
 */
void gemvtile_gemm_config(int *bm, int *bn, int *bk, int *stages, int *threads, int *group_m);

/*
 * gemvtile_gemm_tile -- the output tile (bm x bn) and LDS ring depth the
 * tiled GEMM takes for an M x N output on `num_cus` compute units (gemm_f16
 * and gemm_bf16 when they take the tiled kernel).  Of 256x256 (2
 * stages), 256x128 and 128x256 (3 stages), 128x128 and 128x64 (4 stages),
 * it is the one with the least ceil(#tiles / num_cus) * bm * bn / rate,
 * where rate is the tile's measured work rate relative to 256x256 with
 * tiles to spare (1, 0.9, 0.9, 0.76, 0.55); ties go to the larger tile.
 * The split-K entry points choose the same way among the first four.  Smaller tiles fill the CUs
 * when large ones would leave some idle (an 8192 x 1024 output has 128 tiles
 * of 256x256, 256 of 256x128); their deeper rings cover the load latency
 * over their shorter K tiles.  Any output pointer may be NULL.  Host-only
 * arithmetic; returns GEMVTILE_ERR_INVALID_ARG for M, N or num_cus <= 0 or
 * num_cus > 2^20.
 */
int gemvtile_gemm_tile(int64_t M, int64_t N, int64_t num_cus, int *bm, int *bn, int *stages);

/*
 * gemvtile_device_caps -- the current device's compute-unit count, peak
 * engine clock (kHz), peak memory clock (kHz) and memory bus width (bits),
 * for recomputing the roofline peaks from the part itself.  Any output
 * pointer may be NULL.  Returns GEMVTILE_ERR_DEVICE if a HIP query fails.
 */
int gemvtile_device_caps(int *num_cus, int *clock_khz, int *mem_clock_khz, int *mem_bus_bits);

/*
 * gemvtile_gemv_grid -- the number of workgroups gemv_f16 (and gemv_bf16)
 * launches for an N x K matrix on a device with `num_cus` compute units:
 * ceil(N/R) with R = 2 rows per workgroup (K split 8 ways over the
 * workgroup's 8 waves) when K >= 8192 and N >= 2*num_cus; otherwise R = 16
 * rows per workgroup when N >= 16*num_cus, else 8, 4 or 2 rows (K split 2,
 * 4 or 8 ways) while N >= 8, 4 or 2 times num_cus; else 1 row (K split 8
 * ways).  Host-only arithmetic; returns 0 for N <= 0, K < 0 or num_cus
 * outside [1, 2^20].
 */
int64_t gemvtile_gemv_grid(int64_t N, int64_t K, int64_t num_cus);

/*
 * gemvtile_gemm_grid -- the number of workgroups gemm_f16 launches for an
 * M x N x K product on a device with `num_cus` compute units: the GEMV grid
 * of the other side's rows when M or N is 1; when the smaller side has at
 * most 64 rows (the skinny kernel), ceil(R/p) with R = N if M <= 16, else M
 * if N <= 16, else the larger side, and p rows per workgroup: when
 * R >= 32*num_cus, the one of 32, 48, 64 with the least
 * ceil(ceil(R/p)/num_cus)*p (ties to the larger), else the largest of 16,
 * 8, 4, 2 such that R >= p*num_cus, else 1; except that,
 * when the smaller side S has 17..64 rows and that p is below 8 (or 8 with
 * S <= 32), ceil(S/16)*ceil(R/q) with q the largest of 16, 8, 4, 2 such
 * that ceil(S/16)*ceil(R/q) >= num_cus, else q = 1 (the smaller side split
 * into 16-row blocks); otherwise the persistent grid min(#tiles, num_cus)
 * over the tiles gemvtile_gemm_tile picks.  Host-only arithmetic; returns 0
 * for empty outputs.
 */
int64_t gemvtile_gemm_grid(int64_t M, int64_t N, int64_t K, int64_t num_cus);

/*
 * gemvtile_gemm_f16_variant -- gemm_f16 with an internal kernel variant, for
 * ablation measurements only (same contract and results as gemm_f16).
 *   0  what gemm_f16 runs: on tiled shapes the tile of gemvtile_gemm_tile;
 *      with 256x256 tiles, 4 waves of 128x128, 16x16x32 MFMA blocks, K tiles
 *      of 64 in a 2-stage LDS ring, the next K step's operand reads one every
 *      2 MFMA slots, a refill load every 4 slots, swizzled LDS, persistent
 *      grouped XCD-aware schedule, and the early-free K loop (a second
 *      barrier per K tile, at MFMA slot 48 of K step 0, after which the
 *      wave's stage is refilled, half a K tile sooner than with one barrier);
 *      each K step's MFMAs in serpentine order over the wave's 16x16 blocks
 *   1  as 20 without the LDS swizzle
 *   2  as 10 with single-stage LDS (load, wait, compute: no overlap)
 *   3  as 20 with one workgroup per tile (no persistent loop, no XCD remap)
 *   10 as 30 with 32x32x16 MFMA blocks, one operand read per slot, a refill
 *      load every 2 of its 64 slots per K tile
 *   20 the 256x256 tiled kernel of variant 0, whatever the shape
 *   21, 22, 23 the same schedule on 256x128, 128x256 (3-stage rings) and
 *      128x128 (4-stage ring) output tiles (4 waves of 128x64, 64x128,
 *      64x64): the smaller tiles of variant 0, whatever the shape
 *   24, 25, 26 as 21, 22, 23 with 2-stage rings   27 as 23 with 5 stages
 *   32 the 128x64 tile of variant 0 (4-stage ring, 4 waves of 32x64),
 *      whatever the shape
 *   28 as 20 with D written by ordinary (cached) stores instead of
 *      non-temporal ones
 *   30 as 20 with one barrier per K tile (the ring without the early free)
 *   31 as 20 with the MFMAs of a K step in row-major order over the blocks
 * Variants 1..32 always run the tiled kernel, whatever the shape; variant
 * 0 routes shapes as gemm_f16 does (M or N == 1: the GEMV kernel; M or N
 * <= 16, and some shapes with 17..64 rows on the smaller side: the skinny
 * kernel).  The skinny kernel (only for M <= 16 or N <= 16, and 160 also
 * for 17..64 rows on the smaller side, else GEMVTILE_ERR_UNSUPPORTED):
 *   100 the gemm_f16 choice (32, 48, 64, 16, 8, 4, 2 or 1 rows of the
 *       large side per workgroup, see gemvtile_gemm_grid)
 *   104 operands loaded straight into registers (8 waves, 4 K steps of 32
 *       in flight per wave), 16 large-side rows per workgroup
 *   112 operands staged through a 4-stage LDS ring of 1 KiB row segments,
 *       16 waves, 16 large-side rows per workgroup
 *   130 as 112 with workgroup b starting its K walk at K tile b (mod the
 *       number of K tiles)
 *   147 as 130 with the large side loaded non-temporally
 *   152 as 147 with every workgroup starting its K walk at K tile 0
 *   160 the small side split into blocks of 16 rows along the grid's y
 *       dimension, each workgroup staging one block against 16, 8, 4, 2 or
 *       1 rows of the large side (the most that still give every compute
 *       unit a workgroup); also for 17..64 rows on the smaller side
 * (gemm_f16's choice at 16 rows per workgroup starts workgroup b at K tile
 * b / 8, its index within its XCD, and loads the large side non-temporally
 * from K = 8192 up.)
 * The wave-specialised kernel, whatever the shape:
 *   200, 201 256x128 output tiles, 4 consumer waves (MFMA only, 128x64
 *       each) and 4 loader waves (tile loads only) handing K tiles over at
 *       one barrier per K tile, with a 3-stage (200) or 2-stage (201) ring
 * Other numbers (ablations measured and not kept) return
 * GEMVTILE_ERR_INVALID_ARG.
 */
int gemvtile_gemm_f16_variant(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                              void *stream, int variant);

/*
 * gemvtile_gemm_f16_timed -- measurement only: the 256x256 tiled kernel of
 * gemm_f16 (variant 20) on an M x N x K product (M, N > 16, K > 0; same
 * result as gemm_f16), with one record of 8 uint64 per workgroup written to
 * `stamps` (host-visible or device memory of `stamps_len` uint64, at least
 * 8 * min(#256x256 tiles, #CUs), 8-byte aligned) by its first thread:
 *   [0], [1]  the constant 100 MHz real-time counter and the shader-cycle
 *             counter when the workgroup started
 *   [2], [3]  the same when the K loop of its first output tile ended
 *   [4], [5]  the same when it finished, after every store of every wave
 *             completed
 *   [6], [7]  the HW_ID and XCC_ID hardware registers (XCD in bits 0..3 of
 *             the latter)
 * Cycle deltas over real-time deltas give the clock each workgroup ran at.
 * Returns GEMVTILE_ERR_UNSUPPORTED for shapes gemm_f16 would not run on the
 * tiled kernel, GEMVTILE_ERR_INVALID_ARG for too small a buffer.
 */
int gemvtile_gemm_f16_timed(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, void *stream,
                            uint64_t *stamps, int64_t stamps_len);

/*
 * gemvtile_gemv_f16_variant -- gemv_f16 with an internal launch shape, for
 * measurements only (same contract and results as gemv_f16):
 *   0  the gemv_f16 default (picks one of 8..12 from N, K and the
 *      compute-unit count, see gemvtile_gemv_grid, or its cached twin
 *      37..41 when W holds fewer than 2^25 elements)
 *   6  2 rows per wave, 8 waves, 4 chunk steps in flight, ordinary (cached)
 *      loads of W, each wave starting its walk along K at a different group
 *   7  as 6 with non-temporal loads of W and every wave starting at the
 *      row's first column
 *   8..11  2 rows per wave, 8 waves, 4 steps, non-temporal W, rotated start,
 *      K split over 1, 2, 4, 8 waves per row group (16, 8, 4, 2 rows per
 *      workgroup)
 *   12 1 row per workgroup, K split 8 ways
 *   20 as 8 with grid-strided rows: local row r (0..15) of workgroup b is
 *      row r*G + b (G = the grid size), so workgroups running side by side
 *      read adjacent rows, instead of 16 consecutive rows per workgroup
 *   21 as 8 with x staged in LDS once per workgroup (K <= 16384, else
 *      GEMVTILE_ERR_INVALID_ARG) instead of loaded by every wave
 *   28 as 7 with 8 chunk steps in flight
 *   29 as 7 with 4 rows per wave and 4 waves
 *   37..41 as 8..12 with cached (not non-temporal) loads of W
 * Other numbers return GEMVTILE_ERR_INVALID_ARG.
 */
int gemvtile_gemv_f16_variant(const void *x, const void *W, void *y, int64_t N, int64_t K, void *stream,
                              int variant);

/*
 * gemvtile_ring_trace -- the K-loop schedule of the tiled GEMM kernel, for
 * checking on the CPU (host-only; no GPU needed).  The kernel's K loop is a
 * walker over K tiles that issues tile loads, operand reads, MFMAs, waits
 * and barriers; this runs the same walker on the host for the kernel of
 * tiled variant `variant` (a gemvtile_gemm_f16_variant number: 0 = 20, the
 * 256x256 default; 1 and 3 share its ring; 10, 20..27, 30 and 31) over `ktu`
 * K tiles (of 64 elements), recording each event instead of issuing it.
 * The ring follows "使用 TMA 为 GEMM 建立 Pipeline" (TVM TIRx GEMM chapter),
 * step 5 (Pipeline 机制): K tile k in stage k % stages, refilled with tile
 * k + stages once consumed; completion is tracked by in-order vmcnt waits
 * instead of the chapter's per-stage mbarrier phases.
 *
 *   ktu     K tiles the loop walks (1 .. 2^20): ceil(K / 64), or one K slice
 *           of a split-K unit
 *   events  host memory for `cap` events of five int32 {code, a, b, c, d}:
 *             1 load      a = K tile, b = load index, c = ring stage
 *             2 wait      a = vmcnt (vector-memory operations allowed to
 *                         stay in flight)
 *             3 LDS wait  (the wave's LDS reads are complete)
 *             4 barrier   (workgroup barrier)
 *             5 read      a = K tile, b = K step, c = read index, d = stage;
 *                         with nA x nB MFMA blocks per wave, read index 0
 *                         fetches A block 0, 1..nB the B blocks 0..nB-1,
 *                         and nB+1.. the A blocks 1..nA-1
 *             6 MFMA      a = fragment buffer, b = MFMA index in the K step,
 *                         c = its block row (A block), d = its block
 *                         column (B block)
 *             7 prep      a = K tile, b = part: part b of working out the
 *                         addresses of that K tile's refill loads (the
 *                         early-free schedule), ahead of those loads
 *             8 init      the accumulators are zeroed (once, after the
 *                         prologue's loads are issued)
 *           events beyond `cap` are counted but not written; may be NULL
 *           when cap == 0
 *   info    if not NULL, 10 ints: loads per wave per K tile, operand reads
 *           per wave per K step, K steps per K tile, MFMAs per wave per K
 *           step, ring stages, output tile rows and columns, 1 for the
 *           early-free schedule (two barriers per K tile) or 0, and the
 *           waves along the tile's rows and along its columns
 * Each wave of the workgroup runs this same sequence.  Returns the number
 * of events, or -1 for a variant without a multi-stage ring or arguments
 * out of range.
 */
int64_t gemvtile_ring_trace(int variant, int64_t ktu, int32_t *events, int64_t cap, int *info);

/*
 * gemvtile_xcd_logical_id -- the logical workgroup id the persistent GEMM
 * gives hardware workgroup `w` of a `grid`-wide launch.  Workgroups are
 * dispatched to the 8 XCDs round-robin; when grid % 8 == 0 the renumbering
 * gives each XCD one contiguous range of ids (so neighbouring tiles in the
 * grouped order share an L2), otherwise it is the identity.  Host-only;
 * returns -1 for w outside [0, grid) or grid <= 0.
 */
int64_t gemvtile_xcd_logical_id(int64_t w, int64_t grid);

#ifdef __cplusplus
}
#endif

#endif /* GEMVTILE_H */
