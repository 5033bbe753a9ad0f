// gemv.hip -- batch-1 FP16 / BF16 GEMV for gfx950: y = x · Wᵀ.
//
//   x [K], W [N,K] row-major (nn.Linear layout), y [N]; fp16 in and out, FP32
//   accumulation, one round-to-nearest-even per output ("Learning TileLang
//   with GEMV", §01 GEMV).
//
// The product reads every byte of W once and does one multiply-add per two
// bytes, so its time is the time to stream W from HBM (§02 Bandwidth Bound).
// What the page found to matter -- enough blocks in flight, neighbouring
// lanes reading neighbouring addresses, 16 bytes per lane per load (§4.5
// thread_vectorized_split_k), and a register/shuffle reduction with no shared
// memory round trip (§4.6 thread_tvm_reduce_split_k) -- is re-derived here for
// 64-wide waves:
//
//  * one wave owns ROWS consecutive rows of W; its 64 lanes walk each row in
//    16-byte chunks, lane l taking chunks l, l+64, l+128, ..., so one wave
//    load instruction reads 1 KiB of contiguous row;
//  * the x chunk a lane needs is the same for all ROWS rows, so it is loaded
//    once and reused from registers;
//  * UNROLL chunk steps are issued back to back, keeping UNROLL*(ROWS+1)
//    16-byte loads in flight per lane; whole groups of steps run without a
//    bounds test, and only the ragged end of a row takes a guarded group;
//  * the waves of a launch start their walk along K at different groups
//    and wrap around, so at any moment they read different column windows;
//  * W is read with non-temporal loads (streamed once, no reuse);
//  * v_dot2_f32_f16 multiplies fp16 pairs and accumulates in FP32;
//  * the 64 lane partial sums of a row are combined with DPP lane moves
//    inside the wave (no LDS, no atomics, no second kernel), so each row sum
//    is deterministic; a wave's rows are reduced together so that the short
//    dependent chains overlap;
//  * when N is too small to give every CU a workgroup of whole-row waves, the
//    waves of a workgroup also split K (the page's "enough blocks" lesson,
//    §5.2 block_split_k, which splits K over blocks and adds the partial sums
//    with FP32 atomics): KSPLIT waves share each row group, each walks one
//    slice of K, and the slices' FP32 row sums meet in LDS and are added in
//    slice order, so the result stays deterministic and no workspace is
//    needed.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace gt {

// acc + a · b over 8 elements, products and sums in FP32 (v_dot2_f32_f16 or
// v_dot2_f32_bf16 on pairs).
template <int DT>
__device__ inline float dot8_acc(half8_t a, half8_t b, float acc) {
  if constexpr (DT == kF16) {
    acc = __builtin_amdgcn_fdot2(half2_t{a[0], a[1]}, half2_t{b[0], b[1]}, acc, false);
    acc = __builtin_amdgcn_fdot2(half2_t{a[2], a[3]}, half2_t{b[2], b[3]}, acc, false);
    acc = __builtin_amdgcn_fdot2(half2_t{a[4], a[5]}, half2_t{b[4], b[5]}, acc, false);
    acc = __builtin_amdgcn_fdot2(half2_t{a[6], a[7]}, half2_t{b[6], b[7]}, acc, false);
  } else {
    const bf16x8_t x = __builtin_bit_cast(bf16x8_t, a);
    const bf16x8_t w = __builtin_bit_cast(bf16x8_t, b);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{x[0], x[1]}, bf16x2_t{w[0], w[1]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{x[2], x[3]}, bf16x2_t{w[2], w[3]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{x[4], x[5]}, bf16x2_t{w[4], w[5]}, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{x[6], x[7]}, bf16x2_t{w[6], w[7]}, acc, false);
  }
  return acc;
}

// One DPP step: v + (v as seen through the lane pattern `ctrl`), restricted
// to the rows of 16 lanes selected by ROW_MASK (other rows add zero).
template <int CTRL, int ROW_MASK = 0xF>
__device__ inline float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false);
  return v + __builtin_bit_cast(float, moved);
}

// Sum of the 64 lane values of a wave, returned to every lane.  The data
// moves through DPP lane patterns of the VALU (a few cycles each) instead of
// LDS permutes (a round trip each): swap neighbours, swap pairs, mirror
// within 8 and within 16 lanes leave the 16-lane sum in every lane of each
// row; row_bcast:15 then adds row 0 into row 1 and row 2 into row 3, and
// row_bcast:31 adds lane 31 into rows 2 and 3, so lane 63 holds the total,
// which v_readlane broadcasts.  Several independent sums interleave well.
__device__ inline float wave_sum(float v) {
  v = dpp_add<0xB1>(v);        // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);        // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);       // row_half_mirror
  v = dpp_add<0x140>(v);       // row_mirror
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Rows of W a wave works on.  ROWMAP 0: workgroup b owns the kRows
// consecutive rows starting at b * kRows, and its row group g (of ROWS rows)
// the ROWS consecutive rows g * ROWS .. of those.  ROWMAP 1 (grid-strided):
// workgroup b owns rows b, b + G, b + 2G, ... (G = the grid size), so the
// workgroups running side by side read adjacent rows -- one contiguous
// front through W, as a plain read stream would -- instead of regions
// kRows rows apart.
template <int ROWMAP, int ROWS>
__device__ inline int64_t wave_row(int group, int r, int rows_per_wg) {
  const int local = group * ROWS + r;
  if constexpr (ROWMAP == 0) return static_cast<int64_t>(blockIdx.x) * rows_per_wg + local;
  else return static_cast<int64_t>(local) * gridDim.x + blockIdx.x;
}

// XLDS: x is staged in LDS once per workgroup (K <= kGemvXldsMaxK) and each
// wave reads its chunks from there, instead of every wave loading x from the
// caches alongside its rows of W.
constexpr int kGemvXldsMaxK = 16384;

template <int ROWS, int WAVES, int UNROLL, bool NONTEMPORAL, bool ROTATE = false, int DT = kF16, int KSPLIT = 1,
          int ROWMAP = 0, bool XLDS = false>
__global__ void __launch_bounds__(WAVES * 64)
gemv_kernel(const _Float16 *__restrict__ x, const _Float16 *__restrict__ W, _Float16 *__restrict__ y, int N,
                int K) {
  static_assert(KSPLIT >= 1 && WAVES % KSPLIT == 0, "K slices divide the waves");
  constexpr int kRowGroups = WAVES / KSPLIT;
  constexpr int kRows = kRowGroups * ROWS;  // rows per workgroup
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = wave % KSPLIT;
  const int group = wave / KSPLIT;
  const int chunks = K >> 3;
  const half8_t *xv = reinterpret_cast<const half8_t *>(x);
  __shared__ half8_t x_lds[XLDS ? kGemvXldsMaxK / 8 : 1];
  if constexpr (XLDS) {
    // every wave takes part, before any wave may leave
    for (int c = threadIdx.x; c < chunks; c += WAVES * 64) x_lds[c] = xv[c];
    __syncthreads();
  }
  const int64_t first_row = wave_row<ROWMAP, ROWS>(group, 0, kRows);
  if constexpr (KSPLIT == 1) {
    if (first_row >= N) return;  // wave-uniform; later rows of the wave are past N too
  }
  // This wave's chunks [c_begin, c_end): all of K, or its slice, cut on
  // 64-chunk steps (steps * slice / KSPLIT is below steps, so c_begin < chunks).
  // A row group wholly past N (last workgroup only) walks nothing but still
  // meets the others at the barrier below.
  int c_begin = 0, c_end = chunks;
  if constexpr (KSPLIT > 1) {
    const int steps = (chunks + 63) >> 6;
    c_begin = (steps * slice / KSPLIT) * 64;
    c_end = min(chunks, (steps * (slice + 1) / KSPLIT) * 64);
    if (first_row >= N) c_end = c_begin;
  }
  const half8_t *wrow[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    // Rows past N re-read the last row (always valid memory); their sums
    // are never stored.
    int64_t row = wave_row<ROWMAP, ROWS>(group, r, kRows);
    if (row >= N) row = static_cast<int64_t>(N) - 1;
    wrow[r] = reinterpret_cast<const half8_t *>(W + row * K);
  }

  float acc[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) acc[r] = 0.0f;

  // One group = UNROLL chunk steps of 64 lanes: every load of a group is
  // issued before the first product, so a lane has UNROLL*(ROWS+1) 16-byte
  // loads in flight.  Whole groups need no bounds test; the ragged rest of
  // the row (fewer than 64*UNROLL chunks) is one guarded group at the end.
  auto group_step = [&](int base, bool guarded) {
    half8_t xs[UNROLL];
    half8_t ws[UNROLL][ROWS];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int c = base + u * 64 + lane;
      if (!guarded || c < c_end) {
        if constexpr (XLDS) xs[u] = x_lds[c];
        else xs[u] = xv[c];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) ws[u][r] = NONTEMPORAL ? __builtin_nontemporal_load(wrow[r] + c) : wrow[r][c];
      } else {
        xs[u] = half8_t{};
#pragma unroll
        for (int r = 0; r < ROWS; ++r) ws[u][r] = half8_t{};
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int r = 0; r < ROWS; ++r) acc[r] = dot8_acc<DT>(xs[u], ws[u][r], acc[r]);
  };

  // With ROTATE, each wave starts its walk over the whole groups at a
  // different group (and wraps around), so the waves running at one moment
  // read different column windows of their rows.
  constexpr int kGroup = 64 * UNROLL;
  const int span = c_end - c_begin;
  const int full = span / kGroup;
  const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * kRowGroups + group;
  int g = (ROTATE && full > 0) ? static_cast<int>(wave_id % full) : 0;
  for (int it = 0; it < full; ++it) {
    group_step(c_begin + g * kGroup, false);
    if (++g == full) g = 0;
  }
  if (full * kGroup < span) group_step(c_begin + full * kGroup, true);

  // Row sums: DPP reductions inside the wave; lane r < ROWS holds row r's.
  float sums[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) sums[r] = wave_sum(acc[r]);
  float mine = sums[0];
#pragma unroll
  for (int r = 1; r < ROWS; ++r) mine = (lane == r) ? sums[r] : mine;
  const int64_t my_row = wave_row<ROWMAP, ROWS>(group, lane < ROWS ? lane : 0, kRows);
  if constexpr (KSPLIT == 1) {
    if (lane < ROWS && my_row < N) y[my_row] = round_out<DT>(mine);
  } else {
    // Each slice's row sums go to LDS; the slice-0 wave of the row group adds
    // them in slice order and stores the rounded total.
    __shared__ float part[kRowGroups][ROWS][KSPLIT];
    if (lane < ROWS) part[group][lane][slice] = mine;
    __syncthreads();
    if (slice == 0 && lane < ROWS && my_row < N) {
      float total = part[group][lane][0];
#pragma unroll
      for (int s2 = 1; s2 < KSPLIT; ++s2) total += part[group][lane][s2];
      y[my_row] = round_out<DT>(total);
    }
  }
}

template <int ROWS, int WAVES, int UNROLL, bool NT, bool ROT = false, int DT = kF16, int KSPLIT = 1, int ROWMAP = 0,
          bool XLDS = false>
static hipError_t launch(const void *x, const void *W, void *y, int N, int K, hipStream_t stream) {
  if (XLDS && K > kGemvXldsMaxK) return hipErrorInvalidValue;
  const int64_t rows_per_block = static_cast<int64_t>(ROWS) * WAVES / KSPLIT;
  const int64_t grid = (N + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((gemv_kernel<ROWS, WAVES, UNROLL, NT, ROT, DT, KSPLIT, ROWMAP, XLDS>),
                     dim3(static_cast<unsigned>(grid)), dim3(WAVES * 64), 0, stream, static_cast<const _Float16 *>(x),
                     static_cast<const _Float16 *>(W), static_cast<_Float16 *>(y), N, K);
  return hipGetLastError();
}

// The default launch (gemv_default_launch): 16, 8, 4 or 2 rows per workgroup
// with 1, 2, 4 or 8 K slices, or 1 row in 8 slices, from N, K and the CU
// count, with non-temporal or cached loads of W by its size.
template <int DT, bool NT>
static hipError_t launch_auto_nt(const GemvLaunch &l, const void *x, const void *W, void *y, int N, int K,
                                 hipStream_t stream) {
  static_assert(kGemvWaves == 8, "the instantiations below use 8 waves");
  if (l.rows_per_wave == 1) return launch<1, 8, 4, NT, true, DT, 8>(x, W, y, N, K, stream);
  switch (l.ksplit) {
    case 1: return launch<2, 8, 4, NT, true, DT, 1>(x, W, y, N, K, stream);
    case 2: return launch<2, 8, 4, NT, true, DT, 2>(x, W, y, N, K, stream);
    case 4: return launch<2, 8, 4, NT, true, DT, 4>(x, W, y, N, K, stream);
    default: return launch<2, 8, 4, NT, true, DT, 8>(x, W, y, N, K, stream);
  }
}

template <int DT>
static hipError_t launch_auto(const void *x, const void *W, void *y, int N, int K, int num_cus, hipStream_t stream) {
  const GemvLaunch l = gemv_default_launch(N, K, num_cus);
  return l.nontemporal ? launch_auto_nt<DT, true>(l, x, W, y, N, K, stream)
                       : launch_auto_nt<DT, false>(l, x, W, y, N, K, stream);
}

hipError_t launch_gemv_f16(int variant, const void *x, const void *W, void *y, int N, int K, int num_cus,
                           hipStream_t stream) {
  // <rows per wave, waves per workgroup, chunk steps in flight, non-temporal W, rotated start, type, K slices>
  // Numbers of launch shapes measured and not kept are not reused.
  switch (variant) {
    case 0: return launch_auto<kF16>(x, W, y, N, K, num_cus, stream);
    case 6: return launch<2, 8, 4, false, true>(x, W, y, N, K, stream);
    case 7: return launch<2, 8, 4, true, false>(x, W, y, N, K, stream);
    case 8: return launch<2, 8, 4, true, true, kF16, 1>(x, W, y, N, K, stream);
    case 9: return launch<2, 8, 4, true, true, kF16, 2>(x, W, y, N, K, stream);
    case 10: return launch<2, 8, 4, true, true, kF16, 4>(x, W, y, N, K, stream);
    case 11: return launch<2, 8, 4, true, true, kF16, 8>(x, W, y, N, K, stream);
    case 12: return launch<1, 8, 4, true, true, kF16, 8>(x, W, y, N, K, stream);
    // grid-strided rows; x staged in LDS once per workgroup
    case 20: return launch<2, 8, 4, true, true, kF16, 1, 1>(x, W, y, N, K, stream);
    case 21: return launch<2, 8, 4, true, true, kF16, 1, 0, true>(x, W, y, N, K, stream);
    // no rotated start: 8 chunk steps in flight; 4 rows per wave, 4 waves
    case 28: return launch<2, 8, 8, true, false>(x, W, y, N, K, stream);
    case 29: return launch<4, 4, 4, true, false>(x, W, y, N, K, stream);
    // as 8..12 with cached (not non-temporal) loads of W
    case 37: return launch<2, 8, 4, false, true, kF16, 1>(x, W, y, N, K, stream);
    case 38: return launch<2, 8, 4, false, true, kF16, 2>(x, W, y, N, K, stream);
    case 39: return launch<2, 8, 4, false, true, kF16, 4>(x, W, y, N, K, stream);
    case 40: return launch<2, 8, 4, false, true, kF16, 8>(x, W, y, N, K, stream);
    case 41: return launch<1, 8, 4, false, true, kF16, 8>(x, W, y, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

// y[i] = +0 (or D[i] = +0) for i < count: the K == 0 case (empty sums).  A
// kernel rather than a memset so the call stays capturable in a HIP graph.
__global__ void fill_zero_f16_kernel(_Float16 *__restrict__ p, int64_t count) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride)
    p[i] = static_cast<_Float16>(0.0f);
}

hipError_t launch_gemv_bf16(const void *x, const void *W, void *y, int N, int K, int num_cus, hipStream_t stream) {
  return launch_auto<kBF16>(x, W, y, N, K, num_cus, stream);
}

hipError_t launch_fill_zero_f16(void *p, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const int64_t threads = 256;
  int64_t blocks = (count + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_zero_f16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream,
                     static_cast<_Float16 *>(p), count);
  return hipGetLastError();
}

}  // namespace gt
