// gemv.hip -- batch-1 FP16 GEMV for gfx950: y = x · Wᵀ.
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
//    16-byte loads in flight per lane;
//  * W is read with non-temporal loads (streamed once, no reuse);
//  * v_dot2_f32_f16 multiplies fp16 pairs and accumulates in FP32;
//  * the 64 lane partial sums of a row are combined with cross-lane
//    exchanges inside the wave (no LDS, no atomics, no second kernel), so
//    each row sum is deterministic.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace gt {

__device__ inline float dot8_acc(half8_t a, half8_t b, float acc) {
  acc = __builtin_amdgcn_fdot2(half2_t{a[0], a[1]}, half2_t{b[0], b[1]}, acc, false);
  acc = __builtin_amdgcn_fdot2(half2_t{a[2], a[3]}, half2_t{b[2], b[3]}, acc, false);
  acc = __builtin_amdgcn_fdot2(half2_t{a[4], a[5]}, half2_t{b[4], b[5]}, acc, false);
  acc = __builtin_amdgcn_fdot2(half2_t{a[6], a[7]}, half2_t{b[6], b[7]}, acc, false);
  return acc;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int ROWS, int WAVES, int UNROLL, bool NONTEMPORAL>
__global__ void __launch_bounds__(WAVES * 64)
gemv_f16_kernel(const _Float16 *__restrict__ x, const _Float16 *__restrict__ W, _Float16 *__restrict__ y, int N,
                int K) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * WAVES + wave) * ROWS;
  if (row0 >= N) return;  // wave-uniform
  const int chunks = K >> 3;
  const half8_t *xv = reinterpret_cast<const half8_t *>(x);
  const half8_t *wrow[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    // Rows past N re-read the last row (always valid memory); their sums
    // are never stored.
    const int64_t row = (row0 + r < N) ? row0 + r : static_cast<int64_t>(N) - 1;
    wrow[r] = reinterpret_cast<const half8_t *>(W + row * K);
  }

  float acc[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) acc[r] = 0.0f;

  for (int base = 0; base < chunks; base += 64 * UNROLL) {
    half8_t xs[UNROLL];
    half8_t ws[UNROLL][ROWS];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int c = base + u * 64 + lane;
      if (c < chunks) {
        xs[u] = xv[c];
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
          ws[u][r] = NONTEMPORAL ? __builtin_nontemporal_load(wrow[r] + c) : wrow[r][c];
      } else {
        xs[u] = half8_t{};
#pragma unroll
        for (int r = 0; r < ROWS; ++r) ws[u][r] = half8_t{};
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int r = 0; r < ROWS; ++r) acc[r] = dot8_acc(xs[u], ws[u][r], acc[r]);
  }

#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const float s = wave_sum(acc[r]);
    if (lane == r && row0 + r < N) y[row0 + r] = static_cast<_Float16>(s);
  }
}

template <int ROWS, int WAVES, int UNROLL, bool NT>
static hipError_t launch(const void *x, const void *W, void *y, int N, int K, hipStream_t stream) {
  const int64_t rows_per_block = static_cast<int64_t>(ROWS) * WAVES;
  const int64_t grid = (N + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((gemv_f16_kernel<ROWS, WAVES, UNROLL, NT>), dim3(static_cast<unsigned>(grid)), dim3(WAVES * 64),
                     0, stream, static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(W),
                     static_cast<_Float16 *>(y), N, K);
  return hipGetLastError();
}

hipError_t launch_gemv_f16(int variant, const void *x, const void *W, void *y, int N, int K, hipStream_t stream) {
  // <rows per wave, waves per workgroup, chunk steps in flight, non-temporal W>
  switch (variant) {
    case 0: return launch<2, 8, 4, true>(x, W, y, N, K, stream);
    case 1: return launch<4, 4, 4, true>(x, W, y, N, K, stream);
    case 2: return launch<2, 8, 8, true>(x, W, y, N, K, stream);
    case 3: return launch<1, 8, 8, true>(x, W, y, N, K, stream);
    case 4: return launch<2, 4, 8, true>(x, W, y, N, K, stream);
    case 5: return launch<1, 16, 4, true>(x, W, y, N, K, stream);
    case 6: return launch<2, 8, 4, false>(x, W, y, N, K, stream);
    case 7: return launch<4, 4, 2, true>(x, W, y, N, K, stream);
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
