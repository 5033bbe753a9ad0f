// skinny.hip -- FP16 GEMM with one side of at most 16 rows, for gfx950:
// D = A · Bᵀ when M <= 16 (a decode batch of M activation rows against a
// weight matrix B [N,K]) or when N <= 16.
//
// Same operation and contract as the tiled GEMM ("使用 TMA 为 GEMM 建立
// Pipeline", step 4 full kernel: A [M,K], B [N,K], FP32 accumulation, fp16
// out), but with 16 or fewer rows on one side the 256x256 output tiles of the
// tiled kernel would leave all but a few CUs idle, and the work is bound by
// reading the large matrix once, like the batch-1 product of "Learning
// TileLang with GEMV" (§02 Bandwidth Bound).  The kernel follows that page's
// summary for bandwidth-bound kernels (§07 Summary: enough blocks -- splitting
// K when one dimension alone does not give them --, neighbouring lanes on
// neighbouring addresses, 16 bytes per lane per load), and uses the matrix
// cores only because with up to 16 small-side rows a plain dot-product loop
// would be VALU-bound:
//
//  * P [R,K] is the large matrix (streamed once, non-temporal loads), Q
//    [S,K] the small one (S <= 16; it stays in the caches).  A workgroup owns
//    16 rows of P and all S outputs for them.
//  * v_mfma_f32_16x16x32_f16 with P rows as the first operand and Q rows as
//    the second: per 32-wide K step, lane l brings 16 bytes of P row (l % 16)
//    and of Q row (l % 16) at K offset 8*(l / 16), so one wave instruction
//    reads 64 contiguous bytes from each of 16 rows.  Rows of Q past S and
//    rows of P past R are clamped to the last valid row: they only feed
//    outputs that are never stored.  K chunks past K read as zero.
//  * The WAVES waves of a workgroup split the K steps (wave w takes UNROLL
//    consecutive steps out of every WAVES*UNROLL), each keeping UNROLL pairs
//    of loads in flight.  Their 16x16 partial sums meet in LDS and are added
//    in wave order, so every output is deterministic.
//  * Output: D[s*R + r] (D = Q·Pᵀ, the M <= 16 case) or D[r*S + s]
//    (TRANS, D = P·Qᵀ, the N <= 16 case), rounded to nearest-even fp16.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace gt {

template <int WAVES, int UNROLL, bool TRANS>
__global__ void __launch_bounds__(WAVES * 64)
gemm_skinny_kernel(const _Float16 *__restrict__ P, const _Float16 *__restrict__ Q, _Float16 *__restrict__ D, int R,
                   int S, int K) {
  __shared__ float partial[WAVES][16][17];  // [wave][s][r], padded row
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = blockIdx.x * 16;
  const int frow = lane & 15;
  const int kgrp = lane >> 4;
  const int prow = min(r0 + frow, R - 1);
  const int qrow = min(frow, S - 1);
  const half8_t *pr = reinterpret_cast<const half8_t *>(P + static_cast<int64_t>(prow) * K);
  const half8_t *qr = reinterpret_cast<const half8_t *>(Q + static_cast<int64_t>(qrow) * K);
  const int chunks = K >> 3;         // 16-byte chunks per row
  const int steps = (K + 31) >> 5;  // 32-wide K steps

  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int base = wave * UNROLL; base < steps; base += WAVES * UNROLL) {
    half8_t pv[UNROLL], qv[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int c = (base + u) * 4 + kgrp;  // chunk index along K
      if (c < chunks) {
        pv[u] = __builtin_nontemporal_load(pr + c);
        qv[u] = qr[c];
      } else {
        pv[u] = half8_t{};
        qv[u] = half8_t{};
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(pv[u], qv[u], acc, 0, 0, 0);
  }

  // acc[e] of lane l is the partial sum for P row r0 + 4*(l/16) + e and Q row
  // l % 16.
#pragma unroll
  for (int e = 0; e < 4; ++e) partial[wave][frow][4 * kgrp + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int s = threadIdx.x >> 4;
    const int r = threadIdx.x & 15;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += partial[w][s][r];
    if (s < S && r0 + r < R) {
      const int64_t idx = TRANS ? static_cast<int64_t>(r0 + r) * S + s : static_cast<int64_t>(s) * R + r0 + r;
      D[idx] = static_cast<_Float16>(sum);
    }
  }
}

template <int WAVES, int UNROLL>
static hipError_t launch(const void *P, const void *Q, void *D, int R, int S, int K, bool trans,
                         hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((R + 15) / 16));
  const auto *p = static_cast<const _Float16 *>(P);
  const auto *q = static_cast<const _Float16 *>(Q);
  auto *d = static_cast<_Float16 *>(D);
  if (trans)
    hipLaunchKernelGGL((gemm_skinny_kernel<WAVES, UNROLL, true>), grid, dim3(WAVES * 64), 0, stream, p, q, d, R, S,
                       K);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<WAVES, UNROLL, false>), grid, dim3(WAVES * 64), 0, stream, p, q, d, R, S,
                       K);
  return hipGetLastError();
}

hipError_t launch_gemm_skinny_f16(int variant, const void *A, const void *B, void *D, int M, int N, int K,
                                  hipStream_t stream) {
  // The small side is Q.  M <= 16: Q = A, P = B, D = Q·Pᵀ.  Otherwise
  // (N <= 16): Q = B, P = A, D = P·Qᵀ.
  const bool small_m = M <= kSkinnyMaxRows;
  if (!small_m && N > kSkinnyMaxRows) return hipErrorInvalidValue;
  const void *P = small_m ? B : A;
  const void *Q = small_m ? A : B;
  const int R = small_m ? N : M;
  const int S = small_m ? M : N;
  // <waves per workgroup, K steps in flight per wave>
  switch (variant) {
    case 0: return launch<8, 4>(P, Q, D, R, S, K, !small_m, stream);
    case 1: return launch<8, 2>(P, Q, D, R, S, K, !small_m, stream);
    case 2: return launch<8, 8>(P, Q, D, R, S, K, !small_m, stream);
    case 3: return launch<16, 4>(P, Q, D, R, S, K, !small_m, stream);
    case 4: return launch<4, 8>(P, Q, D, R, S, K, !small_m, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gt
