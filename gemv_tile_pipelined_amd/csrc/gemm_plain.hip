// gemm_plain.hip -- the plain (unfused) tiled GEMM launches: gemm_f16's
// default and its ablation variants, and gemm_bf16.  Kept apart from
// gemm.hip so the two translation units compile in parallel.
#include "gemm_kernel.hpp"

namespace gt {

hipError_t launch_gemm_f16(int variant, const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                           hipStream_t stream) {
  // Numbers of ablations measured and not kept are not reused.
  switch (variant) {
    case 0: return launch_default<kF16>(A, B, D, M, N, K, num_cus, stream);
    case 1: return launch<GemmNoSwizzle>(A, B, D, M, N, K, num_cus, stream);
    case 2: return launch<Gemm32x32OneStage>(A, B, D, M, N, K, num_cus, stream);
    case 3: return launch<GemmNonPersistent>(A, B, D, M, N, K, num_cus, stream);
    case 10: return launch<Gemm32x32>(A, B, D, M, N, K, num_cus, stream);
    // Forced output tiles and ring depths (the default picks among them).
    case 20: return launch<GemmDefault>(A, B, D, M, N, K, num_cus, stream);
    case 21: return launch<GemmTile256x128<kF16, 3>>(A, B, D, M, N, K, num_cus, stream);
    case 22: return launch<GemmTile128x256<kF16, 3>>(A, B, D, M, N, K, num_cus, stream);
    case 23: return launch<GemmTile128x128<kF16, 4>>(A, B, D, M, N, K, num_cus, stream);
    case 24: return launch<GemmTile256x128<kF16, 2>>(A, B, D, M, N, K, num_cus, stream);
    case 25: return launch<GemmTile128x256<kF16, 2>>(A, B, D, M, N, K, num_cus, stream);
    case 26: return launch<GemmTile128x128<kF16, 2>>(A, B, D, M, N, K, num_cus, stream);
    case 27: return launch<GemmTile128x128<kF16, 5>>(A, B, D, M, N, K, num_cus, stream);
    case 28: return launch<GemmDefault, kEpiCachedStores>(A, B, D, M, N, K, num_cus, stream);
    case 30: return launch<GemmOneBarrier>(A, B, D, M, N, K, num_cus, stream);
    case 31: return launch<GemmRowMajorMfma>(A, B, D, M, N, K, num_cus, stream);
    case 32: return launch<GemmTile128x64<kF16, 4>>(A, B, D, M, N, K, num_cus, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_bf16(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                            hipStream_t stream) {
  return launch_default<kBF16>(A, B, D, M, N, K, num_cus, stream);
}


hipError_t launch_gemm_f16_timed(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                                 uint64_t *stamps, hipStream_t stream) {
  return launch<GemmDefault, kEpiTimed>(A, B, D, M, N, K, num_cus, stream, nullptr, 0,
                                        reinterpret_cast<float *>(stamps), 1);
}

}  // namespace gt
