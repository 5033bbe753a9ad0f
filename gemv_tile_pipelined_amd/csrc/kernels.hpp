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
constexpr int kGemmVariants = 13;
constexpr int kGemvVariants = 8;
// GEMMs with at most this many rows on one side (M or N) take the skinny
// kernel (skinny.hip); it has kSkinnyVariants launch shapes.
constexpr int kSkinnyMaxRows = 16;
constexpr int kSkinnyVariants = 12;
// Skinny launch shapes from this index on stage only 8 rows of the small side.
constexpr int kSkinnyFirstQ8Variant = 9;

// s_waitcnt immediate for "lgkmcnt(0)" alone on gfx9-family targets
// (vmcnt field [3:0]|[15:14] = 63, expcnt [6:4] = 7, lgkmcnt [11:8] = 0).
// Issued through the builtin so the compiler knows the LDS reads are done.
constexpr unsigned kWaitLgkm0 = 0xC07F;

hipError_t launch_gemm_f16(int variant, const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                           hipStream_t stream);
hipError_t launch_gemm_skinny_f16(int variant, const void *A, const void *B, void *D, int M, int N, int K,
                                  hipStream_t stream);
hipError_t launch_gemv_f16(int variant, const void *x, const void *W, void *y, int N, int K, hipStream_t stream);
hipError_t launch_fill_zero_f16(void *p, int64_t count, hipStream_t stream);
// bf16 operands and results: the default launch shape of each kernel.
hipError_t launch_gemm_bf16(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                            hipStream_t stream);
hipError_t launch_gemm_skinny_bf16(const void *A, const void *B, void *D, int M, int N, int K, hipStream_t stream);
hipError_t launch_gemv_bf16(const void *x, const void *W, void *y, int N, int K, hipStream_t stream);

}  // namespace gt
