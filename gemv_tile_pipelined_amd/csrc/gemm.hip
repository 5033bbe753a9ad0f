// gemm.hip -- persistent, pipelined FP16 / BF16 GEMM for gfx950: D = A · Bᵀ.
//
//   A [M,K], B [N,K] row-major (K-contiguous) fp16 or bf16; D [M,N]
//   row-major in the same format; FP32 accumulation in the matrix cores, one
//   round-to-nearest-even per output (bf16 in and out is the SM120 page's
//   own kernel: nv_bfloat16 operands at §2.2 entrance, _rn rounding of the
//   FP32 accumulators in the §2.3 kernel).  The operation and layout are those of the TVM TIRx GEMM chapter
//   ("使用 TMA 为 GEMM 建立 Pipeline", step 4 full kernel) and of the SM120
//   walk-through "TensorCore_GEMM_with_TMA" (§2.2 entrance, §2.3 kernel).
//
// Structure (one workgroup per CU, 4 waves; with the default 256x256 output
// tile each wave holds a 128x128 sub-tile):
//
//  * Tile shape -- 256x256 output tiles while they give every CU one; an
//    output with fewer takes 256x128, 128x256 or 128x128 tiles, whose shorter
//    K tiles get deeper LDS rings (gemm_default_tile, kernels.hpp).
//
//  * Tile scheduler -- a persistent grid of min(#tiles, #CUs) workgroups walks
//    tile indices t = id, id + grid, ... in the grouped order of tile_order.hpp
//    (GROUP_M = 8 as on both GEMM pages), with workgroup ids renumbered so
//    each XCD owns a contiguous range of the order (shared L2).  Step 6 of the
//    TVM chapter is the persistent/scheduler design this follows; the grouped
//    formula is §2.3 of the SM120 page.
//
//  * Global -> LDS movement -- each K tile of A [BM,BK] and B [BN,BK] is moved
//    by direct-to-LDS buffer loads (16 bytes per lane, 1 KiB per wave
//    instruction), which frees the waves' VGPRs the way TMA frees threads on
//    the pages (TVM chapter step 4; Croqtile ch. 7 on TMA vs DMA).  Rows at or
//    past M/N lie beyond the buffer descriptor's range and K chunks at or past
//    K get an out-of-range offset, so both read as zero: the `.zfill`
//    behaviour of Croqtile ch. 7 (irregular access), which keeps the MFMA
//    loop uniform on edge tiles.
//
//  * LDS layout -- rows of BK fp16 in 16-byte chunks; chunk c of row r is
//    stored at chunk c ^ swz(r).  The loader applies the XOR by choosing which
//    global chunk each lane fetches (the LDS side of a DMA instruction is
//    fixed: lane i -> 16*i), and the MFMA operand reads apply the same XOR, so
//    writer and reader agree (Croqtile ch. 7 swizzle rule; the 128-byte
//    swizzle of the TVM chapter and of the SM120 page's ldmatrix addressing
//    play the same role there).
//
//  * LDS ring -- STAGES buffers; K tile t lives in stage t % STAGES.  In the
//    final K step of tile k each wave waits (vmcnt) until tile k+1 has landed
//    while younger tiles stay in flight, completes its LDS reads, and meets
//    the other waves at the one barrier of the K tile; that barrier frees
//    stage k, whose refill with tile k + STAGES starts at once, the loads
//    threaded between the MFMAs that follow.  Tile k+1's first operands are
//    fetched during the same MFMAs.  Stage index and wait count follow from
//    the loop counter, so nothing resets between output tiles (a ragged
//    K = 4104 has an odd number of K tiles).  TVM chapter step 5 (Pipeline
//    机制) and the SM120 page's multistage main loop describe the same ring
//    with mbarriers.
//
//  * MFMA micro-kernel -- v_mfma_f32_16x16x32_f16 (or _bf16), written as
//    inline asm with the accumulators bound to AGPRs (the compiler's builtin
//    moves them around the loop); the compiler does not see these as MFMAs,
//    so their hazards are padded by hand, and the build checks the generated
//    code for accumulator moves near them (build.py).  B rows feed the first
//    operand and A rows the second, so each lane holds four consecutive
//    output columns of one output row.  Operand fetches for the next K step
//    are interleaved with the current step's MFMAs.  A 32x32x16 form through
//    the compiler's builtin remains for ablation.
//
//  * Epilogue -- FP32 -> fp16 or bf16 with round-to-nearest-even (the `_rn`
//    conversion of the SM120 page's epilogue), staged through LDS so D is
//    written in whole 16-byte row segments (the TVM chapter likewise stages D
//    in shared memory before its bulk store), masked to the M x N region.
//    The fused instantiations add bias[n] and apply ReLU before the rounding
//    (gemm_bias_*; not on the pages).  With split K (gemm_splitk_*) the units
//    are (tile, K slice) pairs that store FP32 partial sums to a workspace,
//    and a second kernel adds the slices in order and rounds.
//
// This file holds the fused-epilogue and split-K launches, the static scratch
// of gemm_splitk_f16_noalloc and the host-side trace of the ring schedule;
// the kernel template is in gemm_kernel.hpp and the plain launches in
// gemm_plain.hip.
#include <hip/hip_runtime.h>

#include <atomic>

#include "gemm_kernel.hpp"

namespace gt {

// D[m,n] = act(bias[n]) (+0 where bias is NULL): the K == 0 case of the
// fused epilogue, whose sums are empty.  A kernel rather than a memset so
// the call stays capturable in a HIP graph.

template <int DT>
__global__ void fill_bias_kernel(_Float16 *__restrict__ D, const uint16_t *__restrict__ bias, int64_t M, int64_t N,
                                 int relu) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < M * N; i += stride) {
    float v = bias ? widen_in<DT>(bias[i % N]) : 0.0f;
    if (relu) v = relu_act(v);
    D[i] = round_out<DT>(v);
  }
}


hipError_t launch_gemm_bias(int dtype, const void *A, const void *B, const void *bias, int relu, void *D, int M, int N,
                            int K, int num_cus, hipStream_t stream) {
  if (K == 0) {
    const int64_t count = static_cast<int64_t>(M) * N;
    const int64_t threads = 256;
    int64_t blocks = (count + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    if (count <= 0) return hipSuccess;
    auto kernel = dtype == kBF16 ? fill_bias_kernel<kBF16> : fill_bias_kernel<kF16>;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream,
                       static_cast<_Float16 *>(D), static_cast<const uint16_t *>(bias), static_cast<int64_t>(M),
                       static_cast<int64_t>(N), relu);
    return hipGetLastError();
  }
  return dtype == kBF16 ? launch_default<kBF16, kEpiFused>(A, B, D, M, N, K, num_cus, stream, bias, relu)
                        : launch_default<kF16, kEpiFused>(A, B, D, M, N, K, num_cus, stream, bias, relu);
}

// D[i] = rne(ws[0][i] + ws[1][i] + ... + ws[splits-1][i]): the K slices of a
// split-K GEMM added in slice order, so every output is deterministic.
template <int DT>
__global__ void splitk_reduce_kernel(const float *__restrict__ ws, _Float16 *__restrict__ D, int64_t count,
                                     int splits) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  // Four outputs per thread with 16-byte loads where the layout allows
  // (count % 4 == 0 keeps every slice's start 16-byte aligned), else one.
  // The slices' loads go out up to 8 at a time before their sums, which
  // stay in slice order: one load in flight per thread would leave a small
  // output's reduction waiting on memory latency once per slice.
  if (count % 4 == 0) {
    const int64_t quads = count / 4;
    for (int64_t q = first; q < quads; q += stride) {
      const float4_t *src = reinterpret_cast<const float4_t *>(ws) + q;
      const int64_t step = count / 4;
      float4_t v = src[0];
      for (int s = 1; s < splits; s += 8) {
        float4_t t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (s + j < splits) t[j] = src[(s + j) * step];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (s + j < splits) v += t[j];
      }
      half4_t h;
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = round_out<DT>(v[e]);
      _Float16 *dst = D + 4 * q;
      if ((reinterpret_cast<uintptr_t>(dst) & 7) == 0) {
        *reinterpret_cast<half4_t *>(dst) = h;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = h[e];
      }
    }
    return;
  }
  for (int64_t i = first; i < count; i += stride) {
    float v = ws[i];
    for (int s = 1; s < splits; s += 8) {
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s + j < splits) t[j] = ws[(s + j) * count + i];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s + j < splits) v += t[j];
    }
    D[i] = round_out<DT>(v);
  }
}

hipError_t launch_splitk_reduce(int dtype, const float *ws, void *D, int64_t count, int splits, hipStream_t stream) {
  const int64_t threads = 256;
  const int64_t items = count % 4 == 0 ? count / 4 : count;  // the reduction's per-thread items
  int64_t blocks = (items + threads - 1) / threads;
  if (blocks > 8192) blocks = 8192;
  auto kernel = dtype == kBF16 ? splitk_reduce_kernel<kBF16> : splitk_reduce_kernel<kF16>;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream, ws,
                     static_cast<_Float16 *>(D), count, splits);
  return hipGetLastError();
}

hipError_t launch_gemm_splitk(int dtype, const void *A, const void *B, void *D, int M, int N, int K, void *ws,
                              int splits, int num_cus, hipStream_t stream) {
  float *w = static_cast<float *>(ws);
  const hipError_t e = dtype == kBF16
                           ? launch_default<kBF16, kEpiPartial>(A, B, D, M, N, K, num_cus, stream, nullptr, 0, w, splits)
                           : launch_default<kF16, kEpiPartial>(A, B, D, M, N, K, num_cus, stream, nullptr, 0, w, splits);
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(dtype, w, D, static_cast<int64_t>(M) * N, splits, stream);
}

// ---- static scratch of the non-allocating split-K entry point ------------
// gemm_splitk_f16_noalloc keeps its FP32 partial sums here instead of in a
// caller's workspace.  Each device the library runs on holds one copy of the
// array, at its own address, until the process ends.  In host code the name
// `scratch` is a host-side stand-in, not a device address: the kernels only
// ever receive the address hipGetSymbolAddress returns for the current
// device (noalloc_scratch below).
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> per_device[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = per_device[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // Once per device, with that device current (two threads racing here
    // both obtain the same address).
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    per_device[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

// ---- the ring schedule on the host -------------------------------------
// The walker gemm_kernel runs (ring.hpp), run on the host with an Ops object
// that records each event instead of issuing it.
namespace {
template <class S>
struct RingRecorder {
  int stages;
  int32_t *ev;
  int64_t cap;
  int64_t n = 0;
  void push(int32_t code, int32_t a = 0, int32_t b = 0, int32_t c = 0, int32_t d = 0) {
    if (ev != nullptr && n < cap) {
      int32_t *e = ev + 5 * n;
      e[0] = code;
      e[1] = a;
      e[2] = b;
      e[3] = c;
      e[4] = d;
    }
    ++n;
  }
  void mfma(int buf, int idx) { push(kRingMfma, buf, idx, S::mfma_i(idx), S::mfma_j(idx)); }
  void read(int buf, int kt, int ks, int r) { push(kRingRead, kt, ks, r, ring_stage(kt, stages)); }
  void load(int tile, int d) { push(kRingLoad, tile, d, ring_stage(tile, stages)); }
  void mfma_load(int buf, int idx, int tile, int d) {
    mfma(buf, idx);
    load(tile, d);
  }
  void prep(int tile, int part) { push(kRingPrep, tile, part); }
  void init_acc() { push(kRingInit); }
  void wait_tile(int vmcnt) { push(kRingWaitTile, vmcnt); }
  void wait_lds() { push(kRingWaitLds); }
  void barrier() { push(kRingBarrier); }
  void fence() {}
};

template <class S>
int64_t record_ring(int ktu, int32_t *events, int64_t cap) {
  RingRecorder<S> rec{S::STAGES, events, cap};
  if constexpr (S::EARLY_FREE)
    ring_k_loop_ef<S>(rec, ktu);
  else
    ring_k_loop<S>(rec, ktu);
  return rec.n;
}
}  // namespace

int64_t ring_trace(int variant, int ktu, int32_t *events, int64_t cap, int *info) {
  auto run = [&](auto shape) {
    using S = decltype(shape);
    info[0] = S::kDmaPerStage;
    info[1] = S::kReads;
    info[2] = S::kKSub;
    info[3] = S::kMfma;
    info[4] = S::STAGES;
    info[5] = S::BM;
    info[6] = S::BN;
    info[7] = S::EARLY_FREE ? 1 : 0;
    info[8] = S::WAVES_M;
    info[9] = S::WAVES_N;
    return record_ring<S>(ktu, events, cap);
  };
  switch (variant) {
    case 0:
    case 1:
    case 3:
    case 20:
    case 28: return run(GemmDefault{});
    case 10: return run(Gemm32x32{});
    case 21: return run(GemmTile256x128<kF16, 3>{});
    case 22: return run(GemmTile128x256<kF16, 3>{});
    case 23: return run(GemmTile128x128<kF16, 4>{});
    case 24: return run(GemmTile256x128<kF16, 2>{});
    case 25: return run(GemmTile128x256<kF16, 2>{});
    case 26: return run(GemmTile128x128<kF16, 2>{});
    case 27: return run(GemmTile128x128<kF16, 5>{});
    case 30: return run(GemmOneBarrier{});
    case 31: return run(GemmRowMajorMfma{});
    case 32: return run(GemmTile128x64<kF16, 4>{});
    default: return -1;
  }
}

}  // namespace gt