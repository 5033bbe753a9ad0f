// gemm.hip -- persistent, pipelined FP16 GEMM for gfx950: D = A · Bᵀ.
//
//   A [M,K], B [N,K] row-major (K-contiguous) fp16; D [M,N] row-major fp16;
//   FP32 accumulation in the matrix cores, one round-to-nearest-even per
//   output.  The operation and layout are those of the TVM TIRx GEMM chapter
//   ("使用 TMA 为 GEMM 建立 Pipeline", step 4 full kernel) and of the SM120
//   walk-through "TensorCore_GEMM_with_TMA" (§2.2 entrance, §2.3 kernel).
//
// Structure (one workgroup per CU, 4 waves, each wave a 128x128 sub-tile):
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
//  * LDS layout -- rows of BK fp16 (128 bytes) in 16-byte chunks; chunk c of
//    row r is stored at chunk c ^ swz(r).  The loader applies the XOR by
//    choosing which global chunk each lane fetches (the LDS side of a DMA
//    instruction is fixed: lane i -> 16*i), and the MFMA operand reads apply
//    the same XOR, so writer and reader agree (Croqtile ch. 7 swizzle rule;
//    the 128-byte swizzle of the TVM chapter and of the SM120 page's
//    ldmatrix addressing play the same role there).
//
//  * LDS ring -- STAGES buffers, all filled by the prologue.  In the last
//    16-wide K step of K tile k, each wave waits (vmcnt) for tile k+1 while
//    younger tiles stay in flight, finishes its LDS reads of stage k, meets
//    the other waves at one barrier, refills stage k with tile k + STAGES, and
//    fetches tile k+1's first MFMA operands while the step's MFMAs run.  The
//    wait count and the stage index come from the loop counter, so nothing
//    resets between output tiles (a ragged K = 4104 has 65 K tiles).  TVM chapter step 5 (Pipeline 机制) and the
//    SM120 page's multistage main loop describe the same ring with mbarriers.
//
//  * MFMA micro-kernel -- v_mfma_f32_32x32x16_f16.  B rows feed the first
//    operand and A rows the second, so each lane ends up holding four
//    consecutive output columns of one output row (8-byte stores).
//
//  * Epilogue -- FP32 -> fp16 with round-to-nearest-even (the `_rn`
//    conversion of the SM120 page's epilogue), masked to the M x N region.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"
#include "tile_order.hpp"

namespace gt {

template <int BM_, int BN_, int BK_, int STAGES_, int WAVES_M_, int WAVES_N_, bool SWIZZLE_, bool PERSISTENT_>
struct GemmShape {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int BK = BK_;
  static constexpr int STAGES = STAGES_;
  static constexpr int WAVES_M = WAVES_M_;
  static constexpr int WAVES_N = WAVES_N_;
  static constexpr bool SWIZZLE = SWIZZLE_;
  static constexpr bool PERSISTENT = PERSISTENT_;

  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kWaveM = BM / WAVES_M;  // rows of D per wave
  static constexpr int kWaveN = BN / WAVES_N;  // cols of D per wave
  static constexpr int kFragM = kWaveM / 32;   // 32x32 MFMA blocks per wave, M
  static constexpr int kFragN = kWaveN / 32;   // 32x32 MFMA blocks per wave, N
  static constexpr int kRowBytes = BK * 2;
  static constexpr int kChunks = BK / 8;           // 16-byte chunks per LDS row
  static constexpr int kRowsPerDma = 64 / kChunks;  // rows one wave DMA fills
  static constexpr int kDmaA = BM / kRowsPerDma / kWaves;  // per-wave DMA instrs for A
  static constexpr int kDmaB = BN / kRowsPerDma / kWaves;
  static constexpr int kDmaPerStage = kDmaA + kDmaB;
  static constexpr int kStageA = BM * kRowBytes;
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kLdsBytes = STAGES * kStageBytes;
  static constexpr int kKSub = BK / 16;  // MFMA K steps per K tile

  static_assert(BK == 64, "the swizzle and fragment addressing assume 128-byte LDS rows");
  static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be whole 32x32 MFMA blocks");
  static_assert(BM % (kRowsPerDma * kWaves) == 0 && BN % (kRowsPerDma * kWaves) == 0, "DMA split");
  static_assert(kLdsBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");
  static_assert(STAGES >= 1 && (STAGES - 1) * kDmaPerStage <= 63, "vmcnt range");

  // Physical 16-byte chunk of logical chunk c in LDS row r.  With 8 chunks
  // per 128-byte row, any 8 consecutive rows read at one logical chunk land
  // on 8 different chunk positions (conflict-free with 8 lanes per LDS
  // cycle), and any 16 consecutive rows cover all 16 chunk positions of a
  // 256-byte bank window (conflict-free with 16 lanes per cycle).
  __host__ __device__ static constexpr int swz(int row) { return SWIZZLE ? ((row & 7) ^ ((row >> 3) & 1)) : 0; }
};

// Wave-uniform wait until the K tile this wave needs next has landed in LDS,
// while `younger` K tiles issued after it may stay in flight.  Loads complete
// in issue order, so "at most younger*kDmaPerStage outstanding" means every
// load of the needed tile is done.  vmcnt takes an immediate, so the count is
// picked from the few values the ring can produce (falling back to a full
// drain, which is always correct).
template <class S>
__device__ inline void wait_tile_landed(int younger) {
  if constexpr (S::STAGES >= 2) {
    if (younger >= S::STAGES - 1) {
      wait_vmcnt<(S::STAGES - 1) * S::kDmaPerStage>();
      return;
    }
  }
  if constexpr (S::STAGES >= 3) {
    if (younger >= S::STAGES - 2) {
      wait_vmcnt<(S::STAGES - 2) * S::kDmaPerStage>();
      return;
    }
  }
  wait_vmcnt<0>();
}

template <class S>
__global__ void __launch_bounds__(S::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_f16_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B, _Float16 *__restrict__ D,
                int M, int N, int K, int tiles_m, int tiles_n, int vec_store) {
  __shared__ __attribute__((aligned(1024))) char smem[S::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WAVES_N;
  const int wn = wave % S::WAVES_N;
  const uint32_t lds0 = lds_addr(smem);
  const int KT = (K + S::BK - 1) / S::BK;
  const int64_t num_tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  const int64_t grid = gridDim.x;

  // ---- loader geometry ----------------------------------------------------
  // DMA instruction i of this wave fills the kRowsPerDma LDS rows starting at
  // row (i*kWaves + wave)*kRowsPerDma; lane l writes physical chunk l % 8 of
  // row i*kRowsPerDma*kWaves + ld_row, so it fetches logical chunk
  // (l % 8) ^ swz(row) of that row.  swz() only sees row & 15, which does not
  // depend on i, so one offset per lane serves every instruction (instruction
  // i adds i * kRowsPerDma*kWaves rows).  A and B tiles use the same pattern.
  const int ld_row = wave * S::kRowsPerDma + lane / S::kChunks;
  const int ld_kcol = ((lane % S::kChunks) ^ S::swz(ld_row)) * 8;
  const uint32_t ld_off = static_cast<uint32_t>(ld_row) * static_cast<uint32_t>(K) * 2u +
                          static_cast<uint32_t>(ld_kcol) * 2u;
  const uint32_t ld_step = static_cast<uint32_t>(S::kRowsPerDma * S::kWaves) * static_cast<uint32_t>(K) * 2u;
  constexpr uint32_t kLdsStep = S::kRowsPerDma * S::kWaves * S::kRowBytes;

  // ---- operand-read geometry ---------------------------------------------
  // MFMA 32x32x16: lane l supplies row (l % 32) of a 32-row block and 8
  // consecutive K values starting at 8*(l / 32) of a 16-wide K step.  Both
  // operands use the same lane -> K mapping, so the products pair up.
  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  // Fragment row blocks start at multiples of 32, so swz() of every
  // fragment row equals swz(lane % 32).
  const int frag_swz = S::swz(frag_row);
  const uint32_t a_row_base = static_cast<uint32_t>(wm * S::kWaveM + frag_row) * S::kRowBytes;
  const uint32_t b_row_base = static_cast<uint32_t>(wn * S::kWaveN + frag_row) * S::kRowBytes + S::kStageA;

  int64_t t = S::PERSISTENT ? xcd_logical_id(blockIdx.x, grid) : static_cast<int64_t>(blockIdx.x);
  for (; t < num_tiles; t += grid) {
    const TileCoord tc = grouped_tile(t, tiles_m, tiles_n, kGemmGroupM);
    const int m0 = static_cast<int>(tc.tm) * S::BM;
    const int n0 = static_cast<int>(tc.tn) * S::BN;
    const int rows_a = min(S::BM, M - m0);
    const int rows_b = min(S::BN, N - n0);
    const int4_t rsrc_a = make_buffer_rsrc(A + static_cast<int64_t>(m0) * K, static_cast<uint32_t>(rows_a) * K * 2u);
    const int4_t rsrc_b = make_buffer_rsrc(B + static_cast<int64_t>(n0) * K, static_cast<uint32_t>(rows_b) * K * 2u);

    // Re-materialise the per-lane loader offsets inside the tile loop: left to
    // itself the compiler hoists every per-instruction offset out of the
    // persistent loop and spills them, and spill reloads are vector-memory
    // operations that would force vmcnt waits on the in-flight ring.
    uint32_t tile_ld_off = ld_off;
    int tile_ld_kcol = ld_kcol;
    asm volatile("" : "+v"(tile_ld_off), "+v"(tile_ld_kcol));

    auto issue_tile = [&](int kt) {
      const int k0 = kt * S::BK;
      // K chunks at or past K read as zero (the ragged K tail).
      const uint32_t off = (k0 + tile_ld_kcol < K) ? tile_ld_off + static_cast<uint32_t>(k0) * 2u : kOobOffset;
      const uint32_t stage_lds = lds0 + static_cast<uint32_t>((kt % S::STAGES) * S::kStageBytes) +
                                 static_cast<uint32_t>(wave * S::kRowsPerDma * S::kRowBytes);
#pragma unroll
      for (int i = 0; i < S::kDmaA; ++i)
        lds_dma_b128(rsrc_a, off + i * ld_step, __builtin_amdgcn_readfirstlane(stage_lds + i * kLdsStep));
#pragma unroll
      for (int i = 0; i < S::kDmaB; ++i)
        lds_dma_b128(rsrc_b, off + i * ld_step,
                     __builtin_amdgcn_readfirstlane(stage_lds + S::kStageA + i * kLdsStep));
    };

    half8_t fa[2][S::kFragM], fb[2][S::kFragN];
    auto load_frags = [&](int buf, int kt, int ks) {
      const char *stage_ptr = smem + (kt % S::STAGES) * S::kStageBytes;
      const uint32_t chunk = static_cast<uint32_t>(((ks * 2 + frag_half) ^ frag_swz) * 16);
#pragma unroll
      for (int i = 0; i < S::kFragM; ++i)
        fa[buf][i] = *reinterpret_cast<const half8_t *>(stage_ptr + a_row_base + i * 32 * S::kRowBytes + chunk);
#pragma unroll
      for (int j = 0; j < S::kFragN; ++j)
        fb[buf][j] = *reinterpret_cast<const half8_t *>(stage_ptr + b_row_base + j * 32 * S::kRowBytes + chunk);
    };

    float16_t acc[S::kFragM][S::kFragN];
#pragma unroll
    for (int i = 0; i < S::kFragM; ++i)
#pragma unroll
      for (int j = 0; j < S::kFragN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    auto mfma_step = [&](int buf) {
#pragma unroll
      for (int i = 0; i < S::kFragM; ++i)
#pragma unroll
        for (int j = 0; j < S::kFragN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
    };

    // Every wave must be done with the previous output tile's LDS before the
    // ring is refilled, and the previous tile's stores must have left the
    // counter so the ring's vmcnt accounting below counts only its own loads.
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    workgroup_barrier();

    if constexpr (S::STAGES == 1) {
      // No overlap: load, wait, compute -- the serial order the TVM chapter
      // starts from before its step 5 adds a second stage.
      for (int kt = 0; kt < KT; ++kt) {
        issue_tile(kt);
        wait_vmcnt<0>();
        workgroup_barrier();
#pragma unroll
        for (int ks = 0; ks < S::kKSub; ++ks) {
          load_frags(0, kt, ks);
          mfma_step(0);
        }
        wait_lgkmcnt0();
        workgroup_barrier();
      }
    } else {
      // Prologue: every stage of the ring gets a K tile.
#pragma unroll
      for (int s = 0; s < S::STAGES; ++s)
        if (s < KT) issue_tile(s);
      // Tile 0 is needed; tiles 1 .. min(KT, STAGES) - 1 are younger.
      wait_tile_landed<S>(min(KT, S::STAGES) - 1);
      workgroup_barrier();
      load_frags(0, 0, 0);

      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int ks = 0; ks < S::kKSub; ++ks) {
          const int cur = ks & 1;
          if (ks + 1 < S::kKSub) {
            load_frags(cur ^ 1, kt, ks + 1);
          } else if (kt + 1 < KT) {
            // Last K step of this tile.  Its fragments are already in
            // registers; once every wave's reads of this stage are complete
            // and K tile kt+1 has landed, the stage is refilled with tile
            // kt + STAGES and the first fragments of tile kt+1 are fetched
            // while this step's MFMAs run.
            // Issued so far: tiles 0 .. min(KT, kt + STAGES) - 1.
            wait_tile_landed<S>(min(KT, kt + S::STAGES) - 1 - (kt + 1));
            wait_lgkmcnt0();
            workgroup_barrier();
            if (kt + S::STAGES < KT) issue_tile(kt + S::STAGES);
            load_frags(cur ^ 1, kt + 1, 0);
          }
          mfma_step(cur);
        }
      }
    }

    // ---- epilogue: fp32 -> fp16 (nearest even), masked stores ------------
    // acc[i][j][4g + e] is D[m][n] with m = m0 + wm*kWaveM + 32i + (lane % 32)
    // and n = n0 + wn*kWaveN + 32j + 8g + 4*(lane / 32) + e.
#pragma unroll
    for (int i = 0; i < S::kFragM; ++i) {
      const int m = m0 + wm * S::kWaveM + i * 32 + frag_row;
      const bool row_ok = m < M;
      _Float16 *drow = D + static_cast<int64_t>(row_ok ? m : 0) * N;
#pragma unroll
      for (int j = 0; j < S::kFragN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * S::kWaveN + j * 32 + g * 8 + frag_half * 4;
          half4_t h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = static_cast<_Float16>(acc[i][j][4 * g + e]);
          if (row_ok) {
            if (vec_store && n + 3 < N) {
              *reinterpret_cast<half4_t *>(drow + n) = h;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < N) drow[n + e] = h[e];
            }
          }
        }
        // Keep the scheduler from pulling every accumulator out of the
        // matrix-core registers at once.
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// ---- instantiations ------------------------------------------------------
// Default: 256x256 output tile, BK = 64, two 64 KiB LDS stages, 2x2 waves of
// 128x128, swizzled LDS, persistent grouped scheduler.
using GemmDefault = GemmShape<256, 256, 64, 2, 2, 2, true, true>;
using GemmNoSwizzle = GemmShape<256, 256, 64, 2, 2, 2, false, true>;
using GemmOneStage = GemmShape<256, 256, 64, 1, 2, 2, true, true>;
using GemmNonPersistent = GemmShape<256, 256, 64, 2, 2, 2, true, false>;

static_assert(GemmDefault::BM == kGemmBM && GemmDefault::BN == kGemmBN && GemmDefault::BK == kGemmBK &&
                  GemmDefault::STAGES == kGemmStages && GemmDefault::kThreads == kGemmThreads,
              "kernels.hpp constants must describe the default kernel");

template <class S>
static hipError_t launch(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                         hipStream_t stream) {
  const int tiles_m = (M + S::BM - 1) / S::BM;
  const int tiles_n = (N + S::BN - 1) / S::BN;
  const int64_t tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  const int64_t grid = S::PERSISTENT ? (tiles < num_cus ? tiles : num_cus) : tiles;
  const int vec_store = (N % 4 == 0) && (reinterpret_cast<uintptr_t>(D) % 8 == 0);
  hipLaunchKernelGGL(gemm_f16_kernel<S>, dim3(static_cast<unsigned>(grid)), dim3(S::kThreads), 0, stream,
                     static_cast<const _Float16 *>(A), static_cast<const _Float16 *>(B), static_cast<_Float16 *>(D),
                     M, N, K, tiles_m, tiles_n, vec_store);
  return hipGetLastError();
}

hipError_t launch_gemm_f16(int variant, const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                           hipStream_t stream) {
  switch (variant) {
    case 0: return launch<GemmDefault>(A, B, D, M, N, K, num_cus, stream);
    case 1: return launch<GemmNoSwizzle>(A, B, D, M, N, K, num_cus, stream);
    case 2: return launch<GemmOneStage>(A, B, D, M, N, K, num_cus, stream);
    case 3: return launch<GemmNonPersistent>(A, B, D, M, N, K, num_cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gt
