// gemm_ws.hip -- wave-specialised (producer / consumer) FP16 / BF16 GEMM for
// gfx950: D = A · Bᵀ, the same operation, layout and rounding as gemm.hip.
//
// The pages' last pipeline step separates the roles: producer warps only
// move tiles (TMA) and consumer warps only compute, handing stages back and
// forth through full / empty barriers (the TVM TIRx GEMM chapter's warp
// specialisation step; Croqtile ch. 7, its producer / consumer example with
// full and empty events).  This kernel is that design on gfx950:
//
//  * 8 waves per workgroup.  Waves 0..3 are consumers: each owns a 128x64
//    sub-tile of a 256x128 output tile as 8x4 blocks of
//    v_mfma_f32_16x16x32 (128 FP32 accumulators per lane, in AGPRs) and
//    issues no vector-memory instruction in the K loop -- only LDS operand
//    reads and MFMAs.  Waves 4..7 are loaders: they only issue the
//    direct-to-LDS tile loads (12 one-KiB loads per wave per K tile) and wait
//    for them.
//  * gfx950 gives every wave of a kernel the same register allocation, and a
//    SIMD holds 512 registers per lane in all.  A consumer of the default
//    kernel's 128x128 sub-tile needs 256 accumulators alone, so a loader wave
//    could not share its SIMD; with 128x64 sub-tiles both roles fit in 256
//    registers and each SIMD runs one consumer and one loader.  The price is
//    a smaller output tile: 1.5x the LDS traffic per flop of the 256x256 tile.
//  * Hand-off: one workgroup barrier per K tile plays both the "full" and
//    the "empty" barrier.  A loader arrives once the next K tile has landed
//    (its own vmcnt); a consumer arrives once it has read the last operands of
//    the current K tile (lgkmcnt), before its final MFMAs.  After the barrier
//    the consumers finish the tile and read the next one's first operands,
//    and the loaders refill the stage just freed with the tile STAGES ahead.
//  * Tile order, LDS layout and swizzle, zero-filled edges and the LDS-staged
//    epilogue are those of gemm.hip.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "tile_order.hpp"

namespace gt {

template <int STAGES, int DT>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_ws_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B, _Float16 *__restrict__ D, int M,
               int N, int K, int tiles_m, int tiles_n, int vec16) {
  constexpr int BM = 256, BN = 128, BK = 64;
  constexpr int kConsumers = 4, kLoaders = 4;
  constexpr int WAVES_N = 2;
  constexpr int kWaveM = 128, kWaveN = 64;  // consumer sub-tile
  constexpr int MI = 16, kKStep = 32;
  constexpr int kFragM = kWaveM / MI;  // 8
  constexpr int kFragN = kWaveN / MI;  // 4
  constexpr int kRowBytes = BK * 2;    // 128: one whole line per LDS row
  constexpr int kChunks = BK / 8;
  constexpr int kRowsPerDma = 64 / kChunks;                   // rows one load fills
  constexpr int kDmaA = BM / kRowsPerDma / kLoaders;          // per loader wave per K tile
  constexpr int kDmaB = BN / kRowsPerDma / kLoaders;
  constexpr int kDmaPerStage = kDmaA + kDmaB;
  constexpr int kStageA = BM * kRowBytes;
  constexpr int kStageBytes = (BM + BN) * kRowBytes;
  constexpr int kStagePitch = kWaveN * 2 + 16;
  constexpr int kStagingBytes = kConsumers * kWaveM * kStagePitch;
  constexpr int kRingBytes = STAGES * kStageBytes;
  constexpr int kLdsBytes = kRingBytes > kStagingBytes ? kRingBytes : kStagingBytes;
  constexpr int kKSub = BK / kKStep;                // MFMA K steps per K tile
  constexpr int kReads = kFragM + kFragN;           // operand reads per K step
  constexpr int kMfma = kFragM * kFragN;            // MFMAs per K step
  constexpr int kReadStride = 2;                    // MFMA slots between operand reads
  constexpr int kBarrierAt = kMfma - kReads * kReadStride;
  static_assert(kBarrierAt >= 0 && kKSub % 2 == 0, "K step schedule");
  static_assert(kLdsBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");
  static_assert(STAGES >= 2 && STAGES * kDmaPerStage <= 63, "vmcnt range");
  static_assert(kRowsPerDma * kLoaders % 16 == 0, "load row blocks must keep swz() per-lane");
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

  auto swz = [](int row) { return (row & 7) ^ ((row >> 3) & 1); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = wave >= kConsumers;  // wave-uniform
  const uint32_t lds0 = lds_addr(smem);
  const int KT = (K + BK - 1) / BK;
  const int64_t num_tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  const int64_t grid = gridDim.x;

  for (int64_t t = xcd_logical_id(blockIdx.x, grid); t < num_tiles; t += grid) {
    const TileCoord tc = grouped_tile(t, tiles_m, tiles_n, kGemmGroupM);
    const int m0 = static_cast<int>(tc.tm) * BM;
    const int n0 = static_cast<int>(tc.tn) * BN;

    // Every wave is done with the previous output tile's LDS (ring and
    // epilogue staging) before the loaders refill the ring.
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    workgroup_barrier();

    if (loader) {
      // ---- producer -------------------------------------------------------
      // Load d of a K tile fills the kRowsPerDma LDS rows starting at row
      // (d*kLoaders + lw)*kRowsPerDma of the A tile (d < kDmaA) or the B tile;
      // lane l fetches logical chunk (l % kChunks) ^ swz(row) so the LDS
      // holds the swizzled layout the operand reads expect.
      const int lw = wave - kConsumers;
      const int rows_a = min(BM, M - m0);
      const int rows_b = min(BN, N - n0);
      const int4_t rsrc_a = make_buffer_rsrc(A + static_cast<int64_t>(m0) * K, static_cast<uint32_t>(rows_a) * K * 2u);
      const int4_t rsrc_b = make_buffer_rsrc(B + static_cast<int64_t>(n0) * K, static_cast<uint32_t>(rows_b) * K * 2u);
      const int ld_row = lw * kRowsPerDma + lane / kChunks;
      const int ld_kcol = ((lane % kChunks) ^ swz(ld_row)) * 8;
      const uint32_t ld_off =
          static_cast<uint32_t>(ld_row) * static_cast<uint32_t>(K) * 2u + static_cast<uint32_t>(ld_kcol) * 2u;
      const uint32_t ld_step = static_cast<uint32_t>(kRowsPerDma * kLoaders) * static_cast<uint32_t>(K) * 2u;
      constexpr uint32_t kLdsStep = kRowsPerDma * kLoaders * kRowBytes;
      auto issue = [&](int kt) {
        const int k0 = kt * BK;
        const uint32_t off = (k0 + ld_kcol < K) ? ld_off + static_cast<uint32_t>(k0) * 2u : kOobOffset;
        const uint32_t stage_lds = lds0 + static_cast<uint32_t>((kt % STAGES) * kStageBytes) +
                                   static_cast<uint32_t>(lw * kRowsPerDma * kRowBytes);
#pragma unroll
        for (int d = 0; d < kDmaPerStage; ++d) {
          if (d < kDmaA)
            lds_dma_b128(rsrc_a, off + d * ld_step,
                         static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(stage_lds + d * kLdsStep)));
          else
            lds_dma_b128(rsrc_b, off + (d - kDmaA) * ld_step,
                         static_cast<uint32_t>(
                             __builtin_amdgcn_readfirstlane(stage_lds + kStageA + (d - kDmaA) * kLdsStep)));
        }
      };
      // Every stage starts free: tiles 0 .. STAGES-1 go out at once.
#pragma unroll
      for (int s = 0; s < STAGES; ++s)
        if (s < KT) issue(s);
      // Tile 0 landed ("full"), then one hand-off per K tile: tile kt+1 has
      // landed, and past the barrier stage kt is free ("empty") for tile
      // kt + STAGES.
      wait_younger<kDmaPerStage, STAGES - 1>(min(KT, STAGES) - 1);
      workgroup_barrier();
      for (int kt = 0; kt + 1 < KT; ++kt) {
        wait_younger<kDmaPerStage, STAGES - 1>(min(KT, kt + STAGES) - (kt + 2));
        workgroup_barrier();
        if (kt + STAGES < KT) issue(kt + STAGES);
      }
      workgroup_barrier();  // the consumers' epilogue may now reuse the ring
    } else {
      // ---- consumer -------------------------------------------------------
      const int wm = wave / WAVES_N;
      const int wn = wave % WAVES_N;
      const int frag_row = lane % MI;
      const int frag_kgrp = lane / MI;
      // Chunks 0, 2, 1, 3 of the K step for lane groups 0..3: lanes l and
      // l + 32, which the LDS serves together, then read chunks an odd XOR
      // apart (conflict-free under the row swizzle), as in gemm.hip.
      const int frag_kchunk = ((frag_kgrp & 1) << 1) | (frag_kgrp >> 1);
      const int frag_swz = swz(frag_row);
      const uint32_t a_row_base = static_cast<uint32_t>(wm * kWaveM + frag_row) * kRowBytes;
      const uint32_t b_row_base = static_cast<uint32_t>(wn * kWaveN + frag_row) * kRowBytes + kStageA;

      half8_t fa[2][kFragM], fb[2][kFragN];
      auto read_frag = [&](int buf, int kt, int ks, int r) {
        const char *stage_ptr = smem + (kt % STAGES) * kStageBytes;
        const uint32_t chunk = static_cast<uint32_t>(((ks * (kKStep / 8) + frag_kchunk) ^ frag_swz) * 16);
        if (r == 0) {
          fa[buf][0] = *reinterpret_cast<const half8_t *>(stage_ptr + a_row_base + chunk);
        } else if (r <= kFragN) {
          const int j = r - 1;
          fb[buf][j] = *reinterpret_cast<const half8_t *>(stage_ptr + b_row_base + j * MI * kRowBytes + chunk);
        } else {
          const int i = r - kFragN;
          fa[buf][i] = *reinterpret_cast<const half8_t *>(stage_ptr + a_row_base + i * MI * kRowBytes + chunk);
        }
      };

      float4_t acc[kFragM][kFragN];
#pragma unroll
      for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      // The zeros are VALU writes first read by hand-written MFMAs the
      // compiler's hazard padding does not see: these statements take every
      // accumulator and carry wait states after the zeros are materialised.
      static_assert(kFragN == 4, "accumulator fence covers 4 blocks per row");
#pragma unroll
      for (int i = 0; i < kFragM; ++i)
        asm volatile("s_nop 1" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]));

      // 16x16x32 MFMA on AGPR-pinned accumulators (see gemm.hip for why the
      // builtin is not used).  B rows feed the first operand, A rows the second.
      auto mfma = [&](int buf, int idx) {
        const int i = idx / kFragN;
        const int j = idx % kFragN;
        if constexpr (DT == kF16)
          asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(fb[buf][j]), "v"(fa[buf][i]));
        else
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(fb[buf][j]), "v"(fa[buf][i]));
      };

      // One K tile, instruction order pinned: a non-final K step carries one
      // operand read for the next step every kReadStride MFMA slots; the
      // final step reads its last operands in the previous step, waits for
      // its LDS reads, meets the loaders at the hand-off after kBarrierAt
      // MFMAs, and reads the next K tile's first operands during the rest.
      auto ktile = [&](int kt, auto next_c) {
        constexpr bool kNext = decltype(next_c)::value;
#pragma unroll
        for (int ks = 0; ks < kKSub; ++ks) {
          const int cur = ks & 1;
          const bool last = ks == kKSub - 1;
#pragma unroll
          for (int idx = 0; idx < kMfma; ++idx) {
            if (last && kNext && idx == kBarrierAt) {
              __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
              workgroup_barrier();
              __builtin_amdgcn_sched_barrier(0);
            }
            mfma(cur, idx);
            __builtin_amdgcn_sched_barrier(0);
            if (!last) {
              if (idx % kReadStride == 0 && idx / kReadStride < kReads) {
                read_frag(cur ^ 1, kt, ks + 1, idx / kReadStride);
                __builtin_amdgcn_sched_barrier(0);
              }
            } else if (kNext && idx >= kBarrierAt && (idx - kBarrierAt) % kReadStride == 0) {
              read_frag(cur ^ 1, kt + 1, 0, (idx - kBarrierAt) / kReadStride);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      };

      workgroup_barrier();  // tile 0 has landed
#pragma unroll
      for (int r = 0; r < kReads; ++r) read_frag(0, 0, 0, r);
      using yes = std::true_type;
      using no = std::false_type;
      int kt = 0;
      for (; kt + 1 < KT; ++kt) ktile(kt, yes{});
      ktile(kt, no{});

      // Wait states between the last hand-written MFMA and the accumulator
      // reads below.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      workgroup_barrier();  // every wave is done with the ring

      // ---- epilogue: FP32 -> 16-bit, nearest even, staged through LDS ------
      // acc[i][j][e] is D[m][n] with m = m0 + wm*kWaveM + 16i + (lane % 16)
      // and n = n0 + wn*kWaveN + 16j + 4*(lane / 16) + e.
      const uint32_t stage_base = static_cast<uint32_t>(wave * kWaveM * kStagePitch);
#pragma unroll
      for (int i = 0; i < kFragM; ++i) {
#pragma unroll
        for (int j = 0; j < kFragN; ++j) {
          half4_t h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = round_out<DT>(acc[i][j][e]);
          const int col = j * 16 + frag_kgrp * 4;
          const uint32_t off = stage_base + static_cast<uint32_t>((i * MI + frag_row) * kStagePitch + col * 2);
          *reinterpret_cast<half4_t *>(smem + off) = h;
        }
      }
      constexpr int kRowChunks = kWaveN / 8;
      constexpr int kRowsPerPass = 64 / kRowChunks;
      const int chunk = lane % kRowChunks;
      const int n = n0 + wn * kWaveN + chunk * 8;
#pragma unroll 4
      for (int r0 = 0; r0 < kWaveM; r0 += kRowsPerPass) {
        const int r = r0 + lane / kRowChunks;
        const half8_t v = *reinterpret_cast<const half8_t *>(smem + stage_base + r * kStagePitch + chunk * 16);
        const int m = m0 + wm * kWaveM + r;
        if (m < M) {
          _Float16 *dst = D + static_cast<int64_t>(m) * N + n;
          if (vec16 && n + 8 <= N) {
            *reinterpret_cast<half8_t *>(dst) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (n + e < N) dst[e] = v[e];
          }
        }
      }
    }
  }
}

template <int STAGES, int DT>
static hipError_t launch_ws(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                            hipStream_t stream) {
  const int tiles_m = (M + 255) / 256;
  const int tiles_n = (N + 127) / 128;
  const int64_t tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  const int64_t grid = tiles < num_cus ? tiles : num_cus;
  const int vec16 = (N % 8 == 0) && (reinterpret_cast<uintptr_t>(D) % 16 == 0);
  hipLaunchKernelGGL((gemm_ws_kernel<STAGES, DT>), dim3(static_cast<unsigned>(grid)), dim3(512), 0, stream,
                     static_cast<const _Float16 *>(A), static_cast<const _Float16 *>(B), static_cast<_Float16 *>(D),
                     M, N, K, tiles_m, tiles_n, vec16);
  return hipGetLastError();
}

hipError_t launch_gemm_ws_f16(int variant, const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                              hipStream_t stream) {
  switch (variant) {
    case 0: return launch_ws<3, kF16>(A, B, D, M, N, K, num_cus, stream);
    case 1: return launch_ws<2, kF16>(A, B, D, M, N, K, num_cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gt
