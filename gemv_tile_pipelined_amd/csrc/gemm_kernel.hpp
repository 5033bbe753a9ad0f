// gemm_kernel.hpp -- the persistent, pipelined tiled GEMM kernel (D = A·Bᵀ)
// as a template, its launch shapes, and the launchers the translation units
// gemm.hip and gemm_plain.hip instantiate.  The structure of the kernel is
// described at the top of gemm.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "ring.hpp"
#include "tile_order.hpp"

namespace gt {

template <int BM_, int BN_, int BK_, int STAGES_, int WAVES_M_, int WAVES_N_, bool SWIZZLE_, bool PERSISTENT_,
          int DMA_STRIDE_, int MI_ = 32, int READ_STRIDE_ = 1, int DMA_OFFSET_ = 0, int DTYPE_ = kF16,
          bool EARLY_FREE_ = false, int WAR_AT_ = 0, bool SERPENTINE_ = false>
struct GemmShape {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int BK = BK_;
  static constexpr int STAGES = STAGES_;
  static constexpr int WAVES_M = WAVES_M_;
  static constexpr int WAVES_N = WAVES_N_;
  static constexpr bool SWIZZLE = SWIZZLE_;
  static constexpr bool PERSISTENT = PERSISTENT_;
  // MFMA slots between two consecutive loads of the ring refill.
  static constexpr int DMA_STRIDE = DMA_STRIDE_;
  // MFMA block edge: 32 (v_mfma_f32_32x32x16_f16) or 16 (v_mfma_f32_16x16x32_f16).
  static constexpr int MI = MI_;
  static_assert(MI == 32 || MI == 16, "MFMA shape");
  static_assert(MI == 32 || STAGES_ >= 2, "16x16x32 blocks need the pipelined (multi-stage) loop");
  static constexpr int kKStep = MI == 32 ? 16 : 32;  // K consumed by one MFMA
  static constexpr int kAccRegs = MI * MI / 64;      // FP32 accumulator registers per lane per block
  // MFMA slots between two operand reads for the next K step (1: one read
  // per slot from the start of the step), and the slot offset of the refill
  // loads, which lets them fall between the reads.
  static constexpr int READ_STRIDE = READ_STRIDE_;
  static constexpr int DMA_OFFSET = DMA_OFFSET_;
  // Element format of A, B and D (kF16 or kBF16; bf16 only with the
  // hand-written 16x16x32 MFMAs).
  static constexpr int DTYPE = DTYPE_;
  static_assert(DTYPE == kF16 || (DTYPE == kBF16 && MI_ == 16), "bf16 uses the 16x16x32 MFMA path");
  // K loop schedule: the one-barrier ring (ring_k_loop), or the early-free
  // one (ring_k_loop_ef) with its free barrier at slot WAR_AT of K step 0.
  static constexpr bool EARLY_FREE = EARLY_FREE_;
  static constexpr int WAR_AT = WAR_AT_;
  // MFMA order within a K step: row-major over the wave's blocks (i, j), or
  // serpentine (odd block rows run j downwards), so that consecutive MFMAs
  // always share one operand, also across block rows.
  static constexpr bool SERPENTINE = SERPENTINE_;
  static_assert((BK / kKStep) >= 1 && (BM / WAVES_M / MI) * (BN / WAVES_N / MI) % READ_STRIDE == 0,
                "the read spacing must divide the MFMA slots of a K step");

  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kWaveM = BM / WAVES_M;  // rows of D per wave
  static constexpr int kWaveN = BN / WAVES_N;  // cols of D per wave
  static constexpr int kFragM = kWaveM / MI;   // MFMA blocks per wave, M
  static constexpr int kFragN = kWaveN / MI;   // MFMA blocks per wave, N
  static constexpr int kRowBytes = BK * 2;
  static constexpr int kChunks = BK / 8;            // 16-byte chunks per LDS row
  static constexpr int kRowsPerDma = 64 / kChunks;  // rows one wave DMA fills
  static constexpr int kDmaA = BM / kRowsPerDma / kWaves;  // per-wave DMA instrs for A
  static constexpr int kDmaB = BN / kRowsPerDma / kWaves;
  static constexpr int kDmaPerStage = kDmaA + kDmaB;
  static constexpr int kStageA = BM * kRowBytes;
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  // Epilogue staging: each wave's kWaveM x kWaveN fp16 tile, rows padded by
  // 16 bytes (keeps 16-byte row alignment for the read-back and spreads the
  // column-wise writes over the banks).
  static constexpr int kStagePitch = kWaveN * 2 + 16;
  static constexpr int kStagingBytes = kWaves * kWaveM * kStagePitch;
  static constexpr int kRingBytes = STAGES * kStageBytes;
  static constexpr int kLdsBytes = kRingBytes > kStagingBytes ? kRingBytes : kStagingBytes;
  static constexpr int kKSub = BK / kKStep;  // MFMA K steps per K tile
  static constexpr int kReads = kFragM + kFragN;  // operand reads per wave per K step
  static constexpr int kMfma = kFragM * kFragN;   // MFMAs per wave per K step
  // Block row and column of MFMA slot idx of a K step.
  __host__ __device__ static constexpr int mfma_i(int idx) { return idx / kFragN; }
  __host__ __device__ static constexpr int mfma_j(int idx) {
    return (SERPENTINE && (idx / kFragN) % 2 == 1) ? kFragN - 1 - idx % kFragN : idx % kFragN;
  }

  static_assert(BK == 32 || BK == 64, "LDS rows of 64 or 128 bytes");
  // The pipelined loop double-buffers the operand fragments by K-step parity
  // (step ks of a K tile computes from buffer ks & 1 and fills the other), so
  // a K tile must hold an even number of K steps for the parity to carry
  // over to the next tile: K tiles of 64 with 16x16x32 blocks, of 32 or 64
  // with 32x32x16 blocks.
  static_assert(STAGES_ == 1 || (BK / kKStep) % 2 == 0, "pipelined loop needs an even number of K steps per K tile");
  static_assert(kWaveM % MI == 0 && kWaveN % MI == 0, "wave tile must be whole MFMA blocks");
  static_assert(BM % (kRowsPerDma * kWaves) == 0 && BN % (kRowsPerDma * kWaves) == 0, "DMA split");
  static_assert(kLdsBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS per CU");
  static_assert(STAGES >= 1 && (STAGES - 1) * kDmaPerStage <= 63, "vmcnt range");

  // Physical 16-byte chunk of logical chunk c in LDS row r is c ^ swz(r);
  // swz depends only on r & 15.  An operand fetch reads one logical chunk
  // from 32 consecutive rows.  128-byte rows (8 chunks): any 8 consecutive
  // rows land on 8 different chunk positions (conflict-free when 8 lanes
  // share an LDS cycle) and any 16 consecutive rows cover the 16 positions of
  // a 256-byte bank window (conflict-free with 16 lanes per cycle).  64-byte
  // rows (4 chunks, two rows per 128 bytes): the same two properties hold
  // with the XOR taken from rows' bits 1..3.
  __host__ __device__ static constexpr int swz(int row) {
    if (!SWIZZLE) return 0;
    if (BK == 64) return (row & 7) ^ ((row >> 3) & 1);
    return ((row >> 1) ^ ((row >> 3) & 1)) & 3;
  }
};

// Wait until at most `n` vector-memory operations of this wave are in flight,
// where n is one of 0, PER, 2*PER, ..., MAXY*PER (the values ring_vmcnt
// produces for a ring of MAXY+2 stages); vmcnt takes an immediate, so the
// value is matched against that set, and anything else drains fully (always
// correct).
template <int PER, int MAXY>
__device__ inline void wait_vmcnt_n(int n) {
  if constexpr (MAXY > 0) {
    if (n == MAXY * PER) {
      wait_vmcnt<MAXY * PER>();
      return;
    }
    wait_vmcnt_n<PER, MAXY - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// The kernel's side of the ring walker (ring.hpp): each event becomes the
// instruction(s) it stands for.
template <class S, class Mfma, class Read, class Load, class MfmaLoad, class Prep, class InitAcc>
struct KernelRingOps {
  Mfma mfma_fn;
  Read read_fn;
  Load load_fn;
  MfmaLoad mfma_load_fn;
  Prep prep_fn;
  InitAcc init_acc_fn;
  __device__ __attribute__((always_inline)) void mfma(int buf, int idx) { mfma_fn(buf, idx); }
  __device__ __attribute__((always_inline)) void read(int buf, int kt, int ks, int r) { read_fn(buf, kt, ks, r); }
  __device__ __attribute__((always_inline)) void load(int tile, int d) { load_fn(tile, d); }
  __device__ __attribute__((always_inline)) void mfma_load(int buf, int idx, int tile, int d) {
    mfma_load_fn(buf, idx, tile, d);
  }
  __device__ __attribute__((always_inline)) void prep(int tile, int part) { prep_fn(tile, part); }
  __device__ __attribute__((always_inline)) void init_acc() { init_acc_fn(); }
  __device__ __attribute__((always_inline)) void wait_tile(int n) {
    if constexpr (S::EARLY_FREE) {
      constexpr int kSteady = RingEarly<S>::kSteadyVmcnt;
      if (n == kSteady) {
        wait_vmcnt<kSteady>();
        return;
      }
      wait_vmcnt_n<S::kDmaPerStage, S::STAGES - 1>(n);
    } else {
      wait_vmcnt_n<S::kDmaPerStage, S::STAGES - 2>(n);
    }
  }
  __device__ __attribute__((always_inline)) void wait_lds() { __builtin_amdgcn_s_waitcnt(kWaitLgkm0); }
  __device__ __attribute__((always_inline)) void barrier() { workgroup_barrier(); }
  __device__ __attribute__((always_inline)) void fence() { __builtin_amdgcn_sched_barrier(0); }
};

// Epilogue modes.  kEpiPlain: round and store D.  kEpiFused: add bias[n]
// and apply ReLU when `relu` is set (gemm_bias_*), then round and store D.
// kEpiPartial (split K, gemm_splitk_*): the grid walks (tile, K slice) units,
// `splits` slices per tile; each unit sums only its slice of K tiles and
// stores the FP32 sums, unrounded, to ws[slice][m][n]; splitk_reduce_kernel
// adds the slices.  kEpiTimed: as kEpiPlain, and thread 0 of each workgroup
// records when it started, when the K loop of its first output tile ended
// and when it finished (its stores complete), in the constant 100 MHz
// real-time counter and the shader-cycle counter, with its XCC and hardware
// ids, into 8 uint64 at ws + 16 * blockIdx.x bytes (a measurement of the
// clock the MFMAs run at and of where the time goes; gemvtile_gemm_f16_timed).
// kEpiCachedStores: as kEpiPlain with ordinary (cached) stores of D instead
// of non-temporal ones (an ablation).  Each mode ignores the arguments of the
// others.
enum : int { kEpiPlain = 0, kEpiFused = 1, kEpiPartial = 2, kEpiTimed = 3, kEpiCachedStores = 4 };

template <class S, int EPI = kEpiPlain>
__global__ void __launch_bounds__(S::kThreads) __attribute__((amdgpu_waves_per_eu(S::kWaves / 4, S::kWaves / 4)))
gemm_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B, _Float16 *__restrict__ D,
                int M, int N, int K, int tiles_m, int tiles_n, int vec16, const uint16_t *__restrict__ bias,
                int relu, float *__restrict__ ws, int splits) {
  static_assert(EPI != kEpiPartial || (S::MI == 16 && S::STAGES >= 2), "split K uses the pipelined 16x16x32 loop");
  __shared__ __attribute__((aligned(1024))) char smem[S::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // kEpiTimed: thread 0 writes each stamp as it is taken (none is held in
  // registers across the K loop, whose accumulators fill the register file).
  uint64_t *const stamps =
      EPI == kEpiTimed ? reinterpret_cast<uint64_t *>(ws) + static_cast<int64_t>(blockIdx.x) * 8 : nullptr;
  bool first_tile = true;
  if constexpr (EPI == kEpiTimed) {
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    const uint64_t c = __builtin_amdgcn_s_memtime();
    if (tid == 0) {
      stamps[0] = r;
      stamps[1] = c;
    }
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WAVES_N;
  const int wn = wave % S::WAVES_N;
  const uint32_t lds0 = lds_addr(smem);
  const int KT = (K + S::BK - 1) / S::BK;
  const int64_t num_tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  const int64_t grid = gridDim.x;

  // ---- loader geometry ----------------------------------------------------
  // DMA instruction i of this wave fills the kRowsPerDma LDS rows starting at
  // row (i*kWaves + wave)*kRowsPerDma; lane l writes physical chunk
  // l % kChunks of the row i*kRowsPerDma*kWaves + ld_row, so it fetches the
  // logical chunk (l % kChunks) ^ swz(row) of that row.  Each instruction
  // starts at a multiple of 16 rows, so swz(row) does not depend on i: one
  // offset per lane serves every instruction (instruction i adds
  // i*kRowsPerDma*kWaves rows).  A and B tiles use the same pattern.
  static_assert(S::kRowsPerDma * S::kWaves % 16 == 0, "DMA row blocks must keep swz() per-lane");
  const int ld_row = wave * S::kRowsPerDma + lane / S::kChunks;
  const int ld_kcol = ((lane % S::kChunks) ^ S::swz(ld_row)) * 8;
  const uint32_t ld_off = static_cast<uint32_t>(ld_row) * static_cast<uint32_t>(K) * 2u +
                          static_cast<uint32_t>(ld_kcol) * 2u;
  const uint32_t ld_step = static_cast<uint32_t>(S::kRowsPerDma * S::kWaves) * static_cast<uint32_t>(K) * 2u;
  constexpr uint32_t kLdsStep = S::kRowsPerDma * S::kWaves * S::kRowBytes;

  // ---- operand-read geometry ---------------------------------------------
  // An MFMA with MI x MI blocks takes, from lane l, row (l % MI) of an MI-row
  // block and the 8 consecutive K values starting at 8*(l / MI) of its K step
  // (16 wide for MI = 32, 32 wide for MI = 16), i.e. one 16-byte LDS chunk.
  // Both operands use the same lane -> K mapping, so the products pair up.
  const int frag_row = lane % S::MI;
  const int frag_kgrp = lane / S::MI;
  // Which 16-byte chunk of the K step lane group frag_kgrp reads.  The MFMA
  // only needs A and B to agree, so the order is free.  The LDS serves a
  // 16-byte-per-lane read in lane groups that pair lane l with lane l + 32;
  // with 16x16 blocks those lanes read the same rows, and chunks c and c + 2
  // (an even XOR apart) would land two rows on the same banks under the row
  // swizzle.  Groups 0..3 therefore read chunks 0, 2, 1, 3 of the step, so
  // lanes l and l + 32 differ by an odd XOR.  With 32x32 blocks (two groups:
  // chunks c, c + 1) the plain order already has that property.
  const int frag_kchunk = S::MI == 16 ? ((frag_kgrp & 1) << 1) | (frag_kgrp >> 1) : frag_kgrp;
  // Fragment row blocks start at multiples of MI (16 or 32), and swz()
  // depends only on row & 15, so swz() of every fragment row equals
  // swz(lane % MI).
  const int frag_swz = S::swz(frag_row);
  const uint32_t a_row_base = static_cast<uint32_t>(wm * S::kWaveM + frag_row) * S::kRowBytes;
  const uint32_t b_row_base = static_cast<uint32_t>(wn * S::kWaveN + frag_row) * S::kRowBytes + S::kStageA;

  // Work units: output tiles, or (tile, K slice) pairs with split K, slice
  // major, so that units running side by side share K ranges.
  const int64_t num_units = EPI == kEpiPartial ? num_tiles * splits : num_tiles;
  int64_t u = S::PERSISTENT ? xcd_logical_id(blockIdx.x, grid) : static_cast<int64_t>(blockIdx.x);
  for (; u < num_units; u += grid) {
    const int64_t t = EPI == kEpiPartial ? u % num_tiles : u;
    const TileCoord tc = tile_of(t, tiles_m, tiles_n, kGemmGroupM);
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

    // Loads [first, last) of the kDmaPerStage per-wave DMA instructions of K
    // tile kt (A tile first, then B tile).
    // K tile kt of the loop reads K tile kt + kofs of the matrices; the loop
    // runs over KTu K tiles (all KT of them, or one K slice), and kofs + KTu
    // <= KT.
    int kofs = 0;
    int KTu = KT;
    int slice = 0;
    if constexpr (EPI == kEpiPartial) {
      slice = static_cast<int>(u / num_tiles);
      const int per = (KT + splits - 1) / splits;  // the host keeps every slice non-empty
      kofs = slice * per;
      KTu = min(per, KT - kofs);
    }
    // Operands of load d of K tile kt: buffer descriptor, per-lane byte
    // offset, and the (wave-uniform) LDS address of its 1 KiB destination.
    struct DmaArgs {
      int4_t rsrc;
      uint32_t voffset;
      uint32_t lds;
    };
    auto dma_args = [&](int kt, int d) -> DmaArgs {
      const int k0 = (kt + kofs) * S::BK;
      // K chunks at or past K read as zero (the ragged K tail).
      const uint32_t off = (k0 + tile_ld_kcol < K) ? tile_ld_off + static_cast<uint32_t>(k0) * 2u : kOobOffset;
      const uint32_t stage_lds = lds0 + static_cast<uint32_t>((kt % S::STAGES) * S::kStageBytes) +
                                 static_cast<uint32_t>(wave * S::kRowsPerDma * S::kRowBytes);
      if (d < S::kDmaA)
        return DmaArgs{rsrc_a, off + d * ld_step,
                       static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(stage_lds + d * kLdsStep))};
      const int i = d - S::kDmaA;
      return DmaArgs{rsrc_b, off + i * ld_step,
                     static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(stage_lds + S::kStageA + i * kLdsStep))};
    };
    auto issue_loads = [&](int kt, int first, int last) {
#pragma unroll
      for (int d = 0; d < S::kDmaPerStage; ++d) {
        if (d < first || d >= last) continue;
        const DmaArgs g = dma_args(kt, d);
        lds_dma_b128(g.rsrc, g.voffset, g.lds);
      }
    };

    half8_t fa[2][S::kFragM], fb[2][S::kFragN];
    // Operand read r (of kReads) of K step ks of K tile kt into buffer buf.
    // Reads go out as fa[0], fb[0..kFragN-1], fa[1..kFragM-1], which is the
    // order the MFMA sequence below (block row 0 first, in either order)
    // first needs them in.
    constexpr int kReads = S::kReads;
    constexpr int kMfma = S::kMfma;
    auto read_frag = [&](int buf, int kt, int ks, int r) {
      const char *stage_ptr = smem + (kt % S::STAGES) * S::kStageBytes;
      const uint32_t chunk = static_cast<uint32_t>(((ks * (S::kKStep / 8) + frag_kchunk) ^ frag_swz) * 16);
      if (r == 0) {
        fa[buf][0] = *reinterpret_cast<const half8_t *>(stage_ptr + a_row_base + chunk);
      } else if (r <= S::kFragN) {
        const int j = r - 1;
        fb[buf][j] = *reinterpret_cast<const half8_t *>(stage_ptr + b_row_base + j * S::MI * S::kRowBytes + chunk);
      } else {
        const int i = r - S::kFragN;
        fa[buf][i] = *reinterpret_cast<const half8_t *>(stage_ptr + a_row_base + i * S::MI * S::kRowBytes + chunk);
      }
    };
    auto load_frags = [&](int buf, int kt, int ks) {
#pragma unroll
      for (int r = 0; r < kReads; ++r) read_frag(buf, kt, ks, r);
    };

    using AccT = std::conditional_t<S::MI == 32, float16_t, float4_t>;
    AccT acc[S::kFragM][S::kFragN];
    // Zero the accumulators.  The pipelined loop does this after issuing its
    // first tile loads (ring.hpp calls init_acc), so the 256 register writes
    // overlap the loads' latency instead of delaying their issue.
    auto init_acc = [&]() {
#pragma unroll
      for (int i = 0; i < S::kFragM; ++i)
#pragma unroll
        for (int j = 0; j < S::kFragN; ++j)
#pragma unroll
          for (int e = 0; e < S::kAccRegs; ++e) acc[i][j][e] = 0.0f;
      if constexpr (S::MI == 16) {
        // The zeros above are written by VALU instructions and first read by
        // a hand-written MFMA, which the compiler's hazard padding does not
        // know about.  These statements take every accumulator as input and
        // output and carry wait states: the zeros are materialised before
        // them (and cannot be re-created after them), so they precede every
        // MFMA by at least 16 wait states.
        static_assert(S::kFragN % 4 == 0, "accumulator fence covers 4 blocks per statement");
#pragma unroll
        for (int i = 0; i < S::kFragM; ++i)
#pragma unroll
          for (int j = 0; j < S::kFragN; j += 4)
            asm volatile("s_nop 1" : "+a"(acc[i][j]), "+a"(acc[i][j + 1]), "+a"(acc[i][j + 2]), "+a"(acc[i][j + 3]));
      }
    };

    auto mfma = [&](int buf, int idx) {
      const int i = S::mfma_i(idx);
      const int j = S::mfma_j(idx);
      if constexpr (S::MI == 32) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
      } else {
        // Written as inline asm with the accumulator pinned to AGPRs: through
        // the builtin, the register allocator renames the 64 four-register
        // accumulators around the K loop and copies them back on every
        // iteration.  The compiler does not see this as an MFMA, so the read
        // of the accumulators after the K loop is padded by hand (mfma_drain).
        if constexpr (S::DTYPE == kF16)
          asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                       : "+a"(acc[i][j])
                       : "v"(fb[buf][j]), "v"(fa[buf][i]));
        else
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                       : "+a"(acc[i][j])
                       : "v"(fb[buf][j]), "v"(fa[buf][i]));
      }
    };
    // Wait states between the last hand-written MFMA and any read of its
    // result: more than the 16x16x32 MFMA's pass count requires.  The
    // sched_barrier keeps the accumulator reads after the padding.
    auto mfma_drain = [&]() {
      if constexpr (S::MI == 16) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    if constexpr (S::STAGES == 1) {
      // No overlap: load, wait, compute -- the serial order the TVM chapter
      // starts from before its step 5 adds a second stage.  Every wave must
      // first be done with the previous output tile's LDS.
      init_acc();
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      workgroup_barrier();
      for (int kt = 0; kt < KTu; ++kt) {
        issue_loads(kt, 0, S::kDmaPerStage);
        wait_vmcnt<0>();
        workgroup_barrier();
#pragma unroll
        for (int ks = 0; ks < S::kKSub; ++ks) {
          load_frags(0, kt, ks);
#pragma unroll
          for (int idx = 0; idx < kMfma; ++idx) mfma(0, idx);
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        workgroup_barrier();
      }
    } else {
      // The pipelined loop: the ring walker of ring.hpp, in a fixed
      // instruction order (fence() is a sched_barrier).  Every READ_STRIDE-th
      // MFMA slot of a non-final K step carries one operand read for the next
      // step, spread out so that the four waves' reads do not outrun the LDS.
      // The refill's loads go out one every DMA_STRIDE MFMA slots: bunched
      // together, the four waves' loads saturate the texture path and stall
      // MFMA issue, while spread too thin the last load lands too close to
      // the barrier that needs it.  The previous output tile's D stores may
      // still be in flight when the ring starts: they are older than every
      // ring load, so they can only make the ring's vmcnt waits more
      // conservative.
      auto load_one = [&](int tile, int d) { issue_loads(tile, d, d + 1); };
      // The refill's addresses, worked out by prep() in the otherwise empty
      // MFMA slots before the free barrier (computed all at once after the
      // barrier, they held up the next MFMA by about 8 instruction issues):
      // rf_off is this lane's byte offset for the refill's load 0 (each
      // further row block adds ld_step; the A and B tiles share it), or
      // kOobOffset past K; rf_lds is the LDS address of load 0 (this wave's
      // rows of the stage).  The empty asm statements pin each part where
      // the walker puts it.  A lane's chunk lies past K when
      // rf_k0 + tile_ld_kcol >= K, i.e. when rf_lim - rf_k0 is negative; its
      // sign bit then moves rf_off past every buffer's range (as kOobOffset
      // does), without a compare and a select.
      static_assert(kOobOffset == 0x80000000u, "the sign bit is the out-of-range offset");
      const int rf_lim = K - 1 - tile_ld_kcol;
      uint32_t rf_off = 0, rf_lds = 0, rf_past = 0;
      int rf_k0 = 0;
      auto prep = [&](int tile, int part) {
        if (part == 0) {
          rf_k0 = (tile + kofs) * S::BK;
          asm volatile("" : "+s"(rf_k0));
        } else if (part == 1) {
          rf_lds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
              lds0 + static_cast<uint32_t>((tile % S::STAGES) * S::kStageBytes) +
              static_cast<uint32_t>(wave * S::kRowsPerDma * S::kRowBytes)));
          asm volatile("" : "+s"(rf_lds));
        } else if (part == 2) {
          rf_off = tile_ld_off + static_cast<uint32_t>(rf_k0) * 2u;
          asm volatile("" : "+v"(rf_off));
        } else if (part == 3) {
          rf_past = static_cast<uint32_t>(rf_lim - rf_k0);
          asm volatile("" : "+v"(rf_past));
        } else {
          rf_off |= rf_past & kOobOffset;
          asm volatile("" : "+v"(rf_off));
        }
      };
      // A slot's MFMA and its refill load in one asm statement: M0 (the
      // load's LDS address) is written before the MFMA, which then serves as
      // the wait state an LDS DMA needs after an M0 write, instead of an
      // s_nop of its own.  0.8-1.7 % faster at 4096^3 and 8192^3 than the
      // load issued on its own after the MFMA, on uniform data and on zeros.
      // As in lds_dma_b128, M0 is written and used inside the one statement
      // (build.py rejects compiler-emitted M0 uses in such kernels).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      auto mfma_load = [&](int buf, int idx, int tile, int d) {
        if constexpr (S::MI == 16) {
          const int i = S::mfma_i(idx);
          const int j = S::mfma_j(idx);
          (void)tile;  // prep() has worked out this refill's addresses
          const bool is_a = d < S::kDmaA;
          const uint32_t row_block = static_cast<uint32_t>(is_a ? d : d - S::kDmaA);
          const DmaArgs g{is_a ? rsrc_a : rsrc_b, rf_off + row_block * ld_step,
                          rf_lds + (is_a ? 0u : static_cast<uint32_t>(S::kStageA)) + row_block * kLdsStep};
          if constexpr (S::DTYPE == kF16)
            asm volatile(
                "s_mov_b32 m0, %3\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0\n\tbuffer_load_dwordx4 %4, %5, 0 offen lds"
                : "+a"(acc[i][j])
                : "v"(fb[buf][j]), "v"(fa[buf][i]), "s"(g.lds), "v"(g.voffset), "s"(g.rsrc)
                : "memory", "m0");
          else
            asm volatile(
                "s_mov_b32 m0, %3\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\tbuffer_load_dwordx4 %4, %5, 0 offen lds"
                : "+a"(acc[i][j])
                : "v"(fb[buf][j]), "v"(fa[buf][i]), "s"(g.lds), "v"(g.voffset), "s"(g.rsrc)
                : "memory", "m0");
        } else {
          mfma(buf, idx);
          load_one(tile, d);
        }
      };
#pragma clang diagnostic pop
      KernelRingOps<S, decltype(mfma), decltype(read_frag), decltype(load_one), decltype(mfma_load), decltype(prep),
                    decltype(init_acc)>
          ops{mfma, read_frag, load_one, mfma_load, prep, init_acc};
      if constexpr (S::EARLY_FREE)
        ring_k_loop_ef<S>(ops, KTu);
      else
        ring_k_loop<S>(ops, KTu);
    }
    if constexpr (EPI == kEpiTimed) {
      if (first_tile) {
        const uint64_t r = __builtin_amdgcn_s_memrealtime();
        const uint64_t c = __builtin_amdgcn_s_memtime();
        if (tid == 0) {
          stamps[2] = r;
          stamps[3] = c;
        }
        first_tile = false;
      }
    }

    // ---- epilogue: fp32 -> fp16 (nearest even), staged through LDS -------
    // With MI = 32, acc[i][j][4g + e] is D[m][n] with
    // m = m0 + wm*kWaveM + 32i + (lane % 32) and
    // n = n0 + wn*kWaveN + 32j + 8g + 4*(lane / 32) + e; with MI = 16,
    // acc[i][j][e] is D[m][n] with m = m0 + wm*kWaveM + 16i + (lane % 16) and
    // n = n0 + wn*kWaveN + 16j + 4*(lane / 16) + e.  Either way each lane
    // holds 8-byte pieces of many different rows, which written straight to D
    // would cost one partial cache-line write per row.  The wave instead writes its
    // tile to LDS and reads it back row by row, so each store instruction
    // writes whole 16-byte-per-lane row segments (full cache lines).
    mfma_drain();
    workgroup_barrier();  // every wave is done reading the ring
    if constexpr (EPI == kEpiPartial) {
      // FP32 sums of this K slice, unrounded, straight from the accumulators:
      // lane l holds columns 4*(l/16) .. +3 of row l % 16 of each 16x16
      // block, a 16-byte piece (ordinary stores: the reduction reads them
      // next, from the caches).
      float *wsl = ws + static_cast<int64_t>(slice) * M * N;
      const bool vec4 = (N % 4) == 0;
#pragma unroll
      for (int i = 0; i < S::kFragM; ++i) {
        const int m = m0 + wm * S::kWaveM + i * 16 + frag_row;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < S::kFragN; ++j) {
          const int n = n0 + wn * S::kWaveN + j * 16 + frag_kgrp * 4;
          float *dst = wsl + static_cast<int64_t>(m) * N + n;
          if (vec4 && n + 4 <= N) {
            *reinterpret_cast<float4_t *>(dst) = acc[i][j];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) dst[e] = acc[i][j][e];
          }
        }
      }
    } else {
      const uint32_t stage_base = static_cast<uint32_t>(wave * S::kWaveM * S::kStagePitch);
      // Column of this lane's 4 values of group g of block column j inside
      // the wave tile.
      auto lane_col = [&](int j, int g) {
        return S::MI == 32 ? j * 32 + g * 8 + frag_kgrp * 4 : j * 16 + frag_kgrp * 4;
      };
      // The bias of every column this lane holds, loaded once per tile
      // (columns past N read the last bias; their outputs are not stored).
      // The null test is made once, outside the loads: inside them it put
      // every load under its own branch, each waited for before the next.
      float bv[S::kFragN][S::kAccRegs];
      if constexpr (EPI == kEpiFused) {
        if (bias != nullptr) {
          uint16_t raw[S::kFragN][S::kAccRegs];
#pragma unroll
          for (int j = 0; j < S::kFragN; ++j)
#pragma unroll
            for (int g = 0; g < S::kAccRegs / 4; ++g)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                raw[j][4 * g + e] = bias[min(n0 + wn * S::kWaveN + lane_col(j, g) + e, N - 1)];
#pragma unroll
          for (int j = 0; j < S::kFragN; ++j)
#pragma unroll
            for (int r = 0; r < S::kAccRegs; ++r) bv[j][r] = widen_in<S::DTYPE>(raw[j][r]);
        } else {
#pragma unroll
          for (int j = 0; j < S::kFragN; ++j)
#pragma unroll
            for (int r = 0; r < S::kAccRegs; ++r) bv[j][r] = 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < S::kFragM; ++i) {
#pragma unroll
        for (int j = 0; j < S::kFragN; ++j) {
#pragma unroll
          for (int g = 0; g < S::kAccRegs / 4; ++g) {
            half4_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float v = acc[i][j][4 * g + e];
              if constexpr (EPI == kEpiFused) {
                // With no bias this adds +0: every value but -0 stays as it
                // is, and -0 becomes +0, as the exact sum (which starts at
                // +0) would be.
                v += bv[j][4 * g + e];
                if (relu) v = relu_act(v);
              }
              h[e] = round_out<S::DTYPE>(v);
            }
            const uint32_t off =
                stage_base + static_cast<uint32_t>((i * S::MI + frag_row) * S::kStagePitch + lane_col(j, g) * 2);
            *reinterpret_cast<half4_t *>(smem + off) = h;
          }
        }
      }
      constexpr int kRowChunks = S::kWaveN / 8;       // 16-byte chunks per tile row
      constexpr int kRowsPerPass = 64 / kRowChunks;   // rows one wave instruction covers
      static_assert(64 % kRowChunks == 0, "lanes per staged row");
      const int chunk = lane % kRowChunks;
      const int n = n0 + wn * S::kWaveN + chunk * 8;
#pragma unroll 4
      for (int r0 = 0; r0 < S::kWaveM; r0 += kRowsPerPass) {
        const int r = r0 + lane / kRowChunks;
        const half8_t v = *reinterpret_cast<const half8_t *>(smem + stage_base + r * S::kStagePitch + chunk * 16);
        const int m = m0 + wm * S::kWaveM + r;
        if (m < M) {
          _Float16 *dst = D + static_cast<int64_t>(m) * N + n;
          if (vec16 && n + 8 <= N) {
            // Non-temporal (streamed to memory, not kept in the caches): with
            // several tiles per CU, cached D lines would evict the A and B
            // panels the next tiles read (2 % faster at 8192^3, about 1.5 % at
            // 4096^3).  A kernel that reads D next finds it in memory.
            if constexpr (EPI == kEpiCachedStores)
              *reinterpret_cast<half8_t *>(dst) = v;
            else
              __builtin_nontemporal_store(v, reinterpret_cast<half8_t *>(dst));
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (n + e < N) dst[e] = v[e];
          }
        }
      }
    }
  }
  if constexpr (EPI == kEpiTimed) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
    workgroup_barrier();            // ... and every other wave's
    if (tid == 0) {
      const uint64_t t_end_r = __builtin_amdgcn_s_memrealtime();
      const uint64_t t_end_c = __builtin_amdgcn_s_memtime();
      uint64_t *st = stamps;
      st[4] = t_end_r;
      st[5] = t_end_c;
      st[6] = static_cast<uint32_t>(__builtin_amdgcn_s_getreg((31 << 11) | 4));   // HW_ID
      st[7] = static_cast<uint32_t>(__builtin_amdgcn_s_getreg((31 << 11) | 20));  // XCC_ID
    }
  }
}

// ---- instantiations ------------------------------------------------------
// Default: 256x256 output tile, K tiles of 64 (128-byte LDS rows, so every
// tile load is a whole 128-byte line), a two-stage 64 KiB-per-stage LDS ring,
// 2x2 waves of 128x128 made of 16x16x32 MFMA blocks (128 MFMA slots per K
// tile), the next K step's operand reads one every 2 slots, one refill load
// every 4 slots, swizzled LDS, persistent grouped scheduler, and the
// early-free K loop with its free barrier at slot 48 of K step 0 (ring.hpp:
// measured 1.5-3 % faster than one barrier per K tile at 4096^3 and 8192^3,
// 4 % at the maximum clock; the slot, 32..56, and the refill spacing, 3..5,
// made no difference beyond noise).  The 16x16x32 shape moves half the
// accumulator bytes per flop of 32x32x16 and runs at a measurably higher
// sustained clock under the power limit.  MFMAs go in serpentine order, so
// each shares an operand with the one before it: 0.3-0.7 % faster than
// row-major order on uniform data (4096^3, 8192^3, 4000x4032x4104), 0.3 % on
// zeros, where the clock is not power-limited.
using GemmDefault = GemmShape<256, 256, 64, 2, 2, 2, true, true, 4, 16, 2, 1, kF16, true, 48, true>;
// The default shape with bf16 operands and results.
using GemmBf16 = GemmShape<256, 256, 64, 2, 2, 2, true, true, 4, 16, 2, 1, kBF16, true, 48, true>;
// Ablations, each the default with one design choice taken back: no LDS
// swizzle; one workgroup per output tile in launch order (no persistent
// grouped, XCD-aware schedule); one barrier per K tile (the ring without the
// early free); 32x32x16 MFMA blocks through the compiler's builtin (64 slots
// per K tile, one operand read per slot, a refill load every 2 slots; four K
// steps per K tile, so the one-barrier ring); and that with a single LDS
// stage (load, wait, compute); MFMAs in row-major order.
using GemmNoSwizzle = GemmShape<256, 256, 64, 2, 2, 2, false, true, 4, 16, 2, 1, kF16, true, 48, true>;
using GemmNonPersistent = GemmShape<256, 256, 64, 2, 2, 2, true, false, 4, 16, 2, 1, kF16, true, 48, true>;
using GemmOneBarrier = GemmShape<256, 256, 64, 2, 2, 2, true, true, 4, 16, 2, 1, kF16, false, 0, true>;
using GemmRowMajorMfma = GemmShape<256, 256, 64, 2, 2, 2, true, true, 4, 16, 2, 1, kF16, true, 48, false>;
using Gemm32x32 = GemmShape<256, 256, 64, 2, 2, 2, true, true, 2>;
using Gemm32x32OneStage = GemmShape<256, 256, 64, 1, 2, 2, true, true, 1>;
// Smaller output tiles, for outputs whose 256x256 tiles would leave CUs
// idle (gemm_default_tile picks): the one-barrier schedule on 256x128,
// 128x256 and 128x128 tiles (4 waves of 128x64, 64x128 and 64x64; 12, 12 and
// 8 loads per wave per K tile), with the deeper rings of kGemmTileShapes.  A
// K tile of these is 1/2 or 1/4 of the 256x256 one in MFMA time, so two
// stages no longer cover a load's latency.
template <int DT, int STAGES = 2>
using GemmTile256x128 = GemmShape<256, 128, 64, STAGES, 2, 2, true, true, 4, 16, 2, 1, DT, false, 0, true>;
template <int DT, int STAGES = 2>
using GemmTile128x256 = GemmShape<128, 256, 64, STAGES, 2, 2, true, true, 4, 16, 2, 1, DT, false, 0, true>;
template <int DT, int STAGES = 2>
using GemmTile128x128 = GemmShape<128, 128, 64, STAGES, 2, 2, true, true, 4, 16, 2, 1, DT, false, 0, true>;
// A smaller tile, four waves stacked along M (32 rows by 64 columns each):
// 8 MFMAs per K step, so an operand read in every slot.
template <int DT, int STAGES = 4, int DMA_STRIDE = 2>
using GemmTile128x64 = GemmShape<128, 64, 64, STAGES, 4, 1, true, true, DMA_STRIDE, 16, 1, 1, DT, false, 0, true>;

static_assert(GemmDefault::BM == kGemmBM && GemmDefault::BN == kGemmBN && GemmDefault::BK == kGemmBK &&
                  GemmDefault::STAGES == kGemmStages && GemmDefault::kThreads == kGemmThreads,
              "kernels.hpp constants must describe the default kernel");

template <class S, int EPI = kEpiPlain>
static hipError_t launch(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                         hipStream_t stream, const void *bias = nullptr, int relu = 0, float *ws = nullptr,
                         int splits = 1) {
  const int tiles_m = (M + S::BM - 1) / S::BM;
  const int tiles_n = (N + S::BN - 1) / S::BN;
  const int64_t units = static_cast<int64_t>(tiles_m) * tiles_n * (EPI == kEpiPartial ? splits : 1);
  const int64_t grid = S::PERSISTENT ? (units < num_cus ? units : num_cus) : units;
  // Whole 16-byte row segments of D are 16-byte aligned when N % 8 == 0.
  const int vec16 = (N % 8 == 0) && (reinterpret_cast<uintptr_t>(D) % 16 == 0);
  hipLaunchKernelGGL((gemm_kernel<S, EPI>), dim3(static_cast<unsigned>(grid)), dim3(S::kThreads), 0, stream,
                     static_cast<const _Float16 *>(A), static_cast<const _Float16 *>(B), static_cast<_Float16 *>(D),
                     M, N, K, tiles_m, tiles_n, vec16, static_cast<const uint16_t *>(bias), relu, ws, splits);
  return hipGetLastError();
}

// The shape-dependent default: the tile gemm_default_tile picks, with the
// ring depth of kGemmTileShapes.
template <int DT, int EPI = kEpiPlain>
static hipError_t launch_default(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                                 hipStream_t stream, const void *bias = nullptr, int relu = 0, float *ws = nullptr,
                                 int splits = 1) {
  using Big = std::conditional_t<DT == kF16, GemmDefault, GemmBf16>;
  static_assert(Big::BM == kGemmTileShapes[kTile256x256].bm && Big::BN == kGemmTileShapes[kTile256x256].bn &&
                    Big::STAGES == kGemmTileShapes[kTile256x256].stages &&
                    GemmTile256x128<DT, kGemmTileShapes[kTile256x128].stages>::BN ==
                        kGemmTileShapes[kTile256x128].bn &&
                    GemmTile128x256<DT, kGemmTileShapes[kTile128x256].stages>::BM ==
                        kGemmTileShapes[kTile128x256].bm &&
                    GemmTile128x128<DT, kGemmTileShapes[kTile128x128].stages>::BM ==
                        kGemmTileShapes[kTile128x128].bm &&
                    GemmTile128x64<DT, kGemmTileShapes[kTile128x64].stages>::BN ==
                        kGemmTileShapes[kTile128x64].bn,
                "kGemmTileShapes must describe the kernels launched for each tile");
  switch (gemm_default_tile(M, N, num_cus, EPI == kEpiPartial ? kGemmSplitKTiles : kGemmTiles)) {
    case kTile256x128:
      return launch<GemmTile256x128<DT, kGemmTileShapes[kTile256x128].stages>, EPI>(A, B, D, M, N, K, num_cus, stream,
                                                                              bias, relu, ws, splits);
    case kTile128x256:
      return launch<GemmTile128x256<DT, kGemmTileShapes[kTile128x256].stages>, EPI>(A, B, D, M, N, K, num_cus, stream,
                                                                              bias, relu, ws, splits);
    case kTile128x128:
      return launch<GemmTile128x128<DT, kGemmTileShapes[kTile128x128].stages>, EPI>(A, B, D, M, N, K, num_cus, stream,
                                                                              bias, relu, ws, splits);
    case kTile128x64:
      if constexpr (EPI != kEpiPartial)
        return launch<GemmTile128x64<DT, kGemmTileShapes[kTile128x64].stages>, EPI>(A, B, D, M, N, K, num_cus, stream,
                                                                               bias, relu, ws, splits);
      return hipErrorInvalidValue;  // split K keeps to the first kGemmSplitKTiles tiles
    default: return launch<Big, EPI>(A, B, D, M, N, K, num_cus, stream, bias, relu, ws, splits);
  }
}

}  // namespace gt
