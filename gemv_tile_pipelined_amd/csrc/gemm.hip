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
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "ring.hpp"
#include "tile_order.hpp"

namespace gt {

template <int BM_, int BN_, int BK_, int STAGES_, int WAVES_M_, int WAVES_N_, bool SWIZZLE_, bool PERSISTENT_,
          int DMA_STRIDE_, int MI_ = 32, int READ_STRIDE_ = 1, int DMA_OFFSET_ = 0, int DTYPE_ = kF16>
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
template <class S, class Mfma, class Read, class Load>
struct KernelRingOps {
  Mfma mfma_fn;
  Read read_fn;
  Load load_fn;
  __device__ __attribute__((always_inline)) void mfma(int buf, int idx) { mfma_fn(buf, idx); }
  __device__ __attribute__((always_inline)) void read(int buf, int kt, int ks, int r) { read_fn(buf, kt, ks, r); }
  __device__ __attribute__((always_inline)) void load(int tile, int d) { load_fn(tile, d); }
  __device__ __attribute__((always_inline)) void wait_tile(int n) { wait_vmcnt_n<S::kDmaPerStage, S::STAGES - 2>(n); }
  __device__ __attribute__((always_inline)) void wait_lds() { __builtin_amdgcn_s_waitcnt(kWaitLgkm0); }
  __device__ __attribute__((always_inline)) void barrier() { workgroup_barrier(); }
  __device__ __attribute__((always_inline)) void fence() { __builtin_amdgcn_sched_barrier(0); }
};

// One wave per SIMD for 4 waves; with 8 waves two per SIMD, so each is held
// to half the register file.
// Epilogue modes.  kEpiPlain: round and store D.  kEpiFused: add bias[n]
// and apply ReLU when `relu` is set (gemm_bias_*), then round and store D.
// kEpiPartial (split K, gemm_splitk_*): the grid walks (tile, K slice) units,
// `splits` slices per tile; each unit sums only its slice of K tiles and
// stores the FP32 sums, unrounded, to ws[slice][m][n]; splitk_reduce_kernel
// adds the slices.  Each mode ignores the arguments of the others.
enum : int { kEpiPlain = 0, kEpiFused = 1, kEpiPartial = 2 };

template <class S, int EPI = kEpiPlain>
__global__ void __launch_bounds__(S::kThreads) __attribute__((amdgpu_waves_per_eu(S::kWaves / 4, S::kWaves / 4)))
gemm_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B, _Float16 *__restrict__ D,
                int M, int N, int K, int tiles_m, int tiles_n, int vec16, const uint16_t *__restrict__ bias,
                int relu, float *__restrict__ ws, int splits) {
  static_assert(EPI != kEpiPartial || (S::MI == 16 && S::STAGES >= 2), "split K uses the pipelined 16x16x32 loop");
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

    // Loads [first, last) of the kDmaPerStage per-wave DMA instructions of K
    // tile kt (A tile first, then B tile).
    // K tile kt of the loop reads K tile (kt + kofs) mod KT of the matrices;
    // the loop runs over KTu K tiles (all KT of them, or one K slice).
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
      int ka = kt + kofs;
      if (ka >= KT) ka -= KT;
      const int k0 = ka * S::BK;
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
    // order the row-major MFMA sequence below first needs them in.
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
#pragma unroll
    for (int i = 0; i < S::kFragM; ++i)
#pragma unroll
      for (int j = 0; j < S::kFragN; ++j)
#pragma unroll
        for (int e = 0; e < S::kAccRegs; ++e) acc[i][j][e] = 0.0f;
    if constexpr (S::MI == 16) {
      // The zeros above are written by VALU instructions and first read by a
      // hand-written MFMA, which the compiler's hazard padding does not know
      // about.  These statements take every accumulator as input and output
      // and carry wait states: the zeros are materialised before them (and
      // cannot be re-created after them), so they precede every MFMA by at
      // least 16 wait states.
      static_assert(S::kFragN % 4 == 0, "accumulator fence covers 4 blocks per statement");
#pragma unroll
      for (int i = 0; i < S::kFragM; ++i)
#pragma unroll
        for (int j = 0; j < S::kFragN; j += 4)
          asm volatile("s_nop 1" : "+a"(acc[i][j]), "+a"(acc[i][j + 1]), "+a"(acc[i][j + 2]), "+a"(acc[i][j + 3]));
    }

    auto mfma = [&](int buf, int idx) {
      const int i = idx / S::kFragN;
      const int j = idx % S::kFragN;
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
      KernelRingOps<S, decltype(mfma), decltype(read_frag), decltype(load_one)> ops{mfma, read_frag, load_one};
      ring_k_loop<S>(ops, KTu);
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
      float bv[S::kFragN][S::kAccRegs];
      if constexpr (EPI == kEpiFused) {
#pragma unroll
        for (int j = 0; j < S::kFragN; ++j)
#pragma unroll
          for (int g = 0; g < S::kAccRegs / 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int n = min(n0 + wn * S::kWaveN + lane_col(j, g) + e, N - 1);
              bv[j][4 * g + e] = bias ? widen_in<S::DTYPE>(bias[n]) : 0.0f;
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
}

// ---- instantiations ------------------------------------------------------
// Default: 256x256 output tile, K tiles of 64 (128-byte LDS rows, so every
// tile load is a whole 128-byte line), a two-stage 64 KiB-per-stage LDS ring,
// 2x2 waves of 128x128 made of 16x16x32 MFMA blocks (128 MFMA slots per K
// tile), the next K step's operand reads one every 2 slots, one refill load
// every 4 slots (offset by one slot from the reads), swizzled LDS, persistent
// grouped scheduler.  The 16x16x32 shape moves half the accumulator bytes
// per flop of 32x32x16 and runs at a measurably higher sustained clock under
// the power limit.  The others exist for ablation measurements.
using GemmDefault = GemmShape<256, 256, 64, 2, 2, 2, true, true, 4, 16, 2, 1>;
// The default shape with bf16 operands and results.
using GemmBf16 = GemmShape<256, 256, 64, 2, 2, 2, true, true, 4, 16, 2, 1, kBF16>;
// Ablations, each the default with one design choice taken back: no LDS
// swizzle; one workgroup per output tile in launch order (no persistent
// grouped, XCD-aware schedule); 32x32x16 MFMA blocks through the compiler's
// builtin (64 slots per K tile, one operand read per slot, a refill load
// every 2 slots); and the same with a single LDS stage (load, wait, compute).
using GemmNoSwizzle = GemmShape<256, 256, 64, 2, 2, 2, false, true, 4, 16, 2, 1>;
using GemmNonPersistent = GemmShape<256, 256, 64, 2, 2, 2, true, false, 4, 16, 2, 1>;
using Gemm32x32 = GemmShape<256, 256, 64, 2, 2, 2, true, true, 2>;
using Gemm32x32OneStage = GemmShape<256, 256, 64, 1, 2, 2, true, true, 1>;
// Smaller output tiles, for outputs whose 256x256 tiles would leave CUs
// idle (gemm_default_tile picks): the default's schedule on 256x128, 128x256
// and 128x128 tiles (4 waves of 128x64, 64x128 and 64x64; 12, 12 and 8 loads
// per wave per K tile), with the deeper rings of kGemmTileShapes.  A K tile
// of these is 1/2 or 1/4 of the 256x256 one in MFMA time, so two stages no
// longer cover a load's latency.
template <int DT, int STAGES = 2>
using GemmTile256x128 = GemmShape<256, 128, 64, STAGES, 2, 2, true, true, 4, 16, 2, 1, DT>;
template <int DT, int STAGES = 2>
using GemmTile128x256 = GemmShape<128, 256, 64, STAGES, 2, 2, true, true, 4, 16, 2, 1, DT>;
template <int DT, int STAGES = 2>
using GemmTile128x128 = GemmShape<128, 128, 64, STAGES, 2, 2, true, true, 4, 16, 2, 1, DT>;

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
                        kGemmTileShapes[kTile128x128].bm,
                "kGemmTileShapes must describe the kernels launched for each tile");
  switch (gemm_default_tile(M, N, num_cus)) {
    case kTile256x128:
      return launch<GemmTile256x128<DT, kGemmTileShapes[kTile256x128].stages>, EPI>(A, B, D, M, N, K, num_cus, stream,
                                                                              bias, relu, ws, splits);
    case kTile128x256:
      return launch<GemmTile128x256<DT, kGemmTileShapes[kTile128x256].stages>, EPI>(A, B, D, M, N, K, num_cus, stream,
                                                                              bias, relu, ws, splits);
    case kTile128x128:
      return launch<GemmTile128x128<DT, kGemmTileShapes[kTile128x128].stages>, EPI>(A, B, D, M, N, K, num_cus, stream,
                                                                              bias, relu, ws, splits);
    default: return launch<Big, EPI>(A, B, D, M, N, K, num_cus, stream, bias, relu, ws, splits);
  }
}

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
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_bf16(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                            hipStream_t stream) {
  return launch_default<kBF16>(A, B, D, M, N, K, num_cus, stream);
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
  void mfma(int buf, int idx) { push(kRingMfma, buf, idx); }
  void read(int buf, int kt, int ks, int r) { push(kRingRead, kt, ks, r, ring_stage(kt, stages)); }
  void load(int tile, int d) { push(kRingLoad, tile, d, ring_stage(tile, stages)); }
  void wait_tile(int vmcnt) { push(kRingWaitTile, vmcnt); }
  void wait_lds() { push(kRingWaitLds); }
  void barrier() { push(kRingBarrier); }
  void fence() {}
};

template <class S>
int64_t record_ring(int ktu, int32_t *events, int64_t cap) {
  RingRecorder rec{S::STAGES, events, cap};
  ring_k_loop<S>(rec, ktu);
  return rec.n;
}
}  // namespace

int64_t ring_trace(int bm, int bn, int stages, int ktu, int32_t *events, int64_t cap, int *loads_per_tile,
                   int *reads_per_step, int *ksteps, int *mfma_per_step) {
  auto info = [&](auto shape) {
    using S = decltype(shape);
    if (loads_per_tile) *loads_per_tile = S::kDmaPerStage;
    if (reads_per_step) *reads_per_step = S::kReads;
    if (ksteps) *ksteps = S::kKSub;
    if (mfma_per_step) *mfma_per_step = S::kMfma;
    return record_ring<S>(ktu, events, cap);
  };
  if (bm == 256 && bn == 256 && stages == 2) return info(GemmDefault{});
  if (bm == 256 && bn == 128 && stages == 2) return info(GemmTile256x128<kF16, 2>{});
  if (bm == 256 && bn == 128 && stages == 3) return info(GemmTile256x128<kF16, 3>{});
  if (bm == 128 && bn == 256 && stages == 2) return info(GemmTile128x256<kF16, 2>{});
  if (bm == 128 && bn == 256 && stages == 3) return info(GemmTile128x256<kF16, 3>{});
  if (bm == 128 && bn == 128 && stages == 2) return info(GemmTile128x128<kF16, 2>{});
  if (bm == 128 && bn == 128 && stages == 4) return info(GemmTile128x128<kF16, 4>{});
  if (bm == 128 && bn == 128 && stages == 5) return info(GemmTile128x128<kF16, 5>{});
  return -1;
}

}  // namespace gt
