// skinny.hip -- FP16 / BF16 GEMM with one side of at most 16 rows, for gfx950:
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
//  * The WAVES waves of a workgroup split the K steps.  Their 16x16 partial
//    sums meet in LDS and are added in wave order, so every output is
//    deterministic.
//  * Two ways to feed the MFMAs: straight into registers (each wave keeps
//    UNROLL pairs of loads in flight; one load instruction touches 16 rows x
//    64 bytes), or -- the default -- through an LDS ring filled by
//    direct-to-LDS loads of 1 KiB each, one to four whole row segments
//    (gemm_skinny_lds_kernel below).  On 8x4096x14336 the ring takes 23 us against 30 us, because
//    the register form re-reads the small operand in 64-byte pieces from
//    every workgroup.
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

// LDS-staged variant: both operands go through a STAGES-deep LDS ring of K
// tiles of BK = 512 (1 KiB per row), 256 or 128, filled by direct-to-LDS
// loads in which one wave instruction moves 1 KiB: one row segment, or two
// at BK = 256 (the register variant above touches 16 rows x
// 64 bytes per instruction, and every workgroup re-reads the small operand
// that way), or four at BK = 128.  A workgroup owns PR rows of P (48 or 64
// at BK = 128, 32 at BK = 256 or 16 by default;
// 8, 4, 2 or 1 when R is too small to give every CU a workgroup of 16 -- the
// page's "enough blocks" again, here without splitting K, since every
// workgroup re-reading the small Q costs only cache traffic).
// A stage holds the PR rows of P and QROWS rows of Q (rows past R or S and K
// past K read as zero: the buffer descriptors' ranges and an out-of-range
// offset).  The MFMA's 16 P lanes read P row (lane % PR) and its 16 Q lanes
// Q row (lane % QROWS): rows re-read that way only reach outputs that are
// never stored.  QROWS = 8 (for S <= 8) halves the Q traffic.  The load
// instructions of a stage's PR + QROWS rows are spread over the waves;
// spare slots load zeros (out-of-range offset, no memory access) into a
// junk KiB so every wave issues the same number of loads and the vmcnt
// accounting stays uniform.  With PR = 32, 48 or 64 the P rows form two,
// three or four 16-row MFMA blocks.  Each wave computes
// BK/32/WAVES of the stage's K steps.  LDS chunk c of row r holds logical
// chunk c ^ s(r) with s(r) = 2*(r % 8) + (r / 8) (the loader picks the global
// chunk per lane to make it so), and the four lane groups of a K step read
// chunks 0, 2, 1, 3 of the step: lanes l and l + 32, which the LDS serves
// together, then read chunks an odd XOR apart and every read is bank-conflict
// free (lanes that re-read a row read the same address, a broadcast; rows
// of 512 bytes or 1 KiB both start at bank 0, so the argument holds for
// either K tile).  With the grid's y dimension above 1, workgroup (x, y)
// stages Q rows [16y, 16y + 16) (the small-side split).
//
// With SPLIT, K is split across workgroups as well: the grid holds `splits`
// workgroups per block of PR rows (row-block major, so that workgroups side
// by side read different K ranges of Q), workgroup slice j walks only the K
// tiles [j*per, min(KT, (j+1)*per)) with per = ceil(KT / splits) (the host
// keeps every slice non-empty), and its sums go unrounded to
// ws[j][output index] for the ordered reduction kernel.  More workgroups of
// 16 P rows, instead of fewer P rows per workgroup, keep the number of times
// Q is read from the caches at ceil(R / 16).
template <int WAVES, int STAGES, int QROWS, bool TRANS, int DT = kF16, int PR = 16, int KROT = 0, bool NTP = false,
          bool SPLIT = false, int BK = 512>
__global__ void __launch_bounds__(WAVES * 64)
gemm_skinny_lds_kernel(const _Float16 *__restrict__ P, const _Float16 *__restrict__ Q, _Float16 *__restrict__ D,
                       int R, int S, int K, float *__restrict__ ws, int splits) {
  static_assert(BK == 512 || BK == 256 || BK == 128, "K tile");
  constexpr int kRowBytes = BK * 2;                              // one row of a stage
  constexpr int kChunks = BK / 8;                                // 16-byte chunks per row
  constexpr int kRowsPerLoad = 1024 / kRowBytes;                 // rows per 1 KiB wave instruction
  constexpr int kLoads = PR + QROWS;                             // rows per stage
  constexpr int kInstr = (kLoads + kRowsPerLoad - 1) / kRowsPerLoad;  // wave instructions per stage
  constexpr int kDmaPerWave = (kInstr + WAVES - 1) / WAVES;      // per wave per stage
  constexpr bool kJunk = kDmaPerWave * WAVES > kInstr;           // spare slots -> junk KiB kInstr
  constexpr int kTileBytes = PR * kRowBytes;                     // the P rows, then the Q rows
  constexpr int kStageBytes = (kInstr + (kJunk ? 1 : 0)) * 1024;
  static_assert(PR % kRowsPerLoad == 0, "an instruction's rows belong to one operand");
  constexpr int kSteps = BK / 32;                                // 32-wide K steps per stage
  constexpr int kStepsPerWave = kSteps / WAVES;
  static_assert(QROWS == 8 || QROWS == 16 || QROWS == 32 || QROWS == 64, "Q tile rows");
  constexpr int QB = QROWS >= 32 ? QROWS / 16 : 1;  // 16-row blocks of Q (each its own MFMA)
  constexpr int PB = PR > 16 ? PR / 16 : 1;         // 16-row blocks of P
  constexpr int kPRows = 16 * PB;                   // P rows of the partial sums
  // With 64 Q rows the ring takes (nearly) all of the LDS: the wave partial
  // sums then reuse the ring once the K loop is done with it.
  constexpr bool kAliasPartial = QROWS == 64;
  constexpr int kPartialBytes = WAVES * 16 * QB * (kPRows + 1) * 4;
  static_assert(PR == 1 || PR == 2 || PR == 4 || PR == 8 || PR == 16 || PR == 32 || PR == 48 || PR == 64,
                "P rows per workgroup");
  static_assert(kSteps % WAVES == 0, "work split");
  static_assert(STAGES >= 2 && (STAGES - 1) * kDmaPerWave <= 63, "vmcnt range");
  static_assert(STAGES * kStageBytes + (kAliasPartial ? 0 : kPartialBytes) <= 160 * 1024,
                "gfx950 has 160 KiB of LDS per CU");
  static_assert(!kAliasPartial || kPartialBytes <= STAGES * kStageBytes, "partial sums fit the ring");
  __shared__ __attribute__((aligned(1024))) char ring[STAGES * kStageBytes + (kAliasPartial ? 0 : kPartialBytes)];
  auto partial =
      reinterpret_cast<float (*)[16 * QB][kPRows + 1]>(ring + (kAliasPartial ? 0 : STAGES * kStageBytes));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KT = (K + BK - 1) / BK;
  // This workgroup's rows and K tiles [kbeg, kbeg + nkt).
  int rb = static_cast<int>(blockIdx.x), slice = 0, kbeg = 0, nkt = KT;
  if constexpr (SPLIT) {
    rb = static_cast<int>(blockIdx.x / static_cast<unsigned>(splits));
    slice = static_cast<int>(blockIdx.x % static_cast<unsigned>(splits));
    const int per = (KT + splits - 1) / splits;
    kbeg = slice * per;
    nkt = min(per, KT - kbeg);
  }
  const int r0 = rb * PR;
  const int prows = min(PR, R - r0);
  // With the small side split over the grid's y dimension, this workgroup
  // stages Q rows [q0, q0 + QROWS) (q0 = 0 with one Q block).
  const int q0 = static_cast<int>(blockIdx.y) * QROWS;
  const int4_t rsrc_p = make_buffer_rsrc(P + static_cast<int64_t>(r0) * K, static_cast<uint32_t>(prows) * K * 2u);
  const int4_t rsrc_q =
      make_buffer_rsrc(Q + static_cast<int64_t>(q0) * K, static_cast<uint32_t>(S - q0) * K * 2u);
  const uint32_t ring0 = lds_addr(ring);
  // With KROT, workgroup b walks its K tiles from tile j % nkt and wraps, so
  // the workgroups running at one moment read different K ranges: j = b
  // (KROT 1), or j = b / 8, its index within its XCD (KROT 2; workgroups are
  // dispatched to the 8 XCDs in turn), so the workgroups sharing one L2 all
  // start at different K tiles (with j = b they take only two starts per XCD
  // when there are 16 K tiles).
  const int kt0 = KROT == 1   ? static_cast<int>(blockIdx.x % static_cast<unsigned>(nkt))
                  : KROT == 2 ? static_cast<int>((blockIdx.x >> 3) % static_cast<unsigned>(nkt))
                              : 0;
  static_assert(KROT >= 0 && KROT <= 2, "K start rotation mode");
  auto swz = [](int r) { return ((r & 7) << 1) | ((r >> 3) & 1); };

  // Row loads of K tile kt: load d of this wave is the stage's 1 KiB
  // instruction t = d*WAVES + wave, which moves stage rows
  // t*kRowsPerLoad .. +kRowsPerLoad-1 (P rows 0..PR-1, then Q rows
  // 0..QROWS-1; rows past kLoads, and instructions t >= kInstr into the junk
  // KiB, load zeros).
  auto issue = [&](int kt) {
    const uint32_t stage = ring0 + static_cast<uint32_t>((kt % STAGES) * kStageBytes);
    const int ktile = kbeg + (kt + kt0 < nkt ? kt + kt0 : kt + kt0 - nkt);  // the K tile this ring slot holds
#pragma unroll
    for (int d = 0; d < kDmaPerWave; ++d) {
      const int t = d * WAVES + wave;
      const bool junk = kJunk && t >= kInstr;
      const int t0 = t * kRowsPerLoad;                        // the instruction's first stage row
      const int tr = t0 + (kRowsPerLoad > 1 ? lane / kChunks : 0);  // this lane's stage row
      const int row = tr < PR ? tr : tr - PR;                 // row within its operand
      const int k = ktile * BK + (((lane % kChunks) ^ swz(row & 15)) << 3);  // first K element this lane fetches
      const uint32_t off = (k < K && !junk && tr < kLoads)
                               ? static_cast<uint32_t>(row) * K * 2u + static_cast<uint32_t>(k) * 2u
                               : kOobOffset;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(stage + static_cast<uint32_t>(min(t, kInstr) * 1024));
      // With NTP the rows of P, read once, are loaded non-temporally.
      if (NTP && t0 < PR)
        lds_dma_b128<2>(rsrc_p, off, dst);
      else
        lds_dma_b128(t0 < PR ? rsrc_p : rsrc_q, off, dst);
    }
  };

  const int frow = lane & 15;
  const int kgrp = lane >> 4;
  const int kperm = ((kgrp & 1) << 1) | (kgrp >> 1);
  const int prow = frow % (PR < 16 ? PR : 16);  // P row of this lane's fragment in P block 0
  const uint32_t frag_off = static_cast<uint32_t>(prow * kRowBytes);
  const int fswz = swz(prow);
  const int qrow = frow % (QROWS < 16 ? QROWS : 16);  // Q row of this lane's fragment in Q block 0
  const uint32_t qfrag_off = static_cast<uint32_t>(kTileBytes + qrow * kRowBytes);
  const int qswz = swz(qrow);  // also that of the same row of the other Q block (the swizzle repeats every 16 rows)

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nkt) issue(s);

  float4_t acc[PB][QB];
#pragma unroll
  for (int a = 0; a < PB; ++a)
#pragma unroll
    for (int b = 0; b < QB; ++b) acc[a][b] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int kt = 0; kt < nkt; ++kt) {
    // Tile kt has landed once at most `younger` tiles' loads are pending.
    // Loads complete in issue order, so waiting until at most
    // younger*kDmaPerWave are pending leaves only the younger tiles in flight.
    wait_younger<kDmaPerWave, STAGES - 2>(min(nkt, kt + STAGES - 1) - (kt + 1));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    workgroup_barrier();  // tile kt complete for everyone; tile kt-1 no longer read
    if (kt + STAGES - 1 < nkt) issue(kt + STAGES - 1);
    const char *stage = ring + (kt % STAGES) * kStageBytes;
#pragma unroll
    for (int j = 0; j < kStepsPerWave; ++j) {
      const int step = wave * kStepsPerWave + j;
      const int c = step * 4 + kperm;  // logical chunk
      half8_t pf[PB];
#pragma unroll
      for (int a = 0; a < PB; ++a)
        pf[a] = *reinterpret_cast<const half8_t *>(stage + frag_off + a * 16 * kRowBytes + ((c ^ fswz) << 4));
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const half8_t qf =
            *reinterpret_cast<const half8_t *>(stage + qfrag_off + b * 16 * kRowBytes + ((c ^ qswz) << 4));
#pragma unroll
        for (int a = 0; a < PB; ++a) {
          if constexpr (DT == kF16)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[a], qf, acc[a][b], 0, 0, 0);
          else
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, pf[a]), __builtin_bit_cast(bf16x8_t, qf), acc[a][b], 0, 0, 0);
        }
      }
    }
  }

  // Every wave's reads of the ring are done (and no load into it is in
  // flight: the last tile was waited for) before the partials overwrite it.
  if constexpr (kAliasPartial) __syncthreads();
#pragma unroll
  for (int a = 0; a < PB; ++a)
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) partial[wave][16 * b + frow][16 * a + 4 * kgrp + e] = acc[a][b][e];
  __syncthreads();
  // 16*QB x kPRows outputs (Q row s, P row r), each the wave partials in wave order.
  for (int i = threadIdx.x; i < 16 * QB * kPRows; i += WAVES * 64) {
    const int s = i / kPRows;
    const int r = i % kPRows;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += partial[w][s][r];
    const int sg = q0 + s;  // row of Q (column of D when TRANS)
    if (s < QROWS && sg < S && r < PR && r0 + r < R) {
      const int64_t idx = TRANS ? static_cast<int64_t>(r0 + r) * S + sg : static_cast<int64_t>(sg) * R + r0 + r;
      if constexpr (SPLIT)
        ws[static_cast<int64_t>(slice) * R * S + idx] = sum;
      else
        D[idx] = round_out<DT>(sum);
    }
  }
}

// ceil(R / PR) workgroups along x; with qblocks > 1 the small side is split
// into blocks of QROWS rows along y.
template <int WAVES, int STAGES, int QROWS, int DT = kF16, int PR = 16, int KROT = 0, bool NTP = false,
          int BK = 512>
static hipError_t launch_lds(const void *P, const void *Q, void *D, int R, int S, int K, bool trans,
                             hipStream_t stream, int qblocks = 1) {
  const dim3 grid(static_cast<unsigned>((R + PR - 1) / PR), static_cast<unsigned>(qblocks));
  const auto *p = static_cast<const _Float16 *>(P);
  const auto *q = static_cast<const _Float16 *>(Q);
  auto *d = static_cast<_Float16 *>(D);
  float *no_ws = nullptr;
  if (trans)
    hipLaunchKernelGGL((gemm_skinny_lds_kernel<WAVES, STAGES, QROWS, true, DT, PR, KROT, NTP, false, BK>), grid,
                       dim3(WAVES * 64), 0, stream, p, q, d, R, S, K, no_ws, 1);
  else
    hipLaunchKernelGGL((gemm_skinny_lds_kernel<WAVES, STAGES, QROWS, false, DT, PR, KROT, NTP, false, BK>), grid,
                       dim3(WAVES * 64), 0, stream, p, q, d, R, S, K, no_ws, 1);
  return hipGetLastError();
}

// Split-K form: ceil(R / 16) x splits workgroups of 16 P rows write FP32
// partial sums to ws [splits][M*N]; the ordered reduction then rounds D.
template <int WAVES, int STAGES, int QROWS, int DT>
static hipError_t launch_lds_split(const void *P, const void *Q, void *D, int R, int S, int K, bool trans, float *ws,
                                   int splits, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((R + 15) / 16 * splits));
  const auto *p = static_cast<const _Float16 *>(P);
  const auto *q = static_cast<const _Float16 *>(Q);
  auto *d = static_cast<_Float16 *>(D);
  if (trans)
    hipLaunchKernelGGL((gemm_skinny_lds_kernel<WAVES, STAGES, QROWS, true, DT, 16, false, true, true>), grid,
                       dim3(WAVES * 64), 0, stream, p, q, d, R, S, K, ws, splits);
  else
    hipLaunchKernelGGL((gemm_skinny_lds_kernel<WAVES, STAGES, QROWS, false, DT, 16, false, true, true>), grid,
                       dim3(WAVES * 64), 0, stream, p, q, d, R, S, K, ws, splits);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(DT, ws, D, static_cast<int64_t>(R) * S, splits, stream);
}

hipError_t launch_gemm_skinny_splitk(int dtype, const void *A, const void *B, void *D, int M, int N, int K, void *ws,
                                     int splits, hipStream_t stream) {
  const bool small_m = M <= kSkinnyMaxRows;
  if (!small_m && N > kSkinnyMaxRows) return hipErrorInvalidValue;
  const void *P = small_m ? B : A;
  const void *Q = small_m ? A : B;
  const int R = small_m ? N : M;
  const int S = small_m ? M : N;
  float *w = static_cast<float *>(ws);
  if (dtype == kBF16)
    return S <= 8 ? launch_lds_split<8, 4, 8, kBF16>(P, Q, D, R, S, K, !small_m, w, splits, stream)
                  : launch_lds_split<16, 4, 16, kBF16>(P, Q, D, R, S, K, !small_m, w, splits, stream);
  return S <= 8 ? launch_lds_split<8, 4, 8, kF16>(P, Q, D, R, S, K, !small_m, w, splits, stream)
                : launch_lds_split<16, 4, 16, kF16>(P, Q, D, R, S, K, !small_m, w, splits, stream);
}

// The small side in ceil(S / 16) blocks of 16 rows along the grid's y
// dimension, each workgroup staging one block against PR rows of P (the
// launches of the S <= 16 case), PR from skinny_qsplit_rows.
template <int DT>
static hipError_t launch_lds_qsplit(const void *P, const void *Q, void *D, int R, int S, int K, bool trans,
                                    int num_cus, hipStream_t stream) {
  const int qb = (S + 15) / 16;
  switch (skinny_qsplit_rows(R, S, num_cus)) {
    case 16:
      if (K < kSkinnyStreamMinK)
        return launch_lds<16, 4, 16, DT, 16, kSkinnyRotateXcd>(P, Q, D, R, S, K, trans, stream, qb);
      return launch_lds<16, 4, 16, DT, 16, kSkinnyRotateXcd, true>(P, Q, D, R, S, K, trans, stream, qb);
    case 8: return launch_lds<8, 4, 16, DT, 8, kSkinnyRotateXcd>(P, Q, D, R, S, K, trans, stream, qb);
    case 4: return launch_lds<4, 4, 16, DT, 4>(P, Q, D, R, S, K, trans, stream, qb);
    case 2: return launch_lds<4, 4, 16, DT, 2>(P, Q, D, R, S, K, trans, stream, qb);
    default: return launch_lds<4, 4, 16, DT, 1>(P, Q, D, R, S, K, trans, stream, qb);
  }
}

// The default launch (skinny_default_rows): 32, 48 or 64 P rows per
// workgroup, in K tiles of 256 or 128, while R gives every CU 32 rows; else
// 16 P rows: with 16 waves, a 4-stage ring of K tiles of 512 and cached P
// loads below K = kSkinnyStreamMinK, and with 8 waves, a 6-stage ring of K
// tiles of 256 and non-temporal P loads from there up; else 8, 4, 2 or 1 P
// rows, staging 8 Q rows when S <= 8
// (and loading P non-temporally at 8 rows with 8 Q rows; at fewer rows that
// measured slower).  Launches of 32, 16 or 8 P rows start each workgroup's
// K walk at its index within its XCD (KROT 2, kSkinnyRotateXcd): without
// it, rows whose length is a multiple of 8 KiB (K % 4096 == 0) read 17-22 %
// slower, as every workgroup sharing an L2 then reads the same offset of
// its rows at once.  With 17..32 staged Q rows at 16 P rows the rotation is
// taken only for such rows (elsewhere it measured 5 % slower); with 4 or
// fewer P rows never (4-10 % slower: every workgroup re-reads the same Q
// lines, best all at once).  17..64 small-side rows against few P rows take
// the small-side split (skinny_qsplit).
template <int DT>
static hipError_t launch_lds_auto(const void *P, const void *Q, void *D, int R, int S, int K, bool trans,
                                  int num_cus, hipStream_t stream) {
  if (skinny_qsplit(R, S, num_cus)) return launch_lds_qsplit<DT>(P, Q, D, R, S, K, trans, num_cus, stream);
  const int pr = skinny_default_rows(R, num_cus);
  if (pr > 32) {
    // 48 or 64 P rows (three or four 16-row MFMA blocks) in K tiles of 128
    // (256-byte rows, four to a load instruction), 4 waves, a 4-stage ring of
    // (PR + Q rows) x 256 bytes.
    if (S > 32)
      return pr == 48 ? launch_lds<4, 4, 64, DT, 48, kSkinnyRotateXcd, true, 128>(P, Q, D, R, S, K, trans, stream)
                      : launch_lds<4, 4, 64, DT, 64, kSkinnyRotateXcd, true, 128>(P, Q, D, R, S, K, trans, stream);
    if (S > kSkinnyMaxRows)
      return pr == 48 ? launch_lds<4, 4, 32, DT, 48, kSkinnyRotateXcd, true, 128>(P, Q, D, R, S, K, trans, stream)
                      : launch_lds<4, 4, 32, DT, 64, kSkinnyRotateXcd, true, 128>(P, Q, D, R, S, K, trans, stream);
    return pr == 48 ? launch_lds<4, 4, 16, DT, 48, kSkinnyRotateXcd, true, 128>(P, Q, D, R, S, K, trans, stream)
                    : launch_lds<4, 4, 16, DT, 64, kSkinnyRotateXcd, true, 128>(P, Q, D, R, S, K, trans, stream);
  }
  if (pr == 32) {
    // 32 P rows per workgroup (two 16-row MFMA blocks) in K tiles of 256
    // (512-byte rows, two to a load instruction), so the ring holds 3 or 4
    // stages of (32 + Q rows) x 512 bytes: each workgroup reads the staged
    // Q rows once per 32 P rows.
    if (S > 32) return launch_lds<8, 3, 64, DT, 32, kSkinnyRotateXcd, true, 256>(P, Q, D, R, S, K, trans, stream);
    if (S > kSkinnyMaxRows)
      return launch_lds<4, 4, 32, DT, 32, kSkinnyRotateXcd, true, 256>(P, Q, D, R, S, K, trans, stream);
    return launch_lds<8, 4, 16, DT, 32, kSkinnyRotateXcd, true, 256>(P, Q, D, R, S, K, trans, stream);
  }
  if (S > 32) {
    // 33..64 small-side rows at 16 or 8 P rows per workgroup (fewer take the
    // split): 64 staged Q rows, 8 waves (1-4 % ahead of 4, 16 waves 5-17 %
    // behind), a 2-stage ring of (PR + 64) KiB stages, the partial sums
    // reusing the ring.
    return pr == 16 ? launch_lds<8, 2, 64, DT, 16, kSkinnyRotateXcd, true>(P, Q, D, R, S, K, trans, stream)
                    : launch_lds<8, 2, 64, DT, 8, kSkinnyRotateXcd, true>(P, Q, D, R, S, K, trans, stream);
  }
  if (S > kSkinnyMaxRows) {
    // 17..32 small-side rows at 16 P rows per workgroup (fewer take the
    // split): 32 staged Q rows, 4 waves, a 3-stage ring of (16 + 32) KiB
    // stages.
    const bool rot = K % 4096 == 0;
    return rot ? launch_lds<4, 3, 32, DT, 16, kSkinnyRotateXcd, true>(P, Q, D, R, S, K, trans, stream)
               : launch_lds<4, 3, 32, DT, 16, 0, true>(P, Q, D, R, S, K, trans, stream);
  }
  const bool q8 = S <= 8;
  switch (pr) {
    case 16:
      if (K < kSkinnyStreamMinK) return launch_lds<16, 4, 16, DT, 16, kSkinnyRotateXcd>(P, Q, D, R, S, K, trans, stream);
      // from K = 8192: K tiles of 256, 8 waves, a 6-stage ring of 16 KiB
      // (8x4096x14336 19.27 -> 18.93 us, 8x4096x8192 12.39 -> 11.65 us
      // against 16 waves and 4 stages of 512)
      return launch_lds<8, 6, 16, DT, 16, kSkinnyRotateXcd, true, 256>(P, Q, D, R, S, K, trans, stream);
    case 8: return q8 ? launch_lds<8, 4, 8, DT, 8, kSkinnyRotateXcd, true>(P, Q, D, R, S, K, trans, stream)
                      : launch_lds<8, 4, 16, DT, 8, kSkinnyRotateXcd>(P, Q, D, R, S, K, trans, stream);
    case 4: return q8 ? launch_lds<4, 4, 8, DT, 4>(P, Q, D, R, S, K, trans, stream)
                      : launch_lds<4, 4, 16, DT, 4>(P, Q, D, R, S, K, trans, stream);
    case 2: return q8 ? launch_lds<4, 4, 8, DT, 2>(P, Q, D, R, S, K, trans, stream)
                      : launch_lds<4, 4, 16, DT, 2>(P, Q, D, R, S, K, trans, stream);
    default: return q8 ? launch_lds<4, 4, 8, DT, 1>(P, Q, D, R, S, K, trans, stream)
                       : launch_lds<4, 4, 16, DT, 1>(P, Q, D, R, S, K, trans, stream);
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

// Which operand is the small side Q: A when M <= 16, else B when N <= 16;
// with `wide` (the default launch only), shapes whose smaller side has
// 17..64 rows take that side.  Returns false for shapes it does not cover.
static bool skinny_small_m(int M, int N, bool wide, bool *small_m) {
  if (M <= kSkinnyMaxRows) {
    *small_m = true;
  } else if (N <= kSkinnyMaxRows) {
    *small_m = false;
  } else if (wide && (M < N ? M : N) <= kSkinnyWideRows) {
    *small_m = M <= N;
  } else {
    return false;
  }
  return true;
}

hipError_t launch_gemm_skinny_f16(int variant, const void *A, const void *B, void *D, int M, int N, int K,
                                  int num_cus, hipStream_t stream) {
  // The small side is Q.  Q = A, P = B, D = Q·Pᵀ when the small side is M;
  // otherwise Q = B, P = A, D = P·Qᵀ.
  bool small_m = false;
  if (!skinny_small_m(M, N, variant == 0 || variant == 60, &small_m)) return hipErrorInvalidValue;
  const void *P = small_m ? B : A;
  const void *Q = small_m ? A : B;
  const int R = small_m ? N : M;
  const int S = small_m ? M : N;
  // Numbers of launch shapes measured and not kept are not reused.
  switch (variant) {
    case 0: return launch_lds_auto<kF16>(P, Q, D, R, S, K, !small_m, num_cus, stream);
    // operands loaded into registers: <waves per workgroup, K steps in flight per wave>
    case 4: return launch<8, 4>(P, Q, D, R, S, K, !small_m, stream);
    // LDS ring, 16 P rows per workgroup: <waves, stages, Q rows, type, P rows, K start rotation (1: by
    // workgroup index)>
    case 12: return launch_lds<16, 4, 16, kF16, 16>(P, Q, D, R, S, K, !small_m, stream);
    case 30: return launch_lds<16, 4, 16, kF16, 16, true>(P, Q, D, R, S, K, !small_m, stream);
    // as 30 with non-temporal loads of P (the default at 16 P rows)
    case 47: return launch_lds<16, 4, 16, kF16, 16, true, true>(P, Q, D, R, S, K, !small_m, stream);
    // as 47 without the rotated K start
    case 52: return launch_lds<16, 4, 16, kF16, 16, false, true>(P, Q, D, R, S, K, !small_m, stream);
    // the small side in 16-row blocks along the grid's y dimension, whatever the shape
    case 60: return launch_lds_qsplit<kF16>(P, Q, D, R, S, K, !small_m, num_cus, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_skinny_bf16(const void *A, const void *B, void *D, int M, int N, int K, int num_cus,
                                   hipStream_t stream) {
  bool small_m = false;
  if (!skinny_small_m(M, N, true, &small_m)) return hipErrorInvalidValue;
  return launch_lds_auto<kBF16>(small_m ? B : A, small_m ? A : B, D, small_m ? N : M, small_m ? M : N, K, !small_m,
                                num_cus, stream);
}

}  // namespace gt
