// ring.hpp -- the LDS ring schedule of the pipelined GEMM K loop, written
// once as a host- and device-callable walker.
//
// gemm_kernel runs ring_k_loop() with an Ops object whose methods issue the
// kernel's instructions (tile loads, operand reads, MFMAs, waits, barriers).
// The host runs the same walker with an Ops object that records each event
// (gemvtile_ring_trace in the C ABI), so CPU tests check the schedule the
// kernel executes: the ring stage of every K tile, where each tile load is
// issued, the vmcnt each wait takes, and where the barriers fall.
//
// The ring is the one of the TVM TIRx GEMM chapter, step 5 (Software
// Pipeline, Pipeline 机制): K tile k lives in stage k % STAGES, the first
// tiles are prefetched before the loop, and a stage is refilled with the
// tile STAGES ahead as soon as its own tile has been consumed.  The chapter
// tracks completion with one mbarrier per stage whose phase flips on every
// reuse of the stage.  Here a wave's loads complete in issue order, so "K
// tile k has landed" is "at most (loads issued after those of tile k) are
// outstanding", a vmcnt wait, followed by a workgroup barrier so that the
// other waves' loads of the tile have landed too.  The mbarrier phase of the
// chapter corresponds to the parity of ring_round().
//
// Within K tile kt (kKSub K steps of kMfma MFMA slots each):
//  * every READ_STRIDE-th slot of a non-final K step reads one operand
//    fragment of the next K step (kReads per step) from stage kt;
//  * the final K step meets the other waves after kBarrierAt MFMAs: it waits
//    until tile kt+1 has landed (younger tiles may stay in flight), waits for
//    its own LDS reads, and crosses the one barrier of the K tile.  Its
//    operands are already in registers, so the barrier frees stage kt;
//  * right after that barrier the refill of stage kt with tile kt + STAGES
//    starts (load d at slot DMA_OFFSET + d * DMA_STRIDE counted from the
//    barrier), and the first operands of tile kt+1 are read from its stage;
//  * the refill continues through the non-final K steps of tile kt+1, and
//    every load of it is issued before the barrier of tile kt+1 (a static
//    assertion), so the barrier of tile kt always knows exactly which tiles
//    are in flight.
// The stage index and the wait count follow from the loop counter, so nothing
// resets between output tiles, and an odd number of K tiles (65 for
// K = 4104) needs no special case.
#pragma once

#include <stdint.h>

#include "tile_order.hpp"  // GT_HD

namespace gt {

// The walker must be inlined into the kernel: called out of line it would
// reach the kernel's accumulator and fragment arrays through pointers, which
// puts them in scratch memory.
#define GT_RING_INLINE GT_HD __attribute__((always_inline)) inline

GT_HD constexpr int ring_min(int a, int b) { return a < b ? a : b; }
GT_HD constexpr int ring_max(int a, int b) { return a > b ? a : b; }

// Stage of K tile kt, and how many times that stage has been filled before
// it (the mbarrier phase of the TVM chapter is the parity of this).
GT_HD constexpr int ring_stage(int kt, int stages) { return kt % stages; }
GT_HD constexpr int ring_round(int kt, int stages) { return kt / stages; }

// Phases of the loop over ktu K tiles:
//  rest  -- K tile kt carries the rest of the refill with tile kt+STAGES-1
//           (started at the barrier of tile kt-1, or in the prologue);
//  early -- K tile kt starts the refill with tile kt+STAGES at its barrier;
//  next  -- a K tile follows kt (so kt has a barrier at all).
GT_HD constexpr bool ring_rest(int kt, int ktu, int stages) { return kt + stages - 1 < ktu; }
GT_HD constexpr bool ring_early(int kt, int ktu, int stages) { return kt + stages < ktu; }
GT_HD constexpr bool ring_next(int kt, int ktu) { return kt + 1 < ktu; }

// K tiles issued after the one needed next, which may stay in flight at a
// wait: at the barrier of K tile kt, tiles 0 .. min(ktu, kt+STAGES)-1 are
// issued and tile kt+1 is needed; in the prologue, tiles
// 0 .. min(ktu, STAGES-1)-1 are issued and tile 0 is needed.
GT_HD constexpr int ring_younger_at_barrier(int kt, int ktu, int stages) {
  return ring_min(ktu, kt + stages) - (kt + 2);
}
GT_HD constexpr int ring_younger_at_prologue(int ktu, int stages) { return ring_min(ktu, stages - 1) - 1; }

// The vmcnt of a wait that lets `younger` whole K tiles of `per` loads each
// stay in flight (never more than STAGES-2 of them can be).
GT_HD constexpr int ring_vmcnt(int younger, int stages, int per) {
  return ring_max(0, ring_min(younger, stages - 2)) * per;
}

// Index of the refill load issued at slot position `pos` (counted in MFMA
// slots from the barrier that starts the refill), or -1.
template <class S>
GT_HD constexpr int ring_slot_load(int pos) {
  const int q = pos - S::DMA_OFFSET;
  return (q >= 0 && q % S::DMA_STRIDE == 0 && q / S::DMA_STRIDE < S::kDmaPerStage) ? q / S::DMA_STRIDE : -1;
}

// MFMAs of a final K step before its barrier, and slots after it.
template <class S>
struct RingSlots {
  static constexpr int kBarrierAt = S::kMfma - S::kReads * S::READ_STRIDE;
  static constexpr int kAfter = S::kMfma - kBarrierAt;
  static constexpr int kTileSlots = S::kKSub * S::kMfma;
  static_assert(S::STAGES >= 2, "the ring needs two stages or more");
  static_assert(S::kMfma >= S::kReads * S::READ_STRIDE, "MFMA slots for the operand reads");
  static_assert((S::kDmaPerStage - 1) * S::DMA_STRIDE + S::DMA_OFFSET < kTileSlots,
                "a refill must be issued in full within one K tile");
  // The operand fragments are double-buffered by K-step parity, so a K tile
  // must hold an even number of K steps for the parity to carry over.
  static_assert(S::kKSub % 2 == 0, "an even number of K steps per K tile");
};

// One K tile of the loop (see the file comment).  Ops provides
//   mfma(buf, idx), read(buf, kt, ks, r), load(tile, d), wait_tile(vmcnt),
//   wait_lds(), barrier(), fence(), init_acc() (zero the accumulators: the
//   walker calls it once, between the prologue's loads and its first wait),
//   and (used by the early-free loop)
//   mfma_load(buf, idx, tile, d): mfma(buf, idx) then load(tile, d) as one
//   instruction group, and prep(tile, part): work out, in part `part` of
//   RingEarly::kPrepParts, the addresses of the refill of K tile `tile`
//   that the following mfma_load calls issue
// where fence() keeps the instruction order (a scheduling barrier).
template <class S, bool kRest, bool kEarly, bool kNext, class Ops>
GT_RING_INLINE void ring_ktile(Ops &ops, int kt, int ktu) {
  using R = RingSlots<S>;
#pragma unroll
  for (int ks = 0; ks < S::kKSub; ++ks) {
    const int cur = ks & 1;
    const bool last = ks == S::kKSub - 1;
#pragma unroll
    for (int idx = 0; idx < S::kMfma; ++idx) {
      if (last && kNext && idx == R::kBarrierAt) {
        ops.wait_tile(ring_vmcnt(ring_younger_at_barrier(kt, ktu, S::STAGES), S::STAGES, S::kDmaPerStage));
        ops.wait_lds();
        ops.barrier();
        ops.fence();
      }
      ops.mfma(cur, idx);
      ops.fence();
      if (!last) {
        if (idx % S::READ_STRIDE == 0 && idx / S::READ_STRIDE < S::kReads) {
          ops.read(cur ^ 1, kt, ks + 1, idx / S::READ_STRIDE);
          ops.fence();
        }
      } else if (kNext && idx >= R::kBarrierAt && (idx - R::kBarrierAt) % S::READ_STRIDE == 0) {
        ops.read(cur ^ 1, kt + 1, 0, (idx - R::kBarrierAt) / S::READ_STRIDE);
        ops.fence();
      }
      if (last && idx >= R::kBarrierAt) {
        if (kEarly) {
          const int d = ring_slot_load<S>(idx - R::kBarrierAt);
          if (d >= 0) ops.load(kt + S::STAGES, d);
          ops.fence();
        }
      } else if (kRest) {
        const int d = ring_slot_load<S>(R::kAfter + ks * S::kMfma + idx);
        if (d >= 0) ops.load(kt + S::STAGES - 1, d);
        ops.fence();
      }
    }
  }
  if (!kNext) ops.wait_lds();
}

// The whole K loop of one output tile over ktu >= 1 K tiles.
template <class S, class Ops>
GT_RING_INLINE void ring_k_loop(Ops &ops, int ktu) {
  using R = RingSlots<S>;
  // Every wave must be done with the previous output tile's LDS (ring and
  // epilogue staging) before the ring is refilled.
  ops.wait_lds();
  ops.barrier();
  // Prologue: K tiles 0 .. STAGES-2 in flight; once tile 0 has landed, its
  // first operands are read and the loads of tile STAGES-1 that would follow
  // a barrier go out, the rest during K tile 0.
#pragma unroll
  for (int s = 0; s < S::STAGES - 1; ++s)
    if (s < ktu)
#pragma unroll
      for (int d = 0; d < S::kDmaPerStage; ++d) ops.load(s, d);
  // The accumulators are zeroed while the first tiles are in flight.
  ops.fence();
  ops.init_acc();
  ops.fence();
  ops.wait_tile(ring_vmcnt(ring_younger_at_prologue(ktu, S::STAGES), S::STAGES, S::kDmaPerStage));
  ops.barrier();
#pragma unroll
  for (int r = 0; r < S::kReads; ++r) ops.read(0, 0, 0, r);
  if (S::STAGES - 1 < ktu) {
#pragma unroll
    for (int pos = 0; pos < R::kAfter; ++pos) {
      const int d = ring_slot_load<S>(pos);
      if (d >= 0) ops.load(S::STAGES - 1, d);
    }
  }
  int kt = 0;
  for (; ring_early(kt, ktu, S::STAGES); ++kt) ring_ktile<S, true, true, true>(ops, kt, ktu);  // steady state
  if (ring_rest(kt, ktu, S::STAGES) && ring_next(kt, ktu)) {                                  // last refill
    ring_ktile<S, true, false, true>(ops, kt, ktu);
    ++kt;
  }
  for (; ring_next(kt, ktu); ++kt) ring_ktile<S, false, false, true>(ops, kt, ktu);  // the ring drains
  ring_ktile<S, false, false, false>(ops, kt, ktu);                                  // last K tile
}

// ---- the early-free schedule -------------------------------------------
// The loop above has one barrier per K tile, which does two jobs at once:
// every wave is done reading stage kt (so it may be refilled) and tile kt+1
// has landed (so it may be read).  With two stages the refill of stage kt
// then has one K tile of MFMA slots, minus its own issue span, before the
// barrier that needs it.  The early-free schedule (S::EARLY_FREE) splits the
// two jobs: a "free" barrier in K step 0 of tile kt, at slot S::WAR_AT, once
// the wave has read all of stage kt (K step 1's operands are read during K
// step 0), starts the refill of stage kt with tile kt + STAGES there; the
// "landed" barrier stays where it was, in the last K step.  The refill
// starts about half a K tile earlier and the wait for a tile leaves the
// next tile's loads in flight, at the price of a second barrier per K tile.
// The prologue issues tiles 0 .. STAGES-1 at once (every stage is free at
// the start of an output tile).
template <class S>
struct RingEarly {
  static constexpr int kBarrierAt = S::kMfma - S::kReads * S::READ_STRIDE;  // landed barrier, last K step
  static constexpr int kRawPos = (S::kKSub - 1) * S::kMfma + kBarrierAt;    // ... counted from the tile start
  static constexpr int kTileSlots = S::kKSub * S::kMfma;
  static constexpr int kLastLoad = S::WAR_AT + S::DMA_OFFSET + (S::kDmaPerStage - 1) * S::DMA_STRIDE;
  // refill loads issued before the landed barrier of the same K tile
  static constexpr int loads_before_raw() {
    int n = 0;
    for (int d = 0; d < S::kDmaPerStage; ++d)
      if (S::WAR_AT + S::DMA_OFFSET + d * S::DMA_STRIDE < kRawPos) ++n;
    return n;
  }
  static constexpr int kLoadsBeforeRaw = loads_before_raw();
  // The refill's addresses are worked out ahead of its free barrier, in
  // kPrepParts pieces one MFMA slot apart (every other slot from kPrepAt),
  // in the slots after K step 0's last operand read, which carry nothing
  // else.  A wave issues one instruction every 4 cycles at most, so a slot
  // (16 cycles of one MFMA) has room for 3 more before the next MFMA waits.
  static constexpr int kPrepParts = 5;
  static constexpr int kPrepAt = S::kReads * S::READ_STRIDE + 1;
  static constexpr bool is_prep_slot(int idx) {
    return idx >= kPrepAt && (idx - kPrepAt) % 2 == 0 && (idx - kPrepAt) / 2 < kPrepParts;
  }
  // the vmcnt of the landed wait in the steady state: the STAGES-2 whole
  // tiles after the needed one, and the part of the newest refill issued
  static constexpr int kSteadyVmcnt = (S::STAGES - 2) * S::kDmaPerStage + kLoadsBeforeRaw;
  static_assert(S::STAGES >= 2 && S::kKSub == 2, "early free: two K steps per K tile");
  static_assert(S::WAR_AT >= S::kReads * S::READ_STRIDE && S::WAR_AT < S::kMfma,
                "the free barrier follows the last operand read of K step 0, within K step 0");
  // The walker issues a refill only within the K tile whose free barrier
  // starts it: a load placed past that tile's last MFMA slot would never be
  // issued.
  static_assert(S::WAR_AT + S::DMA_OFFSET + (S::kDmaPerStage - 1) * S::DMA_STRIDE < kTileSlots,
                "a refill is issued in full within the K tile that starts it");
  static_assert(kLastLoad < kTileSlots + kRawPos, "a refill is issued in full before the barrier that needs it");
  static_assert(S::STAGES * S::kDmaPerStage <= 63 && kSteadyVmcnt <= 63, "vmcnt range");
  static_assert(kPrepAt + 2 * (kPrepParts - 1) < S::WAR_AT, "the refill's addresses are ready before its free barrier");
};

// vmcnt of the landed wait in K tile kt: loads of whole tiles issued after
// tile kt+1, and the newest refill's loads issued so far.
template <class S, bool kEarly>
GT_HD constexpr int ring_ef_vmcnt(int kt, int ktu) {
  return kEarly ? RingEarly<S>::kSteadyVmcnt
                : ring_max(0, ring_min(ktu, kt + S::STAGES) - (kt + 2)) * S::kDmaPerStage;
}

template <class S, bool kEarly, bool kNext, class Ops>
GT_RING_INLINE void ring_ktile_ef(Ops &ops, int kt, int ktu) {
  using R = RingEarly<S>;
#pragma unroll
  for (int ks = 0; ks < S::kKSub; ++ks) {
    const int cur = ks & 1;
    const bool last = ks == S::kKSub - 1;
#pragma unroll
    for (int idx = 0; idx < S::kMfma; ++idx) {
      if (kEarly && !last && idx == S::WAR_AT) {
        ops.wait_lds();
        ops.barrier();
        ops.fence();
      }
      if (last && kNext && idx == R::kBarrierAt) {
        ops.wait_tile(ring_ef_vmcnt<S, kEarly>(kt, ktu));
        ops.barrier();
        ops.fence();
      }
      // A slot that carries a refill load issues it together with the
      // slot's MFMA (mfma_load: one instruction group, the load after the
      // MFMA).
      const int pos = ks * S::kMfma + idx;
      const int d = (kEarly && pos >= S::WAR_AT) ? ring_slot_load<S>(pos - S::WAR_AT) : -1;
      if (d >= 0)
        ops.mfma_load(cur, idx, kt + S::STAGES, d);
      else
        ops.mfma(cur, idx);
      ops.fence();
      if (!last) {
        if (idx % S::READ_STRIDE == 0 && idx / S::READ_STRIDE < S::kReads) {
          ops.read(cur ^ 1, kt, ks + 1, idx / S::READ_STRIDE);
          ops.fence();
        }
        if (kEarly && R::is_prep_slot(idx)) {
          ops.prep(kt + S::STAGES, (idx - R::kPrepAt) / 2);
          ops.fence();
        }
      } else if (kNext && idx >= R::kBarrierAt && (idx - R::kBarrierAt) % S::READ_STRIDE == 0) {
        ops.read(cur ^ 1, kt + 1, 0, (idx - R::kBarrierAt) / S::READ_STRIDE);
        ops.fence();
      }
    }
  }
  if (!kNext) ops.wait_lds();
}

template <class S, class Ops>
GT_RING_INLINE void ring_k_loop_ef(Ops &ops, int ktu) {
  // Every wave must be done with the previous output tile's LDS first.
  ops.wait_lds();
  ops.barrier();
#pragma unroll
  for (int s = 0; s < S::STAGES; ++s)
    if (s < ktu)
#pragma unroll
      for (int d = 0; d < S::kDmaPerStage; ++d) ops.load(s, d);
  // The accumulators are zeroed while the first tiles are in flight.
  ops.fence();
  ops.init_acc();
  ops.fence();
  ops.wait_tile(ring_min(ktu, S::STAGES) * S::kDmaPerStage - S::kDmaPerStage);
  ops.barrier();
#pragma unroll
  for (int r = 0; r < S::kReads; ++r) ops.read(0, 0, 0, r);
  int kt = 0;
  // The steady state, two K tiles per iteration: the stage of each is then
  // known when the code is generated, and the loop's own bookkeeping comes
  // once per two K tiles.
  for (; ring_early(kt + 1, ktu, S::STAGES); kt += 2) {
    ring_ktile_ef<S, true, true>(ops, kt, ktu);
    ring_ktile_ef<S, true, true>(ops, kt + 1, ktu);
  }
  if (ring_early(kt, ktu, S::STAGES)) ring_ktile_ef<S, true, true>(ops, kt++, ktu);
  for (; ring_next(kt, ktu); ++kt) ring_ktile_ef<S, false, true>(ops, kt, ktu);          // the ring drains
  ring_ktile_ef<S, false, false>(ops, kt, ktu);                                          // last K tile
}

// Event codes of the host-side trace (gemvtile_ring_trace): each event is
// five int32 values {code, a, b, c, d}.
enum RingEvent : int32_t {
  kRingLoad = 1,      // a = K tile (loop index), b = load index d, c = stage
  kRingWaitTile = 2,  // a = vmcnt
  kRingWaitLds = 3,   // (all LDS reads of the wave done)
  kRingBarrier = 4,   // workgroup barrier
  kRingRead = 5,      // a = K tile, b = K step, c = read index r, d = stage
  kRingMfma = 6,      // a = fragment buffer, b = MFMA index within the K step
  kRingPrep = 7,      // a = K tile whose refill addresses are prepared, b = part
  kRingInit = 8,      // the accumulators are zeroed
};

}  // namespace gt
