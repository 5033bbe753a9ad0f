"""The LDS ring of the tiled GEMM's K loop, checked on the CPU.

The kernel's K loop is a walker (ring.hpp) that the library also runs on the
host, recording every event instead of issuing it (gemvtile_ring_trace).
These tests replay those traces through an independent model of what the
events mean on the hardware and check that the schedule is correct:

* loads of one wave complete in issue order, and a wait with count n leaves
  only the n most recent loads in flight;
* a tile is visible to every wave once a barrier follows the wait that saw
  the tile land (each wave runs the same sequence);
* an operand read of tile t must use stage t % STAGES, see tile t there and
  find it visible; a stage may only be refilled after every wave has
  finished reading its previous tile (LDS wait, then a barrier);
* every K tile is loaded once, completely, into its stage, and read in full,
  and nothing is in flight when the loop ends.

The stage and prefetch pattern is also compared with the walk-through
exercise of the TVM chapter ("使用 TMA 为 GEMM 建立 Pipeline", step 5,
Pipeline 机制: PIPE_DEPTH = 2, K_TILES = 5), and the ragged K = 4104 (65 K
tiles, an odd count) and split-K slice lengths are covered.
"""
import os

import pytest

import gemv_tile_pipelined_amd as gt

# Tiled variants with a multi-stage ring (gemvtile_gemm_f16_variant numbers):
# 20 the 256x256 default (early-free schedule), 10 its 32x32x16 form, 21..27
# the smaller tiles with 2..5 stages, 30 the one-barrier ring, 31 the default
# with row-major MFMA order.
VARIANTS = [20, 10, 21, 22, 23, 24, 25, 26, 27, 30, 31, 32]
# 1..9 short loops (every prologue / last-refill / drain branch), 22 and 56
# (split-K slice lengths: ceil(224 / 4) = 56 for K = 14336 in 4 slices), 64
# (K = 4096), 65 (K = 4104: the ragged benchmark shape), 128 (K = 8192).
KTUS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 22, 56, 64, 65, 128]


class RingModel:
    """Replays a trace; raises AssertionError on the first violation."""

    def __init__(self, ktu, info):
        self.S, self.ktu = info["stages"], ktu
        self.per = info["loads_per_tile"]
        self.reads = info["reads_per_step"]
        self.ksteps = info["ksteps"]
        self.mfma = info["mfma_per_step"]
        self.pending = []  # this wave's loads in flight, oldest first: (tile, d)
        self.landed = {}  # tile -> loads of this wave that have landed
        self.issued = {}  # tile -> list of load indices issued
        self.visible = set()  # tiles every wave has landed (a barrier followed)
        self.landed_before_barrier = set()
        self.owner = {}  # stage -> tile loaded into it last
        self.reads_in_flight = set()  # tiles read since the last LDS wait
        self.reads_done = set()  # tiles whose reads completed since the last barrier
        self.released = set()  # tiles whose stage every wave has finished reading
        self.read_log = {}  # tile -> list of (ks, r)
        self.last_read_tile = -1
        self.mfmas = 0
        self.early_free = info["early_free"]
        self.prepared = {}  # tile -> parts of its refill addresses worked out (early-free schedule)
        self.prep_tile = None  # the tile whose refill addresses the kernel holds
        self.prep_parts = None  # parts per refill (the first refill's count; every refill must match)
        self.mfma_since_load = {}  # tile -> MFMAs issued since its last load was issued
        self.overlap = {}  # tile -> MFMAs between its last load and the wait that landed it
        # MFMA blocks per wave: 16x16 blocks with 2 K steps per 64-wide K
        # tile, 32x32 blocks with 4; waves_m x waves_n waves per output tile.
        mi = 16 if self.ksteps == 2 else 32
        self.n_a, self.n_b = info["bm"] // info["waves_m"] // mi, info["bn"] // info["waves_n"] // mi
        assert self.n_a + self.n_b == self.reads and self.n_a * self.n_b == self.mfma
        self.frag = ({}, {})  # fragment buffer -> {("A" | "B", block): (K tile, K step) it holds}
        self.blocks = set()  # (A block, B block) pairs of the current K step's MFMAs
        self.order = []  # (A block, B block) of the MFMAs of K step 0 of K tile 0
        self.inits = 0  # accumulator zeroings
        self.events = []

    def step(self, ev):
        kind, a, b, c, d = ev
        self.events.append(ev)
        getattr(self, "_" + kind)(a, b, c, d)

    def _load(self, tile, d, stage, _):
        assert 0 <= tile < self.ktu, f"load of K tile {tile} outside 0..{self.ktu - 1}"
        assert stage == tile % self.S, f"tile {tile} loaded into stage {stage}"
        got = self.issued.setdefault(tile, [])
        assert d == len(got), f"tile {tile}: load {d} issued after {got}"
        if self.early_free and tile >= self.S:
            # a refill (not the prologue): its addresses were worked out in
            # full beforehand and are still the ones the kernel holds
            assert self.prep_tile == tile, f"refill of tile {tile} issued with the addresses of {self.prep_tile}"
            parts = self.prepared.get(tile, [])
            if self.prep_parts is None:
                self.prep_parts = len(parts)
            assert parts and parts == list(range(self.prep_parts)), f"refill of tile {tile} issued after prep parts {parts}"
        if d == 0:
            prev = self.owner.get(stage)
            if prev is not None:
                assert prev == tile - self.S, f"stage {stage} refilled with {tile} over {prev}"
                assert prev in self.released, f"stage {stage} refilled with tile {tile} before every wave read tile {prev}"
            self.owner[stage] = tile
        got.append(d)
        assert d < self.per
        self.pending.append((tile, d))
        if d == self.per - 1:
            self.mfma_since_load[tile] = 0

    def _wait(self, n, *_):
        assert 0 <= n <= 63, f"vmcnt {n} outside the counter's range"
        while len(self.pending) > n:
            tile, _d = self.pending.pop(0)
            self.landed[tile] = self.landed.get(tile, 0) + 1
            if self.landed[tile] == self.per:
                self.landed_before_barrier.add(tile)
                self.overlap[tile] = self.mfma_since_load.pop(tile)

    def _lds_wait(self, *_):
        self.reads_done |= self.reads_in_flight
        self.reads_in_flight = set()

    def _barrier(self, *_):
        self.visible |= self.landed_before_barrier
        self.landed_before_barrier = set()
        self.released |= self.reads_done
        self.reads_done = set()

    def _read(self, tile, ks, r, stage):
        assert stage == tile % self.S, f"tile {tile} read from stage {stage}"
        assert self.owner.get(stage) == tile, f"tile {tile} read from stage {stage}, which holds {self.owner.get(stage)}"
        assert tile in self.visible, f"tile {tile} read before every wave's loads of it landed"
        assert tile not in self.released, f"tile {tile} read after its stage was released"
        assert tile >= self.last_read_tile, "reads go back to an older K tile"
        self.last_read_tile = tile
        self.reads_in_flight.add(tile)
        self.read_log.setdefault(tile, []).append((ks, r))
        # read index -> fragment: A block 0, the B blocks, the other A blocks;
        # a K step's operands go to fragment buffer (K step parity)
        frag = ("A", 0) if r == 0 else ("B", r - 1) if r <= self.n_b else ("A", r - self.n_b)
        self.frag[ks & 1][frag] = (tile, ks)

    def _prep(self, tile, part, *_):
        assert self.early_free, "address preparation outside the early-free schedule"
        assert self.S <= tile < self.ktu, f"prep for K tile {tile}, which no refill loads"
        if part == 0:
            # the kernel holds one set of refill addresses: the previous
            # refill must have been issued in full before they are replaced
            if self.prep_tile is not None:
                assert len(self.issued.get(self.prep_tile, [])) == self.per, \
                    f"addresses of tile {tile} prepared before tile {self.prep_tile}'s refill was issued"
            assert tile not in self.prepared, f"tile {tile} prepared twice"
            self.prep_tile = tile
        else:
            assert self.prep_tile == tile, f"prep part {part} of tile {tile} during tile {self.prep_tile}'s"
        parts = self.prepared.setdefault(tile, [])
        assert part == len(parts), f"prep part {part} of tile {tile} after {parts}"
        assert not self.issued.get(tile), f"prep part {part} of tile {tile} after its loads began"
        parts.append(part)

    def _init(self, *_):
        # once, after the prologue has issued every load it issues (those of
        # the first min(ktu, S) tiles, or S-1 for the one-barrier ring) and
        # before any wait or MFMA
        assert self.inits == 0 and self.mfmas == 0, "accumulators zeroed twice or after an MFMA"
        before = [e[0] for e in self.events[:-1]]
        assert before and before[-1] == "load", "accumulators zeroed before the prologue's loads were issued"
        assert not {"wait", "read", "mfma"} & set(before), "accumulators zeroed after a wait or read"
        self.inits += 1

    def _mfma(self, buf, idx, i, j):
        assert self.inits == 1, "MFMA before the accumulators were zeroed"
        step = self.mfmas // self.mfma
        tile, ks = divmod(step, self.ksteps)
        assert idx == self.mfmas % self.mfma, f"MFMA index {idx} out of order"
        assert buf == ks & 1, f"K step {ks} computes from fragment buffer {buf}"
        assert 0 <= i < self.n_a and 0 <= j < self.n_b, f"MFMA block ({i}, {j})"
        assert self.frag[buf].get(("A", i)) == (tile, ks), \
            f"MFMA ({i}, {j}) of K tile {tile} step {ks}: A fragment holds {self.frag[buf].get(('A', i))}"
        assert self.frag[buf].get(("B", j)) == (tile, ks), \
            f"MFMA ({i}, {j}) of K tile {tile} step {ks}: B fragment holds {self.frag[buf].get(('B', j))}"
        assert (i, j) not in self.blocks, f"block ({i}, {j}) computed twice in K tile {tile} step {ks}"
        self.blocks.add((i, j))
        if step == 0:
            self.order.append((i, j))
        if len(self.blocks) == self.mfma:
            self.blocks = set()
        self.mfmas += 1
        for t in self.mfma_since_load:
            self.mfma_since_load[t] += 1

    def finish(self):
        assert self.pending == [], f"loads still in flight at the end: {self.pending}"
        assert self.reads_in_flight == set(), "LDS reads not waited for at the end"
        for t in range(self.ktu):
            assert self.issued.get(t) == list(range(self.per)), f"tile {t} loads {self.issued.get(t)}"
            want = [(ks, r) for ks in range(self.ksteps) for r in range(self.reads)]
            assert sorted(self.read_log.get(t, [])) == want, f"tile {t} reads"
        assert self.mfmas == self.ktu * self.ksteps * self.mfma
        assert self.blocks == set(), "a K step ended without all its blocks"
        assert self.inits == 1, "accumulators never zeroed"
        if self.early_free:
            assert sorted(self.prepared) == list(range(self.S, self.ktu)), f"refills prepared: {sorted(self.prepared)}"


def replay(variant, ktu):
    events, info = gt.ring_trace(variant, ktu)
    model = RingModel(ktu, info)
    for ev in events:
        model.step(ev)
    model.finish()
    return model, events


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("ktu", KTUS)
def test_ring_schedule_is_correct(variant, ktu):
    replay(variant, ktu)


# Variants whose MFMAs go in serpentine order over the wave's blocks (each
# shares an operand with the one before it), and those in row-major order.
SERPENTINE = [20, 21, 22, 23, 24, 25, 26, 27, 30]
ROW_MAJOR = [10, 31]


@pytest.mark.parametrize("variant", SERPENTINE + ROW_MAJOR)
def test_mfma_order(variant):
    model, _ = replay(variant, 3)
    n_b = model.n_b
    if variant in ROW_MAJOR:
        assert model.order == [(k // n_b, k % n_b) for k in range(model.mfma)]
    else:
        want = [(k // n_b, k % n_b if (k // n_b) % 2 == 0 else n_b - 1 - k % n_b) for k in range(model.mfma)]
        assert model.order == want
        for (i0, j0), (i1, j1) in zip(model.order, model.order[1:]):
            assert i0 == i1 or j0 == j1, "consecutive MFMAs share an operand"


def _rejects(events, info, ktu):
    model = RingModel(ktu, info)
    try:
        for ev in events:
            model.step(ev)
        model.finish()
    except AssertionError:
        return True
    return False


def test_model_rejects_wrong_mfma_operands():
    """Traces with an MFMA on a transposed block (i, j) -> (j, i), on the
    other fragment buffer, or before its operand was read for its K step
    fail the model."""
    events, info = gt.ring_trace(20, 3)
    assert not _rejects(events, info, 3)
    mfmas = [n for n, e in enumerate(events) if e[0] == "mfma"]
    k = next(n for n in mfmas if events[n][3] != events[n][4])
    name, a, b, c, d = events[k]
    assert _rejects(events[:k] + [(name, a, b, d, c)] + events[k + 1:], info, 3)
    assert _rejects(events[:k] + [(name, a ^ 1, b, c, d)] + events[k + 1:], info, 3)
    # the read of A block 1 for K step 1 of K tile 1, moved after the first
    # MFMA of that step that uses it
    r = next(n for n, e in enumerate(events) if e == ("read", 1, 1, info["bn"] // 32 + 1, 1))
    per_step = info["mfma_per_step"]
    first = next(n for n in mfmas[3 * per_step:4 * per_step] if events[n][3] == 1)
    moved = events[:r] + events[r + 1:first] + [events[first], events[r]] + events[first + 1:]
    assert _rejects(moved, info, 3)


def test_model_rejects_misplaced_accumulator_zeroing():
    """The accumulators are zeroed once, between the prologue's loads and its
    first wait: a trace that zeroes them after the first MFMA, or twice,
    fails the model."""
    events, info = gt.ring_trace(20, 3)
    k = events.index(("init", 0, 0, 0, 0))
    first = next(n for n, e in enumerate(events) if e[0] == "mfma")
    late = events[:k] + events[k + 1:first + 1] + [events[k]] + events[first + 1:]
    assert _rejects(late, info, 3)
    assert _rejects(events[:k + 1] + [events[k]] + events[k + 1:], info, 3)


def test_trace_info_describes_the_kernels():
    want = {20: (256, 256, 2, 16, 1), 10: (256, 256, 2, 16, 0), 21: (256, 128, 3, 12, 0), 22: (128, 256, 3, 12, 0),
            23: (128, 128, 4, 8, 0), 24: (256, 128, 2, 12, 0), 25: (128, 256, 2, 12, 0), 26: (128, 128, 2, 8, 0),
            27: (128, 128, 5, 8, 0), 30: (256, 256, 2, 16, 0), 31: (256, 256, 2, 16, 1), 32: (128, 64, 4, 6, 0)}
    for v, (bm, bn, stages, per, ef) in want.items():
        _, info = gt.ring_trace(v, 4)
        assert (info["bm"], info["bn"], info["stages"], info["loads_per_tile"], info["early_free"]) == \
            (bm, bn, stages, per, ef), v
    for v in (0, 1, 3, 28):  # the default's ring
        assert gt.ring_trace(v, 7)[0] == gt.ring_trace(20, 7)[0]
    with pytest.raises(gt.GemvTileError):
        gt.ring_trace(2, 4)  # the one-stage ablation has no ring


# The tiles and ring depths gemm_f16 picks (gemvtile_gemm_tile), and the
# early-free schedule.
OVERLAPPED = [20, 21, 22, 23, 30]


@pytest.mark.parametrize("variant", OVERLAPPED)
def test_ring_overlaps_loads_with_mfmas(variant):
    """In the steady state each K tile's last load is issued at least one
    whole K step of MFMAs before the wait that needs it: the loads overlap
    the matrix work (the point of the ring)."""
    model, _ = replay(variant, 16)
    for t in range(model.S, 16):
        assert model.overlap[t] >= model.mfma, (t, model.overlap[t])


def test_early_free_lengthens_the_refill_slack():
    """The early-free schedule (the default, 20) starts each refill about
    half a K tile sooner than the one-barrier ring (30), so a tile's last
    load has far more MFMA slots to land before the barrier that needs it."""
    base, _ = replay(30, 16)
    ef, _ = replay(20, 16)
    for t in range(2, 16):
        assert ef.overlap[t] >= base.overlap[t] + 40, (t, ef.overlap[t], base.overlap[t])
    # two barriers per K tile in the steady state, one in the one-barrier ring
    n_ef = sum(1 for e in gt.ring_trace(20, 16)[0] if e[0] == "barrier")
    n_base = sum(1 for e in gt.ring_trace(30, 16)[0] if e[0] == "barrier")
    assert n_base == 2 + 15 and n_ef == 2 + 15 + 14


def test_two_stage_rings_of_small_tiles_barely_overlap():
    """The 2-stage ablations of the smaller tiles: a K tile of them is 1/2
    or 1/4 of the 256x256 one in MFMA slots, so the last load of a refill
    lands only a few MFMAs before it is needed -- which is why those tiles
    get 3- and 4-stage rings by default."""
    for v in (24, 25, 26):
        model, _ = replay(v, 16)
        assert max(model.overlap[t] for t in range(2, 16)) < model.mfma


def test_ring_wait_counts_let_younger_tiles_fly():
    """With 3 or more stages the steady-state wait leaves the younger tiles'
    loads in flight (vmcnt = (stages - 2) x loads per tile) rather than
    draining the ring; with 2 stages nothing younger exists at the wait --
    except in the early-free schedule, whose next refill is already issued
    there (vmcnt = loads per tile)."""
    for v in VARIANTS:
        events, info = gt.ring_trace(v, 32)
        stages, per = info["stages"], info["loads_per_tile"]
        waits = [e[1] for e in events if e[0] == "wait"]
        steady = waits[1:32 - stages]
        assert len(set(steady)) == 1, (v, steady)
        younger = steady[0] - (stages - 2) * per
        if info["early_free"]:
            assert 0 < younger <= per, (v, steady)  # part of the next refill
        else:
            assert younger == 0, (v, steady)
        assert waits[-1] == 0  # the last tile: nothing younger


def _load_golden():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tvm_pipeline_depth2_ktiles5.txt")
    rows = []
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            k, stage, ph_tma, ph_mma, pre = [p.strip() for p in line.split("|")]
            rows.append((int(k), int(stage), int(ph_tma), int(ph_mma), None if pre == "-" else int(pre)))
    return rows


@pytest.mark.parametrize("variant", [20, 30], ids=["early_free", "one_barrier"])
def test_tvm_pipeline_exercise_depth2_ktiles5(variant):
    """PIPE_DEPTH = 2, K_TILES = 5 (the 256x256 kernel's 2-stage ring over 5
    K tiles, in both schedules): each K tile sits in the chapter's stage, the
    stage's fill round has the parity of the chapter's phase_tma, and the
    tile whose refill starts while K tile k is being computed -- into the
    stage k frees -- is the chapter's prefetch (none in the last two
    iterations).  phase_mma has no counterpart here: the MFMA results are
    ordered by register dependences, not by a barrier."""
    golden = _load_golden()
    assert [g[0] for g in golden] == list(range(5))
    events, info = gt.ring_trace(variant, 5)
    replay(variant, 5)
    per_tile = info["ksteps"] * info["mfma_per_step"]
    stage_of = {}
    started_during = {}  # K tile being computed -> tiles whose first load is issued then
    mfmas = 0
    for kind, a, b, c, d in events:
        if kind == "mfma":
            mfmas += 1
        elif kind == "read":
            stage_of.setdefault(a, set()).add(d)
        elif kind == "load" and b == 0 and mfmas > 0:
            started_during.setdefault(mfmas // per_tile, set()).add(a)
    for k, stage, ph_tma, _ph_mma, pre in golden:
        assert stage_of[k] == {stage}
        assert (k // 2) % 2 == ph_tma  # the stage's fill round, mod 2
        assert started_during.get(k, set()) == ({pre} if pre is not None else set()), (k, started_during)


def _replay_events(events, ktu, info):
    model = RingModel(ktu, info)
    for ev in events:
        model.step(ev)
    model.finish()


def test_model_rejects_broken_schedules():
    """The replay model must fail on plausible ring mistakes, each planted in
    a copy of a real trace: a wait that lets the needed tile stay in flight,
    a missing barrier, a refill issued before the barrier that frees its
    stage, a read from the wrong stage, a dropped load."""
    ktu = 8
    events, info = gt.ring_trace(21, ktu)  # 256x128, 3 stages
    stages = info["stages"]
    _replay_events(events, ktu, info)  # the real trace passes
    per = info["loads_per_tile"]
    waits = [i for i, e in enumerate(events) if e[0] == "wait"]
    barriers = [i for i, e in enumerate(events) if e[0] == "barrier"]
    mutants = []
    # 1. a steady-state wait one tile too lax
    m = list(events)
    i = waits[2]
    m[i] = ("wait", m[i][1] + per, 0, 0, 0)
    mutants.append(m)
    # 2. the barrier of K tile 2 dropped
    m = list(events)
    del m[barriers[4]]
    mutants.append(m)
    # 3. the first load of a refill moved before the barrier that frees its stage
    m = list(events)
    j = next(i for i, e in enumerate(m) if e[0] == "load" and e[1] == stages + 1 and e[2] == 0)
    b = max(i for i in barriers if i < j)
    ev = m.pop(j)
    m.insert(b, ev)
    mutants.append(m)
    # 4. a read from the wrong stage
    m = list(events)
    j = next(i for i, e in enumerate(m) if e[0] == "read" and e[1] == 4)
    k, ks, r, st = m[j][1:]
    m[j] = ("read", k, ks, r, (st + 1) % stages)
    mutants.append(m)
    # 5. one load of a tile dropped
    m = list(events)
    j = next(i for i, e in enumerate(m) if e[0] == "load" and e[1] == 5 and e[2] == 3)
    del m[j]
    mutants.append(m)
    for n, m in enumerate(mutants, 1):
        with pytest.raises(AssertionError):
            _replay_events(m, ktu, info)
