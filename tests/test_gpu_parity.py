"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: |d - ref| <= 1e-2 + 1e-2·|ref| elementwise for uniform random inputs;
bit-for-bit (value) equality for integer-valued inputs, whose FP32 partial
sums are exact in any order (|sums| <= K·64 < 2^24), so only the final
round-to-nearest-even can differ -- and must not.

Small and ragged shapes are compared in full, and so are the full-size
workloads 4096^3 (the benchmark's GEMM), 4000x4032x4104 and the GEMV
4096x14336, in the launch shape the benchmark times.  8192^3 is compared on
64 seeded rows plus one seeded row from every 256-row band (so every tile row
of the output is checked against the oracle), and a closed form is checked on
every element.
"""
import os

import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu

TOL_ABS = 1e-2
TOL_REL = 1e-2


@pytest.fixture(scope="module")
def env():
    import torch

    import gemv_tile_pipelined_amd as gt

    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    gt.load_library()  # raises if the HIP library is not built
    return torch, gt, torch.device("cuda:0")


def _tol_violations(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bad = ~(np.abs(got - ref) <= TOL_ABS + TOL_REL * np.abs(ref))
    return int(bad.sum())


def _gemm(env, A, B, variant=0):
    torch, gt, dev = env
    D = gt.gemm_f16(torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev), variant=variant)
    torch.cuda.synchronize(dev)
    return D


def _gemv(env, x, W, variant=0):
    torch, gt, dev = env
    y = gt.gemv_f16(torch.from_numpy(x).to(dev), torch.from_numpy(W).to(dev), variant=variant)
    torch.cuda.synchronize(dev)
    return y.cpu().numpy()


SMALL_SHAPES = [
    (256, 256, 256),  # the 256^3 workload, one full tile
    (1, 1, 8),
    (17, 300, 8),
    (300, 260, 200),
    (257, 255, 136),
    (513, 1000, 520),
    (64, 64, 4104),
    (1000, 33, 64),
    (520, 776, 1032),
]


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_small_uniform(env, shape):
    M, N, K = shape
    cfg = 0 if shape == (256, 256, 256) else 1000 + SMALL_SHAPES.index(shape)
    A = datagen.uniform_f16(cfg, 0, (M, K), -1.0, 1.0)
    B = datagen.uniform_f16(cfg, 1, (N, K), -1.0, 1.0)
    got = _gemm(env, A, B).cpu().numpy()
    ref = oracle.gemm(A, B)
    assert np.isfinite(got).all()
    assert _tol_violations(got, ref) == 0


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_small_integer_exact(env, shape):
    M, N, K = shape
    cfg = 2000 + SMALL_SHAPES.index(shape)
    A = datagen.integer_f16(cfg, 0, (M, K))
    B = datagen.integer_f16(cfg, 1, (N, K))
    got = _gemm(env, A, B).cpu().numpy()
    ref = oracle.gemm(A, B)
    assert np.array_equal(got, ref)


def test_gemm_closed_forms(env):
    torch, gt, dev = env
    # all-ones -> K everywhere (ragged in M, N and K)
    M, N, K = 300, 520, 4104
    D = _gemm(env, np.ones((M, K), np.float16), np.ones((N, K), np.float16))
    assert bool((D == K).all())
    # B = I -> D = A ;  A = I -> D = Bᵀ
    A = datagen.uniform_f16(3000, 0, (300, 512), -1.0, 1.0)
    D = _gemm(env, A, np.eye(512, dtype=np.float16)).cpu().numpy()
    assert np.array_equal(D.view(np.uint16), A.view(np.uint16))
    B = datagen.uniform_f16(3000, 1, (520, 256), -1.0, 1.0)
    D = _gemm(env, np.eye(256, dtype=np.float16), B).cpu().numpy()
    assert np.array_equal(D.view(np.uint16), np.ascontiguousarray(B.T).view(np.uint16))
    # rank-1: A[m,k] = u_m, B[n,k] = v_n -> K·u_m·v_n exactly
    g = np.random.default_rng(3001)
    choices = np.array([-2.0, -1.0, -0.5, -0.25, 0.25, 0.5, 1.0, 2.0])
    u, v = g.choice(choices, 333), g.choice(choices, 270)
    K = 1032
    A = np.repeat(u[:, None], K, axis=1).astype(np.float16)
    B = np.repeat(v[:, None], K, axis=1).astype(np.float16)
    D = _gemm(env, A, B).cpu().numpy().astype(np.float64)
    assert np.array_equal(D, K * np.outer(u, v))


def _load_rne_probe():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rne_probe.txt")
    cases = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        a, b, want, _ = [p.strip() for p in line.split("|")]
        av = [float.fromhex(t) if "p" in t else float(t) for t in a.split()]
        bv = [float.fromhex(t) if "p" in t else float(t) for t in b.split()]
        cases.append((av + [0.0] * 4, bv + [0.0] * 4, int(want, 16)))  # pad K to 8
    return cases


def test_rne_probe_normal_range(env):
    """Ties-to-even and overflow of the final fp16 rounding (printed probes)."""
    for av, bv, want in _load_rne_probe():
        if min(abs(v) for v in av + bv if v) < 2.0**-14:
            continue  # subnormal inputs: next test
        A = np.array([av], np.float16)
        B = np.array([bv], np.float16)
        D = _gemm(env, A, B).cpu().numpy()
        assert int(D.view(np.uint16)[0, 0]) == want, (av, bv)
        y = _gemv(env, A[0], B)
        assert int(y.view(np.uint16)[0]) == want, (av, bv)


def test_rne_probe_subnormal_inputs(env):
    """fp16 subnormal operands must be honoured by the matrix cores."""
    for av, bv, want in _load_rne_probe():
        if min(abs(v) for v in av + bv if v) >= 2.0**-14:
            continue
        A = np.array([av], np.float16)
        B = np.array([bv], np.float16)
        D = _gemm(env, A, B).cpu().numpy()
        assert int(D.view(np.uint16)[0, 0]) == want, (av, bv)
        y = _gemv(env, A[0], B)
        assert int(y.view(np.uint16)[0]) == want, (av, bv)


@pytest.mark.parametrize("integer", [False, True], ids=["uniform", "integer"])
@pytest.mark.parametrize("cfg_id", [1, 2], ids=["4096cube", "ragged_4000x4032x4104"])
def test_gemm_full_size_every_element(env, full_size, cfg_id, integer):
    """4096^3 and 4000x4032x4104 against the oracle on every output element:
    uniform inputs within the tolerance, integer inputs bit for bit."""
    torch, gt, dev = env
    w = datagen.WORKLOADS[cfg_id]
    print(f"[gemm full size] {w.name} M={w.M} N={w.N} K={w.K} integer={integer}", flush=True)
    A, B = full_size.inputs(cfg_id, integer)
    got = _gemm(env, A, B).cpu().numpy()
    ref = full_size.reference(cfg_id, integer)
    if integer:
        assert np.array_equal(got, ref)
    else:
        assert np.isfinite(got).all()
        assert _tol_violations(got, ref) == 0


def test_gemm_8192_sampled_rows_every_tile_band(env):
    """8192^3: the 64 seeded rows plus one seeded row of every 256-row tile
    band, all columns, uniform within the tolerance and integer bit-exact."""
    torch, gt, dev = env
    w = datagen.WORKLOADS[4]
    print(f"[gemm full size] {w.name} M={w.M} N={w.N} K={w.K}", flush=True)
    rows = np.union1d(datagen.sample_rows(4, w.M, 64), datagen.band_rows(4, w.M, 256))
    assert len(np.unique(rows // 256)) == w.M // 256
    trows = torch.from_numpy(rows).to(dev)
    A, B = datagen.gemm_inputs(w)
    D = _gemm(env, A, B)
    assert bool(torch.isfinite(D).all())
    assert _tol_violations(D[trows].cpu().numpy(), oracle.gemm(A, B, rows=rows)) == 0
    Ai, Bi = datagen.gemm_inputs(w, integer=True)
    Di = _gemm(env, Ai, Bi)
    assert np.array_equal(Di[trows].cpu().numpy(), oracle.gemm(Ai, Bi, rows=rows))


@pytest.mark.parametrize("cfg_id", [1, 2, 4], ids=["4096cube", "ragged_4000x4032x4104", "8192cube"])
def test_gemm_full_size_rank1_every_element(env, cfg_id):
    """Closed form on every output: A[m,k] = u_m, B[n,k] = v_n -> K·u_m·v_n."""
    torch, gt, dev = env
    w = datagen.WORKLOADS[cfg_id]
    g = datagen.rng(cfg_id, 20)
    choices = np.array([-1.0, -0.5, -0.25, -0.125, 0.125, 0.25, 0.5, 1.0])
    u, v = g.choice(choices, w.M), g.choice(choices, w.N)
    tu = torch.from_numpy(u.astype(np.float16)).to(dev)
    tv = torch.from_numpy(v.astype(np.float16)).to(dev)
    A = tu[:, None].expand(w.M, w.K).contiguous()
    B = tv[:, None].expand(w.N, w.K).contiguous()
    D = gt.gemm_f16(A, B)
    want = (w.K * torch.outer(tu.double(), tv.double())).half()  # exact: K·u·v is fp16-representable
    torch.cuda.synchronize(dev)
    assert bool((D == want).all())


def test_gemv_workload(env):
    w = datagen.WORKLOADS[3]
    x, W = datagen.gemv_inputs(w)
    got = _gemv(env, x, W)
    ref = oracle.gemv(x, W)
    assert np.isfinite(got).all()
    assert _tol_violations(got, ref) == 0
    xi, Wi = datagen.gemv_inputs(w, integer=True)
    assert np.array_equal(_gemv(env, xi, Wi), oracle.gemv(xi, Wi))
    # unit vectors pick columns of W
    for j in (0, 7, 8, 14335):
        e = np.zeros(w.K, np.float16)
        e[j] = 1.0
        assert np.array_equal(_gemv(env, e, W).view(np.uint16), np.ascontiguousarray(W[:, j]).view(np.uint16))


GEMV_SHAPES = [(1, 8), (7, 520), (4097, 14336), (1000, 14344), (33, 16392), (4096, 64), (16, 1032)]


@pytest.mark.parametrize("shape", GEMV_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemv_ragged(env, shape):
    N, K = shape
    cfg = 4000 + GEMV_SHAPES.index(shape)
    x = datagen.uniform_f16(cfg, 0, (K,), -1.0, 1.0)
    W = datagen.uniform_f16(cfg, 1, (N, K), -0.05, 0.05)
    assert _tol_violations(_gemv(env, x, W), oracle.gemv(x, W)) == 0
    xi = datagen.integer_f16(cfg, 10, (K,))
    Wi = datagen.integer_f16(cfg, 11, (N, K))
    assert np.array_equal(_gemv(env, xi, Wi), oracle.gemv(xi, Wi))


def test_degenerate_shapes(env):
    torch, gt, dev = env
    # K = 0: the empty sum, +0 everywhere (D starts as NaN)
    D = torch.full((33, 70), float("nan"), dtype=torch.float16, device=dev)
    A = torch.empty((33, 0), dtype=torch.float16, device=dev)
    B = torch.empty((70, 0), dtype=torch.float16, device=dev)
    gt.gemm_f16(A, B, D)
    torch.cuda.synchronize(dev)
    assert bool((D.view(torch.int16) == 0).all())
    y = torch.full((9,), float("nan"), dtype=torch.float16, device=dev)
    gt.gemv_f16(torch.empty((0,), dtype=torch.float16, device=dev), torch.empty((9, 0), dtype=torch.float16, device=dev), y)
    torch.cuda.synchronize(dev)
    assert bool((y.view(torch.int16) == 0).all())
    # M = 0 / N = 0: no-op
    gt.gemm_f16(torch.empty((0, 8), dtype=torch.float16, device=dev), torch.ones((5, 8), dtype=torch.float16, device=dev))
    gt.gemm_f16(torch.ones((5, 8), dtype=torch.float16, device=dev), torch.empty((0, 8), dtype=torch.float16, device=dev))
    torch.cuda.synchronize(dev)


def test_output_guard_band(env):
    """Only the M x N region is written: a NaN-filled guard band after D and
    the unwritten part of a larger buffer stay untouched."""
    torch, gt, dev = env
    M, N, K = 300, 260, 72
    A = datagen.integer_f16(5000, 0, (M, K))
    B = datagen.integer_f16(5000, 1, (N, K))
    guard = 4096
    buf = torch.full((M * N + guard,), float("nan"), dtype=torch.float16, device=dev)
    D = buf[: M * N].view(M, N)
    gt.gemm_f16(torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev), D)
    torch.cuda.synchronize(dev)
    assert bool(torch.isnan(buf[M * N :]).all())
    assert np.array_equal(D.cpu().numpy(), oracle.gemm(A, B))


TILED_VARIANTS = [1, 2, 3, 10, 20, 21, 22, 23, 24, 25, 26, 27, 28, 30, 31, 32]


@pytest.mark.parametrize("variant", TILED_VARIANTS)
def test_gemm_variants_bit_identical(env, variant):
    """The ablation kernels (no swizzle, one stage, non-persistent) give the
    same bits as the default on integer data; a pipeline race would not."""
    M, N, K = 520, 776, 4104
    A = datagen.integer_f16(6000, 0, (M, K))
    B = datagen.integer_f16(6000, 1, (N, K))
    base = _gemm(env, A, B, 0).cpu().numpy()
    assert np.array_equal(base, oracle.gemm(A, B))
    assert np.array_equal(_gemm(env, A, B, variant).cpu().numpy(), base)


@pytest.mark.parametrize("variant", [0, 2, 10, 20, 21, 22, 23, 24, 25, 26, 27, 30])
@pytest.mark.parametrize("K", [8, 64, 72, 128, 136, 192, 200, 264, 328])
def test_gemm_variants_few_k_tiles(env, variant, K):
    """1 to 6 K tiles of 64, whole and ragged: the prologue, the last refill
    and the ring drain take their short-K branches for every ring depth
    (2 to 5 stages).  Integer data, so every variant must match the oracle
    bit for bit."""
    M, N = 300, 260
    A = datagen.integer_f16(6100 + K, 0, (M, K))
    B = datagen.integer_f16(6100 + K, 1, (N, K))
    assert np.array_equal(_gemm(env, A, B, variant).cpu().numpy(), oracle.gemm(A, B))


# Outputs whose 256x256 tiles would leave CUs idle take smaller tiles: these
# route (with 256 CUs) to 256x128, 128x256, 128x128 and 128x64 tiles, with ragged M,
# N and K.  Sampled rows against the oracle; integer data bit-exact.
TILE_CHOICE_SHAPES = [(8192, 1000, 264, (256, 128)), (2176, 3832, 200, (128, 256)), (1000, 3000, 136, (128, 128)),
                      (1000, 1000, 264, (128, 64))]


@pytest.mark.parametrize("case", TILE_CHOICE_SHAPES, ids=lambda c: "x".join(map(str, c[:3])))
def test_gemm_tile_choice_shapes(env, case):
    torch, gt, dev = env
    M, N, K, tile = case
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    print(f"[tile choice] {M}x{N}x{K} on {cus} CUs -> {gt.gemm_tile(M, N, cus)}", flush=True)
    if cus == 256:
        assert gt.gemm_tile(M, N, cus)[:2] == tile
    cfg = 6200 + TILE_CHOICE_SHAPES.index(case)
    rows = np.sort(datagen.rng(cfg, 2).choice(M, 64, replace=False))
    A = datagen.uniform_f16(cfg, 0, (M, K), -1.0, 1.0)
    B = datagen.uniform_f16(cfg, 1, (N, K), -1.0, 1.0)
    D = _gemm(env, A, B)
    got = D[torch.from_numpy(rows).to(dev)].cpu().numpy()
    assert np.isfinite(D.float().cpu().numpy()).all()
    assert _tol_violations(got, oracle.gemm(A, B, rows=rows)) == 0
    Ai = datagen.integer_f16(cfg, 10, (M, K))
    Bi = datagen.integer_f16(cfg, 11, (N, K))
    Di = _gemm(env, Ai, Bi)
    assert np.array_equal(Di[torch.from_numpy(rows).to(dev)].cpu().numpy(), oracle.gemm(Ai, Bi, rows=rows))
    # every element of the last rows (the ragged tile row) as well
    last = np.arange(M - 40, M)
    assert np.array_equal(Di[torch.from_numpy(last).to(dev)].cpu().numpy(), oracle.gemm(Ai, Bi, rows=last))


@pytest.mark.parametrize("variant", [6, 7, 8, 9, 10, 11, 12, 20, 21, 28, 29, 37, 38, 39, 40, 41])
def test_gemv_variants_bit_identical(env, variant):
    N, K = 1031, 14344
    x = datagen.integer_f16(6001, 0, (K,))
    W = datagen.integer_f16(6001, 1, (N, K))
    base = _gemv(env, x, W, 0)
    assert np.array_equal(base, oracle.gemv(x, W))
    assert np.array_equal(_gemv(env, x, W, variant), base)


def test_side_stream_and_repeat(env):
    """Stream-ordered on a caller's stream; repeated calls give the same bits."""
    torch, gt, dev = env
    M, N, K = 777, 513, 1032
    A = torch.from_numpy(datagen.uniform_f16(7000, 0, (M, K), -1.0, 1.0)).to(dev)
    B = torch.from_numpy(datagen.uniform_f16(7000, 1, (N, K), -1.0, 1.0)).to(dev)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        D1 = gt.gemm_f16(A, B)
        D2 = gt.gemm_f16(A, B)
    s.synchronize()
    assert torch.equal(D1, D2)
    assert _tol_violations(D1.cpu().numpy(), oracle.gemm(A.cpu().numpy(), B.cpu().numpy())) == 0


def test_misaligned_pointer_is_rejected(env):
    torch, gt, dev = env
    base = torch.zeros((65, 64), dtype=torch.float16, device=dev)
    A = base.view(-1)[1 : 1 + 64 * 64].view(64, 64)  # 2-byte offset
    B = torch.zeros((64, 64), dtype=torch.float16, device=dev)
    with pytest.raises(gt.GemvTileError) as e:
        gt.gemm_f16(A, B)
    assert e.value.status == 2


def test_timed_gemm_matches_and_stamps_are_sane(env):
    """gemvtile_gemm_f16_timed computes what the 256x256 kernel computes, and
    each workgroup's stamps are ordered and give a plausible clock."""
    torch, gt, dev = env
    lib = gt.load_library()
    M, N, K = 1000, 1300, 1032
    Ai = datagen.integer_f16(6300, 10, (M, K))
    Bi = datagen.integer_f16(6300, 11, (N, K))
    tA, tB = torch.from_numpy(Ai).to(dev), torch.from_numpy(Bi).to(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    grid = min(((M + 255) // 256) * ((N + 255) // 256), cus)
    stamps = torch.zeros((grid * 8,), dtype=torch.int64, device=dev)
    D = torch.empty((M, N), dtype=torch.float16, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    assert lib.gemvtile_gemm_f16_timed(tA.data_ptr(), tB.data_ptr(), D.data_ptr(), M, N, K, s, stamps.data_ptr(),
                                       grid * 8 - 1) == 1  # too small a buffer
    assert lib.gemvtile_gemm_f16_timed(tA.data_ptr(), tB.data_ptr(), D.data_ptr(), M, N, K, s, stamps.data_ptr(),
                                       grid * 8) == 0
    torch.cuda.synchronize(dev)
    assert np.array_equal(D.cpu().numpy(), oracle.gemm(Ai, Bi))
    st = stamps.cpu().numpy().reshape(grid, 8).astype(np.int64)
    assert (st[:, 0] > 0).all() and (st[:, 0] <= st[:, 2]).all() and (st[:, 2] <= st[:, 4]).all()
    assert (st[:, 1] <= st[:, 3]).all() and (st[:, 3] <= st[:, 5]).all()
    mhz = (st[:, 5] - st[:, 1]) / np.maximum(st[:, 4] - st[:, 0], 1) * 100.0
    assert ((mhz > 300) & (mhz < 3500)).all(), mhz
    assert set((st[:, 7] & 0xF).tolist()) <= set(range(8))
