"""Parity of the bf16 entry points (gemm_bf16, gemv_bf16) with the CPU oracle.

The SM120 page's §2.3 kernel reads bf16 operands, accumulates in FP32 and
rounds the result to bf16 to nearest.  numpy has no bfloat16 dtype, so every
array on the numpy side holds bf16 bit patterns (uint16) and the oracle takes
and returns those.

Bar, as for fp16: |d - ref| <= 1e-2 + 1e-2·|ref| elementwise for uniform
inputs (a bf16 result may sit one bf16 ulp, 2^-8 relative, from the oracle's
correctly rounded one); bit-for-bit for integer-valued inputs, whose FP32
partial sums are exact in any order (|sums| <= K·64 < 2^24), so only the final
round-to-nearest-even decides.  The tiled path (4096^3, the ragged
4000x4032x4104), the skinny path (decode batch 8x4096x14336, small N) and the
GEMV (4096x14336) are all covered, the full sizes compared with the oracle on
every element, plus a closed form on every element.
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
    gt.load_library()
    return torch, gt, torch.device("cuda:0")


def _dev(env, bits):
    """uint16 bit patterns -> device bfloat16 tensor (same bits)."""
    torch, _, dev = env
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def _bits(t):
    """device bfloat16 tensor -> uint16 bit patterns."""
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _gemm(env, A, B):
    torch, gt, dev = env
    D = gt.gemm_bf16(_dev(env, A), _dev(env, B))
    torch.cuda.synchronize(dev)
    return D


def _gemv(env, x, W):
    torch, gt, dev = env
    y = gt.gemv_bf16(_dev(env, x), _dev(env, W))
    torch.cuda.synchronize(dev)
    return _bits(y)


def _violations(got_bits, ref_bits):
    got = oracle.bf16_to_f64(got_bits)
    ref = oracle.bf16_to_f64(ref_bits)
    return int((~(np.abs(got - ref) <= TOL_ABS + TOL_REL * np.abs(ref))).sum())


def _to_bf16_bits(values):
    """Exactly representable float values -> bf16 bit patterns."""
    f = np.asarray(values, np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), f), "value not bf16-exact"
    return bits


# Tiled shapes (one full tile, ragged M/N/K tails, long K), the shapes that
# route to the GEMV (M or N == 1) and to the skinny kernel (M or N <= 16, and
# 17..64 rows on the smaller side against few large-side rows: 64x64,
# 1000x33 and the three after 520x5).
SHAPES = [
    (256, 256, 256),
    (300, 260, 200),
    (257, 255, 136),
    (513, 1000, 520),
    (64, 64, 4104),
    (1000, 33, 64),
    (520, 776, 1032),
    (1, 1, 8),
    (1, 4096, 1032),
    (777, 1, 520),
    (3, 17, 8),
    (8, 4096, 4104),
    (16, 1000, 1032),
    (4000, 16, 520),
    (520, 5, 1032),
    (32, 4096, 4104),
    (4000, 48, 520),
    (24, 300, 8200),
    # 4 large-side rows per workgroup with 32 and 64 staged small-side rows,
    # and the 64-row staging at 16 large-side rows per workgroup
    (24, 1500, 4104),
    (48, 1500, 1032),
    (1000, 50, 2056),
    (8200, 40, 1032),
    (16, 8192, 2056),
    (10300, 40, 1032),
    (64, 16384, 264),
    (48, 4096, 4104),
    # 32 large-side rows per workgroup
    (20, 8192, 4096),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_bf16_uniform(env, shape):
    M, N, K = shape
    cfg = 8000 + SHAPES.index(shape)
    A = datagen.uniform_bf16(cfg, 0, (M, K), -1.0, 1.0)
    B = datagen.uniform_bf16(cfg, 1, (N, K), -1.0, 1.0)
    got = _bits(_gemm(env, A, B))
    ref = oracle.gemm_bf16(A, B)
    assert np.isfinite(oracle.bf16_to_f64(got)).all()
    assert _violations(got, ref) == 0


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_bf16_integer_exact(env, shape):
    M, N, K = shape
    cfg = 8100 + SHAPES.index(shape)
    A = datagen.integer_bf16(cfg, 0, (M, K))
    B = datagen.integer_bf16(cfg, 1, (N, K))
    assert np.array_equal(_bits(_gemm(env, A, B)), oracle.gemm_bf16(A, B))


@pytest.mark.parametrize("shape", [(8192, 1000, 264), (2176, 3832, 200)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_bf16_smaller_tiles(env, shape):
    """Shapes that take 256x128 and 128x256 tiles: sampled rows, integer data
    bit-exact and uniform data within the bar."""
    torch, gt, dev = env
    M, N, K = shape
    cfg = 8300 + shape[0] % 97
    rows = np.sort(datagen.rng(cfg, 2).choice(M, 48, replace=False))
    Ai = datagen.integer_bf16(cfg, 10, (M, K))
    Bi = datagen.integer_bf16(cfg, 11, (N, K))
    got = _bits(_gemm(env, Ai, Bi)[torch.from_numpy(rows).to(dev)])
    assert np.array_equal(got, oracle.gemm_bf16(Ai, Bi, rows=rows))
    A = datagen.uniform_bf16(cfg, 0, (M, K), -1.0, 1.0)
    B = datagen.uniform_bf16(cfg, 1, (N, K), -1.0, 1.0)
    got = _bits(_gemm(env, A, B)[torch.from_numpy(rows).to(dev)])
    assert _violations(got, oracle.gemm_bf16(A, B, rows=rows)) == 0


def _load_probe():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "bf16_rne_probe.txt")
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


def _probe(env, subnormal_result):
    seen = 0
    for av, bv, want in _load_probe():
        exact = sum(a * b for a, b in zip(av, bv))  # exact in float64 for these probes
        if (0.0 < abs(exact) < 2.0**-126) != subnormal_result:
            continue
        seen += 1
        A = _to_bf16_bits([av])
        B = _to_bf16_bits([bv])
        D = _bits(_gemm(env, A, B))
        assert int(D[0, 0]) == want, ("gemm", av, bv, hex(int(D[0, 0])))
        y = _gemv(env, A[0], B)
        assert int(y[0]) == want, ("gemv", av, bv, hex(int(y[0])))
        # the skinny kernel: the probe row among 7 zero rows (M = 8)
        A8 = np.zeros((8, 8), np.uint16)
        A8[5] = A[0]
        B3 = np.zeros((3, 8), np.uint16)
        B3[1] = B[0]
        D8 = _bits(_gemm(env, A8, B3))
        assert int(D8[5, 1]) == want, ("skinny", av, bv, hex(int(D8[5, 1])))
    assert seen > 0


def test_bf16_rne_probe_normal_results(env):
    """Ties-to-even and overflow of the final bf16 rounding (printed probes)."""
    _probe(env, subnormal_result=False)


def test_bf16_rne_probe_subnormal_results(env):
    """Sums below the smallest normal (2^-126, shared by FP32 and bf16): the
    FP32 accumulator and the conversion must keep subnormals and round them
    to nearest-even."""
    _probe(env, subnormal_result=True)


@pytest.mark.parametrize("integer", [False, True], ids=["uniform", "integer"])
@pytest.mark.parametrize("cfg_id", [1, 2], ids=["4096cube", "ragged_4000x4032x4104"])
def test_gemm_bf16_full_size_every_element(env, full_size, cfg_id, integer):
    """4096^3 and 4000x4032x4104 in bf16 against the oracle on every output
    element: uniform within the tolerance, integer bit for bit."""
    torch, gt, dev = env
    w = datagen.WORKLOADS[cfg_id]
    print(f"[gemm_bf16 full size] {w.name} M={w.M} N={w.N} K={w.K} integer={integer}", flush=True)
    A, B = full_size.inputs(cfg_id, integer, True)
    D = _gemm(env, A, B)
    got = _bits(D)
    ref = full_size.reference(cfg_id, integer, True)
    if integer:
        assert np.array_equal(got, ref)
    else:
        assert bool(torch.isfinite(D).all())
        assert _violations(got, ref) == 0


@pytest.mark.parametrize("cfg_id", [1, 2], ids=["4096cube", "ragged_4000x4032x4104"])
def test_gemm_bf16_full_size_rank1_every_element(env, cfg_id):
    """Closed form on every output: A[m,k] = u_m, B[n,k] = v_n -> K·u_m·v_n."""
    torch, gt, dev = env
    w = datagen.WORKLOADS[cfg_id]
    g = datagen.rng(cfg_id, 21)
    choices = np.array([-1.0, -0.5, -0.25, -0.125, 0.125, 0.25, 0.5, 1.0])
    u, v = g.choice(choices, w.M), g.choice(choices, w.N)
    tu = torch.from_numpy(u).to(dev).to(torch.bfloat16)
    tv = torch.from_numpy(v).to(dev).to(torch.bfloat16)
    A = tu[:, None].expand(w.M, w.K).contiguous()
    B = tv[:, None].expand(w.N, w.K).contiguous()
    D = gt.gemm_bf16(A, B)
    # K·u·v = K·2^-j: K = 4096 is a power of two, 4104 = 2^3·513 needs 10
    # significant bits, so the expected value is K·u·v rounded to bf16.
    want = (w.K * torch.outer(tu.double(), tv.double())).to(torch.bfloat16)
    torch.cuda.synchronize(dev)
    assert bool((D == want).all())


def test_decode_batch_bf16(env):
    """The decode batch 8x4096x14336 on the skinny kernel, compared in full."""
    w = datagen.DECODE_BATCH
    A = datagen.uniform_bf16(w.cfg_id, 0, (w.M, w.K), w.lo_a, w.hi_a)
    B = datagen.uniform_bf16(w.cfg_id, 1, (w.N, w.K), w.lo_b, w.hi_b)
    got = _bits(_gemm(env, A, B))
    assert _violations(got, oracle.gemm_bf16(A, B)) == 0
    Ai = datagen.integer_bf16(w.cfg_id, 10, (w.M, w.K))
    Bi = datagen.integer_bf16(w.cfg_id, 11, (w.N, w.K))
    assert np.array_equal(_bits(_gemm(env, Ai, Bi)), oracle.gemm_bf16(Ai, Bi))


def test_gemv_bf16_workload(env):
    w = datagen.WORKLOADS[3]
    x, W = datagen.gemv_inputs(w, bf16=True)
    got = _gemv(env, x, W)
    assert np.isfinite(oracle.bf16_to_f64(got)).all()
    assert _violations(got, oracle.gemv_bf16(x, W)) == 0
    xi, Wi = datagen.gemv_inputs(w, integer=True, bf16=True)
    assert np.array_equal(_gemv(env, xi, Wi), oracle.gemv_bf16(xi, Wi))
    # unit vectors pick columns of W
    for j in (0, 7, 8, 14335):
        e = np.zeros(w.K, np.uint16)
        e[j] = 0x3F80  # 1.0
        assert np.array_equal(_gemv(env, e, W), np.ascontiguousarray(W[:, j]))


GEMV_SHAPES = [(1, 8), (7, 520), (4097, 14336), (1000, 14344), (33, 16392), (16, 1032)]


@pytest.mark.parametrize("shape", GEMV_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemv_bf16_ragged(env, shape):
    N, K = shape
    cfg = 8200 + GEMV_SHAPES.index(shape)
    x = datagen.uniform_bf16(cfg, 0, (K,), -1.0, 1.0)
    W = datagen.uniform_bf16(cfg, 1, (N, K), -0.05, 0.05)
    assert _violations(_gemv(env, x, W), oracle.gemv_bf16(x, W)) == 0
    xi = datagen.integer_bf16(cfg, 10, (K,))
    Wi = datagen.integer_bf16(cfg, 11, (N, K))
    assert np.array_equal(_gemv(env, xi, Wi), oracle.gemv_bf16(xi, Wi))


def test_bf16_degenerate_and_guard(env):
    torch, gt, dev = env
    bf = torch.bfloat16
    # K = 0: the empty sum, +0 everywhere (D starts as NaN)
    D = torch.full((33, 70), float("nan"), dtype=bf, device=dev)
    gt.gemm_bf16(torch.empty((33, 0), dtype=bf, device=dev), torch.empty((70, 0), dtype=bf, device=dev), D)
    y = torch.full((9,), float("nan"), dtype=bf, device=dev)
    gt.gemv_bf16(torch.empty((0,), dtype=bf, device=dev), torch.empty((9, 0), dtype=bf, device=dev), y)
    torch.cuda.synchronize(dev)
    assert bool((D.view(torch.int16) == 0).all())
    assert bool((y.view(torch.int16) == 0).all())
    # only the M x N region is written (tiled and skinny shapes)
    for M, N, K in ((300, 260, 72), (6, 700, 1032)):
        A = datagen.integer_bf16(8300, 0, (M, K))
        B = datagen.integer_bf16(8300, 1, (N, K))
        guard = 4096
        buf = torch.full((M * N + guard,), float("nan"), dtype=bf, device=dev)
        Dv = buf[: M * N].view(M, N)
        gt.gemm_bf16(_dev(env, A), _dev(env, B), Dv)
        torch.cuda.synchronize(dev)
        assert bool(torch.isnan(buf[M * N :]).all())
        assert np.array_equal(_bits(Dv), oracle.gemm_bf16(A, B))


def test_bf16_rejects_fp16_tensors(env):
    torch, gt, dev = env
    A = torch.zeros((64, 64), dtype=torch.float16, device=dev)
    with pytest.raises(TypeError):
        gt.gemm_bf16(A, A)
    with pytest.raises(TypeError):
        gt.gemv_bf16(A[0], A)
