"""Parity of gemm_bias_f16 / gemm_bias_bf16 (fused bias and ReLU) with the oracle.

D = RNE(act(A·Bᵀ + bias)), bias [N] on every row, act identity or ReLU, one
rounding.  The same bar as the plain GEMM: bit-for-bit on integer data (sums
and bias exact in FP32), |d - ref| <= 1e-2 + 1e-2·|ref| on uniform data.
Shapes cover each output tile the tiled kernel picks, ragged edges (so the
bias columns past N and the masked stores both matter), shapes with 16 or
fewer rows on a side (which the fused epilogue runs on the tiled kernel),
K = 0, a NULL bias, and the 4096^3 workload on sampled rows.
"""
import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu

TOL_ABS = 1e-2
TOL_REL = 1e-2
RELU = oracle.ACT_RELU
NONE = oracle.ACT_NONE


@pytest.fixture(scope="module")
def env():
    import torch

    import gemv_tile_pipelined_amd as gt

    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    gt.load_library()
    return torch, gt, torch.device("cuda:0")


def _violations(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return int((~(np.abs(got - ref) <= TOL_ABS + TOL_REL * np.abs(ref))).sum())


def _run(env, A, B, bias, act, rows=None):
    torch, gt, dev = env
    t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    D = gt.gemm_bias_f16(t(A), t(B), None if bias is None else t(bias), act)
    torch.cuda.synchronize(dev)
    if rows is not None:
        D = D[torch.from_numpy(rows).to(dev)]
    return D.cpu().numpy()


# (M, N, K): 128x128 tiles, ragged; 256x128; 128x256; 256x256 (one full
# wave of tiles); 16 or fewer rows on a side; M = 1; one K tile.
SHAPES = [(300, 260, 200), (8192, 1000, 264), (2176, 3832, 200), (4096, 4096, 136), (8, 4100, 520),
          (1000, 5, 264), (1, 777, 72), (257, 129, 8)]


def _rows(M, cfg):
    if M <= 512:
        return None
    r = datagen.rng(cfg, 2).choice(M, 48, replace=False)
    return np.unique(np.concatenate([r, np.arange(M - 8, M)]))  # and the ragged last rows


@pytest.mark.parametrize("act", [NONE, RELU], ids=["none", "relu"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_bias_integer_exact(env, shape, act):
    M, N, K = shape
    cfg = 9800 + SHAPES.index(shape)
    A = datagen.integer_f16(cfg, 10, (M, K))
    B = datagen.integer_f16(cfg, 11, (N, K))
    bias = datagen.integer_f16(cfg, 3, (N,), -300, 300)
    rows = _rows(M, cfg)
    got = _run(env, A, B, bias, act, rows)
    assert np.array_equal(got, oracle.gemm_bias(A, B, bias, act, rows=rows))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_bias_uniform(env, shape):
    M, N, K = shape
    cfg = 9900 + SHAPES.index(shape)
    A = datagen.uniform_f16(cfg, 0, (M, K), -1.0, 1.0)
    B = datagen.uniform_f16(cfg, 1, (N, K), -1.0, 1.0)
    bias = datagen.uniform_f16(cfg, 3, (N,), -4.0, 4.0)
    rows = _rows(M, cfg)
    for act in (NONE, RELU):
        got = _run(env, A, B, bias, act, rows)
        assert np.isfinite(got).all()
        assert _violations(got, oracle.gemm_bias(A, B, bias, act, rows=rows)) == 0, act


def test_gemm_bias_null_bias_and_k0(env):
    torch, gt, dev = env
    M, N, K = 300, 260, 520
    A = datagen.integer_f16(9850, 10, (M, K))
    B = datagen.integer_f16(9850, 11, (N, K))
    # no bias: identity equals gemm_f16, ReLU clamps the plain sums
    assert np.array_equal(_run(env, A, B, None, NONE), oracle.gemm(A, B))
    assert np.array_equal(_run(env, A, B, None, RELU), oracle.gemm_bias(A, B, None, RELU))
    # K = 0: D = act(bias) on every row (A and B may be NULL)
    bias = np.array([-3.0, -0.5, 0.0, 0.25, 7.0] * 52, np.float16)[:N]
    A0 = torch.empty((M, 0), dtype=torch.float16, device=dev)
    B0 = torch.empty((N, 0), dtype=torch.float16, device=dev)
    for act in (NONE, RELU):
        D = gt.gemm_bias_f16(A0, B0, torch.from_numpy(bias).to(dev), act)
        torch.cuda.synchronize(dev)
        want = oracle.gemm_bias(np.zeros((M, 8), np.float16), np.zeros((N, 8), np.float16), bias, act)
        assert np.array_equal(D.cpu().numpy().view(np.uint16), want.view(np.uint16)), act


def test_gemm_bias_full_size_every_element(env, full_size):
    """The 4096^3 workload with a bias and ReLU against the oracle on every
    output element (uniform inputs), and bit for bit on integer inputs with
    an integer bias."""
    w = datagen.WORKLOADS[1]
    print(f"[gemm_bias full size] {w.name} relu", flush=True)
    A, B = full_size.inputs(1)
    bias = datagen.uniform_f16(1, 3, (w.N,), -4.0, 4.0)
    got = _run(env, A, B, bias, RELU)
    assert _violations(got, oracle.gemm_bias(A, B, bias, RELU)) == 0
    assert (got == 0).mean() > 0.3  # ReLU did clamp a good part of the outputs
    Ai, Bi = full_size.inputs(1, True)
    bias_i = datagen.integer_f16(1, 13, (w.N,), -64, 64)
    assert np.array_equal(_run(env, Ai, Bi, bias_i, RELU), oracle.gemm_bias(Ai, Bi, bias_i, RELU))


@pytest.mark.parametrize("shape", [(300, 260, 200), (8192, 1000, 264), (8, 4100, 520)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_bias_bf16(env, shape):
    torch, gt, dev = env
    M, N, K = shape
    cfg = 9950 + shape[0] % 89
    A = datagen.integer_bf16(cfg, 10, (M, K))
    B = datagen.integer_bf16(cfg, 11, (N, K))
    bias = datagen.integer_bf16(cfg, 3, (N,), -300, 300)
    rows = _rows(M, cfg)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    for act in (NONE, RELU):
        D = gt.gemm_bias_bf16(dev_bf16(A), dev_bf16(B), dev_bf16(bias), act)
        torch.cuda.synchronize(dev)
        if rows is not None:
            D = D[torch.from_numpy(rows).to(dev)]
        got = D.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, oracle.gemm_bias_bf16(A, B, bias, act, rows=rows)), act
