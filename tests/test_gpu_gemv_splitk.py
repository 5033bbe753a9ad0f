"""Parity of the GEMV's K-split launches with the CPU oracle.

For N below 16 rows per compute unit, gemv_f16 splits K over the waves of a
workgroup (2, 4 or 8 slices, or one row per workgroup in 8 slices) and adds
the slices' FP32 row sums in LDS in slice order ("Learning TileLang with
GEMV", §5.2 block_split_k: split K when N alone gives too few blocks); for
K >= 8192 it takes 2 rows per workgroup in 8 slices whatever N.  Each level
is exercised at sizes around its thresholds (on a 256-CU part: N >= 4096,
2048, 1024, 512, else 1 row; K >= 8192), on both sides of the size from
which W is read with non-temporal loads (2^25 elements), with K tails that
leave slices partly or wholly empty (K = 8 is one 16-byte chunk, so only the
last slice has work).

Bar as elsewhere: |d - ref| <= 1e-2 + 1e-2·|ref| for uniform inputs,
bit-for-bit for integer inputs (exact FP32 partial sums in any order).
"""
import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu

TOL_ABS = 1e-2
TOL_REL = 1e-2
SPLIT_VARIANTS = (8, 9, 10, 11, 12)  # 16, 8, 4, 2 rows per workgroup; 1 row in 8 slices


@pytest.fixture(scope="module")
def env():
    import torch

    import gemv_tile_pipelined_amd as gt

    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    gt.load_library()
    return torch, gt, torch.device("cuda:0")


def _gemv(env, x, W, variant=0):
    torch, gt, dev = env
    y = gt.gemv_f16(torch.from_numpy(x).to(dev), torch.from_numpy(W).to(dev), variant=variant)
    torch.cuda.synchronize(dev)
    return y.cpu().numpy()


def _violations(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return int((~(np.abs(got - ref) <= TOL_ABS + TOL_REL * np.abs(ref))).sum())


# (N, K): every split level, both sides of each threshold, ragged K tails
# (K/8 not a multiple of 64), and K shorter than one step per slice.
SHAPES = [
    (4095, 4104),  # 8 rows per workgroup (2 slices)
    (2048, 4096),
    (2047, 520),  # 4 rows (4 slices)
    (1024, 4104),
    (1031, 72),
    (1000, 4096),  # 2 rows (8 slices)
    (4097, 8192),  # K >= 8192: 2 rows (8 slices) whatever N
    (4096, 8184),  # just below: 16 rows, no split
    (8192, 4096),  # W of 2^25 elements: non-temporal loads
    (8192, 4088),  # just below: cached loads
    (2048, 14336),
    (1024, 14344),
    (512, 16392),
    (511, 14336),  # 1 row (8 slices)
    (257, 8),
    (100, 65544),
    (7, 1032),
    (1, 8),
    (1, 14336),
    (3, 520),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemv_split_uniform_and_integer(env, shape):
    N, K = shape
    cfg = 9000 + SHAPES.index(shape)
    x = datagen.uniform_f16(cfg, 0, (K,), -1.0, 1.0)
    W = datagen.uniform_f16(cfg, 1, (N, K), -0.05, 0.05)
    got = _gemv(env, x, W)
    assert np.isfinite(got).all()
    assert _violations(got, oracle.gemv(x, W)) == 0
    xi = datagen.integer_f16(cfg, 10, (K,))
    Wi = datagen.integer_f16(cfg, 11, (N, K))
    assert np.array_equal(_gemv(env, xi, Wi), oracle.gemv(xi, Wi))


@pytest.mark.parametrize("variant", SPLIT_VARIANTS)
@pytest.mark.parametrize("shape", [(1031, 14344), (300, 4104), (17, 8), (64, 1032)], ids=lambda s: "x".join(map(str, s)))
def test_gemv_split_variants_bit_identical(env, variant, shape):
    """Each forced split level gives the oracle's bits on integer data,
    whatever N (a slice that is skipped or read twice would not)."""
    N, K = shape
    cfg = 9100 + variant
    xi = datagen.integer_f16(cfg, 10, (K,))
    Wi = datagen.integer_f16(cfg, 11, (N, K))
    assert np.array_equal(_gemv(env, xi, Wi, variant), oracle.gemv(xi, Wi))


def test_gemv_split_closed_forms(env):
    """Unit vectors pick columns of W (one slice holds the only nonzero
    product); all-ones sums to K on every row."""
    N, K = 700, 14336
    W = datagen.uniform_f16(9200, 1, (N, K), -1.0, 1.0)
    for j in (0, 511, 512, 7167, 14335):
        e = np.zeros(K, np.float16)
        e[j] = 1.0
        assert np.array_equal(_gemv(env, e, W).view(np.uint16), np.ascontiguousarray(W[:, j]).view(np.uint16))
    ones = _gemv(env, np.ones(K, np.float16), np.ones((N, K), np.float16))
    assert np.all(ones == np.float16(K))


def test_gemm_one_row_takes_split_gemv(env):
    """gemm_f16 with M == 1 (or N == 1) runs the GEMV; at 1000 rows that is
    the 8-slice launch."""
    torch, gt, dev = env
    K = 4104
    A = datagen.integer_f16(9300, 0, (1, K))
    B = datagen.integer_f16(9300, 1, (1000, K))
    D = gt.gemm_f16(torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev))
    torch.cuda.synchronize(dev)
    assert np.array_equal(D.cpu().numpy(), oracle.gemm(A, B))
    D2 = gt.gemm_f16(torch.from_numpy(B).to(dev), torch.from_numpy(A).to(dev))
    torch.cuda.synchronize(dev)
    assert np.array_equal(D2.cpu().numpy(), oracle.gemm(B, A))


@pytest.mark.parametrize("shape", [(1024, 14336), (300, 4104), (1, 520)], ids=lambda s: "x".join(map(str, s)))
def test_gemv_bf16_split(env, shape):
    torch, gt, dev = env
    N, K = shape
    cfg = 9400 + N
    for integer in (False, True):
        if integer:
            x = datagen.integer_bf16(cfg, 10, (K,))
            W = datagen.integer_bf16(cfg, 11, (N, K))
        else:
            x = datagen.uniform_bf16(cfg, 0, (K,), -1.0, 1.0)
            W = datagen.uniform_bf16(cfg, 1, (N, K), -0.05, 0.05)
        tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        tW = torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).to(dev)
        y = gt.gemv_bf16(tx, tW)
        torch.cuda.synchronize(dev)
        got = y.view(torch.int16).cpu().numpy().view(np.uint16)
        ref = oracle.gemv_bf16(x, W)
        if integer:
            assert np.array_equal(got, ref)
        else:
            assert _violations(oracle.bf16_to_f64(got), oracle.bf16_to_f64(ref)) == 0
