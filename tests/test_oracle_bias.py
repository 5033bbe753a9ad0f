"""Pins of the oracle's GEMM with a bias and an activation, against
references that share none of its code.

The pages define no fused epilogue; the oracle takes the plain definition
D = RNE(act(A·Bᵀ + bias)), bias [N] added to every row, act the identity or
ReLU (v < 0 -> +0), one rounding at the end.  Each check below fixes one part:
  * the bias is broadcast along rows (indexed by n, not m)  -> zero A, so
    D is the bias itself; integer data with a bias that varies along n;
  * the activation comes after the bias                      -> integer sums
    that the bias moves across zero;
  * the activation is ReLU, not |v| or a shifted clamp      -> negative
    outputs become +0, positive ones are unchanged;
  * one rounding of the exact value                          -> math.fsum of
    the products and the bias, correctly rounded, then numpy's RNE cast (or,
    for bf16, integer round-to-nearest-even on float32 bits);
  * without a bias and activation it is the plain GEMM.
"""
import math

import numpy as np
import pytest

import datagen
import oracle
from test_oracle import _as_f64, _bits, _near_fp16_midpoint, _rne_numpy
from test_oracle_bf16 import _bf16_value, _f32_bits_to_bf16_rne, _near_bf16_midpoint

RELU = oracle.ACT_RELU
NONE = oracle.ACT_NONE


def _relu(v):
    v = np.asarray(v, np.float64)
    return np.where(v < 0, 0.0, v)


def check_bias_broadcast_zero_a(lib):
    """A = 0: every row of D is act(bias), rounded once (exact here)."""
    N, K = 11, 24
    bias = np.array([-65504.0, -3.5, -2.0**-24, -0.0, 0.0, 2.0**-14, 0.5, 1.0, 7.25, 1024.0, 65504.0], np.float16)
    B = datagen.uniform_f16(700, 1, (N, K), -1.0, 1.0)
    A = np.zeros((5, K), np.float16)
    for act in (NONE, RELU):
        D = oracle.gemm_bias(A, B, bias, act, lib=lib)
        want = _rne_numpy(_relu(0.0 + _as_f64(bias)) if act == RELU else 0.0 + _as_f64(bias))
        for row in D:
            assert np.array_equal(_bits(row), _bits(want)), act


def check_bias_integer_exact(lib):
    """Integer A, B and bias: the exact int64 sum plus bias[n], ReLU after
    the bias, and numpy's RNE of the (exact) result."""
    flips = 0
    for i, (M, N, K) in enumerate([(9, 7, 33), (16, 40, 520), (3, 5, 4104)]):
        A = datagen.integer_f16(720 + i, 0, (M, K))
        B = datagen.integer_f16(720 + i, 1, (N, K))
        bias = datagen.integer_f16(720 + i, 3, (N,), -300, 300)
        exact = A.astype(np.int64) @ B.astype(np.int64).T + bias.astype(np.int64)[None, :]
        assert (exact < 0).any() and (exact > 0).any()
        for act in (NONE, RELU):
            D = oracle.gemm_bias(A, B, bias, act, lib=lib)
            want = np.where(exact < 0, 0, exact) if act == RELU else exact
            assert np.array_equal(_bits(D), _bits(_rne_numpy(want))), (M, N, K, act)
        plain = A.astype(np.int64) @ B.astype(np.int64).T
        flips += int(((plain < 0) != (exact < 0)).sum())
    # the bias must be what moves sums across zero in some places, so that
    # ReLU before the bias would give other results
    assert flips > 0


def check_bias_fsum(lib):
    """Uniform data: math.fsum of the exact products and the bias, correctly
    rounded, then ReLU and numpy's RNE; a mismatch is allowed only right at a
    rounding midpoint.  Also on a subset of rows."""
    for i, (M, N, K) in enumerate([(1, 1, 1), (3, 17, 64), (17, 3, 65), (20, 33, 130)]):
        A = datagen.uniform_f16(740 + i, 0, (M, K), -1.0, 1.0)
        B = datagen.uniform_f16(740 + i, 1, (N, K), -1.0, 1.0)
        bias = datagen.uniform_f16(740 + i, 3, (N,), -4.0, 4.0)
        A64, B64, b64 = _as_f64(A), _as_f64(B), _as_f64(bias)
        exact = np.array([[math.fsum((A64[m] * B64[n]).tolist() + [b64[n]]) for n in range(N)] for m in range(M)])
        for act in (NONE, RELU):
            v = _relu(exact) if act == RELU else exact
            D = oracle.gemm_bias(A, B, bias, act, lib=lib)
            same = _bits(D) == _bits(_rne_numpy(v))
            assert np.all(same | _near_fp16_midpoint(v)), (M, N, K, act)
            if M > 2:
                rows = np.array([M - 1, 0, M // 2])
                Dr = oracle.gemm_bias(A, B, bias, act, rows=rows, lib=lib)
                assert np.array_equal(_bits(Dr), _bits(D[rows]))


def check_bias_relu_values(lib):
    """ReLU maps negative outputs to +0 (not |v|, not another threshold) and
    leaves positive ones, and a NaN, as they are."""
    K = 8
    A = np.zeros((1, K), np.float16)
    A[0, 0] = 1.0
    vals = np.array([-5.0, -0.5, -2.0**-20, 0.25, 3.0, 100.0], np.float16)
    B = np.zeros((vals.size, K), np.float16)
    B[:, 0] = vals
    D = oracle.gemm_bias(A, B, None, RELU, lib=lib)
    want = np.where(_as_f64(vals) < 0, 0.0, _as_f64(vals)).astype(np.float16)
    assert np.array_equal(_bits(D[0]), _bits(want))
    assert (_bits(D[0])[:3] == 0).all()  # +0, not -0
    An = A.copy()
    An[0, 0] = np.inf
    Bn = np.zeros((1, K), np.float16)  # inf * 0 = NaN
    assert np.isnan(oracle.gemm_bias(An, Bn, None, RELU, lib=lib).astype(np.float64)).all()


def check_bias_none_is_plain_gemm(lib):
    A = datagen.uniform_f16(760, 0, (13, 72), -1.0, 1.0)
    B = datagen.uniform_f16(760, 1, (21, 72), -1.0, 1.0)
    assert np.array_equal(_bits(oracle.gemm_bias(A, B, None, NONE, lib=lib)), _bits(oracle.gemm(A, B, lib=lib)))
    zero = np.zeros((21,), np.float16)
    assert np.array_equal(_bits(oracle.gemm_bias(A, B, zero, NONE, lib=lib)), _bits(oracle.gemm(A, B, lib=lib)))


def check_bias_bf16(lib):
    """bf16: integer data exact (integer RNE on float32 bits), uniform data
    against math.fsum, both with the bias and ReLU."""
    M, N, K = 7, 19, 520
    A = datagen.integer_bf16(780, 0, (M, K))
    B = datagen.integer_bf16(780, 1, (N, K))
    bias = datagen.integer_bf16(780, 3, (N,), -300, 300)
    Ai, Bi, bi = (_bf16_value(x).astype(np.int64) for x in (A, B, bias))
    exact = Ai @ Bi.T + bi[None, :]
    for act in (NONE, RELU):
        want = np.where(exact < 0, 0, exact) if act == RELU else exact
        got = oracle.gemm_bias_bf16(A, B, bias, act, lib=lib)
        assert np.array_equal(got, _f32_bits_to_bf16_rne(want.astype(np.float32))), act
    Au = datagen.uniform_bf16(781, 0, (5, 64), -1.0, 1.0)
    Bu = datagen.uniform_bf16(781, 1, (9, 64), -1.0, 1.0)
    bu = datagen.uniform_bf16(781, 3, (9,), -4.0, 4.0)
    A64, B64, b64 = _bf16_value(Au), _bf16_value(Bu), _bf16_value(bu)
    ex = np.array([[math.fsum((A64[m] * B64[n]).tolist() + [b64[n]]) for n in range(9)] for m in range(5)])
    v = _relu(ex)
    got = oracle.gemm_bias_bf16(Au, Bu, bu, RELU, lib=lib)
    same = got == _f32_bits_to_bf16_rne(v.astype(np.float32))
    assert np.all(same | _near_bf16_midpoint(v))


ALL_CHECKS = [
    check_bias_broadcast_zero_a,
    check_bias_integer_exact,
    check_bias_fsum,
    check_bias_relu_values,
    check_bias_none_is_plain_gemm,
    check_bias_bf16,
]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_bias_pin(check, oracle_lib):
    check(oracle_lib)


def test_bad_activation_rejected(oracle_lib):
    A = np.ones((2, 8), np.float16)
    with pytest.raises(ValueError):
        oracle.gemm_bias(A, A, None, 2, lib=oracle_lib)
