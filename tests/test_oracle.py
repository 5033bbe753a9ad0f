"""Pins of the CPU oracle against things other than itself.

Each check below is written as a function of the loaded oracle library so
that ``test_oracle_mutants.py`` can run the same checks against copies of
the oracle with a planted mistake and show that some check fails.

What pins what:
  * fp16 decode / RNE encode  -> numpy's own binary16 conversions over every
    bit pattern, every midpoint and off-midpoint points; the printed rounding
    probes in tests/golden/rne_probe.txt.
  * GEMM / GEMV sums          -> math.fsum of the exact products (correctly
    rounded), numpy float64 matmul, exact int64 sums for integer inputs.
  * indexing / orientation    -> closed forms: all-ones, A = I, B = I,
    rank-1 outer products, unit vectors for the GEMV.
"""
import math
import os

import numpy as np
import pytest

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TOL_ABS = 1e-2
TOL_REL = 1e-2


def _as_f64(a):
    return np.asarray(a, dtype=np.float64)


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float16).view(np.uint16)


def _rne_numpy(v):
    """numpy's double -> binary16 cast (round to nearest, ties to even)."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float16)


def _within_tol(d, ref):
    d = _as_f64(d)
    ref = _as_f64(ref)
    return np.abs(d - ref) <= TOL_ABS + TOL_REL * np.abs(ref)


def _near_fp16_midpoint(v, rel=1e-9):
    """True where float64 value v lies within rel of a point halfway between
    two neighbouring fp16 values (where an FP64 summation-order difference may
    legitimately flip the rounding)."""
    v = _as_f64(v)
    lo = v.astype(np.float16)
    lo64 = lo.astype(np.float64)
    up = np.where(lo64 <= v, np.nextafter(lo, np.float16(np.inf)), np.nextafter(lo, np.float16(-np.inf)))
    mid = (lo64 + up.astype(np.float64)) / 2.0
    return np.abs(v - mid) <= rel * np.maximum(np.abs(v), 1e-30)


def fsum_gemm(A, B):
    """Correctly rounded double of each exact sum of products."""
    A64, B64 = _as_f64(A), _as_f64(B)
    M, N = A64.shape[0], B64.shape[0]
    out = np.empty((M, N), np.float64)
    for m in range(M):
        for n in range(N):
            out[m, n] = math.fsum((A64[m] * B64[n]).tolist())
    return out


# --------------------------------------------------------------------------
# checks (each raises AssertionError on failure)
# --------------------------------------------------------------------------
def check_decode_all_patterns(lib):
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.f16_to_f64(bits, lib=lib)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, got[0x8000]) == -1.0


def check_encode_grid_and_midpoints(lib):
    finite = np.arange(65536, dtype=np.uint16).view(np.float16)
    finite = finite[np.isfinite(finite)]
    vals = np.unique(finite.astype(np.float64))  # sorted, -0 merged with +0
    # every representable value maps to itself
    got = oracle.f64_to_f16(vals, lib=lib)
    assert np.array_equal(got.astype(np.float64), vals)
    # midpoints between neighbours, and points just beside them
    mids = (vals[:-1] + vals[1:]) / 2.0
    for pts in (mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)):
        got = oracle.f64_to_f16(pts, lib=lib)
        assert np.array_equal(_bits(got), _bits(_rne_numpy(pts))), "midpoint rounding"
    # random doubles spread over the whole exponent range, both signs
    g = np.random.default_rng(1234)
    r = np.ldexp(g.uniform(1.0, 2.0, 200000), g.integers(-30, 17, 200000)) * g.choice([-1.0, 1.0], 200000)
    got = oracle.f64_to_f16(r, lib=lib)
    assert np.array_equal(_bits(got), _bits(_rne_numpy(r)))
    # special values
    spec = np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 1e10, -1e10, 2.0**-25, 3 * 2.0**-25])
    got = oracle.f64_to_f16(spec, lib=lib)
    assert np.array_equal(_bits(got), _bits(_rne_numpy(spec)))
    assert np.isnan(oracle.f64_to_f16(np.array([np.nan]), lib=lib)[0])


def _load_rne_probe():
    cases = []
    with open(os.path.join(GOLDEN, "rne_probe.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b, want, _why = [p.strip() for p in line.split("|")]
            av = [float.fromhex(t) if "p" in t else float(t) for t in a.split()]
            bv = [float.fromhex(t) if "p" in t else float(t) for t in b.split()]
            cases.append((av, bv, int(want, 16)))
    return cases


def check_rne_probe(lib):
    cases = _load_rne_probe()
    assert len(cases) >= 10
    for av, bv, want in cases:
        A = np.array([av], np.float16)
        B = np.array([bv], np.float16)
        assert np.array_equal(A.astype(np.float64), [av]) and np.array_equal(B.astype(np.float64), [bv])
        D = oracle.gemm(A, B, lib=lib)
        assert int(_bits(D)[0, 0]) == want, (av, bv, hex(int(_bits(D)[0, 0])), hex(want))
        # the same probe through the GEMV (x = a, W row = b)
        y = oracle.gemv(A[0], B, lib=lib)
        assert int(_bits(y)[0]) == want


def check_gemm_brute_force(lib):
    shapes = [(1, 1, 1), (3, 17, 64), (17, 3, 65), (64, 65, 130), (130, 1, 17), (5, 64, 3), (65, 130, 64)]
    for i, (M, N, K) in enumerate(shapes):
        A = datagen.uniform_f16(100 + i, 0, (M, K), -1.0, 1.0)
        B = datagen.uniform_f16(100 + i, 1, (N, K), -1.0, 1.0)
        D = oracle.gemm(A, B, lib=lib)
        exact = fsum_gemm(A, B)
        want = _rne_numpy(exact)
        same = _bits(D) == _bits(want)
        # a mismatch is only acceptable right at an fp16 rounding midpoint
        assert np.all(same | _near_fp16_midpoint(exact)), (M, N, K)
        assert same.mean() > 0.999
        assert np.all(_within_tol(D, exact))
        # and against numpy's float64 matmul
        np_ref = _as_f64(A) @ _as_f64(B).T
        assert np.all(_within_tol(D, np_ref))


def check_gemm_closed_forms(lib):
    # all-ones: every entry equals K exactly (all K used here are fp16-exact)
    for K in (1, 8, 256, 4104, 8192):
        D = oracle.gemm(np.ones((3, K), np.float16), np.ones((5, K), np.float16), lib=lib)
        assert np.all(_as_f64(D) == K), K
    # B = I  ->  D = A ;  A = I  ->  D = Bᵀ   (D = A·Bᵀ)
    A = datagen.uniform_f16(200, 0, (7, 9), -1.0, 1.0)
    D = oracle.gemm(A, np.eye(9, dtype=np.float16), lib=lib)
    assert np.array_equal(_bits(D), _bits(A))
    B = datagen.uniform_f16(200, 1, (11, 7), -1.0, 1.0)
    D = oracle.gemm(np.eye(7, dtype=np.float16), B, lib=lib)
    assert np.array_equal(_bits(D), _bits(np.ascontiguousarray(B.T)))
    # rank-1: A[m,k] = u_m, B[n,k] = v_n  ->  D = K u_m v_n exactly
    g = np.random.default_rng(7)
    choices = np.array([-2.0, -1.0, -0.5, -0.25, 0.25, 0.5, 1.0, 2.0])
    for K in (64, 4104):
        u = g.choice(choices, 13)
        v = g.choice(choices, 6)
        A = np.repeat(u[:, None], K, axis=1).astype(np.float16)
        B = np.repeat(v[:, None], K, axis=1).astype(np.float16)
        D = oracle.gemm(A, B, lib=lib)
        assert np.array_equal(_as_f64(D), K * np.outer(u, v)), K


def check_gemm_integer_exact(lib):
    for i, (M, N, K) in enumerate([(9, 7, 33), (16, 40, 520), (3, 5, 4104)]):
        A = datagen.integer_f16(300 + i, 0, (M, K))
        B = datagen.integer_f16(300 + i, 1, (N, K))
        exact = A.astype(np.int64) @ B.astype(np.int64).T  # exact in int64
        D = oracle.gemm(A, B, lib=lib)
        assert np.array_equal(_as_f64(D), _as_f64(_rne_numpy(exact.astype(np.float64)))), (M, N, K)


def check_gemm_rows_and_degenerate(lib):
    A = datagen.uniform_f16(400, 0, (40, 24), -1.0, 1.0)
    B = datagen.uniform_f16(400, 1, (12, 24), -1.0, 1.0)
    full = oracle.gemm(A, B, lib=lib)
    rows = np.array([0, 7, 39, 20])
    part = oracle.gemm(A, B, rows=rows, lib=lib)
    assert np.array_equal(_bits(part), _bits(full[rows]))
    # K = 0: the empty sum, +0
    D = oracle.gemm(np.zeros((3, 0), np.float16), np.zeros((4, 0), np.float16), lib=lib)
    assert D.shape == (3, 4) and np.all(_bits(D) == 0)
    # M = 0 and N = 0
    assert oracle.gemm(np.zeros((0, 5), np.float16), np.ones((4, 5), np.float16), lib=lib).shape == (0, 4)
    assert oracle.gemm(np.ones((2, 5), np.float16), np.zeros((0, 5), np.float16), lib=lib).shape == (2, 0)


def check_gemv(lib):
    N, K = 37, 520
    W = datagen.uniform_f16(500, 1, (N, K), -0.05, 0.05)
    # unit vectors pick a column of W
    for j in (0, 1, 255, K - 1):
        x = np.zeros(K, np.float16)
        x[j] = 1.0
        y = oracle.gemv(x, W, lib=lib)
        assert np.array_equal(_bits(y), _bits(np.ascontiguousarray(W[:, j])))
    # all ones -> K  (14336 is fp16-exact)
    y = oracle.gemv(np.ones(14336, np.float16), np.ones((3, 14336), np.float16), lib=lib)
    assert np.all(_as_f64(y) == 14336)
    # random values vs the correctly rounded exact sum
    x = datagen.uniform_f16(500, 0, (K,), -1.0, 1.0)
    y = oracle.gemv(x, W, lib=lib)
    exact = np.array([math.fsum((_as_f64(x) * _as_f64(W[n])).tolist()) for n in range(N)])
    same = _bits(y) == _bits(_rne_numpy(exact))
    assert np.all(same | _near_fp16_midpoint(exact))
    assert np.all(_within_tol(y, exact))
    # integers: exact int64 sums
    xi = datagen.integer_f16(501, 0, (K,))
    Wi = datagen.integer_f16(501, 1, (N, K))
    exact_i = Wi.astype(np.int64) @ xi.astype(np.int64)
    yi = oracle.gemv(xi, Wi, lib=lib)
    assert np.array_equal(_as_f64(yi), _as_f64(_rne_numpy(exact_i.astype(np.float64))))
    # the GEMV is the GEMM with M = 1
    assert np.array_equal(_bits(oracle.gemm(x[None, :], W, lib=lib))[0], _bits(y))
    # K = 0
    assert np.all(_bits(oracle.gemv(np.zeros(0, np.float16), np.zeros((4, 0), np.float16), lib=lib)) == 0)


ALL_CHECKS = [
    check_decode_all_patterns,
    check_encode_grid_and_midpoints,
    check_rne_probe,
    check_gemm_brute_force,
    check_gemm_closed_forms,
    check_gemm_integer_exact,
    check_gemm_rows_and_degenerate,
    check_gemv,
]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check, oracle_lib):
    check(oracle_lib)


def test_tolerance_is_tight_enough(oracle_lib):
    """Dropping the ragged K tail (8 of 4104 terms) must break the tolerance
    for most outputs, so the parity bar can see a lost tail tile."""
    A = datagen.uniform_f16(2, 0, (16, 4104), -1.0, 1.0)
    B = datagen.uniform_f16(2, 1, (64, 4104), -1.0, 1.0)
    full = oracle.gemm(A, B, lib=oracle_lib)
    cut = oracle.gemm(np.ascontiguousarray(A[:, :4096]), np.ascontiguousarray(B[:, :4096]), lib=oracle_lib)
    assert (~_within_tol(cut, full)).mean() > 0.5
