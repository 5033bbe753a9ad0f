"""Pins of the CPU oracle's bf16 functions against things other than itself.

bf16 is the upper half of an IEEE binary32, so:
  * decode              -> every one of the 65536 bit patterns, shifted left
                           16 bits and read as numpy float32;
  * RNE encode          -> an independent route: integer round-to-nearest-even
                           on float32 bit patterns (add 0x7fff plus the kept
                           lsb, drop 16 bits), exact wherever the input is a
                           float32 -- every midpoint between bf16 neighbours
                           is one -- plus the hand-derived rounding probes in
                           tests/golden/bf16_rne_probe.txt (ties, overflow,
                           subnormals);
  * GEMM / GEMV sums    -> math.fsum of the exact products; for integer
                           inputs, the exact int64 sum rounded by the float32
                           route above (sums < 2^24 are float32-exact);
  * indexing            -> closed forms (all-ones, identities, rank-1).
Each check takes the loaded oracle library, so the mutant test can run them
against copies of the oracle with planted mistakes.
"""
import math
import os

import numpy as np
import pytest

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f32_bits_to_bf16_rne(f32):
    """Round float32 values to bf16 bit patterns by integer arithmetic on
    their bits (finite inputs)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_value(bits):
    """bf16 bit patterns -> float64, via float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # NaN patterns
        return b.view(np.float32).astype(np.float64)


def _near_bf16_midpoint(v, rel=1e-9):
    v = np.asarray(v, np.float64)
    bits = _f32_bits_to_bf16_rne(v.astype(np.float32))
    lo = _bf16_value(bits)
    # the neighbour on the other side of v
    step = np.where(lo <= v, 1, -1).astype(np.int64)
    mag_bits = bits.astype(np.int64)
    other = _bf16_value((mag_bits + np.where(lo >= 0, step, -step)).astype(np.uint16))
    mid = (lo + other) / 2.0
    return np.abs(v - mid) <= rel * np.maximum(np.abs(v), 1e-300)


def check_bf16_decode_all_patterns(lib):
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.bf16_to_f64(bits, lib=lib)
    ref = _bf16_value(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert math.copysign(1.0, got[0x8000]) == -1.0


def check_bf16_encode(lib):
    bits = np.arange(65536, dtype=np.uint16)
    vals = _bf16_value(bits)
    fin = np.isfinite(vals)
    # every finite bf16 value encodes to its own bit pattern (except -0 -> -0 too)
    assert np.array_equal(oracle.f64_to_bf16(vals[fin], lib=lib), bits[fin])
    # midpoints between neighbours (float32-exact) and their float32 neighbours
    v = np.unique(vals[fin])
    mids = ((v[:-1] + v[1:]) / 2.0).astype(np.float32)
    for pts in (mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))):
        pts = pts[np.isfinite(pts)]
        got = oracle.f64_to_bf16(pts.astype(np.float64), lib=lib)
        assert np.array_equal(got, _f32_bits_to_bf16_rne(pts)), "midpoint rounding"
    # random float32 values over the whole exponent range, both signs
    g = np.random.default_rng(4321)
    r = g.integers(0, 2**32, 300000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    r = r[np.isfinite(r)]
    assert np.array_equal(oracle.f64_to_bf16(r.astype(np.float64), lib=lib), _f32_bits_to_bf16_rne(r))
    # beyond float32: above the overflow tie, infinities, NaN
    big = oracle.f64_to_bf16(np.array([1e39, -1e39, np.inf, -np.inf]), lib=lib)
    assert list(big) == [0x7F80, 0xFF80, 0x7F80, 0xFF80]
    assert _bf16_value(oracle.f64_to_bf16(np.array([np.nan]), lib=lib)).tolist()[0] != _bf16_value(np.array([0], np.uint16))[0]
    assert np.isnan(_bf16_value(oracle.f64_to_bf16(np.array([np.nan]), lib=lib)))[0]


def _load_probe():
    cases = []
    with open(os.path.join(GOLDEN, "bf16_rne_probe.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b, want, _why = [p.strip() for p in line.split("|")]
            av = [float.fromhex(t) if "p" in t else float(t) for t in a.split()]
            bv = [float.fromhex(t) if "p" in t else float(t) for t in b.split()]
            cases.append((av, bv, int(want, 16)))
    return cases


def _to_bf16_exact(values):
    """bf16 bit patterns of values that must be bf16-exact."""
    f = np.asarray(values, np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(_bf16_value(bits), np.asarray(values, np.float64)), values
    return bits


def check_bf16_rne_probe(lib):
    cases = _load_probe()
    assert len(cases) >= 12
    for av, bv, want in cases:
        A = _to_bf16_exact(av)[None, :]
        B = _to_bf16_exact(bv)[None, :]
        D = oracle.gemm_bf16(A, B, lib=lib)
        assert int(D[0, 0]) == want, (av, bv, hex(int(D[0, 0])), hex(want))
        y = oracle.gemv_bf16(A[0], B, lib=lib)
        assert int(y[0]) == want


def check_bf16_gemm_brute_force(lib):
    for i, (M, N, K) in enumerate([(1, 1, 1), (3, 17, 64), (17, 3, 65), (64, 65, 130), (5, 64, 3)]):
        A = datagen.uniform_bf16(600 + i, 0, (M, K), -1.0, 1.0)
        B = datagen.uniform_bf16(600 + i, 1, (N, K), -1.0, 1.0)
        D = oracle.gemm_bf16(A, B, lib=lib)
        Av, Bv = _bf16_value(A), _bf16_value(B)
        exact = np.array([[math.fsum((Av[m] * Bv[n]).tolist()) for n in range(N)] for m in range(M)])
        want = oracle.f64_to_bf16(exact, lib=lib)  # the encoder is pinned on its own above
        same = D == want
        assert np.all(same | _near_bf16_midpoint(exact)), (M, N, K)
        assert same.mean() > 0.999
        # within the bf16 rounding of the exact sum (half a bf16 ulp, 2^-9 relative)
        assert np.all(np.abs(_bf16_value(D) - exact) <= np.abs(exact) * 2.0**-8 + 1e-30)
        np_ref = Av @ Bv.T
        assert np.all(np.abs(_bf16_value(D) - np_ref) <= np.abs(np_ref) * 2.0**-8 + 1e-12)


def check_bf16_closed_forms(lib):
    one = np.uint16(0x3F80)
    for K in (1, 8, 256, 4096, 8192):  # bf16-exact
        D = oracle.gemm_bf16(np.full((3, K), one), np.full((5, K), one), lib=lib)
        assert np.all(_bf16_value(D) == K), K
    A = datagen.uniform_bf16(700, 0, (7, 9), -1.0, 1.0)
    eye9 = np.where(np.eye(9) > 0, one, np.uint16(0)).astype(np.uint16)
    assert np.array_equal(oracle.gemm_bf16(A, eye9, lib=lib), A)
    B = datagen.uniform_bf16(700, 1, (11, 7), -1.0, 1.0)
    eye7 = np.where(np.eye(7) > 0, one, np.uint16(0)).astype(np.uint16)
    assert np.array_equal(oracle.gemm_bf16(eye7, B, lib=lib), np.ascontiguousarray(B.T))
    g = np.random.default_rng(8)
    choices = np.array([-2.0, -1.0, -0.5, -0.25, 0.25, 0.5, 1.0, 2.0])
    for K in (64, 4096):
        u, v = g.choice(choices, 13), g.choice(choices, 6)
        A = np.repeat(_to_bf16_exact(u)[:, None], K, axis=1)
        B = np.repeat(_to_bf16_exact(v)[:, None], K, axis=1)
        assert np.array_equal(_bf16_value(oracle.gemm_bf16(A, B, lib=lib)), K * np.outer(u, v)), K


def check_bf16_integer_exact(lib):
    for i, (M, N, K) in enumerate([(9, 7, 33), (16, 40, 520), (3, 5, 4104)]):
        A = datagen.integer_bf16(800 + i, 0, (M, K))
        B = datagen.integer_bf16(800 + i, 1, (N, K))
        exact = _bf16_value(A).astype(np.int64) @ _bf16_value(B).astype(np.int64).T
        want = _f32_bits_to_bf16_rne(exact.astype(np.float32))  # |sums| < 2^24: float32-exact
        assert np.array_equal(oracle.gemm_bf16(A, B, lib=lib), want), (M, N, K)


def check_bf16_gemv(lib):
    N, K = 37, 520
    W = datagen.uniform_bf16(900, 1, (N, K), -0.05, 0.05)
    for j in (0, 1, 255, K - 1):
        x = np.zeros(K, np.uint16)
        x[j] = 0x3F80
        assert np.array_equal(oracle.gemv_bf16(x, W, lib=lib), np.ascontiguousarray(W[:, j]))
    xi = datagen.integer_bf16(901, 0, (K,))
    Wi = datagen.integer_bf16(901, 1, (N, K))
    exact = _bf16_value(Wi).astype(np.int64) @ _bf16_value(xi).astype(np.int64)
    assert np.array_equal(oracle.gemv_bf16(xi, Wi, lib=lib), _f32_bits_to_bf16_rne(exact.astype(np.float32)))
    x = datagen.uniform_bf16(900, 0, (K,), -1.0, 1.0)
    y = oracle.gemv_bf16(x, W, lib=lib)
    assert np.array_equal(oracle.gemm_bf16(x[None, :], W, lib=lib)[0], y)
    assert np.all(oracle.gemv_bf16(np.zeros(0, np.uint16), np.zeros((4, 0), np.uint16), lib=lib) == 0)


ALL_CHECKS = [
    check_bf16_decode_all_patterns,
    check_bf16_encode,
    check_bf16_rne_probe,
    check_bf16_gemm_brute_force,
    check_bf16_closed_forms,
    check_bf16_integer_exact,
    check_bf16_gemv,
]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_bf16_pin(check, oracle_lib):
    check(oracle_lib)
