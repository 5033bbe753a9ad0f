"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle/oracle.c with one plausible mistake (a
dropped term, a wrong sign, a wrong index, a transposed operand, the wrong
rounding), compiled on the CPU into a temporary library.  The pin checks of
test_oracle.py are run against it and at least one of them must fail.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle
import test_oracle_bf16
import test_oracle_bias

MUTANTS = {
    "drop_last_k_term": ("for (int64_t k = 0; k < K; ++k) sum += arow[k] * brow[k];",
                         "for (int64_t k = 0; k < K - 1; ++k) sum += arow[k] * brow[k];"),
    "wrong_sign": ("sum += arow[k] * brow[k];", "sum -= arow[k] * brow[k];"),
    "reversed_k_index": ("sum += arow[k] * brow[k];", "sum += arow[k] * brow[K - 1 - k];"),
    "transposed_b": ("const double *brow = Bd + n * K;", "const double *brow = Bd + (n % (K ? K : 1)) * N;"),
    "round_toward_zero": ("double q = round_half_even(ldexp(a, 10 - E));", "double q = floor(ldexp(a, 10 - E));"),
    "ties_away_from_zero": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    "subnormal_scale": ("mag = ldexp((double)frac, -24);", "mag = ldexp((double)frac, -25);"),
    "exponent_bias": ("mag = ldexp((double)(1024 + frac), exp - 25);", "mag = ldexp((double)(1024 + frac), exp - 24);"),
    "gemv_transposed_w": ("sum += xd[k] * decode(fmt, W[n * K + k]);",
                          "sum += xd[k] * decode(fmt, W[(k * N + n) % (N * K)]);"),
    "gemv_drop_first": ("for (int64_t k = 0; k < K; ++k) sum += xd[k]", "for (int64_t k = 1; k < K; ++k) sum += xd[k]"),
    "overflow_threshold": ("if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);",
                           "if (a >= 65504.0) return (uint16_t)(sign | 0x7c00);"),
    # bf16
    "bf16_exponent_bias": ("mag = ldexp((double)(128 + frac), exp - 134);", "mag = ldexp((double)(128 + frac), exp - 133);"),
    "bf16_subnormal_scale": ("mag = ldexp((double)frac, -133);", "mag = ldexp((double)frac, -134);"),
    "bf16_round_toward_zero": ("double q = round_half_even(ldexp(a, 7 - E));", "double q = floor(ldexp(a, 7 - E));"),
    "bf16_overflow_threshold": ("if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return (uint16_t)(sign | 0x7f80);",
                                "if (a >= ldexp(2.0 - ldexp(1.0, -7), 127)) return (uint16_t)(sign | 0x7f80);"),
    "bf16_subnormal_encode": ("double q = round_half_even(ldexp(a, 133));", "double q = round_half_even(ldexp(a, 132));"),
    "bf16_decoded_as_fp16": ("return fmt ? oracle_bf16_to_f64(bits) : oracle_f16_to_f64(bits);",
                             "return oracle_f16_to_f64(bits);"),
    "bf16_encoded_as_fp16": ("return fmt ? oracle_f64_to_bf16_rne(v) : oracle_f64_to_f16_rne(v);",
                             "return oracle_f64_to_f16_rne(v);"),
    # bias and activation
    "bias_dropped": ("if (bias) sum += decode(fmt, bias[n]);", "if (0) sum += decode(fmt, bias[n]);"),
    "bias_indexed_by_row": ("if (bias) sum += decode(fmt, bias[n]);", "if (bias) sum += decode(fmt, bias[m % N]);"),
    "bias_subtracted": ("if (bias) sum += decode(fmt, bias[n]);", "if (bias) sum -= decode(fmt, bias[n]);"),
    "relu_before_bias": ("if (bias) sum += decode(fmt, bias[n]);\n                if (act == 1 && sum < 0.0) sum = 0.0;",
                         "if (act == 1 && sum < 0.0) sum = 0.0;\n                if (bias) sum += decode(fmt, bias[n]);"),
    "relu_as_abs": ("if (act == 1 && sum < 0.0) sum = 0.0;", "if (act == 1 && sum < 0.0) sum = -sum;"),
    "relu_threshold": ("if (act == 1 && sum < 0.0) sum = 0.0;", "if (act == 1 && sum < 1.0) sum = 0.0;"),
    "relu_negative_zero": ("if (act == 1 && sum < 0.0) sum = 0.0;", "if (act == 1 && sum < 0.0) sum = -0.0;"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    old, new = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = os.path.join(mutant_dir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib_path = os.path.join(mutant_dir, f"lib{name}.so")
    oracle.compile_oracle(source=path, output=lib_path)
    lib = oracle.load(lib_path)
    caught = []
    for check in test_oracle.ALL_CHECKS + test_oracle_bf16.ALL_CHECKS + test_oracle_bias.ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin detects the planted mistake {name}"
