"""Parity of the wave-specialised (producer / consumer) GEMM with the oracle.

gemvtile_gemm_f16_variant 200 and 201 run gemm_ws.hip whatever the shape:
256x128 output tiles, 4 consumer waves that only read LDS and issue MFMAs, 4
loader waves that only issue tile loads, one hand-off barrier per K tile, and
a 3- or 2-stage LDS ring.  Same bar as the default kernel: bit-for-bit on
integer inputs (exact FP32 partial sums), |d - ref| <= 1e-2 + 1e-2·|ref| on
uniform inputs, a rank-1 closed form on every element at full size.
"""
import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu

TOL_ABS = 1e-2
TOL_REL = 1e-2
WS_VARIANTS = (200, 201)


@pytest.fixture(scope="module")
def env():
    import torch

    import gemv_tile_pipelined_amd as gt

    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    gt.load_library()
    return torch, gt, torch.device("cuda:0")


def _gemm(env, A, B, variant):
    torch, gt, dev = env
    D = gt.gemm_f16(torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev), variant=variant)
    torch.cuda.synchronize(dev)
    return D


def _violations(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return int((~(np.abs(got - ref) <= TOL_ABS + TOL_REL * np.abs(ref))).sum())


# One K tile, ragged M/N/K, more tiles than one CU pass, tiny and skinny shapes.
SHAPES = [(256, 128, 64), (300, 260, 200), (520, 776, 4104), (1, 17, 8), (17, 1000, 72), (1000, 33, 136), (513, 129, 8)]


@pytest.mark.parametrize("variant", WS_VARIANTS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_ws_small(env, shape, variant):
    M, N, K = shape
    cfg = 9500 + SHAPES.index(shape)
    Ai = datagen.integer_f16(cfg, 10, (M, K))
    Bi = datagen.integer_f16(cfg, 11, (N, K))
    assert np.array_equal(_gemm(env, Ai, Bi, variant).cpu().numpy(), oracle.gemm(Ai, Bi))
    A = datagen.uniform_f16(cfg, 0, (M, K), -1.0, 1.0)
    B = datagen.uniform_f16(cfg, 1, (N, K), -1.0, 1.0)
    got = _gemm(env, A, B, variant).cpu().numpy()
    assert np.isfinite(got).all()
    assert _violations(got, oracle.gemm(A, B)) == 0


@pytest.mark.parametrize("variant", WS_VARIANTS)
def test_gemm_ws_full_size(env, full_size, variant):
    """4096^3 (two output tiles per CU in the persistent loop) against the
    oracle on every element, uniform inputs within the tolerance and integer
    inputs bit-exact, and a rank-1 closed form on every element."""
    torch, gt, dev = env
    w = datagen.WORKLOADS[1]
    print(f"[gemm_ws full size] variant {variant} {w.name}", flush=True)
    A, B = full_size.inputs(1)
    got = _gemm(env, A, B, variant).cpu().numpy()
    assert _violations(got, full_size.reference(1)) == 0
    Ai, Bi = full_size.inputs(1, True)
    assert np.array_equal(_gemm(env, Ai, Bi, variant).cpu().numpy(), full_size.reference(1, True))
    g = datagen.rng(1, 22)
    choices = np.array([-1.0, -0.5, -0.25, -0.125, 0.125, 0.25, 0.5, 1.0])
    u, v = g.choice(choices, w.M), g.choice(choices, w.N)
    tu = torch.from_numpy(u.astype(np.float16)).to(dev)
    tv = torch.from_numpy(v.astype(np.float16)).to(dev)
    Dr = gt.gemm_f16(tu[:, None].expand(w.M, w.K).contiguous(), tv[:, None].expand(w.N, w.K).contiguous(), variant=variant)
    want = (w.K * torch.outer(tu.double(), tv.double())).half()
    torch.cuda.synchronize(dev)
    assert bool((Dr == want).all())


def test_gemm_ws_matches_default_bits(env):
    """Integer data: the wave-specialised kernel and the default kernel give
    the same bits on a ragged shape (a race in either would show)."""
    M, N, K = 4000, 4032, 4104
    Ai = datagen.integer_f16(9600, 10, (M, K))
    Bi = datagen.integer_f16(9600, 11, (N, K))
    base = _gemm(env, Ai, Bi, 0)
    for variant in WS_VARIANTS:
        import torch

        assert torch.equal(_gemm(env, Ai, Bi, variant), base)
