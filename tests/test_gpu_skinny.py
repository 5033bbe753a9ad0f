"""Parity of the skinny GEMM path with the CPU oracle.

gemm_f16 sends shapes with at most 16 rows on one side, or 17..64 rows on
the smaller side, to a bandwidth-bound kernel that streams the larger
operand once.  The bar is the one of the
tiled GEMM: |d - ref| <= 1e-2 + 1e-2·|ref| for uniform inputs, bit-for-bit
for integer inputs (exact FP32 partial sums, so only the final rounding to
nearest-even decides, and it must agree).  Every shape is compared in full:
the oracle's cost is M·N·K with one small side.
"""
import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu

TOL_ABS = 1e-2
TOL_REL = 1e-2

# gemvtile_gemm_f16_variant ids of the skinny launch shapes
SKINNY_VARIANTS = [100, 104, 112, 130, 147, 152]


@pytest.fixture(scope="module")
def env():
    import torch

    import gemv_tile_pipelined_amd as gt

    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    gt.load_library()
    return torch, gt, torch.device("cuda:0")


def _gemm(env, A, B, variant=0):
    torch, gt, dev = env
    D = gt.gemm_f16(torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev), variant=variant)
    torch.cuda.synchronize(dev)
    return D.cpu().numpy()


def _violations(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return int((~(np.abs(got - ref) <= TOL_ABS + TOL_REL * np.abs(ref))).sum())


# (M, N, K): small M (D = A·Bᵀ with A the batch), small N (the transposed
# store), both small, ragged row counts and K tails (K not a multiple of 32).
SHAPES = [
    (1, 4096, 14336),
    (2, 520, 1032),
    (8, 4096, 14336),
    # 16 large-side rows per workgroup: cached loads below K = 8192,
    # non-temporal loads from there up; K starts rotated by the workgroup's
    # index within its XCD (8 K tiles at 4096, 16 at 8192, 32 at 16384)
    (8, 4096, 8184),
    (8, 4096, 8192),
    (8, 4096, 10232),
    (8, 4096, 10240),
    (8, 4096, 16384),
    (12, 4096, 4096),
    # 8 large-side rows per workgroup, rotated K starts
    (8, 2048, 8192),
    (13, 3000, 4104),
    (16, 4096, 4096),
    (16, 1000, 4104),
    (3, 17, 8),
    (15, 4097, 520),
    (16, 16, 64),
    (4000, 16, 4104),
    (520, 5, 1032),
    (33, 1, 72),
    # fewer large-side rows than 16 per CU: 8, 4, 2 or 1 rows per workgroup
    # (on a 256-CU part), with 8 or 16 small-side rows staged
    (16, 3000, 1032),
    (8, 2000, 4104),
    (9, 1000, 4104),
    (5, 300, 14336),
    (16, 100, 65544),
    (2, 17, 8),
    (4000, 12, 520),
    (600, 16, 1032),
    (300, 3, 4104),
    # 17..32 rows on the smaller side: two 16-row blocks of the small operand
    # per MFMA step (the default launch only)
    (17, 4096, 4104),
    (32, 4096, 14336),
    (24, 1000, 1032),
    (4000, 32, 4104),
    (1000, 20, 14336),
    (32, 32, 520),
    (30, 17, 72),
    (25, 300, 8200),
    (17, 129, 8),
    # 33..64 rows on the smaller side: four 16-row blocks, the partial sums
    # reusing the LDS ring
    (33, 4096, 4104),
    (64, 4096, 14336),
    (48, 1000, 1032),
    (4000, 64, 520),
    (1000, 40, 4104),
    (64, 64, 72),
    (50, 300, 8200),
    (33, 129, 8),
    # few large-side rows: the small side split into 16-row blocks along the
    # grid's y dimension, 4 large-side rows per workgroup on a 256-CU part
    # (and ragged K), a ragged last block of 2 rows with the transposed
    # store, 16 large-side rows at 8 staged-launch rows with <= 32 small-side
    # rows, and 4 blocks at the 64-row limit
    (24, 1500, 4104),
    (1500, 48, 1032),
    (40, 1100, 8200),
    (1000, 50, 2056),
    (20, 2048, 4096),
    (64, 1024, 14336),
    # 17..32 staged rows with rotated K starts (K % 4096 == 0) at 16
    # large-side rows per workgroup, the small-side split at 8 staged-launch
    # rows with at most 32 small-side rows, and 33..64 staged rows at 8 rows
    # per workgroup
    (24, 4096, 8192),
    (2500, 20, 4096),
    (48, 2600, 4104),
    # 32 large-side rows per workgroup (two 16-row MFMA blocks) in K tiles
    # of 256, from 32 rows per CU up: 16, 32 and 64 staged small-side rows,
    # ragged large side, ragged K (a last K tile of 8 or 16 elements, or one
    # tile and a tail), the transposed store, 1.5 waves of workgroups
    (24, 8192, 4096),
    (32, 12300, 4104),
    (12300, 17, 1032),
    (8210, 17, 1032),
    (20, 12288, 4096),
    (8, 8200, 4104),
    (8210, 12, 1032),
    (3, 8192, 264),
    (64, 8200, 2056),
    (8300, 40, 1032),
    (33, 8192, 4096),
    # 48 and 64 large-side rows per workgroup (three or four MFMA blocks) in
    # K tiles of 128, with 16, 32 and 64 staged rows, ragged large side and
    # K, the transposed store
    (8, 10300, 1032),
    (10300, 20, 2056),
    (64, 14400, 520),
    (16400, 40, 1032),
    (16384, 30, 136),
    (12, 16390, 4104),
    # 17..64 small-side rows against more large-side rows than 128x128
    # tiles would need to fill the CUs (the skinny kernel whatever R)
    (24, 16500, 1032),
    (20000, 40, 520),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_skinny_uniform(env, shape):
    M, N, K = shape
    cfg = 3000 + SHAPES.index(shape)
    A = datagen.uniform_f16(cfg, 0, (M, K), -1.0, 1.0)
    B = datagen.uniform_f16(cfg, 1, (N, K), -1.0, 1.0)
    got = _gemm(env, A, B)
    assert got.shape == (M, N)
    assert np.isfinite(got).all()
    assert _violations(got, oracle.gemm(A, B)) == 0


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_skinny_integer_exact(env, shape):
    M, N, K = shape
    cfg = 3100 + SHAPES.index(shape)
    A = datagen.integer_f16(cfg, 0, (M, K))
    B = datagen.integer_f16(cfg, 1, (N, K))
    assert np.array_equal(_gemm(env, A, B), oracle.gemm(A, B))


@pytest.mark.parametrize("variant", SKINNY_VARIANTS)
@pytest.mark.parametrize(
    "shape", [(8, 1000, 14344), (1000, 8, 1032), (5, 300, 72)], ids=["small_m", "small_n", "k_fewer_tiles_than_waves"]
)
def test_skinny_variants_exact(env, shape, variant):
    M, N, K = shape
    A = datagen.integer_f16(3200, 0, (M, K))
    B = datagen.integer_f16(3200, 1, (N, K))
    assert np.array_equal(_gemm(env, A, B, variant=variant), oracle.gemm(A, B))


def test_decode_batch_workload(env):
    """The 8x4096x14336 decode batch in the launch shape the benchmark times."""
    w = datagen.DECODE_BATCH
    A, B = datagen.gemm_inputs(w)
    got = _gemm(env, A, B)
    assert _violations(got, oracle.gemm(A, B)) == 0


def test_skinny_closed_form_and_guard(env):
    """Rank-1 inputs give exact products; nothing outside D is written."""
    torch, gt, dev = env
    for M, N, K in [(7, 3000, 4104), (3000, 7, 4104), (7, 500, 4104), (500, 7, 1032)]:
        u = np.array([0.25, -0.5, 1.0, 2.0, -1.0, 0.5, -2.0], np.float16)
        v = np.array([0.5, -1.0, 2.0, -0.25], np.float16)
        a = u[np.arange(M) % 7]
        b = v[np.arange(N) % 4]
        A = np.repeat(a[:, None], K, axis=1)
        B = np.repeat(b[:, None], K, axis=1)
        guard = 4096
        buf = torch.full((M * N + guard,), float("nan"), dtype=torch.float16, device=dev)
        D = buf[: M * N].view(M, N)
        gt.gemm_f16(torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev), D)
        torch.cuda.synchronize(dev)
        expect = (K * a.astype(np.float64)[:, None] * b.astype(np.float64)[None, :]).astype(np.float16)
        assert np.array_equal(D.cpu().numpy(), expect)
        assert bool(torch.isnan(buf[M * N :]).all())
