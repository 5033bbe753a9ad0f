"""Seeded random shapes through every entry point, bit-exact on integer data.

The shape rules (GEMV for one row, skinny kernel for 16 rows or fewer, and
the tiled kernel's 256x256 / 256x128 / 128x256 / 128x128 tiles) and the
ragged edges of each are exercised by shapes drawn at random from a fixed
seed: M and N from 1 to 2600 (with extra weight on the rule boundaries 1,
2..16, 17), K a multiple of 8 up to 1040, and 8 outputs of 2000..6200 by
3000..6200 (K up to 552) for the larger tiles (128x256 tiles are rare at
random; test_gpu_parity.py checks them on purpose).  Integer data keeps every FP32
partial sum exact, so each output must equal the oracle's bit for bit, for
gemm_f16, gemm_bf16, gemm_bias_f16 (bias and ReLU) and gemv_f16.
"""
import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu


def _shapes(n, seed):
    g = np.random.default_rng(seed)
    edges = [1, 2, 3, 8, 15, 16, 17, 127, 128, 129, 255, 256, 257]
    out = []
    for _ in range(n):
        M = int(g.choice(edges)) if g.random() < 0.35 else int(g.integers(1, 2600))
        N = int(g.choice(edges)) if g.random() < 0.35 else int(g.integers(1, 2600))
        K = 8 * int(g.integers(1, 131))
        out.append((M, N, K))
    return out


def _large_shapes(n, seed):
    """Outputs large enough for 256x256 and 128x256 tiles (sampled rows)."""
    g = np.random.default_rng(seed)
    return [(int(g.integers(2000, 6200)), int(g.integers(3000, 6200)), 8 * int(g.integers(1, 70))) for _ in range(n)]


SHAPES = _shapes(40, 20261) + _large_shapes(8, 20264)
GEMV_SHAPES = [(int(n), 8 * int(k)) for n, k in zip(np.random.default_rng(20262).integers(1, 5000, 12),
                                                     np.random.default_rng(20263).integers(1, 2000, 12))]


@pytest.fixture(scope="module")
def env():
    import torch

    import gemv_tile_pipelined_amd as gt

    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    gt.load_library()
    return torch, gt, torch.device("cuda:0")


def _rows(M, i):
    if M <= 256:
        return None
    return np.unique(np.concatenate([datagen.rng(7000 + i, 2).choice(M, 24, replace=False), [0, M - 1]]))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_random_shape_all_gemm_entry_points(env, shape):
    torch, gt, dev = env
    M, N, K = shape
    i = SHAPES.index(shape)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    print(f"[random shape] {M}x{N}x{K} tile {gt.gemm_tile(M, N, cus) if min(M, N) > 16 else 'gemv/skinny'}",
          flush=True)
    A = datagen.integer_f16(7000 + i, 10, (M, K))
    B = datagen.integer_f16(7000 + i, 11, (N, K))
    bias = datagen.integer_f16(7000 + i, 3, (N,), -300, 300)
    rows = _rows(M, i)
    sel = (lambda D: D) if rows is None else (lambda D: D[torch.from_numpy(rows).to(dev)])
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    # fp16
    D = sel(gt.gemm_f16(tA, tB)).cpu().numpy()
    assert np.array_equal(D, oracle.gemm(A, B, rows=rows))
    # fused bias + ReLU
    Db = sel(gt.gemm_bias_f16(tA, tB, torch.from_numpy(bias).to(dev), "relu")).cpu().numpy()
    assert np.array_equal(Db, oracle.gemm_bias(A, B, bias, oracle.ACT_RELU, rows=rows))
    # bf16 (the same integers are bf16-exact)
    Ab = datagen.integer_bf16(7000 + i, 10, (M, K))
    Bb = datagen.integer_bf16(7000 + i, 11, (N, K))

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    Dbf = sel(gt.gemm_bf16(dev_bf16(Ab), dev_bf16(Bb))).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(Dbf, oracle.gemm_bf16(Ab, Bb, rows=rows))
    torch.cuda.synchronize(dev)


@pytest.mark.parametrize("shape", GEMV_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_random_shape_gemv(env, shape):
    torch, gt, dev = env
    N, K = shape
    i = GEMV_SHAPES.index(shape)
    x = datagen.integer_f16(7100 + i, 10, (K,))
    W = datagen.integer_f16(7100 + i, 11, (N, K))
    y = gt.gemv_f16(torch.from_numpy(x).to(dev), torch.from_numpy(W).to(dev))
    torch.cuda.synchronize(dev)
    assert np.array_equal(y.cpu().numpy(), oracle.gemv(x, W))
