"""Parity of gemm_splitk_f16 / gemm_splitk_bf16 (K split across workgroups).

Each (tile, K slice) unit stores FP32 partial sums to the workspace and a
second kernel adds the slices in order and rounds once.  The bar is the
plain GEMM's: bit-for-bit on integer data (every partial sum, and their sum,
is exact in FP32), |d - ref| <= 1e-2 + 1e-2·|ref| on uniform data.  The
shapes split into 2 to 21 slices (128x128x14336 is one output tile cut
into 21), with ragged M, N, a ragged last K tile in the last slice, and odd
M·N (the reduction's one-output-per-thread form), also past 8 slices (the
reduction's second batch of loads).  Also: the result does not
depend on what the workspace held before, repeated calls give the same bits,
shapes that do not split give gemm_f16's bits, and a missing, short or
misaligned workspace is an error.  Shapes with 2..16 rows on a side split
on the skinny kernel (16 rows of the large side per workgroup, K tiles of
512 split across workgroups) and are held to the same bar.
"""
import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu

TOL_ABS = 1e-2
TOL_REL = 1e-2

# (M, N, K, slices on 256 CUs)
SHAPES = [(1024, 1024, 4096, 4), (512, 4096, 8192, 2), (300, 260, 4104, 6), (257, 129, 4104, 6),
          (1000, 1000, 4104, 4), (128, 128, 14336, 21), (129, 127, 14336, 21)]


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


def _rows(M, cfg):
    if M <= 256:
        return None
    return np.unique(np.concatenate([datagen.rng(cfg, 2).choice(M, 40, replace=False), [0, M - 1]]))


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "x".join(map(str, c[:3])))
def test_splitk_parity(env, case):
    torch, gt, dev = env
    M, N, K, slices = case
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    print(f"[splitk] {M}x{N}x{K}: {gt.splitk_splits(M, N, K, cus)} slices on {cus} CUs", flush=True)
    if cus == 256:
        assert gt.splitk_splits(M, N, K, cus) == slices
    cfg = 9600 + SHAPES.index(case)
    rows = _rows(M, cfg)
    sel = (lambda D: D) if rows is None else (lambda D: D[torch.from_numpy(rows).to(dev)])
    Ai = datagen.integer_f16(cfg, 10, (M, K))
    Bi = datagen.integer_f16(cfg, 11, (N, K))
    ws = torch.full((max(gt.splitk_workspace_bytes(M, N, K, cus), 16) // 4,), float("nan"), device=dev)
    Di = gt.gemm_splitk_f16(torch.from_numpy(Ai).to(dev), torch.from_numpy(Bi).to(dev), workspace=ws)
    assert np.array_equal(sel(Di).cpu().numpy(), oracle.gemm(Ai, Bi, rows=rows))
    A = datagen.uniform_f16(cfg, 0, (M, K), -1.0, 1.0)
    B = datagen.uniform_f16(cfg, 1, (N, K), -1.0, 1.0)
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    D1 = gt.gemm_splitk_f16(tA, tB, workspace=ws)
    D2 = gt.gemm_splitk_f16(tA, tB, workspace=gt.alloc_splitk_workspace(tA, tB))  # a second, fresh workspace
    torch.cuda.synchronize(dev)
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))  # deterministic
    assert np.isfinite(D1.float().cpu().numpy()).all()
    assert _violations(sel(D1).cpu().numpy(), oracle.gemm(A, B, rows=rows)) == 0


def test_splitk_bf16(env):
    torch, gt, dev = env
    M, N, K = 1024, 1024, 4096
    A = datagen.integer_bf16(9650, 10, (M, K))
    B = datagen.integer_bf16(9650, 11, (N, K))
    rows = _rows(M, 9650)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    tA, tB = dev_bf16(A), dev_bf16(B)
    D = gt.gemm_splitk_bf16(tA, tB, workspace=gt.alloc_splitk_workspace(tA, tB))
    got = D[torch.from_numpy(rows).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.gemm_bf16(A, B, rows=rows))


def test_splitk_no_split_is_plain_gemm(env):
    """Shapes whose tiles fill the CUs, with few K tiles, too little K-loop
    time to save, skinny shapes whose row blocks fill the CUs or with too
    short a K, and one-row shapes (the GEMV) do not split: the result is
    gemm_f16's, and the workspace may be absent."""
    torch, gt, dev = env
    for M, N, K in ((4096, 4096, 256), (1024, 1024, 1024), (2048, 1024, 2048), (8, 3000, 1032), (8, 4096, 4096),
                    (8, 1024, 4096), (1, 700, 520), (1, 1024, 14336)):
        A = torch.from_numpy(datagen.uniform_f16(9660, 0, (M, K), -1.0, 1.0)).to(dev)
        B = torch.from_numpy(datagen.uniform_f16(9660, 1, (N, K), -1.0, 1.0)).to(dev)
        assert gt.splitk_workspace_bytes(M, N, K, torch.cuda.get_device_properties(dev).multi_processor_count) == 0
        D = gt.gemm_splitk_f16(A, B)
        torch.cuda.synchronize(dev)
        assert torch.equal(D.view(torch.int16), gt.gemm_f16(A, B).view(torch.int16)), (M, N, K)


def test_splitk_workspace_errors(env):
    torch, gt, dev = env
    M, N, K = 1024, 1024, 4096
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    need = gt.splitk_workspace_bytes(M, N, K, cus)
    assert need > 0
    A = torch.zeros((M, K), dtype=torch.float16, device=dev)
    B = torch.zeros((N, K), dtype=torch.float16, device=dev)
    D = torch.empty((M, N), dtype=torch.float16, device=dev)
    lib = gt.load_library()
    s = torch.cuda.current_stream(dev).cuda_stream
    args = (A.data_ptr(), B.data_ptr(), D.data_ptr(), M, N, K)
    ws = torch.empty((need + 64,), dtype=torch.uint8, device=dev)
    assert lib.gemm_splitk_f16(*args, None, need, s) == 1  # NULL workspace
    assert lib.gemm_splitk_f16(*args, ws.data_ptr(), need - 4, s) == 1  # too small
    assert lib.gemm_splitk_f16(*args, ws.data_ptr() + 4, need, s) == 2  # misaligned
    assert lib.gemm_splitk_f16(*args, ws.data_ptr(), need, s) == 0
    torch.cuda.synchronize(dev)
    assert bool((D == 0).all())
    # the binding allocates no workspace behind the caller's back
    with pytest.raises(gt.GemvTileError) as e:
        gt.gemm_splitk_f16(A, B, D)
    assert e.value.status == 1


# Skinny shapes (2..16 rows on a side): (M, N, K, slices on 256 CUs).  The
# large side's blocks of 16 rows are split along K in 512-wide K tiles;
# M <= 16 stores D = Q·Pᵀ, N <= 16 the transposed layout; ragged row
# blocks, a ragged last K tile, 16 rows on the small side (16 staged rows),
# and 8 or fewer (8 staged rows).
SKINNY_SHAPES = [(8, 1024, 14336, 4), (16, 256, 14336, 14), (1000, 5, 14336, 4), (3, 300, 8200, 6),
                 (8, 260, 14344, 10), (13, 777, 14336, 5)]


@pytest.mark.parametrize("case", SKINNY_SHAPES, ids=lambda c: "x".join(map(str, c[:3])))
def test_splitk_skinny_parity(env, case):
    torch, gt, dev = env
    M, N, K, slices = case
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    print(f"[splitk skinny] {M}x{N}x{K}: {gt.splitk_splits(M, N, K, cus)} slices on {cus} CUs", flush=True)
    if cus == 256:
        assert gt.splitk_splits(M, N, K, cus) == slices
    cfg = 9700 + SKINNY_SHAPES.index(case)
    Ai = datagen.integer_f16(cfg, 10, (M, K))
    Bi = datagen.integer_f16(cfg, 11, (N, K))
    ws = torch.full((max(gt.splitk_workspace_bytes(M, N, K, cus), 16) // 4,), float("nan"), device=dev)
    Di = gt.gemm_splitk_f16(torch.from_numpy(Ai).to(dev), torch.from_numpy(Bi).to(dev), workspace=ws)
    assert np.array_equal(Di.cpu().numpy(), oracle.gemm(Ai, Bi))
    A = datagen.uniform_f16(cfg, 0, (M, K), -1.0, 1.0)
    B = datagen.uniform_f16(cfg, 1, (N, K), -1.0, 1.0)
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    D1 = gt.gemm_splitk_f16(tA, tB, workspace=ws)
    D2 = gt.gemm_splitk_f16(tA, tB, workspace=gt.alloc_splitk_workspace(tA, tB))
    torch.cuda.synchronize(dev)
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))
    assert np.isfinite(D1.float().cpu().numpy()).all()
    assert _violations(D1.cpu().numpy(), oracle.gemm(A, B)) == 0


def test_splitk_skinny_bf16(env):
    torch, gt, dev = env
    for M, N, K in ((8, 512, 8192), (700, 12, 14336)):
        A = datagen.integer_bf16(9760, 10, (M, K))
        B = datagen.integer_bf16(9760, 11, (N, K))

        def dev_bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        assert gt.splitk_splits(M, N, K, torch.cuda.get_device_properties(dev).multi_processor_count) > 1 or \
            torch.cuda.get_device_properties(dev).multi_processor_count != 256
        tA, tB = dev_bf16(A), dev_bf16(B)
        D = gt.gemm_splitk_bf16(tA, tB, workspace=gt.alloc_splitk_workspace(tA, tB))
        got = D.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, oracle.gemm_bf16(A, B)), (M, N, K)
