"""gemm_splitk_f16_noalloc: the split-K GEMM without a workspace argument,
through the C ABI, against gemm_splitk_f16 with a caller's workspace.

Both run the same kernels in the same order, so the outputs must be
bit-identical; each is also held to the oracle's bar (integer inputs bit
for bit, uniform inputs within |d - ref| <= 1e-2 + 1e-2·|ref|).  Two calls
in a row, the second on a smaller shape, check that the static scratch
keeps no state that matters between calls.  Nothing here allocates between
the non-allocating calls and their checks other than the test's own
tensors.
"""
import ctypes

import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu

TOL_ABS = 1e-2
TOL_REL = 1e-2


@pytest.fixture(scope="module")
def env():
    import torch

    import gemv_tile_pipelined_amd as gt

    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    lib = gt.load_library()
    return torch, gt, lib, torch.device("cuda:0")


def _violations(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return int((~(np.abs(got - ref) <= TOL_ABS + TOL_REL * np.abs(ref))).sum())


def _pair(env, A, B):
    """(D from gemm_splitk_f16_noalloc, D from gemm_splitk_f16 with a
    workspace), both through the C ABI on the current stream."""
    torch, gt, lib, dev = env
    M, K = A.shape
    N = B.shape[0]
    tA = torch.from_numpy(A).to(dev)
    tB = torch.from_numpy(B).to(dev)
    D1 = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    D2 = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    need = gt.splitk_workspace_bytes(M, N, K, cus)
    ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    torch.cuda.synchronize(dev)
    st = lib.gemm_splitk_f16_noalloc(tA.data_ptr(), tB.data_ptr(), D1.data_ptr(), M, N, K, s)
    assert st == 0, gt.status_string(st)
    st = lib.gemm_splitk_f16(tA.data_ptr(), tB.data_ptr(), D2.data_ptr(), M, N, K, ws.data_ptr(),
                             ws.numel() * 4, s)
    assert st == 0, gt.status_string(st)
    torch.cuda.synchronize(dev)
    return D1.cpu().numpy(), D2.cpu().numpy(), gt.splitk_splits(M, N, K, cus)


# (first call, second call on a smaller shape): the tiled split (128x128
# tiles, 16 MiB of partial sums at 512x512x14336 on 256 CUs), then a smaller
# ragged tiled split, then the skinny kernel's split.
SEQUENCES = [
    ((512, 512, 14336), (200, 328, 8200)),
    ((1024, 1024, 14336), (8, 1000, 14344)),
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda q: "_then_".join("x".join(map(str, s)) for s in q))
def test_noalloc_matches_workspace_entry_point(env, seq):
    torch, gt, lib, dev = env
    for n, (M, N, K) in enumerate(seq):
        print(f"[noalloc] call {n}: {M}x{N}x{K}", flush=True)
        cfg = 9900 + 10 * SEQUENCES.index(seq) + n
        Ai = datagen.integer_f16(cfg, 10, (M, K))
        Bi = datagen.integer_f16(cfg, 11, (N, K))
        d1, d2, splits = _pair(env, Ai, Bi)
        assert splits > 1, (M, N, K)  # the shapes do split
        assert np.array_equal(d1.view(np.uint16), d2.view(np.uint16))
        assert np.array_equal(d1, oracle.gemm(Ai, Bi))
        A = datagen.uniform_f16(cfg, 0, (M, K), -1.0, 1.0)
        B = datagen.uniform_f16(cfg, 1, (N, K), -1.0, 1.0)
        d1, d2, _ = _pair(env, A, B)
        assert np.array_equal(d1.view(np.uint16), d2.view(np.uint16))
        assert _violations(d1, oracle.gemm(A, B)) == 0


def test_noalloc_unsplit_shape_and_empty(env):
    """A shape that does not split runs as gemm_f16; an empty one is a no-op."""
    torch, gt, lib, dev = env
    M, N, K = 300, 260, 200
    Ai = datagen.integer_f16(9950, 10, (M, K))
    Bi = datagen.integer_f16(9950, 11, (N, K))
    d1, d2, splits = _pair(env, Ai, Bi)
    assert splits == 1
    assert np.array_equal(d1, oracle.gemm(Ai, Bi)) and np.array_equal(d1, d2)
    assert lib.gemm_splitk_f16_noalloc(None, None, None, 0, 5, 8, None) == 0
