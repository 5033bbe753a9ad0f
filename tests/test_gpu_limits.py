"""The largest sizes the entry points accept, checked by closed forms.

Inputs are built on the device (a host oracle over gigabytes is not needed):
  * gemm_f16 at the largest K (4,194,296: a 256-row panel of A or B then
    spans 2,147,479,552 bytes, just under the 2^31 a buffer descriptor's
    32-bit offsets reach) with A[m,k] = u_m·2^-16 and B[n,k] = v_n, so every
    output is RNE_fp16(K·2^-16·u_m·v_n).  All partial sums are multiples of
    one product below 2^6, exact in FP32 in any order, so the bits must match;
    M = 260 adds a ragged second tile row;
  * the skinny path (8 activation rows) at the same K;
  * gemm_splitk_f16 on both shapes at that K (K split across workgroups:
    42 and 13 slices on 256 CUs), to the same closed form;
  * gemv_f16 at the largest K (2^31 - 8, one row of W is 4 GiB) with unit
    vectors x = e_j at the start, the middle and the end of the row: y[n] is
    then exactly W[n, j], whatever the summation order.
"""
import pytest

pytestmark = pytest.mark.gpu

MAX_GEMM_K = 4194296
MAX_GEMV_K = (1 << 31) - 8


@pytest.fixture(scope="module")
def env():
    import torch

    import gemv_tile_pipelined_amd as gt

    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    gt.load_library()
    return torch, gt, torch.device("cuda:0")


def _rank1(torch, dev, rows, K, scale, seed):
    g = torch.Generator().manual_seed(seed)
    choices = torch.tensor([-1.0, -0.5, 0.5, 1.0], dtype=torch.float64)
    u = choices[torch.randint(0, 4, (rows,), generator=g)]
    t = (u * scale).to(torch.float16).to(dev)
    return u, t[:, None].expand(rows, K).contiguous()


@pytest.mark.parametrize("shape", [(260, 256), (8, 300)], ids=["tiled_260x256", "skinny_8x300"])
def test_gemm_at_largest_k(env, shape):
    torch, gt, dev = env
    M, N = shape
    K = MAX_GEMM_K
    print(f"[limits] gemm {M}x{N}x{K}", flush=True)
    u, A = _rank1(torch, dev, M, K, 2.0**-16, 11)
    v, B = _rank1(torch, dev, N, K, 1.0, 12)
    D = gt.gemm_f16(A, B)
    want = (K * 2.0**-16 * torch.outer(u, v)).to(torch.float16).to(dev)
    torch.cuda.synchronize(dev)
    assert torch.equal(D.view(torch.int16), want.view(torch.int16))
    # split K at the same K: FP32 partial sums of each slice, then their ordered sum
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    print(f"[limits] gemm_splitk {M}x{N}x{K}: {gt.splitk_splits(M, N, K, cus)} slices", flush=True)
    if cus == 256:
        assert gt.splitk_splits(M, N, K, cus) > 1
    Ds = gt.gemm_splitk_f16(A, B, workspace=gt.alloc_splitk_workspace(A, B))
    torch.cuda.synchronize(dev)
    assert torch.equal(Ds.view(torch.int16), want.view(torch.int16))
    del A, B, D, Ds
    torch.cuda.empty_cache()


def test_gemv_at_largest_k(env):
    torch, gt, dev = env
    K = MAX_GEMV_K
    print(f"[limits] gemv 2x{K}", flush=True)
    W = torch.full((2, K), 0.5, dtype=torch.float16, device=dev)
    x = torch.zeros((K,), dtype=torch.float16, device=dev)
    y = torch.empty((2,), dtype=torch.float16, device=dev)
    for j in (0, (1 << 30) + 7, K - 1):
        W[0, j] = 3.0
        W[1, j] = -5.0
        x[j] = 1.0
        gt.gemv_f16(x, W, y)
        torch.cuda.synchronize(dev)
        assert y.tolist() == [3.0, -5.0], j
        x[j] = 0.0
        W[0, j] = 0.5
        W[1, j] = 0.5
    del W, x
    torch.cuda.empty_cache()
