"""The entry points under HIP graph capture.

Every call only enqueues kernels on the caller's stream: no allocation, no
memset (K = 0 writes its zeros with a kernel), no host synchronisation.  A
graph captured around them must therefore give, on every replay, exactly what
the eager calls give.  The graph holds the tiled GEMM, the skinny GEMM, the
K-split GEMV, a bf16 GEMM, a K = 0 fill, a GEMM with the fused bias and
ReLU, the split-K GEMM on a tiled and on a skinny shape (each with its
own workspace) and a 48-row decode batch; it is replayed several times
with eager work between the replays (which also fills the workspaces with
NaN), and every replay is compared bit for bit.
"""
import numpy as np
import pytest

import datagen

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch

    import gemv_tile_pipelined_amd as gt

    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    gt.load_library()
    dev = torch.device("cuda:0")

    def t16(a):
        return torch.from_numpy(a).to(dev)

    A = t16(datagen.uniform_f16(9700, 0, (520, 1032), -1.0, 1.0))
    B = t16(datagen.uniform_f16(9700, 1, (776, 1032), -1.0, 1.0))
    As = t16(datagen.uniform_f16(9700, 2, (8, 4104), -1.0, 1.0))
    Bs = t16(datagen.uniform_f16(9700, 3, (3000, 4104), -0.05, 0.05))
    x = t16(datagen.uniform_f16(9700, 4, (14336,), -1.0, 1.0))
    W = t16(datagen.uniform_f16(9700, 5, (1000, 14336), -0.05, 0.05))
    Ab = A.to(torch.bfloat16)
    Bb = B.to(torch.bfloat16)
    A0 = torch.empty((33, 0), dtype=torch.float16, device=dev)
    B0 = torch.empty((70, 0), dtype=torch.float16, device=dev)
    bias = t16(datagen.uniform_f16(9700, 6, (776,), -4.0, 4.0))

    D = torch.empty((520, 776), dtype=torch.float16, device=dev)
    Ds = torch.empty((8, 3000), dtype=torch.float16, device=dev)
    y = torch.empty((1000,), dtype=torch.float16, device=dev)
    Db = torch.empty((520, 776), dtype=torch.bfloat16, device=dev)
    D0 = torch.empty((33, 70), dtype=torch.float16, device=dev)
    Dr = torch.empty((520, 776), dtype=torch.float16, device=dev)
    # split K: a tiled shape (9 tiles, 6 slices) and a skinny one (32 row blocks, 8 slices)
    Ak = t16(datagen.uniform_f16(9700, 7, (300, 4104), -1.0, 1.0))
    Bk = t16(datagen.uniform_f16(9700, 8, (260, 4104), -1.0, 1.0))
    Aq = t16(datagen.uniform_f16(9700, 9, (8, 8192), -1.0, 1.0))
    Bq = t16(datagen.uniform_f16(9700, 10, (512, 8192), -0.05, 0.05))
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wk = torch.empty((max(gt.splitk_workspace_bytes(300, 260, 4104, cus), 16) // 4,), device=dev)
    wq = torch.empty((max(gt.splitk_workspace_bytes(8, 512, 8192, cus), 16) // 4,), device=dev)
    Dk = torch.empty((300, 260), dtype=torch.float16, device=dev)
    Dq = torch.empty((8, 512), dtype=torch.float16, device=dev)
    # a 48-row decode batch: the skinny kernel with 64 staged rows
    Aw = t16(datagen.uniform_f16(9700, 11, (48, 1032), -1.0, 1.0))
    Bw = t16(datagen.uniform_f16(9700, 12, (1000, 1032), -0.05, 0.05))
    Dw = torch.empty((48, 1000), dtype=torch.float16, device=dev)
    outs = (D, Ds, y, Db, D0, Dr, Dk, Dq, Dw)

    def work():
        gt.gemm_f16(A, B, D)
        gt.gemm_f16(As, Bs, Ds)
        gt.gemv_f16(x, W, y)
        gt.gemm_bf16(Ab, Bb, Db)
        gt.gemm_f16(A0, B0, D0)
        gt.gemm_bias_f16(A, B, bias, "relu", Dr)
        gt.gemm_splitk_f16(Ak, Bk, Dk, workspace=wk)
        gt.gemm_splitk_f16(Aq, Bq, Dq, workspace=wq)
        gt.gemm_f16(Aw, Bw, Dw)

    work()
    torch.cuda.synchronize(dev)
    eager = [o.clone() for o in outs]

    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        work()  # warm-up on the capture stream
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize(dev)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for o in outs + (wk, wq):
            o.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        for got, want in zip(outs, eager):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), rep
    assert bool((D0.view(torch.int16) == 0).all())
    assert np.isfinite(D.float().cpu().numpy()).all()
    if cus == 256:
        assert gt.splitk_splits(300, 260, 4104, cus) == 6 and gt.splitk_splits(8, 512, 8192, cus) == 8
