"""The device operations inside a captured HIP graph: a GEMM, an NCHW
convolution (both of its launches) and a channel-last one recorded once and
replayed several times,
with eager work of the program between the replays; every replay gives the
eager call's bits.  The calls allocate nothing and launch only on the
caller's stream, so capture needs nothing else."""
import pytest
import torch

import tile_size_selection_amd as tss
from tile_size_selection_amd.inputs import draw

pytestmark = pytest.mark.gpu

CUDA = torch.device("cuda:0")


def test_gemm_and_conv_replays_equal_eager():
    A = draw((296, 200), "uniform", -1, 1, "f16", 81).to(CUDA)
    B = draw((200, 328), "uniform", -1, 1, "f16", 82).to(CUDA)
    x = draw((2, 16, 13, 11), "uniform", -1, 1, "f16", 83).to(CUDA)
    w = draw((24, 16, 3, 3), "normal", 0, 0.1, "f16", 84).to(CUDA)
    C = torch.empty(296, 328, dtype=torch.float32, device=CUDA)
    y = torch.empty(2, 24, 7, 11, dtype=torch.float32, device=CUDA)
    cl = torch.channels_last
    xc, wc = x.contiguous(memory_format=cl), w.contiguous(memory_format=cl)
    yc = torch.empty(2, 24, 7, 11, dtype=torch.float32, device=CUDA, memory_format=cl)
    ws = torch.empty(tss.conv2d_workspace_size(2, 16, 13, 11, 24, 3, 3), dtype=torch.uint8, device=CUDA)

    def step():
        tss.gemm(A, B, out_dtype="f32", out=C)
        tss.conv2d(x, w, (2, 1), (1, 1), 1, tile_oh=3, out_dtype="f32", workspace=ws, out=y)
        tss.conv2d(xc, wc, (2, 1), (1, 1), 1, tile_oh=3, out_dtype="f32", out=yc)  # channel-last: one launch

    step()
    torch.cuda.synchronize()
    C_ref, y_ref, yc_ref = C.clone(), y.clone(), yc.clone()
    assert torch.equal(yc.contiguous(), y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # first calls on the capture's stream, outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        C.fill_(float("nan"))
        y.fill_(float("nan"))
        yc.fill_(float("nan"))
        # eager work of the program between replays, on the same operands
        tss.gemm(B.t().contiguous(), A.t().contiguous(), out_dtype="f32")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, C_ref), r
        assert torch.equal(y, y_ref), r
        assert torch.equal(yc, yc_ref), r
