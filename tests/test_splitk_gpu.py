"""Split K on the GPU: the GEMM and the convolution with their K loops cut
into ranges, each range's fp32 partial output in a workspace and a second
pass that adds them in range order.

Integer operands in [-2, 2] keep every partial sum an exact integer in fp32,
so each split count must give exactly the fp64 oracle's result: a range
dropped, counted twice or started at the wrong K tile (or, in the
convolution, at the wrong tap or channel) shows as a mismatch."""
import numpy as np
import pytest
import torch

import tile_size_selection_amd as tss
from oracle import gemm_conv as G
from tile_size_selection_amd.inputs import WORKLOADS, draw
from gpu_util import check_bound, to_f64

pytestmark = pytest.mark.gpu

CUDA = torch.device("cuda:0")

GEMM_CFGS = [tss.TileConfig(64, 64, 64, 2, 256, "mfma16"), tss.TileConfig(128, 128, 32, 3, 256, "mfma32"),
             tss.TileConfig(256, 256, 64, 2, 512, "mfma16"), tss.TileConfig(64, 128, 16, 4, 128, "mfma32")]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gemm_splits_exact_on_ragged_batched_problem(dtype):
    bt, M, N, K = 2, 300, 328, 1000          # ragged in M, N and K for every tile
    A = draw((bt, M, K), "int", -2, 2, dtype, 91)
    B = draw((bt, K, N), "int", -2, 2, dtype, 92)
    ref, _ = G.gemm(A.double().numpy(), B.double().numpy(), with_abs=False)
    dA, dB = A.to(CUDA), B.to(CUDA)
    for cfg in GEMM_CFGS:
        for splits in (2, 3, 4, 5, 6, 7, 8, 64):
            out = torch.full((bt, M, N), float("nan"), dtype=torch.float32, device=CUDA)
            tss.gemm(dA, dB, out_dtype="f32", cfg=cfg, out=out, splits=splits)
            torch.cuda.synchronize()
            assert np.array_equal(to_f64(out), ref), (cfg, splits)


def test_gemm_splits_low_precision_output_and_determinism():
    """fp16/bf16 outputs: the reduction rounds the exact fp32 sum to nearest
    even (exact here: |c| <= 256 for bf16 with K = 64 ... inputs in {-1, 0, 1}
    and K = 192); two runs give the same bits."""
    M, N, K = 200, 264, 192
    for dtype in ("f16", "bf16"):
        A = draw((M, K), "int", -1, 1, dtype, 93)
        B = draw((K, N), "int", -1, 1, dtype, 94)
        ref, _ = G.gemm(A.double().numpy(), B.double().numpy(), with_abs=False)
        dA, dB = A.to(CUDA), B.to(CUDA)
        for splits in (2, 3):
            c1 = tss.gemm(dA, dB, cfg=GEMM_CFGS[1], splits=splits)
            c2 = tss.gemm(dA, dB, cfg=GEMM_CFGS[1], splits=splits)
            torch.cuda.synchronize()
            assert torch.equal(c1, c2)
            assert np.array_equal(to_f64(c1), ref), (dtype, splits)


def test_gemm_splits_float_inputs_within_bound_and_repeatable():
    w = WORKLOADS[1]     # 256^3, U[-1, 1], fp32 out
    A, B = w.make()
    ref, S = G.gemm(A.double().numpy(), B.double().numpy())
    dA, dB = A.to(CUDA), B.to(CUDA)
    for splits in (2, 4, 8):
        got = tss.gemm(dA, dB, out_dtype="f32", splits=splits)
        again = tss.gemm(dA, dB, out_dtype="f32", splits=splits)
        torch.cuda.synchronize()
        check_bound(to_f64(got), ref, S, f"256^3 split {splits}")
        assert torch.equal(got, again)


def test_gemm_split_edges_and_errors():
    A = draw((130, 24), "int", -2, 2, "f16", 95).to(CUDA)
    B = draw((24, 72), "int", -2, 2, "f16", 96).to(CUDA)
    ref, _ = G.gemm(A.double().cpu().numpy(), B.double().cpu().numpy(), with_abs=False)
    # K = 24 is one K step of 64: any split count runs one range
    got = tss.gemm(A, B, out_dtype="f32", cfg=GEMM_CFGS[0], splits=8)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(got), ref)
    # K = 0: zeros, whatever the split count
    Z = tss.gemm(torch.zeros((5, 0), dtype=torch.float16, device=CUDA),
                 torch.zeros((0, 16), dtype=torch.float16, device=CUDA), out_dtype="f32", splits=4)
    torch.cuda.synchronize()
    assert (Z == 0).all().item()
    small = torch.empty(64, dtype=torch.uint8, device=CUDA)
    A2 = draw((64, 512), "int", -2, 2, "f16", 97).to(CUDA)
    B2 = draw((512, 64), "int", -2, 2, "f16", 98).to(CUDA)
    with pytest.raises(ValueError):
        tss.gemm(A2, B2, splits=4, workspace=small)
    with pytest.raises(tss.TssError):
        tss.gemm(A2, B2, splits=-1)
    with pytest.raises(tss.TssError):
        tss.gemm(A2, B2, splits=257)


CONVS = [  # N, C, H, W, Co, kh, kw, stride, pad, dil, tile_oh
    (2, 24, 15, 13, 40, 3, 3, (2, 2), (1, 1), (1, 1), 3),
    (1, 64, 9, 9, 72, 3, 3, (1, 1), (1, 1), (1, 1), 9),
    (3, 12, 10, 12, 8, 3, 2, (1, 1), (1, 0), (1, 1), 4),   # channels padded to the K step
    (2, 130, 8, 8, 16, 1, 1, (1, 1), (0, 0), (1, 1), 8),    # 1x1: the split is over channels only
]


def test_conv_splits_exact():
    for (N, C, H, W, Co, kh, kw, st, pd, dl, toh) in CONVS:
        x = draw((N, C, H, W), "int", -2, 2, "f16", 101)
        w = draw((Co, C, kh, kw), "int", -2, 2, "f16", 102)
        ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), st, pd, dl, with_abs=False)
        dx, dw = x.to(CUDA), w.to(CUDA)
        for cfg in (tss.TileConfig(64, 64, 32, 3, 256, "mfma32"), tss.TileConfig(128, 64, 64, 4, 512, "mfma16")):
            for splits in (2, 3, 5, 8):
                y = tss.conv2d(dx, dw, st, pd, dl, tile_oh=toh, out_dtype="f32", cfg=cfg, splits=splits)
                torch.cuda.synchronize()
                assert np.array_equal(to_f64(y), ref), ((N, C, H, W, Co, kh, kw), cfg, splits)


def test_conv_workload_split_within_bound():
    w = WORKLOADS[5]
    x, wt = w.make()
    ref, S = G.conv2d(x.double().numpy(), wt.double().numpy(), w.stride, w.pad, w.dil)
    dx, dw = x.to(CUDA), wt.to(CUDA)
    for splits in (2, 4):
        y = tss.conv2d(dx, dw, w.stride, w.pad, w.dil, tile_oh=w.tile_oh, out_dtype=w.out_dtype, splits=splits)
        y2 = tss.conv2d(dx, dw, w.stride, w.pad, w.dil, tile_oh=w.tile_oh, out_dtype=w.out_dtype, splits=splits)
        torch.cuda.synchronize()
        check_bound(to_f64(y), ref, S, f"conv split {splits}")
        assert torch.equal(y, y2)


def test_planned_split_count_exact_and_used():
    """splits = 0: the split-K plan's count and tile (tss_splitk_plan) are what
    runs; exact on integer operands."""
    M, N, K = 128, 192, 8192
    S, v = tss.splitk_plan(M, N, K)
    assert S > 1                                  # 2 tiles for 256 CUs: the plan splits
    A = draw((M, K), "int", -2, 2, "f16", 103)
    B = draw((K, N), "int", -2, 2, "f16", 104)
    ref, _ = G.gemm(A.double().numpy(), B.double().numpy(), with_abs=False)
    dA, dB = A.to(CUDA), B.to(CUDA)
    got = tss.gemm(dA, dB, out_dtype="f32", splits=0)
    same = tss.gemm(dA, dB, out_dtype="f32", cfg=v["config"], splits=S)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(got), ref) and torch.equal(got, same)
    x = draw((1, 512, 6, 6), "int", -2, 2, "f16", 105)
    w = draw((8, 512, 3, 3), "int", -2, 2, "f16", 106)
    yref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), (1, 1), (1, 1), (1, 1), with_abs=False)
    Sc, _ = tss.conv_splitk_plan(8, 36, 512, 9)
    assert Sc > 1
    y = tss.conv2d(x.to(CUDA), w.to(CUDA), 1, 1, 1, out_dtype="f32", splits=0)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(y), yref)
