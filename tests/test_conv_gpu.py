"""Convolution parity on the GPU: the implicit GEMM over H-tiles against the
fp64 direct convolution of the oracle, and H-tiled against untiled."""
import numpy as np
import pytest
import torch

import tile_size_selection_amd as tss
from oracle import gemm_conv as G
from tile_size_selection_amd.inputs import WORKLOADS, draw
from gpu_util import check_bound, to_f64

pytestmark = pytest.mark.gpu

CUDA = torch.device("cuda:0")


def test_conv_workload_full_parity():
    w = WORKLOADS[5]
    x, wt = w.make()
    cfg = tss.conv2d_default_config(w.N, w.C, w.H, w.W, w.Co, w.kh, w.kw, w.stride, w.pad, w.dil)
    print("planner choice for", w.name, cfg, flush=True)
    y = tss.conv2d(x.to(CUDA), wt.to(CUDA), w.stride, w.pad, w.dil, tile_oh=w.tile_oh, out_dtype=w.out_dtype)
    ref, S = G.conv2d(x.double().numpy(), wt.double().numpy(), w.stride, w.pad, w.dil)
    assert tuple(y.shape) == ref.shape == (8, 256, 28, 28)
    check_bound(to_f64(y), ref, S, w.name)


def test_conv_htiled_equals_untiled_bitwise():
    """The H-tiles only decide which input rows a block reads; with the same
    tile configuration the sums run in the same order, so every tile_oh gives
    the same bits as one tile covering all 28 output rows."""
    w = WORKLOADS[5]
    x, wt = w.make()
    dx, dw = x.to(CUDA), wt.to(CUDA)
    cfg = tss.TileConfig(128, 128, 64, 2, 256, "mfma32")
    whole = tss.conv2d(dx, dw, w.stride, w.pad, w.dil, tile_oh=28, out_dtype="f32", cfg=cfg)
    for toh in (8, 1, 3, 5, 27):
        part = tss.conv2d(dx, dw, w.stride, w.pad, w.dil, tile_oh=toh, out_dtype="f32", cfg=cfg)
        torch.cuda.synchronize()
        assert torch.equal(whole, part), toh


CASES = [  # N, C, H, W, Co, kh, kw, stride, pad, dil, tile_oh
    (2, 8, 9, 9, 16, 3, 3, (2, 2), (1, 1), (1, 1), 2),       # the worked example's H geometry
    (1, 16, 13, 11, 24, 3, 3, (1, 1), (1, 1), (1, 1), 4),
    (3, 8, 17, 6, 40, 5, 5, (2, 1), (2, 2), (1, 1), 3),
    (2, 32, 15, 7, 8, 3, 3, (1, 2), (2, 1), (2, 1), 5),
    (1, 64, 8, 8, 72, 1, 1, (1, 1), (0, 0), (1, 1), 3),      # 1x1: a plain GEMM
    (2, 8, 11, 4, 16, 2, 2, (3, 2), (0, 1), (1, 2), 1),
    (1, 24, 30, 30, 136, 3, 3, (2, 2), (1, 1), (1, 1), 7),   # ragged channel tiles
    (2, 3, 17, 17, 16, 3, 3, (2, 2), (1, 1), (1, 1), 4),     # 3 channels, padded to 8 in the channel-last copy
    (1, 12, 10, 12, 8, 3, 2, (1, 1), (1, 0), (1, 1), 10),    # C*kh*kw = 72, Cp = 16
    # 6x6 outputs, one row per H-tile: groups of 4 pixels that are one aligned
    # run of y, that straddle two images, or that start misaligned
    (3, 16, 12, 12, 24, 3, 3, (2, 2), (1, 1), (1, 1), 1),
    # pads of 2 at stride 3 (rows) and stride 2 (columns) with 1-tap windows:
    # the first and last output rows or columns read only padding, so their
    # tiles' input slices are empty and their outputs are zero
    (3, 16, 3, 6, 68, 1, 4, (3, 3), (2, 2), (1, 2), 1),
    (3, 27, 12, 5, 68, 5, 1, (2, 2), (0, 2), (2, 2), 2),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_conv_small_exact(case, dtype):
    """Integer inputs: the fp32 result is exact, for the planner's choice and
    for a spread of tile configurations."""
    N, Ci, H, W, Co, kh, kw, st, pd, dl, toh = case
    x = draw((N, Ci, H, W), "int", -2, 2, dtype, 51)
    w = draw((Co, Ci, kh, kw), "int", -2, 2, dtype, 52)
    ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), st, pd, dl)
    dx, dw = x.to(CUDA), w.to(CUDA)
    cfgs = [None, tss.TileConfig(64, 64, 16, 2, 128, "mfma32"), tss.TileConfig(128, 64, 64, 3, 256, "mfma16"),
            tss.TileConfig(64, 128, 32, 4, 256, "mfma32"), tss.TileConfig(256, 128, 32, 2, 512, "mfma32")]
    for cfg in cfgs:
        y = tss.conv2d(dx, dw, st, pd, dl, tile_oh=toh, out_dtype="f32", cfg=cfg)
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(y), ref), (case, cfg)


TILINGS = {  # case index in CASES -> (tile_n, tile_oh, tile_ow) triples, ragged tiles included
    0: [(1, 2, 2), (2, 5, 3), (1, 1, 5), (2, 3, 1)],
    1: [(1, 4, 3), (1, 13, 4), (1, 5, 11)],
    2: [(2, 3, 4), (1, 9, 1), (3, 2, 5)],
    3: [(1, 5, 3), (2, 7, 2), (1, 15, 1)],
    5: [(1, 1, 1), (2, 2, 2), (1, 3, 1)],
    9: [(2, 1, 4), (1, 6, 5), (3, 4, 6)],
    10: [(1, 1, 2), (3, 1, 1), (2, 2, 1)],
    11: [(2, 2, 1), (1, 1, 1), (3, 2, 5)],
}


@pytest.mark.parametrize("idx", sorted(TILINGS))
def test_conv_2d_and_batch_tiles_exact(idx):
    """Tiles of images x output rows x output columns, each reading its row
    and column slices with the H/W formulas' pads: integer inputs give the
    exact result, and every tiling gives the bits of the untiled run with the
    same tile configuration."""
    N, Ci, H, W, Co, kh, kw, st, pd, dl, _ = CASES[idx]
    x = draw((N, Ci, H, W), "int", -2, 2, "f16", 71)
    w = draw((Co, Ci, kh, kw), "int", -2, 2, "f16", 72)
    ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), st, pd, dl)
    dx, dw = x.to(CUDA), w.to(CUDA)
    for cfg in (None, tss.TileConfig(64, 64, 16, 2, 128, "mfma32"), tss.TileConfig(128, 64, 64, 3, 256, "mfma16")):
        whole = tss.conv2d(dx, dw, st, pd, dl, out_dtype="f32", cfg=cfg)
        for tn, toh, tow in TILINGS[idx]:
            y = tss.conv2d(dx, dw, st, pd, dl, tile_oh=toh, tile_ow=tow, tile_n=tn, out_dtype="f32", cfg=cfg)
            torch.cuda.synchronize()
            assert np.array_equal(to_f64(y), ref), (idx, cfg, tn, toh, tow)
            assert torch.equal(y, whole), (idx, cfg, tn, toh, tow)


def test_conv_workload_2d_tiles():
    """The conv workload cut into 8x8-pixel tiles of 2 images: within the
    bound of the fp64 oracle, and the same bits as its H-tiles alone."""
    w = WORKLOADS[5]
    x, wt = w.make()
    dx, dw = x.to(CUDA), wt.to(CUDA)
    y = tss.conv2d(dx, dw, w.stride, w.pad, w.dil, tile_oh=8, tile_ow=8, tile_n=2, out_dtype=w.out_dtype)
    h_only = tss.conv2d(dx, dw, w.stride, w.pad, w.dil, tile_oh=8, out_dtype=w.out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y, h_only)
    ref, S = G.conv2d(x.double().numpy(), wt.double().numpy(), w.stride, w.pad, w.dil)
    check_bound(to_f64(y), ref, S, w.name + " 2-D tiles")


def test_conv_low_precision_output():
    w = WORKLOADS[5]
    x, wt = w.make()
    x, wt = x[:2, :64].contiguous(), wt[:64, :64].contiguous()
    ref, S = G.conv2d(x.double().numpy(), wt.double().numpy(), w.stride, w.pad, w.dil)
    y = tss.conv2d(x.to(CUDA), wt.to(CUDA), w.stride, w.pad, w.dil, tile_oh=8)
    assert y.dtype == torch.float16
    check_bound(to_f64(y), ref, S, "conv f16 out")


def test_conv_two_operand_sets_alternate_exact():
    """A workspace with room for two sets of the operand copies: consecutive
    calls alternate between the sets (one call writes the set the previous
    call's GEMM did not read).  Five calls in a row on two problems, one pass
    and split K (two sets, then the partial outputs after both): every
    output exact, whichever set a call took."""
    shapes = ((2, 16, 13, 11, 24, 3, 3), (1, 8, 9, 9, 16, 3, 3))
    set_bytes = max((tss.conv2d_workspace_size(*sh) + 255) // 256 * 256 for sh in shapes)
    part = 4 * 2 * 24 * 7 * 11 * 4                       # 4 ranges of the first problem's fp32 output
    ws = torch.empty(2 * set_bytes + part, dtype=torch.uint8, device=CUDA)
    for call in range(5):
        N, Ci, H, W, Co, kh, kw = shapes[call % 2]
        x = draw((N, Ci, H, W), "int", -2, 2, "f16", 90 + call)
        w = draw((Co, Ci, kh, kw), "int", -2, 2, "f16", 95 + call)
        ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), (2, 1), (1, 1), (1, 1))
        for splits in (1, 4):
            y = tss.conv2d(x.to(CUDA), w.to(CUDA), (2, 1), (1, 1), 1, tile_oh=2, out_dtype="f32", workspace=ws,
                           splits=splits)
            torch.cuda.synchronize()
            assert np.array_equal(to_f64(y), ref), (call, splits)


def test_conv_workspace_reuse_and_errors():
    """A caller-owned workspace serves calls of different sizes in a row on
    one stream; a workspace below tss_conv2d_workspace_size is rejected
    before anything is launched."""
    big = (2, 16, 13, 11, 24, 3, 3)
    small = (1, 8, 9, 9, 16, 3, 3)
    nbytes = tss.conv2d_workspace_size(*big)
    assert nbytes == 2 * 13 * 11 * 64 * 2 + 24 * 9 * 64 * 2     # channels padded to 64; 36608 B is 256-aligned
    ws = torch.empty(nbytes, dtype=torch.uint8, device=CUDA)
    for shape, seed in ((big, 61), (small, 63), (big, 65)):
        N, Ci, H, W, Co, kh, kw = shape
        x = draw((N, Ci, H, W), "int", -2, 2, "f16", seed)
        w = draw((Co, Ci, kh, kw), "int", -2, 2, "f16", seed + 1)
        ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), (2, 1), (1, 1), (1, 1))
        y = tss.conv2d(x.to(CUDA), w.to(CUDA), (2, 1), (1, 1), 1, tile_oh=2, out_dtype="f32", workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(y), ref), shape
    x = torch.zeros((2, 16, 13, 11), dtype=torch.float16, device=CUDA)
    w = torch.zeros((24, 16, 3, 3), dtype=torch.float16, device=CUDA)
    with pytest.raises(ValueError):
        tss.conv2d(x, w, 1, 1, 1, workspace=ws[: nbytes - 1])
