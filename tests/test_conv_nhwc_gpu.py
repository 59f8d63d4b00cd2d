"""Channel-last convolution (tss_conv2d_nhwc): x, w and y in torch's
channels_last format, read and written in place by the implicit GEMM.
Parity against the fp64 direct convolution of the oracle (which takes NCHW /
OIHW arrays: the tests permute on the host), exact for integer inputs."""
import numpy as np
import pytest
import torch

import tile_size_selection_amd as tss
from oracle import gemm_conv as G
from oracle import planner as OP
from tile_size_selection_amd.inputs import WORKLOADS, draw
from gpu_util import check_bound, to_f64

pytestmark = pytest.mark.gpu

CUDA = torch.device("cuda:0")
CL = torch.channels_last


def _cl(t):
    """A host NCHW tensor as a channels_last device tensor (same values)."""
    return t.to(CUDA).contiguous(memory_format=CL)


def _configs():
    g = OP.device_gfx950()
    return [tss.TileConfig(c.block_m, c.block_n, c.block_k, c.stages, c.threads, c.instr)
            for c in OP.candidates(g, 1 << 20, ["mfma32", "mfma16"]) if OP.evaluate(c, g).feasible]


def test_conv_nhwc_workload_matches_oracle_and_nchw_path():
    """The conv workload (8x256x56x56, 3x3, stride 2, pad 1) on channel-last
    tensors: within the bound of the fp64 oracle, and the same bits as the
    NCHW path (C = 256 is a multiple of every K step, so both paths run the
    same kernel on the same K order)."""
    wl = WORKLOADS[5]
    x, w = wl.make()
    y = tss.conv2d(_cl(x), _cl(w), wl.stride, wl.pad, wl.dil, tile_oh=wl.tile_oh, out_dtype=wl.out_dtype)
    assert y.is_contiguous(memory_format=CL) and tuple(y.shape) == (8, 256, 28, 28)
    ref, S = G.conv2d(x.double().numpy(), w.double().numpy(), wl.stride, wl.pad, wl.dil)
    check_bound(to_f64(y), ref, S, wl.name + " nhwc")
    y_nchw = tss.conv2d(x.to(CUDA), w.to(CUDA), wl.stride, wl.pad, wl.dil, tile_oh=wl.tile_oh, out_dtype=wl.out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y.contiguous(), y_nchw)


def test_conv_nhwc_workload_exact_integer():
    """Integer inputs on the workload's geometry: every output exact."""
    wl = WORKLOADS[5]
    x = draw((wl.N, wl.C, wl.H, wl.W), "int", -2, 2, "f16", 611)
    w = draw((wl.Co, wl.C, wl.kh, wl.kw), "int", -2, 2, "f16", 612)
    ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), wl.stride, wl.pad, wl.dil)
    y = tss.conv2d(_cl(x), _cl(w), wl.stride, wl.pad, wl.dil, tile_oh=wl.tile_oh, out_dtype="f32")
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(y), ref)


# (N, C, H, W, Cout, kh, kw, stride, pad, dilation, (tile_n, tile_oh, tile_ow))
CASES = [
    (2, 8, 9, 7, 13, 3, 3, (1, 1), (1, 1), (1, 1), (2, 9, 7)),
    (1, 16, 12, 12, 40, 5, 5, (2, 2), (2, 2), (1, 1), (1, 3, 2)),
    (3, 24, 10, 13, 70, 3, 1, (1, 2), (0, 3), (2, 1), (2, 4, 5)),
    (2, 40, 15, 6, 33, 1, 1, (1, 1), (0, 0), (1, 1), (1, 15, 6)),
    (1, 64, 17, 17, 130, 3, 3, (2, 2), (1, 1), (1, 1), (1, 2, 3)),
    (2, 96, 8, 8, 64, 3, 3, (1, 1), (1, 1), (1, 1), (1, 8, 8)),
    (2, 128, 7, 9, 96, 2, 3, (3, 2), (1, 0), (1, 2), (2, 1, 4)),
    (1, 8, 5, 5, 7, 5, 5, (1, 1), (4, 4), (1, 1), (1, 2, 9)),   # windows mostly in the padding
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_conv_nhwc_exact(case, dtype):
    """Ragged geometries and tilings (C = 8, 24, 40: below or between the K
    steps, so each tap's channel padding is read as zero), the plan's tile
    and a spread of explicit tiles: exact for integer inputs, fp32 output,
    every output element."""
    N, C, H, W, Co, kh, kw, st, pd, dl, (tn, toh, tow) = CASES[case]
    OH = (H + 2 * pd[0] - (kh - 1) * dl[0] - 1) // st[0] + 1
    OW = (W + 2 * pd[1] - (kw - 1) * dl[1] - 1) // st[1] + 1
    toh, tow = min(toh, OH), min(tow, OW)
    x = draw((N, C, H, W), "int", -2, 2, dtype, 620 + case)
    w = draw((Co, C, kh, kw), "int", -2, 2, dtype, 640 + case)
    ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), st, pd, dl)
    dx, dw = _cl(x), _cl(w)
    cfgs = [None] + _configs()[case::37]
    for cfg in cfgs:
        y = tss.conv2d(dx, dw, st, pd, dl, tile_oh=toh, tile_ow=tow, tile_n=tn, out_dtype="f32", cfg=cfg)
        torch.cuda.synchronize()
        assert y.is_contiguous(memory_format=CL)
        assert np.array_equal(to_f64(y), ref), (CASES[case], cfg)


def test_every_conv_kernel_exact_nhwc():
    """Every compiled convolution kernel on channel-last tensors, ragged
    everywhere (C = 40: every K step pads the channels of each tap), tiles of
    1 image x 3 rows x 4 columns."""
    N, C, H, W, Co, kh, kw, st, pd, dl = 2, 40, 11, 9, 70, 3, 3, (2, 1), (1, 2), (1, 1)
    x = draw((N, C, H, W), "int", -2, 2, "f16", 651)
    w = draw((Co, C, kh, kw), "int", -2, 2, "f16", 652)
    ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), st, pd, dl)
    dx, dw = _cl(x), _cl(w)
    bad = []
    cfgs = _configs()
    assert len(cfgs) == 292
    for cfg in cfgs:
        y = tss.conv2d(dx, dw, st, pd, dl, tile_oh=3, tile_ow=4, tile_n=1, out_dtype="f32", cfg=cfg)
        torch.cuda.synchronize()
        if not np.array_equal(to_f64(y), ref):
            bad.append(cfg)
    assert not bad, bad[:4]


def test_conv_nhwc_low_precision_output_and_split_k():
    """fp16 / bf16 output: the exact sum (integer inputs, exact in fp32)
    rounded once to nearest even; and split K over 2, 3 and 5 ranges: the
    exact fp32 result."""
    N, C, H, W, Co, kh, kw, st, pd, dl = 2, 32, 10, 10, 48, 3, 3, (1, 1), (1, 1), (1, 1)
    for dtype in ("f16", "bf16"):
        x = draw((N, C, H, W), "int", -1, 1, dtype, 661)
        w = draw((Co, C, kh, kw), "int", -1, 1, dtype, 662)
        ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), st, pd, dl)
        dx, dw = _cl(x), _cl(w)
        y = tss.conv2d(dx, dw, st, pd, dl, out_dtype=dtype)
        torch.cuda.synchronize()
        tdt = torch.float16 if dtype == "f16" else torch.bfloat16
        want = torch.from_numpy(ref).to(tdt).to(torch.float64).numpy()  # the exact sum rounded once (RNE)
        assert np.array_equal(to_f64(y), want), dtype
        cfg = tss.TileConfig(64, 64, 32, 2, 256, "mfma16")
        for s in (2, 3, 5):
            ys = tss.conv2d(dx, dw, st, pd, dl, out_dtype="f32", splits=s, cfg=cfg)
            torch.cuda.synchronize()
            assert np.array_equal(to_f64(ys), ref), (dtype, s)


def test_conv_nhwc_split_plan_and_errors():
    """The split-K plan's count (splits = 0) on a problem with few output
    tiles and a long K, exact; C not a multiple of 8 and tensors in the
    wrong memory format are refused."""
    x = draw((1, 48, 6, 6), "int", -1, 1, "f16", 673)
    w = draw((8, 48, 3, 3), "int", -1, 1, "f16", 674)
    ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), (1, 1), (1, 1), (1, 1))
    for splits in (0, 1, 4):
        y = tss.conv2d(_cl(x), _cl(w), 1, 1, 1, out_dtype="f32", splits=splits)
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(y), ref), splits
    xb = draw((1, 12, 6, 6), "int", -1, 1, "f16", 671)
    wb = draw((8, 12, 3, 3), "int", -1, 1, "f16", 672)
    with pytest.raises(tss.TssError):
        tss.conv2d(_cl(xb), _cl(wb), 1, 1, 1)                # C = 12
    with pytest.raises(ValueError):
        tss.conv2d(_cl(x), w.to(CUDA), 1, 1, 1, layout="nhwc")  # OIHW weights
    with pytest.raises(ValueError):
        tss.conv2d(x.to(CUDA), _cl(w), 1, 1, 1, layout="nhwc")  # NCHW input


def test_random_conv_geometries_nhwc_exact():
    """Random geometries (C a multiple of 8 up to 264, windows up to 7x7,
    strides up to 4, dilations up to 3, pads up to 4, random tiles), each
    with a random feasible tile configuration and dtype, channel-last
    tensors: exact for integer inputs."""
    rng = np.random.default_rng(2027)
    cfgs = _configs()
    bad = []
    n = 0
    while n < 40:
        N, C, Co = int(rng.integers(1, 3)), 8 * int(rng.integers(1, 34)), int(rng.integers(1, 140))
        H, W = int(rng.integers(1, 20)), int(rng.integers(1, 20))
        kh, kw = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        st = (int(rng.integers(1, 5)), int(rng.integers(1, 5)))
        pd = (int(rng.integers(0, 5)), int(rng.integers(0, 5)))
        dl = (int(rng.integers(1, 4)), int(rng.integers(1, 4)))
        if H + 2 * pd[0] < (kh - 1) * dl[0] + 1 or W + 2 * pd[1] < (kw - 1) * dl[1] + 1:
            continue
        OH = (H + 2 * pd[0] - (kh - 1) * dl[0] - 1) // st[0] + 1
        OW = (W + 2 * pd[1] - (kw - 1) * dl[1] - 1) // st[1] + 1
        toh, tow, tn = int(rng.integers(1, OH + 1)), int(rng.integers(1, OW + 1)), int(rng.integers(1, N + 1))
        cfg = cfgs[int(rng.integers(0, len(cfgs)))]
        dtype = ["f16", "bf16"][int(rng.integers(0, 2))]
        x = draw((N, C, H, W), "int", -2, 2, dtype, 700 + n)
        w = draw((Co, C, kh, kw), "int", -2, 2, dtype, 800 + n)
        ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), st, pd, dl)
        y = tss.conv2d(_cl(x), _cl(w), st, pd, dl, tile_oh=toh, tile_ow=tow, tile_n=tn, out_dtype="f32", cfg=cfg,
                       layout="nhwc")
        torch.cuda.synchronize()
        if not (y.is_contiguous(memory_format=CL) and np.array_equal(to_f64(y), ref)):
            bad.append((N, C, H, W, Co, kh, kw, st, pd, dl, toh, tow, tn, cfg, dtype))
        n += 1
    assert not bad, bad[:3]
