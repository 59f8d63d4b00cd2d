"""Randomized parity: seeded random shapes and convolution geometries through
the C ABI with the planner's own tile, against the fp64 oracle.  Inputs are
integers in [-2, 2], so every fp32 partial sum is an exact integer and the
GPU result must equal the oracle's bit for bit, whatever the tile, the K
split into steps or the order of accumulation."""
import numpy as np
import pytest
import torch

import tile_size_selection_amd as tss
from oracle import gemm_conv as G
from tile_size_selection_amd.inputs import draw
from gpu_util import to_f64

pytestmark = pytest.mark.gpu

CUDA = torch.device("cuda:0")


def _gemm_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        bt = int(rng.integers(1, 4))
        M = int(rng.integers(1, 700))
        N = 8 * int(rng.integers(1, 90))
        K = 8 * int(rng.integers(1, 80))
        dtype = ["f16", "bf16"][int(rng.integers(0, 2))]
        cases.append((bt, M, N, K, dtype))
    return cases


def _conv_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        N, C, Co = int(rng.integers(1, 4)), int(rng.integers(1, 41)), int(rng.integers(1, 80))
        H, W = int(rng.integers(1, 24)), int(rng.integers(1, 24))
        kh, kw = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        sh, sw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        ph, pw = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        dh, dw = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        if H + 2 * ph < (kh - 1) * dh + 1 or W + 2 * pw < (kw - 1) * dw + 1:
            continue
        OH = (H + 2 * ph - (kh - 1) * dh - 1) // sh + 1
        OW = (W + 2 * pw - (kw - 1) * dw - 1) // sw + 1
        toh, tow, tn = int(rng.integers(1, OH + 1)), int(rng.integers(1, OW + 1)), int(rng.integers(1, N + 1))
        dtype = ["f16", "bf16"][int(rng.integers(0, 2))]
        cases.append((N, C, H, W, Co, kh, kw, (sh, sw), (ph, pw), (dh, dw), toh, tow, tn, dtype))
    return cases


GEMM_CASES = _gemm_cases(60, 2024)
CONV_CASES = _conv_cases(60, 2025)


def test_random_gemm_shapes_exact():
    bad = []
    for idx, (bt, M, N, K, dtype) in enumerate(GEMM_CASES):
        print("gemm case", idx, (bt, M, N, K, dtype), flush=True)
        A = draw((bt, M, K), "int", -2, 2, dtype, 100 + idx)
        B = draw((bt, K, N), "int", -2, 2, dtype, 200 + idx)
        ref, _ = G.gemm(A.double().numpy(), B.double().numpy())
        got = tss.gemm(A.to(CUDA), B.to(CUDA), out_dtype="f32")
        torch.cuda.synchronize()
        if not np.array_equal(to_f64(got), ref):
            bad.append((idx, bt, M, N, K, dtype))
    assert not bad, bad[:5]


def test_random_conv_geometries_exact():
    bad = []
    for idx, (N, C, H, W, Co, kh, kw, st, pd, dl, toh, tow, tn, dtype) in enumerate(CONV_CASES):
        print("conv case", idx, (N, C, H, W, Co, kh, kw, st, pd, dl, toh, tow, tn, dtype), flush=True)
        x = draw((N, C, H, W), "int", -2, 2, dtype, 300 + idx)
        w = draw((Co, C, kh, kw), "int", -2, 2, dtype, 400 + idx)
        ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), st, pd, dl)
        got = tss.conv2d(x.to(CUDA), w.to(CUDA), st, pd, dl, tile_oh=toh, tile_ow=tow, tile_n=tn, out_dtype="f32")
        torch.cuda.synchronize()
        if not np.array_equal(to_f64(got), ref):
            bad.append((idx, N, C, H, W, Co, kh, kw, st, pd, dl, toh, tow, tn, dtype))
    assert not bad, bad[:5]


def _feasible_configs():
    from oracle import planner as OP
    g = OP.device_gfx950()
    return [tss.TileConfig(c.block_m, c.block_n, c.block_k, c.stages, c.threads, c.instr)
            for c in OP.candidates(g, 1 << 20, ["mfma32", "mfma16"]) if OP.evaluate(c, g).feasible]


def test_every_conv_kernel_exact_on_ragged_tiles():
    """Every compiled convolution kernel on one geometry that is ragged
    everywhere (channels, output rows and columns, images, K tiles) and cut
    into tiles of 1 image x 3 rows x 4 columns: exact for integer inputs."""
    N, C, H, W, Co, kh, kw, st, pd, dl = 2, 20, 11, 9, 70, 3, 3, (2, 1), (1, 2), (1, 1)
    x = draw((N, C, H, W), "int", -2, 2, "f16", 501)
    w = draw((Co, C, kh, kw), "int", -2, 2, "f16", 502)
    ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), st, pd, dl)
    dx, dw = x.to(CUDA), w.to(CUDA)
    bad = []
    for cfg in _feasible_configs():
        y = tss.conv2d(dx, dw, st, pd, dl, tile_oh=3, tile_ow=4, tile_n=1, out_dtype="f32", cfg=cfg)
        torch.cuda.synchronize()
        if not np.array_equal(to_f64(y), ref):
            bad.append(cfg)
    assert not bad, bad[:4]


def test_random_conv_geometries_and_tile_configs_exact():
    """Wider random geometries (up to 300 channels, 7x7 windows, stride 4,
    dilation 3, pad 4), each with a random feasible tile configuration."""
    rng = np.random.default_rng(2026)
    cfgs = _feasible_configs()
    bad = []
    n = 0
    while n < 40:
        N, C, Co = int(rng.integers(1, 3)), int(rng.integers(1, 301)), int(rng.integers(1, 140))
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
        case = (N, C, H, W, Co, kh, kw, st, pd, dl, toh, tow, tn, dtype, cfg)
        print("conv case", n, case, flush=True)
        x = draw((N, C, H, W), "int", -2, 2, dtype, 600 + n)
        w = draw((Co, C, kh, kw), "int", -2, 2, dtype, 700 + n)
        ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), st, pd, dl)
        got = tss.conv2d(x.to(CUDA), w.to(CUDA), st, pd, dl, tile_oh=toh, tile_ow=tow, tile_n=tn, out_dtype="f32",
                         cfg=cfg)
        torch.cuda.synchronize()
        if not np.array_equal(to_f64(got), ref):
            bad.append(case)
        n += 1
    assert not bad, bad[:5]


def test_random_gemm_shapes_and_tile_configs_exact():
    """Random shapes, each with a random feasible tile configuration, both
    input dtypes and fp32 output: exact for integer inputs."""
    rng = np.random.default_rng(2027)
    cfgs = _feasible_configs()
    bad = []
    for n in range(60):
        bt, M = int(rng.integers(1, 4)), int(rng.integers(1, 600))
        N, K = 8 * int(rng.integers(1, 80)), 8 * int(rng.integers(1, 70))
        cfg = cfgs[int(rng.integers(0, len(cfgs)))]
        dtype = ["f16", "bf16"][int(rng.integers(0, 2))]
        print("gemm case", n, (bt, M, N, K, dtype, cfg), flush=True)
        A = draw((bt, M, K), "int", -2, 2, dtype, 800 + n)
        B = draw((bt, K, N), "int", -2, 2, dtype, 900 + n)
        ref, _ = G.gemm(A.double().numpy(), B.double().numpy())
        got = tss.gemm(A.to(CUDA), B.to(CUDA), out_dtype="f32", cfg=cfg)
        torch.cuda.synchronize()
        if not np.array_equal(to_f64(got), ref):
            bad.append((n, bt, M, N, K, dtype, cfg))
    assert not bad, bad[:5]


def test_random_low_precision_outputs_exact():
    """fp16 and bf16 outputs on random shapes: with inputs in [-2, 2] and
    K <= 512 (fp16) or K <= 64 (bf16) every exact result is at most 2048 or
    256 in magnitude, an integer the output type holds exactly, so the stored
    value must equal the oracle's; GEMM and convolution, planner's tiles."""
    rng = np.random.default_rng(2028)
    bad = []
    for n in range(40):
        dtype = ["f16", "bf16"][n % 2]
        kmax = 512 if dtype == "f16" else 64
        bt, M = int(rng.integers(1, 3)), int(rng.integers(1, 600))
        N, K = 8 * int(rng.integers(1, 80)), 8 * int(rng.integers(1, kmax // 8 + 1))
        A = draw((bt, M, K), "int", -2, 2, dtype, 1100 + n)
        B = draw((bt, K, N), "int", -2, 2, dtype, 1200 + n)
        ref, _ = G.gemm(A.double().numpy(), B.double().numpy())
        got = tss.gemm(A.to(CUDA), B.to(CUDA))
        torch.cuda.synchronize()
        assert got.dtype == A.dtype
        if not np.array_equal(to_f64(got), ref):
            bad.append(("gemm", n, bt, M, N, K, dtype))
    for n in range(30):
        dtype = ["f16", "bf16"][n % 2]
        N, Co = int(rng.integers(1, 3)), int(rng.integers(1, 100))
        kh = kw = int(rng.integers(1, 4))
        C = int(rng.integers(1, (512 if dtype == "f16" else 64) // (kh * kw) + 1))
        H, W = int(rng.integers(kh, 20)), int(rng.integers(kw, 20))
        st, pd = int(rng.integers(1, 3)), int(rng.integers(0, 2))
        OH, OW = (H + 2 * pd - kh) // st + 1, (W + 2 * pd - kw) // st + 1
        toh, tow = int(rng.integers(1, OH + 1)), int(rng.integers(1, OW + 1))
        x = draw((N, C, H, W), "int", -2, 2, dtype, 1300 + n)
        w = draw((Co, C, kh, kw), "int", -2, 2, dtype, 1400 + n)
        ref, _ = G.conv2d(x.double().numpy(), w.double().numpy(), (st, st), (pd, pd), (1, 1))
        got = tss.conv2d(x.to(CUDA), w.to(CUDA), st, pd, 1, tile_oh=toh, tile_ow=tow)
        torch.cuda.synchronize()
        assert got.dtype == x.dtype
        if not np.array_equal(to_f64(got), ref):
            bad.append(("conv", n, N, C, H, W, Co, kh, st, pd, toh, tow, dtype))
    assert not bad, bad[:5]
