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
