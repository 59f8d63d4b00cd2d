"""Pins of the fp64 GEMM / conv oracle: exact rationals, closed forms, an
independent library routine, and direct == H-tiled bit for bit."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import gemm_conv as G
from tile_size_selection_amd.inputs import draw


def _exact_matmul(A, B):
    M, K = A.shape
    N = B.shape[1]
    Af = [[Fraction(float(A[i, k])) for k in range(K)] for i in range(M)]
    Bf = [[Fraction(float(B[k, j])) for j in range(N)] for k in range(K)]
    return [[sum(Af[i][k] * Bf[k][j] for k in range(K)) for j in range(N)] for i in range(M)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gemm_vs_exact_rationals_tiny(dtype):
    A = draw((5, 7), "uniform", -1, 1, dtype, 11).double().numpy()
    B = draw((7, 3), "uniform", -1, 1, dtype, 12).double().numpy()
    C, S = G.gemm(A, B)
    E = _exact_matmul(A, B)
    for i in range(5):
        for j in range(3):
            # fp16/bf16 values are dyadic: the exact sum is a rational; fp64
            # accumulation of 7 exact products errs by at most 7 ulp of S
            assert abs(Fraction(C[i, j]) - E[i][j]) <= Fraction(7 * 2.0 ** -52) * Fraction(S[i, j])
            assert S[i, j] == pytest.approx(float(sum(abs(Fraction(A[i, k]) * Fraction(B[k, j])) for k in range(7))))


def test_gemm_integer_inputs_exact():
    A = draw((2, 9, 33), "int", -2, 2, "f16", 21).double().numpy()
    B = draw((2, 33, 6), "int", -2, 2, "f16", 22).double().numpy()
    C, _ = G.gemm(A, B)
    for b in range(2):
        E = _exact_matmul(A[b], B[b])
        assert all(C[b, i, j] == E[i][j] for i in range(9) for j in range(6))


def test_gemm_closed_forms():
    B = draw((16, 24), "uniform", -1, 1, "f16", 31).double().numpy()
    C, _ = G.gemm(np.eye(16), B)
    assert np.array_equal(C, B)                                  # I x B = B
    C, _ = G.gemm(np.ones((3, 16)), B)
    assert np.array_equal(C[1], np.cumsum(B, axis=0)[-1])        # ones x B = column sums (k ascending)
    a = draw((10, 1), "uniform", -1, 1, "f16", 32).double().numpy()
    b = draw((1, 12), "uniform", -1, 1, "f16", 33).double().numpy()
    C, S = G.gemm(a, b)
    assert np.array_equal(C, a * b) and np.array_equal(S, np.abs(a * b))   # K = 1: outer product


def test_gemm_orientation_and_batch():
    """Non-square shapes with distinct operands: a transposed operand or a
    mixed-up batch cannot pass."""
    A = draw((3, 13, 29), "normal", 0, 0.5, "f16", 41).double().numpy()
    B = draw((3, 29, 17), "normal", 0, 0.5, "f16", 42).double().numpy()
    C, S = G.gemm(A, B)
    ref = np.matmul(A, B)                                        # independent library routine
    assert np.all(np.abs(C - ref) <= 29 * 2.0 ** -52 * S + 1e-300)
    for b in range(3):
        Cb, _ = G.gemm(A[b], B[b])
        assert np.array_equal(Cb, C[b])


def test_gemm_entries_equal_full():
    A = draw((2, 40, 64), "uniform", -1, 1, "bf16", 51).double().numpy()
    B = draw((2, 64, 48), "uniform", -1, 1, "bf16", 52).double().numpy()
    C, S = G.gemm(A, B)
    rng = np.random.default_rng(5)
    b, i, j = rng.integers(0, 2, 100), rng.integers(0, 40, 100), rng.integers(0, 48, 100)
    c, s = G.gemm_entries(A, B, b, i, j)
    assert np.array_equal(c, C[b, i, j]) and np.array_equal(s, S[b, i, j])


def _conv_bruteforce(x, w, stride, pad, dil):
    N, Ci, Hh, W = x.shape
    Co, _, kh, kw = w.shape
    xp = np.pad(x, ((0, 0), (0, 0), (pad[0], pad[0]), (pad[1], pad[1])))
    OH = (Hh + 2 * pad[0] - (kh - 1) * dil[0] - 1) // stride[0] + 1
    OW = (W + 2 * pad[1] - (kw - 1) * dil[1] - 1) // stride[1] + 1
    y = [[[[Fraction(0)] * OW for _ in range(OH)] for _ in range(Co)] for _ in range(N)]
    for n in range(N):
        for co in range(Co):
            for oh in range(OH):
                for ow in range(OW):
                    acc = Fraction(0)
                    for ci in range(Ci):
                        for r in range(kh):
                            for s in range(kw):
                                acc += Fraction(float(xp[n, ci, oh * stride[0] + r * dil[0], ow * stride[1] + s * dil[1]])) \
                                    * Fraction(float(w[co, ci, r, s]))
                    y[n][co][oh][ow] = acc
    return y


@pytest.mark.parametrize("stride,pad,dil", [((1, 1), (0, 0), (1, 1)), ((2, 2), (1, 1), (1, 1)),
                                            ((2, 1), (1, 2), (2, 1)), ((3, 2), (2, 0), (1, 2))])
def test_conv_vs_bruteforce(stride, pad, dil):
    x = draw((2, 3, 9, 8), "int", -3, 3, "f16", 61).double().numpy()
    w = draw((4, 3, 3, 2), "int", -3, 3, "f16", 62).double().numpy()
    y, _ = G.conv2d(x, w, stride, pad, dil)
    E = _conv_bruteforce(x, w, stride, pad, dil)
    assert y.shape == (len(E), len(E[0]), len(E[0][0]), len(E[0][0][0]))
    assert all(y[n, c, h, q] == E[n][c][h][q] for n in range(y.shape[0]) for c in range(y.shape[1])
               for h in range(y.shape[2]) for q in range(y.shape[3]))


def test_conv_delta_kernel_is_identity():
    x = draw((1, 2, 7, 6), "uniform", -1, 1, "f16", 71).double().numpy()
    w = np.zeros((2, 2, 3, 3))
    w[0, 0, 1, 1] = 1.0
    w[1, 1, 1, 1] = 1.0
    y, _ = G.conv2d(x, w, (1, 1), (1, 1), (1, 1))
    assert np.array_equal(y, x)


def test_conv_1x1_equals_gemm():
    x = draw((2, 24, 5, 7), "uniform", -1, 1, "f16", 81).double().numpy()
    w = draw((10, 24, 1, 1), "uniform", -1, 1, "f16", 82).double().numpy()
    y, _ = G.conv2d(x, w)
    for n in range(2):
        C, _ = G.gemm(w[:, :, 0, 0], x[n].reshape(24, 35))
        assert np.array_equal(C.reshape(10, 5, 7), y[n])


@pytest.mark.parametrize("H,W,k,stride,pad,dil,toh", [(9, 9, 3, 2, 1, 1, 2), (56, 12, 3, 2, 1, 1, 8),
                                                      (13, 5, 3, 1, 1, 1, 3), (17, 6, 5, 2, 2, 1, 4),
                                                      (15, 7, 3, 1, 2, 2, 5), (11, 4, 2, 3, 0, 1, 1)])
def test_conv_htiled_equals_direct_bitwise(H, W, k, stride, pad, dil, toh):
    x = draw((2, 5, H, W), "uniform", -1, 1, "f16", 91).double().numpy()
    w = draw((3, 5, k, k), "normal", 0, 0.05, "f16", 92).double().numpy()
    y, _ = G.conv2d(x, w, (stride, stride), (pad, pad), (dil, dil))
    yt = G.conv2d_htiled(x, w, (stride, stride), (pad, pad), (dil, dil), toh)
    assert np.array_equal(y, yt)


@pytest.mark.parametrize("H,W,kh,kw,stride,pad,dil,tilings", [
    (9, 9, 3, 3, (2, 2), (1, 1), (1, 1), [(1, 2, 2), (2, 4, 1), (3, 1, 3)]),          # the worked example, both axes
    (56, 56, 3, 3, (2, 2), (1, 1), (1, 1), [(1, 8, 8), (2, 28, 5), (3, 3, 28)]),      # the conv workload's geometry
    (13, 11, 3, 5, (1, 2), (1, 2), (1, 1), [(1, 3, 2), (2, 13, 1), (3, 1, 6)]),
    (15, 17, 3, 3, (2, 1), (2, 1), (2, 2), [(2, 4, 5), (1, 8, 17), (3, 2, 3)]),
    (11, 12, 2, 3, (3, 2), (0, 1), (1, 2), [(1, 1, 1), (2, 2, 3), (3, 4, 2)]),
    # pads of 2 at stride 3 with 1-row / 1-column windows: the first and last
    # output rows and columns read only padding, so their tiles' slices are
    # empty (the formulas give min(in_end, H) <= in_start)
    (3, 6, 1, 4, (3, 3), (2, 2), (1, 2), [(1, 1, 1), (3, 1, 2), (2, 2, 1)]),
    (12, 5, 5, 1, (2, 2), (0, 2), (2, 2), [(1, 2, 1), (3, 1, 1), (2, 2, 5)]),
])
def test_conv_tiled_equals_direct_bitwise(H, W, kh, kw, stride, pad, dil, tilings):
    """Tiles over images, output rows and output columns, the columns taking
    their slice and pads from the same formulas as the rows: the direct
    convolution's bits for every tiling (ragged tiles, pads on both sides,
    dilation, unequal strides)."""
    x = draw((3, 5, H, W), "uniform", -1, 1, "f16", 93).double().numpy()
    w = draw((4, 5, kh, kw), "normal", 0, 0.05, "f16", 94).double().numpy()
    y, _ = G.conv2d(x, w, stride, pad, dil)
    for tn, toh, tow in tilings:
        yt = G.conv2d_tiled(x, w, stride, pad, dil, toh, min(tow, y.shape[3]), tn)
        assert np.array_equal(y, yt), (tn, toh, tow)


def test_conv_tiled_columns_are_rows_transposed():
    """Column tiles are row tiles of the transposed problem: tiling W of x
    gives the transpose of tiling H of x with H and W swapped."""
    x = draw((2, 3, 10, 13), "uniform", -1, 1, "f16", 95).double().numpy()
    w = draw((4, 3, 3, 2), "normal", 0, 0.05, "f16", 96).double().numpy()
    st, pd, dl = (2, 1), (1, 0), (1, 2)
    y = G.conv2d_tiled(x, w, st, pd, dl, tile_oh=5, tile_ow=3)
    xt, wt = np.ascontiguousarray(x.transpose(0, 1, 3, 2)), np.ascontiguousarray(w.transpose(0, 1, 3, 2))
    yt = G.conv2d_tiled(xt, wt, st[::-1], pd[::-1], dl[::-1], tile_oh=3, tile_ow=5)
    assert np.array_equal(y, yt.transpose(0, 1, 3, 2))
