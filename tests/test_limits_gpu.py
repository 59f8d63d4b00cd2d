"""The largest operands the C ABI accepts: a GEMM whose B is just under
2 GiB and a convolution whose input and channel-last copy are just under
2 GiB, where the kernels' 32-bit byte offsets reach their top.  Integer
inputs in [-2, 2] make every fp32 sum exact (|sum| < 2^24), so sampled
outputs -- corners, ragged tile edges, tile boundaries and random ones --
must equal the oracle's fp64 value exactly.  The operands are generated on
the device; the oracle gets the rows, columns and input windows it needs."""
import numpy as np
import pytest
import torch

import tile_size_selection_amd as tss
from oracle import gemm_conv as G

pytestmark = pytest.mark.gpu

CUDA = torch.device("cuda:0")


def _ints(shape, seed):
    g = torch.Generator(device=CUDA)
    g.manual_seed(seed)
    return torch.randint(-2, 3, shape, generator=g, device=CUDA, dtype=torch.int8).to(torch.float16)


def test_gemm_b_just_under_2_gib():
    M, K, N = 264, 32768, 32760
    assert K * N * 2 < 2 ** 31 and K * N * 2 > 2 ** 31 - 2 ** 20
    A, B = _ints((M, K), 91), _ints((K, N), 92)
    C = tss.gemm(A, B, out_dtype="f32")
    torch.cuda.synchronize()
    rng = np.random.default_rng(93)
    rows = sorted(set([0, 1, 255, 256, M - 1] + rng.integers(0, M, 5).tolist()))
    cols = sorted(set([0, 255, 256, N - 8, N - 1] + rng.integers(0, N, 5).tolist()))
    a = A[rows].double().cpu().numpy()
    b = B[:, cols].double().cpu().numpy()
    ref, _ = G.gemm(a, b)
    got = C[rows][:, cols].double().cpu().numpy()
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]
    del A, B, C
    torch.cuda.empty_cache()


def test_conv_input_just_under_2_gib():
    N, Ci, H, W, Co = 1, 1024, 1023, 1023, 64
    assert N * Ci * H * W * 2 < 2 ** 31
    ws_bytes = tss.conv2d_workspace_size(N, Ci, H, W, Co, 3, 3)
    assert ws_bytes - Co * 9 * Ci * 2 < 2 ** 31                      # the channel-last copy itself
    x, w = _ints((N, Ci, H, W), 94), _ints((Co, Ci, 3, 3), 95)
    y = tss.conv2d(x, w, 1, 1, 1, tile_oh=64, out_dtype="f32")
    torch.cuda.synchronize()
    rng = np.random.default_rng(96)
    pts = [(0, 0, 0), (Co - 1, H - 1, W - 1), (5, 63, 700), (6, 64, 0), (7, 1022, 511)]
    pts += [(int(c), int(h), int(v)) for c, h, v in zip(rng.integers(0, Co, 8), rng.integers(0, H, 8),
                                                        rng.integers(0, W, 8))]
    wd = w.double().cpu().numpy()
    for co, oh, ow in pts:
        patch = np.zeros((1, Ci, 3, 3))
        for r in range(3):
            for s in range(3):
                ih, iw = oh - 1 + r, ow - 1 + s
                if 0 <= ih < H and 0 <= iw < W:
                    patch[0, :, r, s] = x[0, :, ih, iw].double().cpu().numpy()
        ref, _ = G.conv2d(patch, wd[co:co + 1])
        assert y[0, co, oh, ow].item() == ref[0, 0, 0, 0], (co, oh, ow)
    del x, w, y
    torch.cuda.empty_cache()
