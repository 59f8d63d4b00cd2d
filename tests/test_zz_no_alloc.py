"""The convolution entry point that allocates nothing
(tss_conv2d_splitk_noalloc: its workspace is the library's static device
array) against the same convolution with a workspace the caller allocates
(tss_conv2d_splitk), through the C ABI: the same bits, on two calls in a row
whose second is smaller (the array keeps the first call's contents), with and
without split K; a problem needing more than the array holds is refused
before any launch."""
import numpy as np
import pytest
import torch

import tile_size_selection_amd as tss
from tile_size_selection_amd import _capi as C
from oracle import gemm_conv as G
from tile_size_selection_amd.inputs import draw
from gpu_util import to_f64

pytestmark = pytest.mark.gpu

CUDA = torch.device("cuda:0")


def _pair(N, Ci, H, W, Co, stride, seed, splits, tile_oh, cfg=None, dtype="f16", out_dtype="f32"):
    x = draw((N, Ci, H, W), "uniform", -1, 1, dtype, seed).to(CUDA)
    w = draw((Co, Ci, 3, 3), "normal", 0, 0.05, dtype, seed + 1).to(CUDA)
    ref = tss.conv2d(x, w, stride, 1, 1, tile_oh=tile_oh, out_dtype=out_dtype, cfg=cfg, splits=splits)
    OH = (H + 2 - 3) // stride + 1
    OW = (W + 2 - 3) // stride + 1
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out_dtype]
    out = torch.full((N, Co, OH, OW), float("nan"), dtype=tdt, device=CUDA)
    tss.conv2d_noalloc(x, w, stride, 1, 1, tile_oh=tile_oh, cfg=cfg, out=out, splits=splits)
    torch.cuda.synchronize()
    return x, w, ref, out


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_noalloc_equals_the_workspace_entry_point_twice(splits):
    # the convolution workload's shape first, then a smaller one in the same array
    x, w, ref, out = _pair(8, 256, 56, 56, 256, 2, 301, splits, 8)
    assert torch.equal(out, ref)
    x2, w2, ref2, out2 = _pair(2, 40, 17, 13, 24, 1, 303, splits, 5)
    assert torch.equal(out2, ref2)
    # and exact against the oracle on integer inputs
    xi = draw((2, 24, 11, 9), "int", -2, 2, "f16", 305)
    wi = draw((16, 24, 3, 3), "int", -2, 2, "f16", 306)
    yref, _ = G.conv2d(xi.double().numpy(), wi.double().numpy(), (1, 1), (1, 1), (1, 1), with_abs=False)
    y = torch.full((2, 16, 11, 9), float("nan"), dtype=torch.float32, device=CUDA)
    tss.conv2d_noalloc(xi.to(CUDA), wi.to(CUDA), 1, 1, 1, tile_oh=4, out=y, splits=splits)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(y), yref)


def test_noalloc_refuses_a_problem_beyond_the_array():
    # 8 x 512 x 112 x 112 fp16 input: its channel-last copy alone is 102 MB > 64 MiB
    need = C.lib().tss_conv2d_splitk_workspace_size(8, 512, 112, 112, 64, 3, 3, 1, 1, 1, 1, 1, 1, 1)
    assert need > C.TSS_SCRATCH_BYTES
    x = torch.zeros((8, 512, 112, 112), dtype=torch.float16, device=CUDA)
    w = torch.zeros((64, 512, 3, 3), dtype=torch.float16, device=CUDA)
    y = torch.full((8, 64, 112, 112), 7.0, dtype=torch.float32, device=CUDA)
    with pytest.raises(tss.TssError) as e:
        tss.conv2d_noalloc(x, w, 1, 1, 1, out=y)
    assert e.value.status == C.TSS_E_SCRATCH
    torch.cuda.synchronize()
    assert (y == 7.0).all().item()          # refused before any launch: the output is untouched
