"""The measured tile choice (tss_gemm_autotune): it returns one of the
planner's first topk candidates, the product it leaves in C and the product
of tss_gemm with the chosen tile are exact, and bad arguments are refused."""
import numpy as np
import pytest
import torch

import tile_size_selection_amd as tss
from oracle import gemm_conv as G
from tile_size_selection_amd.inputs import draw
from gpu_util import to_f64

pytestmark = pytest.mark.gpu

CUDA = torch.device("cuda:0")


def test_autotune_picks_a_ranked_candidate_and_stays_exact():
    A = draw((2, 300, 200), "int", -2, 2, "f16", 901)
    B = draw((2, 200, 328), "int", -2, 2, "f16", 902)
    ref, _ = G.gemm(A.double().numpy(), B.double().numpy())
    dA, dB = A.to(CUDA), B.to(CUDA)
    out = torch.empty(2, 300, 328, dtype=torch.float32, device=CUDA)
    cfg, us = tss.autotune_gemm(dA, dB, out_dtype="f32", topk=12, iters=3, out=out)
    torch.cuda.synchronize()
    _, ranked, _ = tss.tile_plan(300, 328, 200, batch=2, cap=12)
    assert cfg in [v["config"] for v in ranked]
    assert us > 0
    assert np.array_equal(to_f64(out), ref)            # the last candidate's product, left in C
    C = tss.gemm(dA, dB, out_dtype="f32", cfg=cfg)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(C), ref)


def test_autotune_arguments():
    dA = draw((64, 64), "int", -1, 1, "f16", 903).to(CUDA)
    dB = draw((64, 64), "int", -1, 1, "f16", 904).to(CUDA)
    for topk, iters in ((0, 3), (2000, 3), (4, 0)):
        with pytest.raises(tss.TssError):
            tss.autotune_gemm(dA, dB, topk=topk, iters=iters)
    with pytest.raises(tss.TssError):   # K not a multiple of 8
        tss.autotune_gemm(draw((64, 60), "int", -1, 1, "f16", 905).to(CUDA),
                          draw((60, 64), "int", -1, 1, "f16", 906).to(CUDA), topk=2, iters=1)
    empty = torch.empty(0, 64, dtype=torch.float16, device=CUDA)
    cfg, us = tss.autotune_gemm(empty, dB, topk=3, iters=2)   # nothing to launch: the plan's first candidate
    assert isinstance(cfg, tss.TileConfig) and us >= 0
