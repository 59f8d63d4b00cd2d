"""Exact parity of the headline tiles over whole outputs.

Integer operands in [-2, 2] are exact in fp16 and bf16, and every partial sum
of a K = 4096 (or 8192) dot product is an integer of magnitude at most
4 * K < 2^24, so the fp32 accumulator holds the exact result whatever the
summation order.  The fp32 output must therefore equal the fp64 oracle bit
for bit, and a low-precision output must equal the oracle's value rounded to
nearest even (the conversion the epilogue performs).  A K step dropped or
counted twice, a misplaced tile or a stale LDS stage changes whole rows of
the output by integers, which this comparison cannot miss (a tolerance
check at this K cannot see one lost 64-wide K step)."""
import numpy as np
import pytest
import torch

import tile_size_selection_amd as tss
from oracle import gemm_conv as G
from tile_size_selection_amd.inputs import draw
from gpu_util import to_f64

pytestmark = pytest.mark.gpu

CUDA = torch.device("cuda:0")


def _rne(ref: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    # the exact integers fit fp32; torch's fp32 -> fp16/bf16 cast rounds to nearest even
    return torch.from_numpy(ref.astype(np.float32)).to(dtype)


def test_headline_4096_full_output_exact():
    M = N = K = 4096
    cfg = tss.default_config(M, N, K, 1, "f16")
    print("4096^3 f16, planner tile", cfg, flush=True)
    A = draw((M, K), "int", -2, 2, "f16", 2100)
    B = draw((K, N), "int", -2, 2, "f16", 2101)
    ref, _ = G.gemm(A.double().numpy(), B.double().numpy(), with_abs=False)
    dA, dB = A.to(CUDA), B.to(CUDA)
    got = torch.full((M, N), float("nan"), dtype=torch.float32, device=CUDA)
    tss.gemm(dA, dB, out_dtype="f32", cfg=cfg, out=got)
    torch.cuda.synchronize()
    g = to_f64(got)
    bad = g != ref
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} outputs differ, first at {np.argwhere(bad)[:4].tolist()}"
    # the headline's own output dtype: fp16, rounded to nearest even
    got16 = tss.gemm(dA, dB, cfg=cfg)
    torch.cuda.synchronize()
    assert torch.equal(got16.cpu(), _rne(ref, torch.float16))


def test_8192_bf16_row_slab_exact():
    """8192^3 bf16 with the planner's tile: two rows of every 256-row tile
    band (one inside, the band's last row) over every column, exact in fp32
    and rounded to nearest even in bf16."""
    M = N = K = 8192
    cfg = tss.default_config(M, N, K, 1, "bf16")
    print("8192^3 bf16, planner tile", cfg, flush=True)
    A = draw((M, K), "int", -2, 2, "bf16", 4100)
    B = draw((K, N), "int", -2, 2, "bf16", 4101)
    rows = np.array(sorted({256 * t + (37 * t + 11) % 256 for t in range(M // 256)}
                           | {256 * t + 255 for t in range(M // 256)}), dtype=np.int64)
    ref, _ = G.gemm(A[torch.from_numpy(rows)].double().numpy(), B.double().numpy(), with_abs=False)
    dA, dB = A.to(CUDA), B.to(CUDA)
    idx = torch.from_numpy(rows).to(CUDA)
    got = torch.full((M, N), float("nan"), dtype=torch.float32, device=CUDA)
    tss.gemm(dA, dB, out_dtype="f32", cfg=cfg, out=got)
    torch.cuda.synchronize()
    g = to_f64(got[idx])
    assert np.array_equal(g, ref), f"{int((g != ref).sum())} of {g.size} sampled outputs differ"
    assert torch.isfinite(got).all().item()   # every output written
    del got
    gotb = tss.gemm(dA, dB, cfg=cfg)
    torch.cuda.synchronize()
    assert torch.equal(gotb[idx].cpu(), _rne(ref, torch.bfloat16))
