"""GEMM parity on the GPU: every path through the C ABI against the fp64
oracle, element by element (small and ragged sizes) or on sampled entries
(full workload sizes, in the configuration the benchmark times)."""
import numpy as np
import pytest
import torch

import tile_size_selection_amd as tss
from oracle import gemm_conv as G
from oracle import planner as OP
from tile_size_selection_amd.inputs import WORKLOADS, draw
from gpu_util import check_bound, sample_indices, to_f64

pytestmark = pytest.mark.gpu

CUDA = torch.device("cuda:0")


def _feasible_configs():
    g = OP.device_gfx950()
    out = []
    for c in OP.candidates(g, 1 << 20, ["mfma32", "mfma16"]):
        if OP.evaluate(c, g).feasible:
            out.append(tss.TileConfig(c.block_m, c.block_n, c.block_k, c.stages, c.threads, c.instr))
    return out


ALL_CONFIGS = _feasible_configs()


def test_single_mfma_tile_exact():
    A = draw((32, 32), "int", -3, 3, "f16", 1)
    B = draw((32, 32), "int", -3, 3, "f16", 2)
    ref, _ = G.gemm(A.double().numpy(), B.double().numpy())
    for cfg in (tss.TileConfig(64, 64, 32, 2, 128, "mfma32"), tss.TileConfig(64, 64, 64, 2, 256, "mfma16")):
        got = tss.gemm(A.to(CUDA), B.to(CUDA), out_dtype="f32", cfg=cfg)
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(got), ref), cfg


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_every_kernel_exact_on_ragged_problem(dtype):
    """Integer inputs in [-2, 2]: every partial sum is an exact integer in
    fp32, so any dropped, doubled or misplaced tile, K step or element shows as
    a mismatch.  M, N, K are ragged for every tile size (300 = 256 + 44,
    328 = 256 + 72, K = 200 = 3*64 + 8) and the batch has two members."""
    bt, M, N, K = 2, 300, 328, 200
    A = draw((bt, M, K), "int", -2, 2, dtype, 11)
    B = draw((bt, K, N), "int", -2, 2, dtype, 12)
    ref, _ = G.gemm(A.double().numpy(), B.double().numpy())
    dA, dB = A.to(CUDA), B.to(CUDA)
    out = torch.empty((bt, M, N), dtype=torch.float32, device=CUDA)
    bad = []
    for cfg in ALL_CONFIGS:
        out.fill_(float("nan"))
        tss.gemm(dA, dB, out_dtype="f32", cfg=cfg, out=out)
        torch.cuda.synchronize()
        if not np.array_equal(to_f64(out), ref):
            bad.append(cfg)
    assert not bad, f"{len(bad)} of {len(ALL_CONFIGS)} configs wrong, e.g. {bad[:4]}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_low_precision_output_exact(dtype):
    """Output rounded to the input dtype: exact when every result is an
    integer the format holds (|c| <= 256 for bf16: K = 64, inputs in [-2, 2])."""
    bt, M, N, K = 1, 130, 136, 64
    A = draw((M, K), "int", -2, 2, dtype, 21)
    B = draw((K, N), "int", -2, 2, dtype, 22)
    ref, _ = G.gemm(A.double().numpy(), B.double().numpy())
    dA, dB = A.to(CUDA), B.to(CUDA)
    for cfg in ALL_CONFIGS[::7]:
        if cfg.bk > K:
            continue
        got = tss.gemm(dA, dB, cfg=cfg)
        torch.cuda.synchronize()
        assert got.dtype == dA.dtype
        assert np.array_equal(to_f64(got), ref), cfg


def test_rounding_of_fp16_and_bf16_outputs():
    """Non-integer results: the stored value is the fp32 accumulator rounded
    to nearest even, so it lies within half an ulp of the output format (plus
    the fp32 accumulation error, at most K * 2^-24 * sum|a*b|) of the oracle."""
    M, N, K = 64, 64, 64
    for dtype, mant in (("f16", 10), ("bf16", 7)):
        A = draw((M, K), "uniform", -1, 1, dtype, 31)
        B = draw((K, N), "uniform", -1, 1, dtype, 32)
        ref, S = G.gemm(A.double().numpy(), B.double().numpy())
        got = to_f64(tss.gemm(A.to(CUDA), B.to(CUDA)))
        expo = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -14)))
        half_ulp = 2.0 ** (expo - mant - 1)
        assert np.all(np.abs(got - ref) <= half_ulp * 1.0000001 + K * 2.0 ** -24 * S), dtype
        check_bound(got, ref, S, dtype)


def test_workload_256_full_parity():
    w = WORKLOADS[1]
    A, B = w.make()
    ref, S = G.gemm(A.double().numpy(), B.double().numpy())
    got = to_f64(tss.gemm(A.to(CUDA), B.to(CUDA), out_dtype=w.out_dtype))
    check_bound(got, ref, S, w.name)


def _sampled_parity(w, cfg=None, n=6000, seed=0):
    A, B = w.make()
    if A.dim() == 2:
        A3, B3 = A[None], B[None]
    else:
        A3, B3 = A, B
    got = tss.gemm(A.to(CUDA), B.to(CUDA), out_dtype=w.out_dtype, cfg=cfg)
    torch.cuda.synchronize()
    got = got.reshape(w.batch, w.M, w.N)
    rng = np.random.default_rng(seed)
    b, i, j = sample_indices((w.batch, w.M, w.N), n, rng)
    ref, S = G.gemm_entries(A3.double().numpy(), B3.double().numpy(), b, i, j)
    g = got[torch.from_numpy(b).to(CUDA), torch.from_numpy(i).to(CUDA), torch.from_numpy(j).to(CUDA)]
    check_bound(to_f64(g), ref, S, w.name)
    # no NaN / Inf and nothing left unwritten anywhere
    assert torch.isfinite(got).all().item()
    return got


def test_workload_4096_headline_sampled():
    w = WORKLOADS[2]
    cfg = tss.default_config(w.M, w.N, w.K, w.batch, w.dtype)
    print("planner choice for", w.name, cfg, flush=True)
    _sampled_parity(w)


def test_workload_ragged_batched_sampled():
    _sampled_parity(WORKLOADS[3])


def test_workload_8192_bf16_sampled():
    _sampled_parity(WORKLOADS[4], n=3000)


def test_k_zero_and_empty_shapes():
    A = torch.zeros((5, 0), dtype=torch.float16, device=CUDA)
    B = torch.zeros((0, 16), dtype=torch.float16, device=CUDA)
    out = torch.full((5, 16), float("nan"), dtype=torch.float32, device=CUDA)
    tss.gemm(A, B, out_dtype="f32", out=out)
    torch.cuda.synchronize()
    assert (out == 0).all().item()
    # K == 0 over several tile rows and columns (and batches): every block's
    # operand ranges are empty, so C is all zeros
    A = torch.zeros((2, 300, 0), dtype=torch.float16, device=CUDA)
    B = torch.zeros((2, 0, 520), dtype=torch.float16, device=CUDA)
    out = torch.full((2, 300, 520), float("nan"), dtype=torch.float32, device=CUDA)
    tss.gemm(A, B, out_dtype="f32", out=out)
    torch.cuda.synchronize()
    assert (out == 0).all().item()
    # M == 0: nothing launched, nothing written
    A0 = torch.zeros((0, 8), dtype=torch.float16, device=CUDA)
    B0 = torch.ones((8, 8), dtype=torch.float16, device=CUDA)
    assert tss.gemm(A0, B0).shape == (0, 8)


def test_minimal_and_thin_shapes():
    for (M, N, K) in [(1, 8, 8), (1, 8, 4096), (257, 8, 24), (3, 520, 16), (64, 64, 8)]:
        A = draw((M, K), "int", -2, 2, "f16", M + N)
        B = draw((K, N), "int", -2, 2, "f16", K + 1)
        ref, _ = G.gemm(A.double().numpy(), B.double().numpy())
        got = tss.gemm(A.to(CUDA), B.to(CUDA), out_dtype="f32")
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(got), ref), (M, N, K)


def test_planner_choice_is_what_runs_and_is_deterministic():
    w = WORKLOADS[3]
    A, B = w.make()
    dA, dB = A.to(CUDA), B.to(CUDA)
    best, _, _ = tss.tile_plan(w.M, w.N, w.K, batch=w.batch)
    c1 = tss.gemm(dA, dB, out_dtype="f32")
    c2 = tss.gemm(dA, dB, out_dtype="f32", cfg=best["config"])
    c3 = tss.gemm(dA, dB, out_dtype="f32")
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(c1, c3)


def test_side_stream_and_errors():
    A = draw((128, 64), "int", -2, 2, "f16", 41).to(CUDA)
    B = draw((64, 128), "int", -2, 2, "f16", 42).to(CUDA)
    ref, _ = G.gemm(A.double().cpu().numpy(), B.double().cpu().numpy())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = tss.gemm(A, B, out_dtype="f32", stream=s)
    s.synchronize()
    assert np.array_equal(to_f64(got), ref)
    with pytest.raises(tss.TssError):
        tss.gemm(A, B, cfg=tss.TileConfig(256, 256, 64, 3, 256, "mfma32"))   # C1 infeasible
    with pytest.raises(tss.TssError):
        tss.gemm(A[:, :60].contiguous(), B[:60].contiguous())                # K % 8
    with pytest.raises(ValueError):
        tss.gemm(A, B, out_dtype="f32", out=torch.empty(128, 128))             # output in host memory
    with pytest.raises(ValueError):
        tss.gemm(A.double(), B.double())                                      # fp64 operands
    x = torch.zeros((1, 8, 9, 9), dtype=torch.float16, device=CUDA)
    w = torch.zeros((8, 8, 3, 3), dtype=torch.float16, device=CUDA)
    with pytest.raises(ValueError):
        tss.conv2d(x, w, 1, 1, 1, out_dtype="f32", out=torch.empty(1, 8, 9, 9))
    with pytest.raises(ValueError):
        tss.conv2d(x, w, 1, 1, 1, workspace=torch.empty(1 << 20, dtype=torch.uint8))
