"""Time every workload with the planner's tile and report microseconds,
TFLOP/s and the fraction of MI355X's dense fp16/bf16 MFMA peak.

    python -m tile_size_selection_amd.workloads_report [--out profiles/workloads.md]

Inputs are the seeded synthetic operands of each workload, resident on the
device.  The launches of n back-to-back calls are captured in one HIP graph
(so a small workload's time is the GPU's, not the Python call's), and HIP
events on the stream time its replay: the median of 5 replays, divided by n.
The graph's output is checked against the eager call's, bit for bit.  The
convolution is timed twice: the whole tss_conv2d call on NCHW tensors
(operand layout pass + implicit GEMM) and the tss_conv2d_nhwc call on the
same values as channel-last tensors (the implicit GEMM alone).  The 4096^3 GEMM is also timed cold: a 512 MB device write before
every launch evicts its operands from the caches (L2 and the 256 MB cache in
front of HBM), and HIP events bracket each launch alone (median of 30).
"""
from __future__ import annotations

import argparse
import statistics
import sys

import torch

from . import api
from .inputs import WORKLOADS, ConvWorkload

PEAK_TFLOPS = 2516.6  # MI355X dense fp16 / bf16 MFMA


def _time(fn, n: int) -> float:
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3  # microseconds


def _time_graph(fn, out, n: int, rounds: int) -> float:
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # the first call on this stream, outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    times = []
    for _ in range(rounds):
        out.zero_()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise RuntimeError("graph replay differs from the eager result")
        times.append(e0.elapsed_time(e1) / n * 1e3)
    return statistics.median(times)


def cold_gemm_us(w, n: int = 30) -> float:
    A, B = w.make()
    dA, dB = A.cuda(), B.cuda()
    C = api.gemm(dA, dB, out_dtype=w.out_dtype)
    flush = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device="cuda")  # 512 MB
    times = []
    for i in range(n + 3):
        flush.fill_(float(i))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        api.gemm(dA, dB, out_dtype=w.out_dtype, out=C)
        e1.record()
        torch.cuda.synchronize()
        if i >= 3:
            times.append(e0.elapsed_time(e1) * 1e3)
    return statistics.median(times)


def run_one(w, rounds: int = 5):
    if isinstance(w, ConvWorkload):
        x, wt = w.make()
        dx, dw = x.cuda(), wt.cuda()
        ws = torch.empty(api.conv2d_workspace_size(w.N, w.C, w.H, w.W, w.Co, w.kh, w.kw), dtype=torch.uint8,
                         device="cuda")
        y = api.conv2d(dx, dw, w.stride, w.pad, w.dil, tile_oh=w.tile_oh, out_dtype=w.out_dtype, workspace=ws)
        OH, OW = y.shape[2], y.shape[3]
        flops = 2 * w.N * w.Co * OH * OW * w.C * w.kh * w.kw
        cfg = api.conv2d_default_config(w.N, w.C, w.H, w.W, w.Co, w.kh, w.kw, w.stride, w.pad, w.dil)
        out = y
        fn = lambda: api.conv2d(dx, dw, w.stride, w.pad, w.dil, tile_oh=w.tile_oh, out_dtype=w.out_dtype,
                                workspace=ws, out=y)
    else:
        A, B = w.make()
        dA, dB = A.cuda(), B.cuda()
        C = api.gemm(dA, dB, out_dtype=w.out_dtype)
        flops = w.flops()
        cfg = api.default_config(w.M, w.N, w.K, batch=w.batch, dtype=w.dtype)
        out = C
        fn = lambda: api.gemm(dA, dB, out_dtype=w.out_dtype, out=C)
    torch.cuda.synchronize()
    t1 = _time(fn, 5)  # warm-up, and a launch count that keeps each replay near 20 ms
    n = max(20, min(2000, int(20000 / max(t1, 1.0))))
    us = _time_graph(fn, out, n, rounds)
    tf = flops / (us * 1e-6) / 1e12
    r = {"name": w.name, "us": us, "tflops": tf, "frac": tf / PEAK_TFLOPS, "launches": n,
         "tile": f"{cfg.bm}x{cfg.bn}x{cfg.bk}/s{cfg.stages}/t{cfg.threads}/{cfg.instr}"}
    if not isinstance(w, ConvWorkload):
        return [r]
    # the same convolution on channel-last tensors: one launch, x and w read in place
    cl = torch.channels_last
    cx, cw = dx.contiguous(memory_format=cl), dw.contiguous(memory_format=cl)
    yc = api.conv2d(cx, cw, w.stride, w.pad, w.dil, tile_oh=w.tile_oh, out_dtype=w.out_dtype)
    fnc = lambda: api.conv2d(cx, cw, w.stride, w.pad, w.dil, tile_oh=w.tile_oh, out_dtype=w.out_dtype, out=yc)
    torch.cuda.synchronize()
    t1 = _time(fnc, 5)
    n = max(20, min(2000, int(20000 / max(t1, 1.0))))
    usc = _time_graph(fnc, yc, n, rounds)
    tfc = flops / (usc * 1e-6) / 1e12
    return [r, {"name": w.name + " (channel-last)", "us": usc, "tflops": tfc, "frac": tfc / PEAK_TFLOPS,
                "launches": n, "tile": r["tile"]}]


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    rows = []
    for i in sorted(WORKLOADS):
        for r in run_one(WORKLOADS[i]):
            rows.append(r)
            print(f"{r['name']}: {r['us']:.2f} us, {r['tflops']:.1f} TFLOP/s ({100 * r['frac']:.1f}% of peak),"
                  f" tile {r['tile']}", flush=True)
    cold = cold_gemm_us(WORKLOADS[2])
    warm = next(r for r in rows if r["name"] == WORKLOADS[2].name)
    print(f"{WORKLOADS[2].name} cold (512 MB written before each launch): {cold:.2f} us "
          f"({WORKLOADS[2].flops() / (cold * 1e-6) / 1e12:.1f} TFLOP/s)", flush=True)
    txt = ("# Every workload with the planner's tile\n\n"
           "Command (repository root, MI355X): `python3 -m tile_size_selection_amd.workloads_report"
           + (f" --out {a.out}" if a.out else "") + "`\n\n"
           "n back-to-back launches captured in one HIP graph, HIP events around its replay, median of 5 replays /"
           " n, on resident inputs (each replay's output checked against the eager call's); % of the 2516.6"
           " TFLOP/s dense fp16/bf16 MFMA peak.\n\n"
           "| workload | tile | us | TFLOP/s | % of peak |\n|---|---|---|---|---|\n"
           + "\n".join(f"| {r['name']} | {r['tile']} | {r['us']:.2f} | {r['tflops']:.1f} | {100 * r['frac']:.1f} |"
                       for r in rows) + "\n\n"
           f"{WORKLOADS[2].name} cold (512 MB written before each launch, one launch per event pair, median of 30):"
           f" {cold:.2f} us = {WORKLOADS[2].flops() / (cold * 1e-6) / 1e12:.1f} TFLOP/s"
           f" (warm, graph-timed: {warm['us']:.2f} us)\n")
    print(txt, flush=True)
    if a.out:
        with open(a.out, "w", encoding="utf-8") as f:
            f.write(txt)
    return 0


if __name__ == "__main__":
    sys.exit(main())
