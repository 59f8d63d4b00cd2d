#!/usr/bin/env python3
"""Headline benchmark: fp16 GEMM at M = N = K = 4096 on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the hot path over the resident synthetic operands:
the tile decision (the planner's choice, cached per shape after its first
evaluation) and the tiled GEMM kernel it selects, launched through the C ABI
on the current stream.  Prints one JSON line.

Warm-up runs at least `warmup` launches and at least one second of GPU work.
The timed region holds exactly `steps` launches, bracketed by
torch.cuda.synchronize(); HIP events recorded on the launch stream give the
average kernel duration the roofline figure uses.  The launches are queued
behind a GPU-side spin so that the interval between the events is the
kernels running back to back, not the host's per-call cost.  Beside it: the convolution
workload (8x256x56x56, 3x3, stride 2, pad 1, H-tiles of 8 output rows) timed
the same way, and the oracle timed on the host cores on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6      # MI355X dense fp16/bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
COUNTER_PROFILE = os.path.join(ROOT, "profiles", "gemm_f16_4096_counters.md")
KERNEL_SOURCES = [os.path.join(ROOT, "tile_size_selection_amd", "csrc", f)
                  for f in ("gemm_kernel.h", "registry.h", "instances.inc")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(cfg_str: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source and tile configuration."""
    if not os.path.exists(COUNTER_PROFILE):
        return None
    txt = open(COUNTER_PROFILE, encoding="utf-8").read()
    kv = dict(re.findall(r"^(\w+):\s*(\S+)\s*$", txt, flags=re.M))
    if kv.get("kernel_source_hash") != kernel_source_hash() or kv.get("config") != cfg_str:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(A, B, budget_s: float = 12.0):
    """The fp64 oracle on the host cores, on the first rows of the same
    problem: a short calibration run sizes the sample to about budget_s."""
    from oracle import gemm_conv as G
    Ad = A.double().numpy()
    Bd = B.double().numpy()
    K, N = Bd.shape
    t0 = time.perf_counter()
    G.gemm(Ad[:64], Bd)
    dt = max(time.perf_counter() - t0, 1e-6)
    rows = int(min(A.shape[0], max(64, budget_s / dt * 64)))
    t0 = time.perf_counter()
    G.gemm(Ad[:rows], Bd)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * N * K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": G.threads(), "kind": "oracle",
            "sample": f"first {rows} of {A.shape[0]} rows of the 4096^3 problem (C and sum|a*b| in fp64), "
                      f"{dt:.1f} s wall on {cpu_model()}"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "an unknown CPU"


def warm_up(launch, n_min: int, min_s: float = 1.0):
    """At least n_min launches and at least min_s seconds of GPU work (the
    engine clock settles under sustained load, not in a few launches).
    Returns the launches made and the host's enqueue cost per launch (us)."""
    import torch
    n, t0 = 0, time.perf_counter()
    enq_s, enq_n = 0.0, 0
    while n < n_min or time.perf_counter() - t0 < min_s:
        t1 = time.perf_counter()
        for _ in range(20):
            launch()
        enq_s += time.perf_counter() - t1
        enq_n += 20
        n += 20
        torch.cuda.synchronize()
    return n, enq_s / enq_n * 1e6


def timed(launch, steps: int, host_us: float, stream):
    """Exactly `steps` launches between two HIP events on the launch stream.
    The launches are queued behind a GPU-side spin long enough for the host
    to enqueue all of them, so the events see the kernels run back to back
    rather than the host's per-call cost (Python marshalling of the call);
    the spin itself lies before the first event.  Returns (ms per step,
    wall seconds of the bracketed region, spin cycles)."""
    import torch
    torch.cuda.synchronize()
    spin_us = min(max(2000.0, 1.5 * steps * host_us), 2.0e6)
    cycles = int(spin_us * 2400)          # at most 2.4 GHz: the spin lasts at least spin_us
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    torch.cuda._sleep(cycles)
    e0.record(stream)
    for _ in range(steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall, cycles


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the GEMM shards by output tiles "
              "with no exchange, so a multi-GPU figure is N independent single-GPU runs.", file=sys.stderr)
        return 2

    import torch
    import tile_size_selection_amd as tss
    from tile_size_selection_amd.inputs import WORKLOADS

    w = WORKLOADS[2]
    A, B = w.make()
    dA, dB = A.to("cuda:0"), B.to("cuda:0")
    out = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda:0")
    cfg = tss.default_config(w.M, w.N, w.K, w.batch, w.dtype)
    stream = torch.cuda.current_stream()

    def launch():
        tss.gemm(dA, dB, out=out)          # planner choice (cached) + kernel

    warm_n, host_us = warm_up(launch, args.warmup)
    ms_per_step, wall, _ = timed(launch, args.steps, host_us, stream)
    flops = w.flops()
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    # a few sampled entries against the oracle (outside the timed region)
    from oracle import gemm_conv as G
    import numpy as np
    rng = np.random.default_rng(0)
    i, j = rng.integers(0, w.M, 64), rng.integers(0, w.N, 64)
    ref, S = G.gemm_entries(A.double().numpy(), B.double().numpy(), np.zeros(64, np.int64), i, j)
    got = out[torch.from_numpy(i).cuda(), torch.from_numpy(j).cuda()].double().cpu().numpy()
    parity_ok = bool(np.all(np.abs(got - ref) <= 5e-3 * S + 1e-3))

    # the convolution workload, same timing method
    cw = WORKLOADS[5]
    x, wt = cw.make()
    dx, dwt = x.to("cuda:0"), wt.to("cuda:0")
    y = tss.conv2d(dx, dwt, cw.stride, cw.pad, cw.dil, tile_oh=cw.tile_oh, out_dtype=cw.out_dtype)
    # room for two sets of the operand copies: consecutive calls alternate between them
    ws_set = (tss.conv2d_workspace_size(cw.N, cw.C, cw.H, cw.W, cw.Co, cw.kh, cw.kw) + 255) // 256 * 256
    ws = torch.empty(2 * ws_set, dtype=torch.uint8, device="cuda:0")

    def launch_conv():
        tss.conv2d(dx, dwt, cw.stride, cw.pad, cw.dil, tile_oh=cw.tile_oh, out_dtype=cw.out_dtype, out=y,
                   workspace=ws)

    _, conv_host_us = warm_up(launch_conv, 10, min_s=0.2)
    conv_ms, _, _ = timed(launch_conv, 200, conv_host_us, stream)
    conv_us = conv_ms * 1e3

    # the same convolution on channel-last tensors (torch's channels_last
    # format), read and written in place: one launch, no operand copies
    cx = dx.contiguous(memory_format=torch.channels_last)
    cwt = dwt.contiguous(memory_format=torch.channels_last)
    yc = tss.conv2d(cx, cwt, cw.stride, cw.pad, cw.dil, tile_oh=cw.tile_oh, out_dtype=cw.out_dtype)
    torch.cuda.synchronize()
    nhwc_same = bool(torch.equal(yc.contiguous(), y))  # the same bits as the NCHW path

    def launch_conv_nhwc():
        tss.conv2d(cx, cwt, cw.stride, cw.pad, cw.dil, tile_oh=cw.tile_oh, out_dtype=cw.out_dtype, out=yc)

    _, nhwc_host_us = warm_up(launch_conv_nhwc, 10, min_s=0.2)
    nhwc_ms, _, _ = timed(launch_conv_nhwc, 200, nhwc_host_us, stream)
    nhwc_us = nhwc_ms * 1e3
    OH = OW = 28
    conv_flops = 2 * cw.N * cw.Co * OH * OW * cw.C * cw.kh * cw.kw
    conv_cfg = tss.conv2d_default_config(cw.N, cw.C, cw.H, cw.W, cw.Co, cw.kh, cw.kw, cw.stride, cw.pad, cw.dil)

    cfg_str = f"{cfg.bm}x{cfg.bn}x{cfg.bk}/s{cfg.stages}/t{cfg.threads}/{cfg.instr}"
    achieved = flops / (ms_per_step * 1e-3) / 1e12
    line = {
        "metric": "fp16 GEMM TFLOP/s at 4096^3 and % of MI355X dense MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "gemm_f16_4096: C = A x B, M=N=K=4096, fp16 row-major operands U[-1,1] "
                               "(seeds 2000/2001), fp32 accumulation, fp16 output",
                   "tile": cfg_str, "parallelism": "single GPU", "wall_s": round(wall, 4),
                   "sampled_parity_ok": parity_ok},
        "timing": {"warmup_launches": warm_n, "timed_launches": args.steps,
                   "host_enqueue_us_per_call": round(host_us, 2),
                   "method": "HIP events on the launch stream around the timed launches, queued behind a "
                             "GPU-side spin so that the host's per-call cost is not in the interval; warm-up "
                             "runs at least --warmup launches and at least 1 s of GPU work"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                     "traffic": profiled_traffic(cfg_str)},
        "conv": {"workload": "conv_f16_n8c256h56_k3s2p1 (tileOh 8, fp32 out), NCHW x / OIHW w / NCHW y: "
                             "layout pass + implicit GEMM (a workspace of two operand sets, which consecutive calls alternate)",
                             "us": round(conv_us, 2),
                 "tflops": round(conv_flops / (conv_us * 1e-6) / 1e12, 2),
                 "tile": f"{conv_cfg.bm}x{conv_cfg.bn}x{conv_cfg.bk}/s{conv_cfg.stages}/t{conv_cfg.threads}/"
                         f"{conv_cfg.instr}"},
        "conv_nhwc": {"workload": "the same convolution, NHWC x / OHWI w / NHWC y (channels_last tensors) read "
                                  "and written in place: the implicit GEMM alone", "us": round(nhwc_us, 2),
                      "tflops": round(conv_flops / (nhwc_us * 1e-6) / 1e12, 2),
                      "same_bits_as_nchw": nhwc_same},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(A, B)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
