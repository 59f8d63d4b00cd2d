"""How the way of timing changes the 4096^3 fp16 GEMM's per-launch figure.

    python3 -m tile_size_selection_amd.timing_study

HIP events on the launch stream around n launches of the planner's kernel
through the Python binding, in five ways: (a) after 5 warm-up launches,
events recorded with an empty queue (so the first kernel waits for the
host's call); (b) the same after 1 s of warm-up; (c) after 1 s of warm-up
with the launches queued behind a GPU-side spin, so the interval holds only
the kernels; (d) and (e): 2000 launches with and without the spin.  Also
prints the host's enqueue cost per call.  The benchmark uses (c).
"""
from __future__ import annotations

import time


def main() -> int:
    import torch
    from . import api
    from .inputs import WORKLOADS
    w = WORKLOADS[2]
    A, B = w.make()
    dA, dB = A.cuda(), B.cuda()
    out = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    s = torch.cuda.current_stream()

    def run(steps, spin):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if spin:
            torch.cuda._sleep(int(5e6))
        e0.record(s)
        for _ in range(steps):
            api.gemm(dA, dB, out=out)
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    for _ in range(5):
        api.gemm(dA, dB, out=out)
    print(f"a: 5 warm-ups, no spin, 20 launches: {run(20, False):.2f} us", flush=True)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        for _ in range(20):
            api.gemm(dA, dB, out=out)
        torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(200):
        api.gemm(dA, dB, out=out)
    t2 = time.perf_counter()
    torch.cuda.synchronize()
    print(f"host enqueue per call: {(t2 - t1) / 200 * 1e6:.1f} us", flush=True)
    print(f"b: 1 s warm-up, no spin, 20 launches: {run(20, False):.2f} us", flush=True)
    print(f"c: 1 s warm-up, spin, 20 launches: {run(20, True):.2f} us", flush=True)
    print(f"d: spin, 2000 launches: {run(2000, True):.2f} us", flush=True)
    print(f"e: no spin, 2000 launches: {run(2000, False):.2f} us", flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
