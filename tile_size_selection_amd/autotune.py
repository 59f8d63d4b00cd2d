"""Measured sweep over the planner's candidate tiles (the autotuning loop of
the "Tiling（分块）" page: enumerate the candidates, drop the ones that break
a hardware constraint, time every survivor on the device, keep the fastest).

    python -m tile_size_selection_amd.autotune --m 4096 --n 4096 --k 4096 [--out report.md]
    python -m tile_size_selection_amd.autotune --conv [--out report.md]     (the conv workload)
    python -m tile_size_selection_amd.autotune summarize report1.md report2.md ...   (one row per report)
    python -m tile_size_selection_amd.autotune library [--topk 64] [--out report.md]   (tss_gemm_autotune's choice
        against the full sweep on nine GEMM shapes)

Prints, for every feasible configuration, its measured time and TFLOP/s, its
rank in the planner's order, and how the planner's first choice compares with
the fastest measured one.
"""
from __future__ import annotations

import argparse
import sys
import time
from typing import List, Optional, Tuple

import torch

from . import api
from .inputs import draw


def time_config(A, B, out, cfg, iters: int, warmup: int, out_dtype: str) -> float:
    for _ in range(warmup):
        api.gemm(A, B, out_dtype=out_dtype, cfg=cfg, out=out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e6))   # the launches queue behind a GPU spin: the host's call cost stays out
    e0.record()
    for _ in range(iters):
        api.gemm(A, B, out_dtype=out_dtype, cfg=cfg, out=out)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters * 1e3  # microseconds


def sweep(M: int, N: int, K: int, batch: int = 1, dtype: str = "f16", out_dtype: Optional[str] = None,
          iters: int = 20, warmup: int = 5, rounds: int = 2) -> Tuple[List[dict], dict]:
    best, ranked, n = api.tile_plan(M, N, K, batch=batch, cap=1024)
    shapeA = (batch, M, K) if batch > 1 else (M, K)
    shapeB = (batch, K, N) if batch > 1 else (K, N)
    A = draw(shapeA, "uniform", -1, 1, dtype, 2000).cuda()
    B = draw(shapeB, "uniform", -1, 1, dtype, 2001).cuda()
    od = out_dtype or dtype
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[od]
    out = torch.empty(((batch,) if batch > 1 else ()) + (M, N), dtype=tdt, device="cuda")
    # bring the clocks up before the first measurement
    t_end = time.time() + 1.0
    while time.time() < t_end:
        api.gemm(A, B, out_dtype=od, cfg=ranked[0]["config"], out=out)
    torch.cuda.synchronize()
    rows = []
    for rank, v in enumerate(ranked):
        rows.append({"rank": rank, "config": v["config"], "verdict": v, "us": float("inf")})
    # several rounds, interleaved, keep each config's best round
    for _ in range(rounds):
        for r in rows:
            r["us"] = min(r["us"], time_config(A, B, out, r["config"], iters, warmup, od))
    flops = 2.0 * batch * M * N * K
    for r in rows:
        r["tflops"] = flops / (r["us"] * 1e-6) / 1e12
    fastest = min(rows, key=lambda r: r["us"])
    summary = {"n_feasible": n, "planner": rows[0], "fastest": fastest,
               "planner_over_fastest": rows[0]["us"] / fastest["us"]}
    return rows, summary


def sweep_conv(iters: int = 20, warmup: int = 3, rounds: int = 2) -> Tuple[List[dict], dict]:
    """The conv workload (8x256x56x56, 3x3, stride 2, pad 1, H-tiles of 8
    rows, fp32 out) under every feasible tile of its implicit GEMM."""
    from .inputs import WORKLOADS
    cw = WORKLOADS[5]
    OH = (cw.H + 2 * cw.pad[0] - cw.kh) // cw.stride[0] + 1
    OW = (cw.W + 2 * cw.pad[1] - cw.kw) // cw.stride[1] + 1
    M, N, K = cw.Co, cw.N * OH * OW, cw.C * cw.kh * cw.kw
    best, ranked, n = api.conv_plan(cw.Co, N, cw.C, cw.kh * cw.kw, cap=1024)
    x, w = cw.make()
    x, w = x.cuda(), w.cuda()
    y = torch.empty((cw.N, cw.Co, OH, OW), dtype=torch.float32, device="cuda")
    run = lambda cfg: api.conv2d(x, w, cw.stride, cw.pad, cw.dil, tile_oh=cw.tile_oh, out_dtype="f32", cfg=cfg,
                                 out=y)
    t_end = time.time() + 1.0
    while time.time() < t_end:
        run(ranked[0]["config"])
    torch.cuda.synchronize()
    rows = [{"rank": i, "config": v["config"], "verdict": v, "us": float("inf")} for i, v in enumerate(ranked)]
    for _ in range(rounds):
        for r in rows:
            for _ in range(warmup):
                run(r["config"])
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(int(2e6))
            e0.record()
            for _ in range(iters):
                run(r["config"])
            e1.record()
            torch.cuda.synchronize()
            r["us"] = min(r["us"], e0.elapsed_time(e1) / iters * 1e3)
    flops = 2.0 * M * N * K
    for r in rows:
        r["tflops"] = flops / (r["us"] * 1e-6) / 1e12
    fastest = min(rows, key=lambda r: r["us"])
    return rows, {"n_feasible": n, "planner": rows[0], "fastest": fastest,
                  "planner_over_fastest": rows[0]["us"] / fastest["us"], "shape": (M, N, K)}


def report(M, N, K, batch, rows, summary) -> str:
    c = lambda cfg: f"{cfg.bm}x{cfg.bn}x{cfg.bk} s{cfg.stages} t{cfg.threads} {cfg.instr}"
    lines = [f"# Measured tile sweep: GEMM {batch}x{M}x{N}x{K}", "",
             f"feasible candidates: {summary['n_feasible']}",
             f"planner's choice: {c(summary['planner']['config'])}: {summary['planner']['us']:.1f} us "
             f"({summary['planner']['tflops']:.1f} TFLOP/s)",
             f"fastest measured: {c(summary['fastest']['config'])} (planner rank {summary['fastest']['rank']}): "
             f"{summary['fastest']['us']:.1f} us ({summary['fastest']['tflops']:.1f} TFLOP/s)",
             f"planner time / fastest time: {summary['planner_over_fastest']:.4f}", "",
             "| planner rank | config | us | TFLOP/s | LDS KiB | blocks/CU | waves | C4 warnings |",
             "|---|---|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: r["us"]):
        v = r["verdict"]
        lines.append(f"| {r['rank']} | {c(r['config'])} | {r['us']:.1f} | {r['tflops']:.1f} | "
                     f"{v['smem_total'] / 1024:.0f} | {v['blocks_per_core']} | {v['waves']} | "
                     f"{','.join(v['warnings']) or '-'} |")
    return "\n".join(lines) + "\n"


def summarize(paths: List[str]) -> str:
    """One table row per sweep report written by this module (--out): the
    planner's choice, the fastest configuration and their time ratio."""
    import re
    rows = ["| M x N x K | planner's choice | us | fastest measured (planner rank) | us | planner / fastest |",
            "|---|---|---|---|---|---|"]
    for p in paths:
        txt = open(p, encoding="utf-8").read()
        shape = re.search(r"GEMM (\d+)x(\d+)x(\d+)x(\d+)", txt).groups()
        plan = re.search(r"planner's choice: (.+?): ([\d.]+) us", txt).groups()
        fast = re.search(r"fastest measured: (.+?) \(planner rank (\d+)\): ([\d.]+) us", txt).groups()
        ratio = re.search(r"planner time / fastest time: ([\d.]+)", txt).group(1)
        b, M, N, K = shape
        rows.append(f"| {M} x {N} x {K}{'' if b == '1' else f' (batch {b})'} | {plan[0]} | {plan[1]} | "
                    f"{fast[0]} ({fast[1]}) | {fast[2]} | {ratio} |")
    return "\n".join(rows) + "\n"


LIBRARY_SHAPES = [(2048, 2048, 2048), (1024, 4096, 4096), (8192, 1024, 8192), (3000, 3000, 3000),
                  (512, 512, 8192), (4096, 4096, 72), (2048, 8192, 136), (4096, 4096, 200), (4096, 4096, 4096)]


def library_check(shapes, topk: int = 64, iters: int = 20) -> str:
    """For each shape: the full measured sweep (every feasible tile, as
    `sweep`), then the library's own measured choice (tss_gemm_autotune over
    the planner's first `topk` candidates), re-timed the way the sweep times
    every tile, against the sweep's fastest and against the model's plan.
    Writes a markdown report."""
    rows = []
    for (M, N, K) in shapes:
        srows, summ = sweep(M, N, K, iters=iters, warmup=3, rounds=2)
        A = draw((M, K), "uniform", -1, 1, "f16", 2000).cuda()
        B = draw((K, N), "uniform", -1, 1, "f16", 2001).cuda()
        out = torch.empty((M, N), dtype=torch.float16, device="cuda")
        torch.cuda.synchronize()
        t0 = time.time()
        cfg, us_lib = api.autotune_gemm(A, B, topk=topk, iters=iters, out=out)
        wall = time.time() - t0
        t_pick = min(time_config(A, B, out, cfg, iters, 3, "f16") for _ in range(2))
        fastest = summ["fastest"]
        key = lambda c: f"{c.bm}x{c.bn}x{c.bk} s{c.stages} t{c.threads} {c.instr}"
        rank = next(r["rank"] for r in srows if r["config"] == cfg)
        rows.append(f"| {M} x {N} x {K} | {key(cfg)} (planner rank {rank}) | {t_pick:.1f} | "
                    f"{key(fastest['config'])} | {fastest['us']:.1f} | {t_pick / fastest['us']:.4f} | "
                    f"{summ['planner_over_fastest']:.4f} | {wall * 1e3:.0f} |")
        print(rows[-1], flush=True)
    head = ("| M x N x K | library's measured choice | us | fastest of the full sweep | us | choice / fastest |"
            " model plan / fastest | autotune wall ms |\n|---|---|---|---|---|---|---|---|\n")
    return head + "\n".join(rows) + "\n"


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "summarize":
        sys.stdout.write(summarize(sys.argv[2:]))
        return 0
    if len(sys.argv) > 1 and sys.argv[1] == "library":
        lp = argparse.ArgumentParser()
        lp.add_argument("cmd")
        lp.add_argument("--topk", type=int, default=64)
        lp.add_argument("--iters", type=int, default=20)
        lp.add_argument("--out", default=None)
        la = lp.parse_args()
        txt = ("# The library's measured tile choice (tss_gemm_autotune) against the full sweep\n\n"
               "Command (repository root, MI355X): `python3 -m tile_size_selection_amd.autotune library"
               + (f" --out {la.out}" if la.out else "") + "`\n\n"
               f"Per shape (fp16, fp16 out): every feasible tile timed as `sweep` does ({la.iters} launches behind a"
               " GPU spin, best of 2 rounds), then tss_gemm_autotune over the planner's first"
               f" {la.topk} candidates ({la.iters} launches each, best of 2 interleaved rounds), its choice re-timed like"
               " the sweep; model plan = the planner's first candidate.\n\n"
               + library_check(LIBRARY_SHAPES, la.topk, la.iters))
        if la.out:
            with open(la.out, "w") as f:
                f.write(txt)
        return 0
    ap = argparse.ArgumentParser()
    ap.add_argument("--m", type=int, default=4096)
    ap.add_argument("--n", type=int, default=4096)
    ap.add_argument("--k", type=int, default=4096)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--dtype", default="f16")
    ap.add_argument("--out-dtype", default=None)
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--out", default=None)
    ap.add_argument("--conv", action="store_true")
    a = ap.parse_args()
    if a.conv:
        rows, summary = sweep_conv(a.iters)
        M, N, K = summary["shape"]
        txt = report(M, N, K, 1, rows, summary).replace("# Measured tile sweep: GEMM",
                                                        "# Measured tile sweep: conv workload as implicit GEMM")
    else:
        rows, summary = sweep(a.m, a.n, a.k, a.batch, a.dtype, a.out_dtype, a.iters)
        txt = report(a.m, a.n, a.k, a.batch, rows, summary)
    if a.out:
        with open(a.out, "w") as f:
            f.write(txt)
    print("\n".join(txt.splitlines()[:8]), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
