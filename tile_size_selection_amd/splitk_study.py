"""Measured effect of split K (tss_gemm_splitk / tss_conv2d_splitk) on
problems whose output tiles leave CUs idle.

    python3 -m tile_size_selection_amd.splitk_study [--out report.md]

For every problem and split count S: the tile the planner picks for the
split problem (batch * S GEMMs of M x N x ceil(K / S), K rounded to whole
K steps of 64), the time of the whole call (the split GEMM and the
reduction pass) from HIP events around 20 launches queued behind a GPU
spin, best of 3 rounds after a warm-up, against the one-pass GEMM with the
planner's tile (S = 1)."""
from __future__ import annotations

import argparse
import sys

import torch

from . import api
from .inputs import draw

GEMMS = [(1, 256, 256, 256), (1, 512, 512, 8192), (1, 1024, 1024, 8192), (1, 768, 768, 4096),
         (1, 128, 128, 16384), (1, 256, 1024, 4096), (1, 2048, 2048, 2048), (1, 4096, 4096, 4096),
         (1, 1024, 4096, 4096)]
SPLITS = (1, 2, 3, 4, 6, 8, 12, 16)


def _time(fn, n=20, rounds=3):
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(2e6))
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / n * 1e3)
    return best


def split_tile(batch, M, N, K, S):
    ks = -(-K // S)
    ks = -(-ks // 64) * 64
    return api.tile_plan(M, N, ks, batch=batch * S)[0]["config"]


def study_gemm(batch, M, N, K):
    A = draw((batch, M, K) if batch > 1 else (M, K), "uniform", -1, 1, "f16", 11).cuda()
    B = draw((batch, K, N) if batch > 1 else (K, N), "uniform", -1, 1, "f16", 12).cuda()
    out = torch.empty(((batch,) if batch > 1 else ()) + (M, N), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(api.gemm_splitk_workspace_size(batch, M, N, max(SPLITS)), 16), dtype=torch.uint8,
                     device="cuda")
    rows = []
    for S in SPLITS:
        cfg = split_tile(batch, M, N, K, S)
        t = _time(lambda: api.gemm(A, B, cfg=cfg, out=out, splits=S, workspace=ws))
        rows.append((S, cfg, t))
    return rows


def study_conv():
    from .inputs import WORKLOADS
    cw = WORKLOADS[5]
    x, w = cw.make()
    dx, dw = x.cuda(), w.cuda()
    y = torch.empty((cw.N, cw.Co, 28, 28), dtype=torch.float32, device="cuda")
    rows = []
    for S in (1, 2, 3, 4, 6):
        best, _, _ = api.conv_plan(cw.Co, cw.N * 28 * 28 * S, cw.C, cw.kh * cw.kw)   # S times the tiles
        cfg = best["config"]
        t = _time(lambda: api.conv2d(dx, dw, cw.stride, cw.pad, cw.dil, tile_oh=cw.tile_oh, out_dtype="f32",
                                     cfg=cfg, out=y, splits=S))
        rows.append((S, cfg, t))
    return rows


def fmt(cfg):
    return f"{cfg.bm}x{cfg.bn}x{cfg.bk}/s{cfg.stages}/t{cfg.threads}/{cfg.instr}"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    lines = ["| problem | S | tile | us | speed-up over S = 1 |", "|---|---|---|---|---|"]
    for (b, M, N, K) in GEMMS:
        rows = study_gemm(b, M, N, K)
        t1 = rows[0][2]
        for S, cfg, t in rows:
            lines.append(f"| GEMM {b}x{M}x{N}x{K} | {S} | {fmt(cfg)} | {t:.2f} | {t1 / t:.2f} |")
        print(lines[-len(rows):], flush=True)
    rows = study_conv()
    t1 = rows[0][2]
    for S, cfg, t in rows:
        lines.append(f"| conv 8x256x56x56 3x3 s2 | {S} | {fmt(cfg)} | {t:.2f} | {t1 / t:.2f} |")
    text = "\n".join(lines) + "\n"
    print(text, flush=True)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
