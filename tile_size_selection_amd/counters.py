"""Hardware counters of the headline GEMM kernel: HBM traffic, MFMA
utilisation and LDS bank conflicts.

HBM traffic, two rocprofv3 runs (one counter per pass):

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -o run -- python3 -m tile_size_selection_amd.counters run
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write -o run -- python3 -m tile_size_selection_amd.counters run
    python3 -m tile_size_selection_amd.counters summarize <dir> [--trace <kernel_stats.csv>] > summary.md

MFMA utilisation and LDS bank conflicts (the rocprofiler derived metrics
MfmaUtil = sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) x SIMDs) and
LdsBankConflict = conflict cycles per LDS access cycle), for the GEMM and for
every pattern of the LDS bank table:

    rocprofv3 --pmc MfmaUtil LdsBankConflict SQ_INSTS_LDS --output-format csv -d <dir>/util -o run -- python3 -m tile_size_selection_amd.counters run
    rocprofv3 --pmc MfmaUtil LdsBankConflict SQ_INSTS_LDS --output-format csv -d <dir>/ldsutil -o run -- python3 -m tile_size_selection_amd.counters run-lds
    python3 -m tile_size_selection_amd.counters summarize-util <dir> > summary.md

Kernel durations of any rocprofv3 --kernel-trace run (its results database
or kernel_trace.csv), with the mean of each kernel's last N launches:

    python3 -m tile_size_selection_amd.counters trace-summary <dir>/run_results.db --last 20

`run` launches a plain elementwise pass over 256 MiB (y = -x: known bytes
read and written) and then the 4096^3 fp16 GEMM in the configuration the
benchmark times.  That pass calibrates the counters: the GEMM's FETCH_SIZE / WRITE_SIZE (KiB per
dispatch, summed over the L2 channels) are scaled by bytes_known / bytes_read
of the copy.  `summarize` writes the figures the benchmark reads back
(kernel_source_hash, config, hbm_bytes_per_launch).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_BYTES = 256 << 20


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm_kernel.h", "registry.h", "instances.inc"):
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def run(launches: int = 5):
    import torch
    from . import api
    from .inputs import WORKLOADS
    src = torch.ones(COPY_BYTES // 2, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)      # reads and writes COPY_BYTES
    torch.cuda.synchronize()
    w = WORKLOADS[2]
    A, B = w.make()
    dA, dB = A.cuda(), B.cuda()
    out = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    for _ in range(launches):
        api.gemm(dA, dB, out=out)
    torch.cuda.synchronize()
    cfg = api.default_config(w.M, w.N, w.K)
    print(f"config {cfg.bm}x{cfg.bn}x{cfg.bk}/s{cfg.stages}/t{cfg.threads}/{cfg.instr}", flush=True)


def run_conv(launches: int = 5):
    """The convolution workload: `launches` NCHW calls (layout pass + implicit
    GEMM), then `launches` calls on the same values as channel-last tensors
    (the implicit GEMM alone), then `launches` 4096^3 GEMMs for comparison."""
    import torch
    from . import api
    from .inputs import WORKLOADS
    cw = WORKLOADS[5]
    x, w = cw.make()
    dx, dw = x.cuda(), w.cuda()
    cl = torch.channels_last
    cx, cwt = dx.contiguous(memory_format=cl), dw.contiguous(memory_format=cl)
    y = api.conv2d(dx, dw, cw.stride, cw.pad, cw.dil, tile_oh=cw.tile_oh, out_dtype=cw.out_dtype)
    yc = api.conv2d(cx, cwt, cw.stride, cw.pad, cw.dil, tile_oh=cw.tile_oh, out_dtype=cw.out_dtype)
    ws = torch.empty(api.conv2d_workspace_size(cw.N, cw.C, cw.H, cw.W, cw.Co, cw.kh, cw.kw), dtype=torch.uint8,
                     device="cuda")
    for _ in range(launches):
        api.conv2d(dx, dw, cw.stride, cw.pad, cw.dil, tile_oh=cw.tile_oh, out_dtype=cw.out_dtype, out=y,
                   workspace=ws)
    for _ in range(launches):
        api.conv2d(cx, cwt, cw.stride, cw.pad, cw.dil, tile_oh=cw.tile_oh, out_dtype=cw.out_dtype, out=yc)
    g = WORKLOADS[2]
    A, B = g.make()
    dA, dB = A.cuda(), B.cuda()
    out = torch.empty((g.M, g.N), dtype=torch.float16, device="cuda")
    for _ in range(launches):
        api.gemm(dA, dB, out=out)
    torch.cuda.synchronize()
    print("conv and GEMM launches done", flush=True)


# hardware counter passes of `run-conv` (each within one pass's counter limits)
CONV_PASSES = [
    "MfmaUtil LdsUtil",
    "LdsLatency",
    "VmemLatency",
    "SQ_WAIT_INST_LDS SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_LDS "
    "SQ_LDS_BANK_CONFLICT SQ_INSTS_MFMA",
    "SQ_INSTS_LDS SQ_INSTS_VMEM SQ_INSTS_VALU SQ_INSTS_SALU SQ_WAVES SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL "
    "SQ_VMEM_TA_CMD_FIFO_FULL",
]


def summarize_conv(d: str) -> str:
    """Per kernel of a `run-conv` run, the mean of every counter over its
    dispatches (pass directories <d>/p1 ... <d>/pN, one per CONV_PASSES
    entry).  A conv GEMM dispatch that follows a layout pass is the NCHW
    call's; the others are the channel-last call's."""
    vals = defaultdict(lambda: defaultdict(list))
    for i in range(1, len(CONV_PASSES) + 1):
        files = glob.glob(os.path.join(d, f"p{i}", "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"counter pass p{i} missing under {d}")
        prev = ""
        for _, name, c in per_dispatch_all(files[0]):
            if "conv_layout" in name:
                kind = "layout pass (NCHW call)"
            elif "tiled_gemm_kernel" in name and "Lb1E" in name:
                kind = "conv implicit GEMM, NCHW call" if "conv_layout" in prev else \
                    "conv implicit GEMM, channel-last call"
            elif "tiled_gemm_kernel" in name:
                kind = "GEMM 4096^3"
            else:
                prev = name
                continue
            prev = name
            for k, v in c.items():
                vals[kind][k].append(v)
    kinds = ["conv implicit GEMM, channel-last call", "conv implicit GEMM, NCHW call", "layout pass (NCHW call)",
             "GEMM 4096^3"]
    counters = sorted({k for kind in kinds for k in vals[kind]})
    lines = ["| counter | " + " | ".join(kinds) + " |", "|---|" + "---|" * len(kinds)]
    for k in counters:
        lines.append(f"| {k} | " + " | ".join(f"{_mean(vals[kind][k]):.4g}" if vals[kind][k] else "—"
                                               for kind in kinds) + " |")
    per_mfma = []
    for kind in kinds[:2] + kinds[3:]:
        v = vals[kind]
        if v["SQ_INSTS_MFMA"] and v["SQ_INSTS_LDS"]:
            m = _mean(v["SQ_INSTS_MFMA"])
            per_mfma.append(f"| {kind} | {_mean(v['SQ_INSTS_LDS']) / m:.3f} | {_mean(v['SQ_INSTS_VMEM']) / m:.3f} | "
                            f"{_mean(v['SQ_WAIT_INST_ANY']) / _mean(v['SQ_WAVE_CYCLES']):.3f} |")
    lines += ["", "| kernel | LDS instructions per MFMA | VMEM instructions per MFMA | "
              "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES |", "|---|---|---|---|"] + per_mfma
    return "\n".join(lines) + "\n"


def run_lds():
    """Every pattern of the LDS bank table, one launch each, in table order."""
    from . import api
    from .ldsbench import ROWS
    for p, stride, _ in ROWS:
        api.lds_probe(p, stride, iters=2000, blocks=256)
        print(f"lds pattern {p} stride {stride}", flush=True)


def per_dispatch_all(csv_path: str):
    """[(dispatch id, kernel name, {counter: value})] in dispatch order."""
    acc = defaultdict(lambda: defaultdict(float))
    names = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            acc[d][r["Counter_Name"]] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
    return [(d, names[d], dict(acc[d])) for d in sorted(acc)]


def summarize_util(d: str) -> str:
    from .ldsbench import ROWS, WHAT
    util = glob.glob(os.path.join(d, "util", "**", "*counter_collection.csv"), recursive=True)
    ldsu = glob.glob(os.path.join(d, "ldsutil", "**", "*counter_collection.csv"), recursive=True)
    if not util or not ldsu:
        raise SystemExit("counter files missing")
    gemm = [c for _, k, c in per_dispatch_all(util[0]) if "tiled_gemm_kernel" in k]
    probes = [c for _, k, c in per_dispatch_all(ldsu[0]) if "lds_probe_kernel" in k]
    if not gemm or len(probes) != len(ROWS):
        raise SystemExit(f"expected GEMM dispatches and {len(ROWS)} probe dispatches, got {len(gemm)}, {len(probes)}")
    mean = lambda key: _mean([c.get(key, float("nan")) for c in gemm])
    lines = [
        "# MFMA utilisation and LDS bank conflicts (rocprofv3 derived metrics)",
        "",
        "Commands (from the repository root, on the MI355X):",
        "",
        "    rocprofv3 --pmc MfmaUtil LdsBankConflict SQ_INSTS_LDS --output-format csv -d <dir>/util -o run -- "
        "python3 -m tile_size_selection_amd.counters run",
        "    rocprofv3 --pmc MfmaUtil LdsBankConflict SQ_INSTS_LDS --output-format csv -d <dir>/ldsutil -o run -- "
        "python3 -m tile_size_selection_amd.counters run-lds",
        "    python3 -m tile_size_selection_amd.counters summarize-util <dir>",
        "",
        "MfmaUtil = sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) x SIMDs) x 100;"
        " LdsBankConflict = SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT), conflict cycles per"
        " conflict-free LDS access cycle.",
        "",
        f"4096^3 fp16 GEMM (planner's tile), mean of {len(gemm)} dispatches: MfmaUtil {mean('MfmaUtil'):.1f} %,"
        f" LdsBankConflict {mean('LdsBankConflict'):.4f}, SQ_INSTS_LDS {mean('SQ_INSTS_LDS'):.0f}",
        f"kernel_source_hash: {kernel_source_hash()}",
        "",
        "| LDS probe pattern | lane stride (4-byte words) | LdsBankConflict |",
        "|---|---|---|",
    ]
    for (p, stride, _), c in zip(ROWS, probes):
        st = "—" if p.startswith("gemm") else str(stride)
        lines.append(f"| {WHAT[p]} | {st} | {c.get('LdsBankConflict', float('nan')):.3f} |")
    return "\n".join(lines) + "\n"


def per_dispatch(csv_path: str, counter: str):
    """{kernel name: [value per dispatch]} (rows of one dispatch summed)."""
    acc = defaultdict(float)
    names = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = r["Dispatch_Id"]
            acc[d] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
    out = defaultdict(list)
    for d, v in acc.items():
        out[names[d]].append(v)
    return out


def _mean(v):
    return sum(v) / len(v)


def summarize(d: str, trace: str = None) -> str:
    from . import api
    fetch = per_dispatch(glob.glob(os.path.join(d, "fetch", "**", "*counter_collection.csv"), recursive=True)[0],
                         "FETCH_SIZE")
    write = per_dispatch(glob.glob(os.path.join(d, "write", "**", "*counter_collection.csv"), recursive=True)[0],
                         "WRITE_SIZE")
    # the calibration pass is the non-GEMM kernel that reads the most
    copy_k = sorted((k for k in fetch if "tiled_gemm_kernel" not in k), key=lambda k: -_mean(fetch[k]))
    gemm_k = [k for k in fetch if "tiled_gemm_kernel" in k]
    if not copy_k or not gemm_k:
        raise SystemExit("calibration or GEMM dispatches missing from the counter files")
    ck, gk = copy_k[0], gemm_k[0]
    f_copy = _mean(fetch[ck]) * 1024.0
    w_copy = _mean(write[ck]) * 1024.0
    f_scale = COPY_BYTES / f_copy
    w_scale = COPY_BYTES / w_copy
    f_gemm = _mean(fetch[gk]) * 1024.0 * f_scale
    w_gemm = _mean(write[gk]) * 1024.0 * w_scale
    cfg = api.default_config(4096, 4096, 4096)
    cfg_s = f"{cfg.bm}x{cfg.bn}x{cfg.bk}/s{cfg.stages}/t{cfg.threads}/{cfg.instr}"
    algo = 3 * 4096 * 4096 * 2
    lines = [
        "# HBM traffic of the 4096^3 fp16 GEMM kernel (rocprofv3 counters)",
        "",
        "Commands (from the repository root, on the MI355X):",
        "",
        "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -o run -- "
        "python3 -m tile_size_selection_amd.counters run",
        "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write -o run -- "
        "python3 -m tile_size_selection_amd.counters run",
        "    python3 -m tile_size_selection_amd.counters summarize <dir>",
        "",
        f"copy calibration: {COPY_BYTES} B copied; FETCH_SIZE read {f_copy:.0f} B (scale {f_scale:.4f}), "
        f"WRITE_SIZE read {w_copy:.0f} B (scale {w_scale:.4f}); kernel `{ck[:60]}`",
        f"GEMM kernel `{gk[:90]}`: {len(fetch[gk])} dispatches",
        f"GEMM FETCH_SIZE {_mean(fetch[gk]):.0f} KiB/dispatch raw -> {f_gemm:.0f} B scaled",
        f"GEMM WRITE_SIZE {_mean(write[gk]):.0f} KiB/dispatch raw -> {w_gemm:.0f} B scaled",
        f"algorithmic bytes (A and B read once, C written once): {algo} B; measured / algorithmic = "
        f"{(f_gemm + w_gemm) / algo:.3f}",
        "",
        "Values read by bench.py:",
        "",
        f"kernel_source_hash: {kernel_source_hash()}",
        f"config: {cfg_s}",
        f"hbm_bytes_per_launch: {f_gemm + w_gemm:.0f}",
        f"fetch_bytes_per_launch: {f_gemm:.0f}",
        f"write_bytes_per_launch: {w_gemm:.0f}",
    ]
    if trace and os.path.exists(trace):
        lines += ["", "Kernel trace of the benchmark, same build:", "",
                  "    rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/ktrace -o bench -- "
                  "python3 bench.py --no-cpu-baseline"]
        with open(trace) as f:
            for r in csv.DictReader(f):
                if "tiled_gemm_kernel" in r["Name"]:
                    lines += ["", f"kernel trace (same build): {r['Name'][:90]} calls {r['Calls']} "
                                  f"average {float(r['AverageNs']) / 1e3:.2f} us, min {float(r['MinNs']) / 1e3:.2f} us"]
    return "\n".join(lines) + "\n"


def trace_summary(path: str, last: int = 0, until: str = "", after: str = "") -> str:
    """Per-kernel durations of a rocprofv3 kernel trace: the run's results
    database (<dir>/<name>_results.db, the default output) or its
    kernel_trace.csv.  last > 0 adds, per kernel, the mean of its last `last`
    launches (the timed region of a benchmark run) and the mean gap between
    them.  until / after (a kernel-name substring K): only the dispatches up
    to the one right after K's last dispatch / only those starting after K's
    last dispatch has ended (to split a run into phases)."""
    rows = []   # (name, start_ns, end_ns)
    if path.endswith(".db"):
        import sqlite3
        con = sqlite3.connect(path)
        rows = list(con.execute("select name, start, end from kernels order by start"))
    else:
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        rows.sort(key=lambda r: r[1])
    rows.sort(key=lambda r: r[1])
    for key, keep_until in ((until, True), (after, False)):
        if not key:
            continue
        idx = [i for i, r in enumerate(rows) if key in r[0]]
        if not idx:
            raise SystemExit(f"no kernel named like {key!r} in {path}")
        i = idx[-1]
        rows = rows[:i + 2] if keep_until else [r for r in rows if r[1] >= rows[i][2]]
    by = defaultdict(list)
    for name, st, en in rows:
        by[name].append((st, en))
    out = ["| kernel | launches | average us | min us | max us |" + (f" last {last}: average us | gap us |" if last else ""),
           "|---|---|---|---|---|" + ("---|---|" if last else "")]
    for name, ev in sorted(by.items(), key=lambda kv: -sum(e - s for s, e in kv[1])):
        d = [e - s for s, e in ev]
        line = f"| `{name[:100]}` | {len(d)} | {_mean(d) / 1e3:.2f} | {min(d) / 1e3:.2f} | {max(d) / 1e3:.2f} |"
        if last:
            tail = ev[-last:]
            gaps = [tail[i + 1][0] - tail[i][1] for i in range(len(tail) - 1)]
            line += f" {_mean([e - s for s, e in tail]) / 1e3:.2f} | {(_mean(gaps) if gaps else 0) / 1e3:.2f} |"
        out.append(line)
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--launches", type=int, default=5)
    sub.add_parser("run-lds")
    rc = sub.add_parser("run-conv")
    rc.add_argument("--launches", type=int, default=5)
    sc = sub.add_parser("summarize-conv")
    sc.add_argument("dir")
    s = sub.add_parser("summarize")
    s.add_argument("dir")
    s.add_argument("--trace", default=None)
    u = sub.add_parser("summarize-util")
    u.add_argument("dir")
    t = sub.add_parser("trace-summary")
    t.add_argument("path")
    t.add_argument("--last", type=int, default=0)
    t.add_argument("--until", default="")
    t.add_argument("--after", default="")
    a = ap.parse_args()
    if a.cmd == "trace-summary":
        sys.stdout.write(trace_summary(a.path, a.last, a.until, a.after))
        return 0
    if a.cmd == "run":
        run(a.launches)
    elif a.cmd == "run-lds":
        run_lds()
    elif a.cmd == "run-conv":
        run_conv(a.launches)
    elif a.cmd == "summarize-conv":
        sys.stdout.write(summarize_conv(a.dir))
    elif a.cmd == "summarize-util":
        sys.stdout.write(summarize_util(a.dir))
    else:
        sys.stdout.write(summarize(a.dir, a.trace))
    return 0


if __name__ == "__main__":
    sys.exit(main())
