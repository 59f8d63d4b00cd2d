"""Build libtss.so (planner, C ABI and every gfx950 kernel) in-tree.

    python -m tile_size_selection_amd.build [--incremental] [--jobs N] [--units NAME ...]

Each instantiation unit under csrc/inst is compiled by its own hipcc process
for --offload-arch=gfx950; the objects are linked into
tile_size_selection_amd/libtss.so, which is what the Python binding loads.
The planner's command line, csrc/tss_plan.c, is built against that library
into tile_size_selection_amd/tss_plan (a host program: gcc, C ABI only).
--units recompiles only the sources whose file names contain one of the
given strings (the other objects are linked as they are).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtss.so")
CLI = os.path.join(PKG, "tss_plan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops off: compiler-made v_pk_{add,mul,fma}_f32 are avoided.
# amdgpu-mfma-vgpr-form: MFMA accumulators stay in the architectural VGPRs.
# Left to its heuristic, the compiler put part of the accumulators of 4-wave
# tiles in AGPRs and copied them into the MFMA's source registers before
# most MFMAs (e.g. 300 accvgpr moves in the 128x128x64/256-thread
# convolution loop); with the flag the accumulators are updated in place.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-variable",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=true",
         "-I", os.path.join(ROOT, "include")]


def sources():
    return ([os.path.join(CSRC, "planner.cpp"), os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "lds_probe.hip"),
             os.path.join(CSRC, "noalloc.cpp")]
            + sorted(glob.glob(os.path.join(CSRC, "inst", "*.hip"))))


def _obj(src):
    rel = os.path.relpath(src, CSRC).replace(os.sep, "_")
    return os.path.join(OUT_DIR, rel + ".o")


def _flags_stamp():
    """A file whose content is the compile flags; rewritten (and so newer
    than every object) when they change."""
    path = os.path.join(OUT_DIR, "flags.txt")
    text = " ".join([HIPCC] + FLAGS)
    if not os.path.exists(path) or open(path).read() != text:
        with open(path, "w") as f:
            f.write(text)
    return path


def _up_to_date(src, obj):
    """True if obj is newer than src, the compile flags and every file its
    dependency list (written by the compiler next to it) names."""
    dep = obj[:-2] + ".d"
    if not (os.path.exists(obj) and os.path.exists(dep)):
        return False
    if os.path.getmtime(_flags_stamp()) >= os.path.getmtime(obj):
        return False
    with open(dep) as f:
        text = f.read().replace("\\\n", " ")
    files = text.split(":", 1)[1].split() if ":" in text else []
    t = os.path.getmtime(obj)
    return all(os.path.exists(d) and os.path.getmtime(d) < t for d in [src] + files)


def _flags_for(src):
    """The wide-accumulator units (256 accumulators per lane) keep the
    compiler's own accumulator placement: the in-VGPR form does not fit them
    (and this compiler fails on them with it)."""
    if src.endswith("_wide.hip"):
        return [f for f in FLAGS if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form=true")]
    return FLAGS


def _compile(src, obj):
    t0 = time.time()
    cmd = [HIPCC, *_flags_for(src), "-x", "hip", "-c", src, "-o", obj, "-MD", "-MF", obj[:-2] + ".d"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return src, time.time() - t0


def build_cli(verbose: bool = True) -> str:
    """tss_plan: the planner's command line, linked to libtss.so beside it."""
    tmp = CLI + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "tss_plan.c"), "-o", tmp, "-L", PKG, "-l:libtss.so", "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for tss_plan.c:\n{r.stderr}")
    os.replace(tmp, CLI)
    if verbose:
        print(f"built {os.path.relpath(CLI, ROOT)}", flush=True)
    return CLI


def build(incremental: bool = False, jobs: int = 0, verbose: bool = True, units=None) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    todo = []
    for s in sources():
        o = _obj(s)
        if units is not None:
            if not any(u in os.path.basename(s) for u in units) and os.path.exists(o):
                continue
        elif incremental and _up_to_date(s, o):
            continue
        todo.append((s, o))
    jobs = jobs or min(16, os.cpu_count() or 4)
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, dt in ex.map(lambda so: _compile(*so), todo):
            if verbose:
                print(f"  compiled {os.path.relpath(src, ROOT)} in {dt:.1f}s", flush=True)
    objs = [_obj(s) for s in sources()]
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {os.path.relpath(LIB, ROOT)} ({len(todo)} units compiled) in {time.time() - t0:.1f}s",
              flush=True)
    build_cli(verbose)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--incremental", action="store_true")
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--clean", action="store_true")
    ap.add_argument("--units", nargs="+", default=None)
    a = ap.parse_args()
    if a.clean and os.path.isdir(OUT_DIR):
        shutil.rmtree(OUT_DIR)
    build(a.incremental, a.jobs, units=a.units)
    return 0


if __name__ == "__main__":
    sys.exit(main())
