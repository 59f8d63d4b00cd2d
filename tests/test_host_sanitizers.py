"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The planner (csrc/planner.cpp, the C entry points the GEMM and convolution
plans go through), the planner's command line (csrc/tss_plan.c) and the fp64
oracle (oracle/gemm_conv.c) are compiled here with gcc / g++ and
-fsanitize=address,undefined (host code only: no GPU code is built), then
driven over a grid of problems including empty, ragged and bound-sized ones
and bad arguments (tests/sanitize/*.c*).  Any sanitizer finding aborts the
program with its report, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tile_size_selection_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")

pytestmark = pytest.mark.skipif(not (shutil.which("gcc") and shutil.which("g++")), reason="gcc / g++ not found")


def _run(cmd, timeout=600, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=ENV, **kw)
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    return r


def _compile(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0 and ("libasan" in r.stderr or "libubsan" in r.stderr):
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr[-3000:]


def test_planner_entry_points_clean(tmp_path):
    exe = str(tmp_path / "plan_driver")
    _compile(["g++", "-std=c++20", *SAN, "-I", os.path.join(ROOT, "include"),
              os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"), os.path.join(CSRC, "planner.cpp"),
              "-o", exe])
    r = _run([exe])
    assert r.returncode == 0, (r.stdout, r.stderr[-3000:])
    assert "bad 0" in r.stdout


def test_planner_command_line_clean(tmp_path):
    obj = str(tmp_path / "tss_plan.o")
    exe = str(tmp_path / "tss_plan")
    _compile(["gcc", "-std=c11", *SAN, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, "tss_plan.c"),
              "-o", obj])
    _compile(["g++", "-std=c++20", *SAN, "-I", os.path.join(ROOT, "include"), obj,
              os.path.join(CSRC, "planner.cpp"), "-o", exe])
    ok = [["--topk", "8"], ["--device", "pages", "--topk", "8"], ["--m", "3000", "--n", "5000", "--k", "2048",
                                                                    "--batch", "4", "--topk", "300"],
          ["--diagnose", "--block-m", "256", "--block-n", "256", "--block-k", "64", "--stages", "2",
           "--threads", "512"],
          ["--device", "pages", "--diagnose", "--block-m", "256", "--block-n", "256", "--block-k", "64",
           "--stages", "4", "--threads", "256"],
          ["--device", "pages", "--instr", "simt", "--sm-count", "108", "--smem-kb", "164", "--m", "1", "--n", "1",
           "--k", "1"]]
    for args in ok:
        r = _run([exe, *args])
        assert r.returncode == 0, (args, r.stdout[-2000:], r.stderr[-2000:])
    for args in (["--m", "-5"], ["--instr", "bogus"], ["--device", "nope"], ["--topk"]):
        r = _run([exe, *args])
        assert r.returncode == 2, (args, r.returncode)


def test_oracle_clean(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _compile(["gcc", "-std=c11", *SAN, os.path.join(ROOT, "oracle", "gemm_conv.c"),
              os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"])
    r = _run([exe])
    assert r.returncode == 0, (r.stdout, r.stderr[-3000:])
