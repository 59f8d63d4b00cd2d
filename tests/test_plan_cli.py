"""The planner's command line (tss_plan, a C program over the C ABI): the
README page's commands give the output that page prints, token by token, and
the gfx950 mode lists the oracle's ranking.  No GPU involved."""
import os
import subprocess

import pytest

from oracle import planner as OP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLI = os.path.join(ROOT, "tile_size_selection_amd", "tss_plan")
GOLD = os.path.join(ROOT, "tests", "golden")


def _run(*args, rc=0):
    if not os.path.exists(CLI):
        pytest.fail(f"{CLI} is missing: build with python -m tile_size_selection_amd.build")
    r = subprocess.run([CLI, *args], capture_output=True, text=True, timeout=60)
    assert r.returncode == rc, (args, r.returncode, r.stderr)
    return r.stdout.splitlines()


def _gold(name):
    with open(os.path.join(GOLD, name), encoding="utf-8") as f:
        return [l.rstrip("\n") for l in f if l.strip() and not l.startswith("#")]


def _after(lines, prefix):
    got = [l for l in lines if l.strip().startswith(prefix)]
    assert len(got) == 1, (prefix, got)
    return got[0].strip()[len(prefix):].strip()


def _table(lines):
    i = next(i for i, l in enumerate(lines) if l.split()[:3] == ["block_M", "block_N", "block_K"])
    rows = []
    for l in lines[i + 1:]:
        if not l.strip():
            break
        rows.append(l.split())
    return rows


def _summary(lines):
    return (int(_after(lines, "feasible configurations found:")),
            int(_after(lines, "configurations tied at the minimum traffic:")),
            _after(lines, "best last-wave fill among feasible configurations:"))


def test_readme_sweep_printout():
    """tile_decision.py --topk 8 on the H100/H200 defaults: 459 feasible, the
    two rows the README page prints first, 8 tied at the least traffic, 94%."""
    out = _run("--device", "pages", "--topk", "8")
    gold = _gold("readme_sweep_topk8.txt")
    want = {l.split()[0]: l.split()[1:] for l in gold if not l.startswith("row ")}
    assert _summary(out) == (int(want["feasible"][0]), int(want["tied"][0]), want["best_fill"][0])
    rows = _table(out)
    assert len(rows) == 8
    for got, w in zip(rows, [l.split()[1:] for l in gold if l.startswith("row ")]):
        assert got == w


def test_readme_overbudget_diagnosis_printout():
    out = _run("--device", "pages", "--diagnose", "--block-m", "256", "--block-n", "256", "--block-k", "64",
               "--stages", "4", "--threads", "256")
    gold = _gold("readme_diagnose_overbudget.txt")
    got = [l.split() for l in out]
    for g in gold[:2]:
        assert g.split() in got, g
    occ = next(l for l in got if l[:1] == ["occupancy:"])
    want_occ = gold[2].split()
    assert occ[:len(want_occ) - 1] == want_occ[:-1]          # the page truncates this line ("...")
    assert [l for l in got if l[:1] == ["FAIL"]] == [g.split() for g in gold if g.startswith("FAIL")]
    assert not any(l[:1] == ["OK"] for l in got)


def test_readme_other_commands():
    """The README's other commands (outputs not printed on the page; the
    values are those of the page's listing, also pinned in the oracle's
    tests): the feasible diagnosis, the mma path and the A100 device."""
    out = _run("--device", "pages", "--diagnose", "--block-m", "128", "--block-n", "256", "--block-k", "64",
               "--stages", "3", "--threads", "256")
    got = [l.split() for l in out]
    assert ["OK", "all", "four", "constraints", "satisfied"] in got
    assert "binding=smem" in next(l for l in got if l[:1] == ["occupancy:"])
    c4 = next(l for l in got if l[:2] == ["C4", "grid"])
    assert c4[2] == "512" and c4[-2] == "87.9%"
    assert _summary(_run("--device", "pages", "--instr", "mma", "--topk", "8")) == (813, 8, "94%")
    out = _run("--device", "pages", "--sm-count", "108", "--smem-kb", "164", "--topk", "8")
    assert _summary(out) == (435, 7, "96%")
    first = _table(out)[0]
    assert first[9:11] == ["3", "37%"]


@pytest.mark.parametrize("shape", [(4096, 4096, 4096), (256, 6272, 2304), (4096, 4096, 72)])
def test_gfx950_sweep_lists_the_oracle_ranking(shape):
    m, n, k = shape
    out = _run("--m", str(m), "--n", str(n), "--k", str(k), "--topk", "40")
    g = OP.device_gfx950()
    res = OP.sweep(m, n, k, g, [s for s, _ in g.instr_shapes])
    rows = _table(out)
    assert len(rows) == min(40, len(res))
    for r, v in zip(rows, res):
        c = v.config
        assert [int(x) for x in r[:5]] == [c.block_m, c.block_n, c.block_k, c.stages, c.threads]
        assert r[-1] == c.instr and r[7] == str(v.regs_per_thread) and r[8] == str(v.blocks_per_core)
    assert int(_after(out, "feasible configurations found:")) == len(res)


def test_gfx950_diagnosis_is_the_oracle_verdict():
    for cfg in [OP.TileConfig(256, 256, 64, 2, 512, "mfma16"), OP.TileConfig(256, 256, 64, 3, 256, "mfma32"),
                OP.TileConfig(64, 64, 16, 2, 256, "mfma32"), OP.TileConfig(64, 64, 32, 2, 512, "mfma32"),
                OP.TileConfig(128, 128, 64, 2, 256, "mfma16")]:
        out = _run("--diagnose", "--block-m", str(cfg.block_m), "--block-n", str(cfg.block_n), "--block-k",
                   str(cfg.block_k), "--stages", str(cfg.stages), "--threads", str(cfg.threads), "--instr", cfg.instr,
                   "--m", "256", "--n", "6272", "--k", "2304")
        v = OP.diagnose(cfg, OP.device_gfx950(), 256, 6272)
        got = [l.split() for l in out]
        want = OP.diagnose_lines(v)
        for w in want:
            ws = w.split()
            if ws[0] in ("C1", "FAIL", "warn", "OK"):
                assert ws in got, (cfg, w)
            elif ws[0] == "C2":
                assert ws[:4] == next(l for l in got if l[:1] == ["C2"])[:4]


def test_bad_command_lines():
    _run("--instr", "wgmma", rc=2)                   # an NVIDIA shape on the gfx950 model
    _run("--device", "pages", "--instr", "mfma16", rc=2)
    _run("--sm-count", "108", rc=2)                  # the pages' device override without --device pages
    _run("--m", "x", rc=2)
    _run("--device", "tpu", rc=2)
    _run("stray", rc=2)
