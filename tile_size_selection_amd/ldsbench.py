"""LDS bank table of gfx950, measured (tss_lds_probe): the counterpart of the
"Tiling（分块）" page's shared-memory bank-conflict table (access stride ->
conflict factor) and of its XOR swizzle, with the GEMM kernel's own fragment
reads beside the plain strides.

    python -m tile_size_selection_amd.ldsbench [--out profiles/lds_banks.md]

For each pattern: shader-clock cycles per read instruction of one wave (the
median over 256 blocks x 8 waves, 8 waves per CU reading concurrently) and the
factor against the contiguous read of the same width.
"""
from __future__ import annotations

import argparse
import sys

from . import api

# (pattern, stride in 4-byte words, the contiguous pattern it is compared with)
ROWS = [("b32", 1, ("b32", 1)), ("b32", 2, ("b32", 1)), ("b32", 4, ("b32", 1)), ("b32", 8, ("b32", 1)),
        ("b32", 16, ("b32", 1)), ("b32", 32, ("b32", 1)), ("b32", 64, ("b32", 1)), ("b32", 65, ("b32", 1)),
        ("b128", 4, ("b128", 4)), ("b128", 8, ("b128", 4)), ("b128", 16, ("b128", 4)), ("b128", 32, ("b128", 4)),
        ("b128", 64, ("b128", 4)),
        ("tr_b64", 2, ("tr_b64", 2)), ("tr_b64", 64, ("tr_b64", 2)),
        ("gemm_a", 0, ("b128", 4)), ("gemm_a_plain", 0, ("b128", 4)),
        ("gemm_b", 0, ("tr_b64", 2)), ("gemm_b_plain", 0, ("tr_b64", 2))]

WHAT = {"b32": "ds_read_b32", "b128": "ds_read_b128", "tr_b64": "ds_read_b64_tr_b16",
        "gemm_a": "GEMM A fragment, swizzled (ds_read_b128)", "gemm_a_plain": "GEMM A fragment, no swizzle",
        "gemm_b": "GEMM B fragment, swizzled (ds_read_b64_tr_b16)", "gemm_b_plain": "GEMM B fragment, no swizzle"}


def measure(iters: int = 2000, blocks: int = 256):
    cache = {}

    def cyc(p, s):
        if (p, s) not in cache:
            cache[(p, s)] = api.lds_probe(p, s, iters=iters, blocks=blocks)
        return cache[(p, s)]

    api.lds_probe("b32", 1, iters=100, blocks=blocks)  # warm-up launch
    out = []
    for p, s, ref in ROWS:
        c = cyc(p, s)
        out.append({"pattern": p, "stride_words": s, "cycles": c, "factor": c / cyc(*ref), "ref": ref})
    return out


def report(rows) -> str:
    lines = ["| read | lane stride (4-byte words) | cycles per wave instruction | factor vs contiguous |",
             "|---|---|---|---|"]
    for r in rows:
        stride = "—" if r["pattern"].startswith("gemm") else str(r["stride_words"])
        lines.append(f"| {WHAT[r['pattern']]} | {stride} | {r['cycles']:.2f} | {r['factor']:.2f} |")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--out", default=None)
    ap.add_argument("--iters", type=int, default=2000)
    a = ap.parse_args(argv)
    rows = measure(a.iters)
    txt = ("# LDS bank table (gfx950), measured\n\n"
           "Command (repository root, MI355X): `python3 -m tile_size_selection_amd.ldsbench"
           + (f" --out {a.out}" if a.out else "") + "`\n\n"
           "Each row: lane l of every wave reads at byte l x stride x 4 (or the GEMM kernel's fragment address),"
           f" {a.iters} x 8 reads per wave, 256 blocks of 8 waves; cycles are the shader clock (s_memtime),"
           " median over all waves.\n\n" + report(rows) + "\n")
    print(txt, flush=True)
    if a.out:
        with open(a.out, "w", encoding="utf-8") as f:
            f.write(txt)
    return 0


if __name__ == "__main__":
    sys.exit(main())
