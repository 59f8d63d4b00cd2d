"""Pins of the H-tile formulas and the intensity arithmetic to the Tiling page."""
import itertools
import os
from fractions import Fraction

from oracle import htile as H
from oracle import intensity as I

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLD, name), encoding="utf-8") as f:
        return [l.rstrip("\n") for l in f if l.strip() and not l.startswith("#")]


def test_worked_halo_example():
    lines = _lines("tiling_halo_example.txt")
    p = dict(kv.split("=") for kv in lines[0].split()[1:])
    Hh, kh, sh, pt, d, OH, toh = (int(p[k]) for k in ("H", "kh", "sh", "pt", "d", "OH", "tileOh"))
    table = H.tile_table(Hh, kh, sh, pt, d, OH, toh)
    tiles = [list(map(int, l.split()[1:])) for l in lines if l.startswith("tile ")]
    assert len(table) == len(tiles)
    for t, want in zip(table, tiles):
        o0, o1, s, e, span, ptp, pbp, first, last = want
        assert (t.o0, t.o1, t.in_start, t.in_end, t.in_span, t.pt, t.pb) == (o0, o1, s, e, span, ptp, pbp)
        assert (t.in_start, min(t.in_end, Hh) - 1) == (first, last)
    halo = int(next(l for l in lines if l.startswith("halo")).split()[1])
    assert all(t.halo == halo for t in table)
    # the shared row: x3 is the last row of tile A and the first of tile B
    assert table[0].in_end - 1 == table[1].in_start == 3


def test_conv_workload_tile_table():
    """8x256x56x56, 3x3, stride 2, pad 1, tileOh 8: 28 output rows, four tiles."""
    OH = H.out_size(56, 3, 2, 1, 1, 1)
    assert OH == 28
    t = H.tile_table(56, 3, 2, 1, 1, OH, 8)
    assert [(x.o0, x.o1) for x in t] == [(0, 8), (8, 16), (16, 24), (24, 28)]
    assert [(x.in_start, x.in_end) for x in t] == [(0, 16), (15, 32), (31, 48), (47, 56)]
    assert [x.pt for x in t] == [1, 0, 0, 0] and [x.pb for x in t] == [0, 0, 0, 0]
    assert t[0].halo == 1


def test_tiles_cover_every_window_brute_force():
    """For every small (H, kh, sh, pt, d, tile) the slice with pads pt'/pb'
    reproduces each output row's window, row for row, and yields exactly the
    tile's output rows.  Pads as tall as the window or taller are included:
    there a tile's windows can lie wholly in the padding; where the slice is
    empty (min(in_end, H) <= in_start) every tap is padding, and pt' +
    (min(in_end, H) - in_start) + pb' is still the window span."""
    n = n_empty = 0
    for Hh, kh, sh, pt, d in itertools.product(range(1, 12), (1, 2, 3, 5), (1, 2, 3), (0, 1, 2, 3, 4), (1, 2)):
        OH = H.out_size(Hh, kh, sh, pt, pt, d)
        if OH <= 0:
            continue
        for toh in range(1, OH + 1):
            for t in H.tile_table(Hh, kh, sh, pt, d, OH, toh):
                rows_in = min(t.in_end, Hh) - t.in_start
                sub_h = t.pt + rows_in + t.pb
                assert sub_h == (t.o1 - 1 - t.o0) * sh + H.window_rows(kh, d)
                assert (sub_h - H.window_rows(kh, d)) // sh + 1 == t.o1 - t.o0
                assert t.in_start - t.pt == t.o0 * sh - pt
                all_pad = all(not 0 <= o * sh - pt + r * d < Hh for o in range(t.o0, t.o1) for r in range(kh))
                if rows_in <= 0:                 # an empty slice: every tap is padding
                    assert all_pad               # (not conversely: dilated taps can straddle slice rows)
                    n_empty += 1
                for o in range(t.o0, t.o1):
                    for r in range(kh):
                        full = o * sh - pt + r * d                 # row in the unpadded image (may be pad)
                        sub = (o - t.o0) * sh + r * d              # row in the padded slice
                        if sub < t.pt:
                            src = None                            # top pad of the slice
                        elif sub < t.pt + rows_in:
                            src = t.in_start + sub - t.pt
                        else:
                            src = None                            # bottom pad of the slice
                        want = full if 0 <= full < Hh else None
                        assert src == want
                n += 1
    assert n > 2000 and n_empty > 100


def test_halo_sign_and_overlap():
    assert H.hw_tile(9, 3, 1, 1, 1, 0, 2).halo == 2      # stride 1: two rows overlap
    assert H.hw_tile(9, 3, 3, 1, 1, 0, 2).halo == 0      # stride = window: none
    assert H.hw_tile(9, 1, 2, 0, 1, 0, 2).halo == -1     # stride past the window: skipped rows
    assert H.hw_tile(9, 3, 1, 0, 2, 0, 2).halo == 4      # dilation 2 widens the window to 5


def test_intensity_numbers_from_page():
    vals = {l.split()[0]: l.split()[1:] for l in _lines("tiling_numbers.txt")}
    K, eb, want = vals["intensity_naive"]
    assert I.intensity_naive(int(K), int(eb)) == Fraction(want)
    bm, bn, eb, want = vals["intensity_tiled"]
    for K in (1, 32, 4096, 4097):
        assert I.intensity_tiled(int(bm), int(bn), K, int(eb)) == int(want)
    ratio = I.intensity_tiled(128, 128, 4096) / I.intensity_naive(4096)
    assert ratio == int(vals["intensity_ratio"][0])
    assert I.gemm_flops(4096, 4096, 4096) == 4096 * 4096 * 2 * 4096
