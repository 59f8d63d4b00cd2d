"""H-dimension tiling of a convolution: input slice, sub-operator pads, halo.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the "Tiling（分块）" page, section on the general H/W tiling formulas
(symbols H, kh, sh, pt, d, output rows [o0, o1)) and its item-by-item
explanation (1)..(5), with the worked example that follows it.  The extracted
text lost its '=', '+' and '-' signs; the reading used here is

    in_start = max(0, o0*sh - pt)
    in_end   = (o1 - 1)*sh - pt + (kh - 1)*d + 1          (exclusive)
    in_span  = in_end - in_start
    pt'      = max(0, pt - o0*sh)
    pb'      = max(0, in_end - H)
    halo     = (kh - 1)*d + 1 - sh

which reproduces every number of the worked example.  The slice handed to the
sub-operator is rows [in_start, min(in_end, H)) of the input, with pt' zero
rows above and pb' zero rows below it.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List


@dataclass(frozen=True)
class HSlice:
    o0: int
    o1: int
    in_start: int
    in_end: int
    in_span: int
    pt: int      # pt' of the sub-operator
    pb: int      # pb' of the sub-operator
    halo: int


def window_rows(kh: int, d: int) -> int:
    """Input rows one output row's window covers: (kh - 1)*d + 1."""
    return (kh - 1) * d + 1


def hw_tile(H: int, kh: int, sh: int, pt: int, d: int, o0: int, o1: int) -> HSlice:
    in_start = max(0, o0 * sh - pt)                      # (1) first window's start, clamped
    in_end = (o1 - 1) * sh - pt + window_rows(kh, d)     # (2) last window's start + its height
    pt_sub = max(0, pt - o0 * sh)                        # (3) top pad the slice still needs
    pb_sub = max(0, in_end - H)                          # (4) rows past the bottom of the image
    halo = window_rows(kh, d) - sh                       # (5) rows shared with the next tile
    return HSlice(o0, o1, in_start, in_end, in_end - in_start, pt_sub, pb_sub, halo)


def out_size(size: int, k: int, stride: int, pad_lo: int, pad_hi: int, d: int) -> int:
    """Output extent of a padded, strided, dilated window sweep."""
    return (size + pad_lo + pad_hi - window_rows(k, d)) // stride + 1


def tile_table(H: int, kh: int, sh: int, pt: int, d: int, OH: int, tile_oh: int) -> List[HSlice]:
    """Output rows [0, OH) cut into consecutive tiles of tile_oh rows (the
    last one ragged)."""
    return [hw_tile(H, kh, sh, pt, d, o0, min(o0 + tile_oh, OH)) for o0 in range(0, OH, tile_oh)]
