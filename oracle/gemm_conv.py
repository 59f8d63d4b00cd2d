"""ctypes front end of the fp64 GEMM / convolution oracle (gemm_conv.c).

TEST INFRASTRUCTURE ONLY (see the package docstring).

``build()`` compiles gemm_conv.c with gcc into oracle/liboracle.so; nothing
of the product library is involved.  Arrays cross as contiguous float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

from . import htile

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_conv.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Plain IEEE double arithmetic: no fast-math, no fused multiply-add.
CFLAGS = ["-O3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11"]

_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        i64, dp, ip = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)
        L.oracle_gemm.argtypes = [i64, i64, i64, i64, dp, dp, dp, dp]
        L.oracle_gemm.restype = None
        L.oracle_gemm_entries.argtypes = [i64, i64, i64, dp, dp, i64, ip, ip, ip, dp, dp]
        L.oracle_gemm_entries.restype = None
        L.oracle_conv2d.argtypes = [i64] * 13 + [dp, dp, dp, dp]
        L.oracle_conv2d.restype = None
        L.oracle_conv2d_htiled.argtypes = [i64] * 14 + [ip, dp, dp, dp]
        L.oracle_conv2d_htiled.restype = ctypes.c_int
        L.oracle_conv2d_tiled.argtypes = [i64] * 14 + [ip, dp, dp, dp]
        L.oracle_conv2d_tiled.restype = ctypes.c_int
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: Optional[np.ndarray], t=ctypes.c_double):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(t))


def gemm(A, B, with_abs: bool = True) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """A: [batch,] M x K, B: [batch,] K x N  ->  C (and S = sum |a*b|), float64."""
    A, B = _f64(A), _f64(B)
    squeeze = A.ndim == 2
    if squeeze:
        A, B = A[None], B[None]
    bt, M, K = A.shape
    bt2, K2, N = B.shape
    assert bt == bt2 and K == K2
    C = np.empty((bt, M, N))
    S = np.empty((bt, M, N)) if with_abs else None
    lib().oracle_gemm(bt, M, N, K, _p(A), _p(B), _p(C), _p(S))
    if squeeze:
        return C[0], (S[0] if S is not None else None)
    return C, S


def gemm_entries(A, B, b: Sequence[int], i: Sequence[int], j: Sequence[int]):
    """Selected entries C[b][i][j] and S[b][i][j]."""
    A, B = _f64(A), _f64(B)
    if A.ndim == 2:
        A, B = A[None], B[None]
    _, M, K = A.shape
    N = B.shape[2]
    bb, ii, jj = (np.ascontiguousarray(np.asarray(v, dtype=np.int64)) for v in (b, i, j))
    n = bb.size
    C, S = np.empty(n), np.empty(n)
    lib().oracle_gemm_entries(M, N, K, _p(A), _p(B), n, _p(bb, ctypes.c_int64), _p(ii, ctypes.c_int64),
                              _p(jj, ctypes.c_int64), _p(C), _p(S))
    return C, S


def conv_out_shape(N, Co, H, W, kh, kw, sh, sw, ph, pw, dh, dw):
    return (N, Co, htile.out_size(H, kh, sh, ph, ph, dh), htile.out_size(W, kw, sw, pw, pw, dw))


def conv2d(x, w, stride=(1, 1), pad=(0, 0), dil=(1, 1), with_abs: bool = True):
    x, w = _f64(x), _f64(w)
    N, Ci, H, W = x.shape
    Co, Ci2, kh, kw = w.shape
    assert Ci == Ci2
    (sh, sw), (ph, pw), (dh, dw) = stride, pad, dil
    y = np.empty(conv_out_shape(N, Co, H, W, kh, kw, sh, sw, ph, pw, dh, dw))
    S = np.empty(y.shape) if with_abs else None
    lib().oracle_conv2d(N, Ci, H, W, Co, kh, kw, sh, sw, ph, pw, dh, dw, _p(x), _p(w), _p(y), _p(S))
    return y, S


def conv2d_htiled(x, w, stride=(1, 1), pad=(0, 0), dil=(1, 1), tile_oh: int = 8):
    """The same convolution assembled from H-tiles whose slices and pads come
    from oracle.htile (the Tiling page's formulas)."""
    x, w = _f64(x), _f64(w)
    N, Ci, H, W = x.shape
    Co, _, kh, kw = w.shape
    (sh, sw), (ph, pw), (dh, dw) = stride, pad, dil
    shape = conv_out_shape(N, Co, H, W, kh, kw, sh, sw, ph, pw, dh, dw)
    table = htile.tile_table(H, kh, sh, ph, dh, shape[2], tile_oh)
    tiles = np.ascontiguousarray(np.array([[t.o0, t.o1, t.in_start, t.in_end, t.pt, t.pb] for t in table],
                                          dtype=np.int64).reshape(-1, 6))
    y = np.full(shape, np.nan)
    rc = lib().oracle_conv2d_htiled(N, Ci, H, W, Co, kh, kw, sh, sw, ph, pw, dh, dw, len(table),
                                    _p(tiles, ctypes.c_int64), _p(x), _p(w), _p(y))
    if rc != 0:
        raise RuntimeError(f"H-tile slice table is inconsistent (rc={rc})")
    return y


def conv2d_tiled(x, w, stride=(1, 1), pad=(0, 0), dil=(1, 1), tile_oh: int = 8, tile_ow: Optional[int] = None,
                 tile_n: Optional[int] = None):
    """The same convolution assembled from tiles of tile_n images x tile_oh
    output rows x tile_ow output columns.  Rows and columns each take their
    slice and pads from oracle.htile (the Tiling page's H/W formulas, applied
    to (H, kh, sh, ph, dh) and to (W, kw, sw, pw, dw)); images split with no
    halo.  tile_ow / tile_n default to the whole width / batch."""
    x, w = _f64(x), _f64(w)
    N, Ci, H, W = x.shape
    Co, _, kh, kw = w.shape
    (sh, sw), (ph, pw), (dh, dw) = stride, pad, dil
    shape = conv_out_shape(N, Co, H, W, kh, kw, sh, sw, ph, pw, dh, dw)
    tile_ow = shape[3] if tile_ow is None else tile_ow
    tile_n = N if tile_n is None else tile_n
    rows = htile.tile_table(H, kh, sh, ph, dh, shape[2], tile_oh)
    cols = htile.tile_table(W, kw, sw, pw, dw, shape[3], tile_ow)
    table = [[n0, min(n0 + tile_n, N), r.o0, r.o1, r.in_start, r.in_end, r.pt, r.pb,
              c.o0, c.o1, c.in_start, c.in_end, c.pt, c.pb]
             for n0 in range(0, N, tile_n) for r in rows for c in cols]
    tiles = np.ascontiguousarray(np.array(table, dtype=np.int64).reshape(-1, 14))
    y = np.full(shape, np.nan)
    rc = lib().oracle_conv2d_tiled(N, Ci, H, W, Co, kh, kw, sh, sw, ph, pw, dh, dw, len(table),
                                   _p(tiles, ctypes.c_int64), _p(x), _p(w), _p(y))
    if rc != 0:
        raise RuntimeError(f"tile slice table is inconsistent (rc={rc})")
    return y


def threads() -> int:
    """OpenMP threads the oracle loops use."""
    return int(lib().oracle_threads())
