"""Arithmetic intensity (FLOPs per byte moved from global memory) of GEMM.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the "Tiling（分块）" page, its numerical example for a 4096^3 fp16
GEMM and the derivation that follows ("案例解释"): every C element costs 2K
FLOPs; computed one element per thread it reads a row of A and a column of B
(2K elements); computed as a BM x BN tile it reads a BM x K panel of A and a
K x BN panel of B once for BM*BN elements, so K cancels.
All results are exact rationals.
"""
from __future__ import annotations

from fractions import Fraction


def flops_per_element(K: int) -> int:
    return 2 * K


def intensity_naive(K: int, elem_bytes: int = 2) -> Fraction:
    """One thread per C[i, j]: 2K FLOPs over 2K elements read."""
    return Fraction(flops_per_element(K), 2 * K * elem_bytes)


def intensity_tiled(BM: int, BN: int, K: int, elem_bytes: int = 2) -> Fraction:
    """One block per BM x BN tile: BM*BN*2K FLOPs over (BM + BN)*K elements."""
    return Fraction(BM * BN * flops_per_element(K), (BM + BN) * K * elem_bytes)


def gemm_flops(M: int, N: int, K: int, batch: int = 1) -> int:
    return batch * M * N * flops_per_element(K)
