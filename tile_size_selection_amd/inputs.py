"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws numbers: it holds none of the GEMM / conv / planner
arithmetic, and imports neither the HIP library nor the oracle.

Recipe: values are drawn in float64 with ``numpy.random.default_rng(seed)``,
narrowed to float32 and then rounded to nearest-even into fp16 or bf16 (by
torch's own conversion).  Both the device path and the oracle receive exactly
these rounded values (the oracle widens them to float64, which is exact).
Workload *i* uses seed ``1000*i + t`` with t = 0 for A / x and t = 1 for B / w.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def seed_for(workload: int, tensor: int) -> int:
    return 1000 * workload + tensor


def draw(shape, dist: str, a: float, b: float, dtype: str, seed: int) -> torch.Tensor:
    """dist 'uniform': U[a, b];  'normal': mean a, standard deviation b;
    'int': integers uniform on [a, b] inclusive (exact in fp16 and bf16 for
    |v| <= 256)."""
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        v = rng.uniform(a, b, size=shape)
    elif dist == "normal":
        v = rng.normal(a, b, size=shape)
    elif dist == "int":
        v = rng.integers(int(a), int(b) + 1, size=shape).astype(np.float64)
    else:
        raise ValueError(dist)
    return torch.from_numpy(v.astype(np.float32)).to(DTYPES[dtype])


@dataclass(frozen=True)
class GemmWorkload:
    index: int
    name: str
    dtype: str
    out_dtype: str
    batch: int
    M: int
    N: int
    K: int
    dist: Tuple[str, float, float]

    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K

    def make(self, dist: Optional[Tuple[str, float, float]] = None, seed_offset: int = 0):
        d = dist or self.dist
        shA = (self.batch, self.M, self.K) if self.batch > 1 else (self.M, self.K)
        shB = (self.batch, self.K, self.N) if self.batch > 1 else (self.K, self.N)
        A = draw(shA, d[0], d[1], d[2], self.dtype, seed_for(self.index, 0) + seed_offset)
        B = draw(shB, d[0], d[1], d[2], self.dtype, seed_for(self.index, 1) + seed_offset)
        return A, B


@dataclass(frozen=True)
class ConvWorkload:
    index: int
    name: str
    dtype: str
    out_dtype: str
    N: int
    C: int
    H: int
    W: int
    Co: int
    kh: int
    kw: int
    stride: Tuple[int, int]
    pad: Tuple[int, int]
    dil: Tuple[int, int]
    tile_oh: int
    x_dist: Tuple[str, float, float]
    w_dist: Tuple[str, float, float]

    def make(self, seed_offset: int = 0):
        x = draw((self.N, self.C, self.H, self.W), *self.x_dist, self.dtype, seed_for(self.index, 0) + seed_offset)
        w = draw((self.Co, self.C, self.kh, self.kw), *self.w_dist, self.dtype, seed_for(self.index, 1) + seed_offset)
        return x, w


U11 = ("uniform", -1.0, 1.0)

WORKLOADS = {
    1: GemmWorkload(1, "gemm_f16_256", "f16", "f32", 1, 256, 256, 256, U11),
    2: GemmWorkload(2, "gemm_f16_4096", "f16", "f16", 1, 4096, 4096, 4096, U11),
    3: GemmWorkload(3, "gemm_f16_b4_3000x5000x2048", "f16", "f32", 4, 3000, 5000, 2048, ("normal", 0.0, 0.5)),
    4: GemmWorkload(4, "gemm_bf16_8192", "bf16", "bf16", 1, 8192, 8192, 8192, U11),
    5: ConvWorkload(5, "conv_f16_n8c256h56_k3s2p1", "f16", "f32", 8, 256, 56, 56, 256, 3, 3, (2, 2), (1, 1),
                    (1, 1), 8, U11, ("normal", 0.0, 0.05)),
}
