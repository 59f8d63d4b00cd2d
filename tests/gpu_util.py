"""Shared helpers of the GPU parity tests."""
import numpy as np
import torch

# Per-element bound on the GPU result against the fp64 oracle:
#   |gpu - oracle| <= 5e-3 * sum_k |a_ik * b_kj| + 1e-3
REL, ABS = 5e-3, 1e-3


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_bound(got: np.ndarray, ref: np.ndarray, S: np.ndarray, what: str = ""):
    err = np.abs(got - ref)
    bound = REL * S + ABS
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of bound; first at "
                             f"{idx.tolist()}: got {got[bad][:5]}, want {ref[bad][:5]}")
    return float((err / bound).max()) if err.size else 0.0


def sample_indices(shape, n, rng, edges=True):
    """n random (b, i, j) triples plus the corners and last row / column of
    every batch (where ragged tiles live)."""
    bt, M, N = shape
    b = rng.integers(0, bt, n)
    i = rng.integers(0, M, n)
    j = rng.integers(0, N, n)
    if edges:
        eb, ei, ej = [], [], []
        for bb in range(bt):
            for ii in (0, M - 1):
                for jj in (0, N - 1):
                    eb.append(bb); ei.append(ii); ej.append(jj)
            cols = rng.integers(0, N, 16)
            rows = rng.integers(0, M, 16)
            eb += [bb] * 32
            ei += [M - 1] * 16 + list(rows)
            ej += list(cols) + [N - 1] * 16
        b = np.concatenate([b, eb]); i = np.concatenate([i, ei]); j = np.concatenate([j, ej])
    return b.astype(np.int64), i.astype(np.int64), j.astype(np.int64)
