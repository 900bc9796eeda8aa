"""Small helpers shared by the GPU tests: tensor transfer, error metrics and
the tolerances the parity tests use.

Tolerances (relative L2 error over a whole tensor, in fp64):
  fp32 activations:  1e-4 on outputs and final states
  bf16 activations:  1e-2 on outputs, 5e-3 on final states
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL_F32 = 1e-4
TOL_BF16_OUT = 1e-2
TOL_BF16_STATE = 5e-3


def say(*a):
    """Print and flush, so a failing GPU step names its case."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.linalg.norm((x - ref).ravel())
    n = np.linalg.norm(ref.ravel())
    return float(d / n) if n > 0 else float(d)


# Both kernels keep the recurrent state in fp32 and form its products to about
# fp32 accuracy, so every (sequence, head) state must match the oracle far
# more tightly than the whole-tensor bf16 tolerance; a per-chain bound catches
# errors confined to a few chains that a whole-tensor norm would average away.
TOL_STATE_PER_CHAIN = 1e-4


def per_chain_max(x, ref) -> float:
    """Largest relative L2 error over the leading two axes (sequence, head)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    a = x.reshape(x.shape[0] * x.shape[1], -1)
    b = ref.reshape(a.shape)
    d = np.linalg.norm(a - b, axis=1)
    n = np.linalg.norm(b, axis=1)
    return float(np.max(np.where(n > 0, d / np.maximum(n, 1e-300), d))) if len(n) else 0.0


# Worst (token, head) output row: the whole-tensor norm can hide one wrong
# row among a million; every row must stay within these relative errors
# (bf16 outputs are rounded to 8 significant bits, about 4e-3 per element).
TOL_ROW_F32 = 1e-3
TOL_ROW_BF16 = 5e-2


def per_row_max(x, ref, row_axes: int = 2) -> float:
    """Largest relative L2 error over rows of the last axis grouped by the
    leading `row_axes` axes (for outputs [T][H][dv]: one row per token and
    head).  A row whose reference is zero counts its absolute error."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    n_rows = int(np.prod(x.shape[:row_axes])) if x.ndim else 0
    if n_rows == 0:
        return 0.0
    a = x.reshape(n_rows, -1)
    b = ref.reshape(a.shape)
    d = np.linalg.norm(a - b, axis=1)
    n = np.linalg.norm(b, axis=1)
    return float(np.max(np.where(n > 0, d / np.maximum(n, 1e-300), d)))


def tol_row(act: str) -> float:
    return TOL_ROW_F32 if act == "f32" else TOL_ROW_BF16


def tols(act: str):
    if act == "f32":
        return TOL_F32, TOL_F32
    return TOL_BF16_OUT, TOL_BF16_STATE


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bytes of a tensor, for bitwise comparisons."""
    return t.detach().contiguous().cpu().view(torch.uint8).numpy().copy()
