"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances (max-abs): bf16 inputs with fp32 accumulation; fp32 end to end.
TOL_BF16_OUT = 2e-2
TOL_BF16_LSE = 1e-3
TOL_F32 = 1e-5


def to_gpu(*ts):
    return [t.to("cuda") for t in ts]


def max_abs(gpu_t, ref: np.ndarray) -> float:
    g = gpu_t.detach().float().cpu().double().numpy()
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


def sample_rows(cu, stride: int = 8):
    """Every stride-th packed row plus the first and last row of every sequence (sorted)."""
    cu = [int(x) for x in cu]
    T = cu[-1]
    rows = set(range(0, T, stride))
    for i in range(len(cu) - 1):
        if cu[i + 1] > cu[i]:
            rows.add(cu[i])
            rows.add(cu[i + 1] - 1)
    return np.array(sorted(rows), dtype=np.int64)


def lse_close(gpu_lse, ref: np.ndarray, tol: float) -> float:
    """Max-abs error of an lse tensor, treating matching -inf entries as exact."""
    g = gpu_lse.detach().float().cpu().double().numpy()
    both_inf = np.isneginf(g) & np.isneginf(ref)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), "-inf pattern differs"
    d = np.where(both_inf, 0.0, np.abs(g - np.where(both_inf, 0.0, ref)))
    err = float(np.max(d)) if d.size else 0.0
    assert err <= tol, err
    return err


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers at |ref| (8 significand bits): the rounding any bf16
    result of ref must carry, on top of the arithmetic error."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def fp32_close(gpu_t, ref: np.ndarray, tol: float = TOL_BF16_OUT) -> float:
    """Plain max-abs check of an fp32 result (no rounding slack: nothing is rounded to bf16)."""
    g = gpu_t.detach().float().cpu().double().numpy()
    err = float(np.max(np.abs(g - ref))) if g.size else 0.0
    assert err <= tol, err
    return err


def boundary_rows(n: int, stride: int = 8, extra=()):
    """Every stride-th row of 0..n-1, the rows on either side of every 64-row and 128-row tile
    edge, the first and last row, and any extra rows (sorted, unique)."""
    rows = set(range(0, n, stride))
    for e in range(0, n + 1, 64):
        rows.update((e - 1, e))
    rows.update((0, n - 1))
    rows.update(int(x) for x in extra)
    return np.array(sorted(r for r in rows if 0 <= r < n), dtype=np.int64)


def grad_close(gpu_t, ref: np.ndarray, tol: float = TOL_BF16_OUT, mean_tol: float = 2e-3):
    """bf16 gradient check: |gpu - ref| <= tol + half a bf16 ulp of ref everywhere, and the mean
    error stays small.  Returns (max error, max error beyond the half ulp, mean error)."""
    g = gpu_t.detach().float().cpu().double().numpy()
    err = np.abs(g - ref)
    over = err - bf16_half_ulp(ref)
    worst = float(np.max(over)) if over.size else 0.0
    mean = float(np.mean(err)) if err.size else 0.0
    assert worst <= tol, (float(np.max(err)), worst)
    assert mean <= mean_tol, mean
    return float(np.max(err)) if err.size else 0.0, worst, mean
