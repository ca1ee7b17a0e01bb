"""Brute-force checker for the oracle, written from a different formulation.

Used only by the CPU pin tests.  It shares nothing with the oracle:
  * candidate scale values come from torch's float8_e4m3fn decoder;
  * the E2M1 cast is a midpoint/threshold table built from the golden grid
    (tests/golden/e2m1_grid.txt), not a nearest-value search;
  * the block error is the output error itself, ||dw^T X_b||^2 / N, taken
    straight from the activations and never forming H (the block-diagonal
    objective of the Local-Hessian weight-scale guide, "Algorithm principle":
    E_b = Delta_b X_b X_b^T Delta_b^T = ||Delta_b X_b||^2).
"""
from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_grid() -> np.ndarray:
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_grid.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, mag = line.split()
            vals[int(code)] = float(mag)
    return np.array([vals[c] for c in range(len(vals))], np.float64)


def load_format() -> dict:
    out = {}
    with open(os.path.join(GOLDEN, "nvfp4_format.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = float(v)
    return out


GRID = load_grid()
MIDPOINTS = (GRID[:-1] + GRID[1:]) / 2.0  # 0.25 0.75 1.25 1.75 2.5 3.5 5


def e4m3_candidates() -> np.ndarray:
    """The positive finite non-zero E4M3FN values, ascending (torch decoder)."""
    v = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    keep = np.isfinite(v) & (v > 0)
    return np.sort(v[keep]).astype(np.float32)


def cast_codes(x: np.ndarray) -> np.ndarray:
    """E2M1 magnitude code of x >= 0 (fp32) by counting passed midpoints;
    at an exact midpoint the even code wins; beyond the grid saturates."""
    x64 = np.asarray(x, np.float64)
    code = np.zeros(x64.shape, np.int64)
    for c, m in enumerate(MIDPOINTS):
        upper_is_even = (c + 1) % 2 == 0
        code += (x64 > m) | ((x64 == m) & upper_is_even)
    return code


def scales(g: float) -> np.ndarray:
    sg = np.float32(g) / np.float32(2688.0)
    return (e4m3_candidates() * sg).astype(np.float32)


def quantize(w: np.ndarray, s: np.float32) -> np.ndarray:
    """fp32 Q = sign(w) * r * s with x = fl32(|w| / s)."""
    w = np.asarray(w, np.float32)
    s = np.float32(s)
    if s == 0:
        return np.zeros_like(w)
    with np.errstate(over="ignore"):
        x = np.abs(w) / s
    r = GRID[cast_codes(x)].astype(np.float32)
    q = (r * s).astype(np.float32)
    q = np.where(w < 0, -q, q)
    return q + np.float32(0.0)  # -0 -> +0


def block_errors_from_x(w16: np.ndarray, xb: np.ndarray, g: float) -> np.ndarray:
    """E_k = ||dw_k^T X_b||^2 / N for all 126 candidates (fp64)."""
    w16 = np.asarray(w16, np.float32)
    xb = np.asarray(xb, np.float64)
    n = xb.shape[1]
    s = scales(g)
    out = np.empty(len(s))
    for k, sk in enumerate(s):
        dw = quantize(w16, sk).astype(np.float64) - w16.astype(np.float64)
        y = dw @ xb
        out[k] = float(y @ y) / n
    return out


def block_errors_mse(w16: np.ndarray, g: float) -> np.ndarray:
    """Plain weight MSE sweep (sum of dw^2), the H = I special case."""
    w16 = np.asarray(w16, np.float32)
    s = scales(g)
    out = np.empty(len(s))
    for k, sk in enumerate(s):
        dw = quantize(w16, sk).astype(np.float64) - w16.astype(np.float64)
        out[k] = float(dw @ dw)
    return out


def argmin_lowest(e: np.ndarray) -> int:
    return int(np.flatnonzero(e == e.min())[0])
