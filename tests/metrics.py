"""Comparison metrics between GPU results and the fp64 oracle.

Output tolerance.  The outputs are bf16, so even an exactly computed value
rounded to bf16 differs from the fp64 reference by up to half a bf16 ulp,
which exceeds 2e-2 once |y| >= 8 (ulp 2^-4).  The output error is therefore
measured beyond that unavoidable rounding:
    e_out = max_i max(0, |y_gpu - y_ref| - ulp_bf16(max(|y_ref|, |y_gpu|)) / 2)
and must stay <= 2e-2.  The literal max-abs error is reported beside it.

State tolerance.  e_state = max over chains of ||S_gpu - S_ref||_F / ||S_ref||_F
(relative error per head; element-wise relative error is undefined near 0),
which must stay <= 1e-3.
"""
from __future__ import annotations

import numpy as np

OUT_TOL = 2e-2
STATE_TOL = 1e-3


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def out_errors(y_gpu: np.ndarray, y_ref: np.ndarray) -> dict:
    d = np.abs(y_gpu - y_ref)
    half = 0.5 * ulp_bf16(np.maximum(np.abs(y_ref), np.abs(y_gpu)))
    beyond = np.maximum(0.0, d - half)
    return {"e_out": float(beyond.max()) if beyond.size else 0.0,
            "max_abs": float(d.max()) if d.size else 0.0,
            "n_large": int((np.abs(y_ref) >= 8).sum()),
            "nonfinite": int((~np.isfinite(y_gpu)).sum())}


def state_error(S_gpu: np.ndarray, S_ref: np.ndarray) -> float:
    """S arrays [n, dk, dv]."""
    num = np.sqrt(((S_gpu.astype(np.float64) - S_ref) ** 2).sum(axis=(1, 2)))
    den = np.sqrt((S_ref ** 2).sum(axis=(1, 2)))
    return float(np.max(num / np.maximum(den, 1e-300)))
