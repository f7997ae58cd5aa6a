"""Parity gates shared by the oracle self-tests and the GPU parity tests.

GEMM gate (a reading of "max relative error 1e-3"; a plain elementwise ratio
is ill-posed where an output cancels to near zero):
    max_i |y_i - ref_i| / max(|ref_i|, mean_j |ref_j|)  <=  tol
"""
from __future__ import annotations

import numpy as np

GEMM_TOL_F32 = 1e-3
# BF16 output adds its own rounding: nearest-even to BF16's 8 significant
# bits (7 stored mantissa bits) is off by at most half an ulp, 2^-8 of |y|,
# on top of the FP32 gate.
GEMM_TOL_BF16 = 2.0 ** -8 + 1e-3


def floored_rel_err(y, ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    floor = float(np.mean(np.abs(ref)))
    den = np.maximum(np.abs(ref), floor)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(y - ref) / den))


def normwise_rel_err(y, ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    return float(np.max(np.abs(y - ref)) / m) if m > 0 else float(np.max(np.abs(y - ref), initial=0.0))


def assert_gemm_close(y, ref, tol=GEMM_TOL_F32, what=""):
    e = floored_rel_err(y, ref)
    assert e <= tol, f"{what}: floored relative error {e:.3e} > {tol:.1e} (normwise {normwise_rel_err(y, ref):.3e})"
    return e
