"""Parity metrics.  TEST INFRASTRUCTURE ONLY.

per-row relative L2:  relL2[m] = ||y[m] - ref[m]||_2 / ||ref[m]||_2
                      (absolute ||y[m] - ref[m]||_2 for an all-zero ref row)
max abs:              max |y - ref|

For outputs stored in bf16 the max-abs bound is widened per element by half
a bf16 unit in the last place of |ref| (the rounding the output store itself
must make); the relative-L2 bound is not widened.
"""

from __future__ import annotations

import numpy as np


def _half_ulp_bf16(a: np.ndarray) -> np.ndarray:
    a = np.abs(a)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    # bf16 spacing in [2**(e-1), 2**e) is 2**(e-8); half of it is 2**(e-9)
    return np.where(a > 0, np.ldexp(1.0, np.maximum(e - 9, -134)), np.ldexp(1.0, -134))


def row_metrics(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = y - ref
    num = np.sqrt(np.sum(d * d, axis=-1))
    den = np.sqrt(np.sum(ref * ref, axis=-1))
    rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return rel, np.abs(d)


def check_close(y, ref, rel_l2: float, max_abs: float, out_is_bf16: bool = False):
    """Return (ok, info).  NaNs in ref must be matched by NaNs in y."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    nan_ref = np.isnan(ref)
    nan_ok = bool(np.array_equal(nan_ref, np.isnan(y)))
    finite_rows = ~np.any(nan_ref, axis=-1) if ref.ndim > 1 else ~nan_ref
    yf = np.where(nan_ref, 0.0, y)
    rf = np.where(nan_ref, 0.0, ref)
    rel, ad = row_metrics(yf, rf)
    bound = np.full(ref.shape, float(max_abs))
    if out_is_bf16:
        bound = bound + _half_ulp_bf16(rf)
    excess = ad - bound
    info = {
        "max_rel_l2": float(np.max(rel[finite_rows])) if np.any(finite_rows) else 0.0,
        "max_abs": float(np.max(ad)) if ad.size else 0.0,
        "worst_abs_excess": float(np.max(excess)) if ad.size else -1.0,
        "nan_pattern_ok": nan_ok,
        "nonfinite_y": int(np.sum(~np.isfinite(y) & ~nan_ref)),
    }
    ok = (nan_ok and info["nonfinite_y"] == 0 and info["max_rel_l2"] <= rel_l2
          and info["worst_abs_excess"] <= 0.0)
    return ok, info
