"""Helpers shared by the GPU parity tests: move seeded inputs to the GPU,
compute oracle references, compare.  The oracle only ever sees the seeded
inputs from ``synth``; nothing computed on the GPU flows into it."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import BF16, F32, stored_to_f64

# Tolerances (FlashNorm parity targets): per-row relative L2 and max abs.
BF16_REL_L2 = 5e-3
BF16_MAX_ABS = 3e-2
F32_REL_L2 = 1e-5
# Kernel-only pin against the deferred form on the same folded operands:
# fp32 accumulation of K products in an unspecified order has a typical
# relative error of about sqrt(K) * 2^-24 (4e-6 at K = 4096), plus the
# float32 reciprocal square root and sum of squares (~1e-7).
KERNEL_REL_L2 = 2e-5


def to_dev(arr: np.ndarray, device="cuda") -> torch.Tensor:
    """Stored numpy tensor (float32 or bf16 bits) -> GPU tensor, same bits."""
    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def from_dev(t: torch.Tensor) -> np.ndarray:
    """GPU output -> float64 numpy (exact)."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def bits_of(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().cpu().numpy().view(np.uint32)


def assert_parity(y_gpu: torch.Tensor, ref: np.ndarray, dtype: str, label: str, out_bf16: bool = False,
                  rel_l2=None, max_abs=None):
    y = from_dev(y_gpu)
    if dtype == F32:
        rl = F32_REL_L2 if rel_l2 is None else rel_l2
        ok, info = oracle.check_close(y, ref, rl, np.inf if max_abs is None else max_abs)
    else:
        rl = BF16_REL_L2 if rel_l2 is None else rel_l2
        ma = BF16_MAX_ABS if max_abs is None else max_abs
        ok, info = oracle.check_close(y, ref, rl, ma, out_is_bf16=out_bf16)
    print(f"[parity] {label}: {info}", flush=True)
    assert ok, f"{label}: {info}"
    return info


def f64(a):
    return stored_to_f64(a) if isinstance(a, np.ndarray) and a.dtype == np.uint16 else np.asarray(a, np.float64)


U32 = 2.0 ** -24


def deferred_bound(x, Ws, eps):
    """Elementwise bound on |fused float32 result - exact deferred form on the
    same folded operands|: a float32 dot product of K terms errs by at most
    about K * u * sum_k |x_k w_k| (u = 2^-24), and the float32 sum of squares
    and reciprocal square root add about K/2 * u + a few u relative."""
    xf, Wf = f64(x), f64(Ws)
    K = xf.shape[1]
    s = 1.0 / oracle.rms(x, eps)
    mag = (np.abs(xf) @ np.abs(Wf).T) * s[:, None]
    return (1.5 * K + 8) * U32 * mag


def assert_within(y_gpu, ref, bound, label):
    y = from_dev(y_gpu)
    excess = np.abs(y - ref) - bound
    worst = float(np.max(excess)) if excess.size else -1.0
    print(f"[bound] {label}: worst excess {worst:.3e}, max bound {float(np.max(bound)):.3e}", flush=True)
    assert np.all(np.isfinite(y)) and worst <= 0.0, f"{label}: worst excess {worst}"


def glu_bound(x, Wg, Wu, eps):
    """Propagate the dot-product bounds of a and b through SiLU(a) * b
    (|SiLU'| < 1.1 everywhere), plus float32 rounding of the epilogue."""
    a = oracle.deferred_on_folded(x, Wg, eps)
    b = oracle.deferred_on_folded(x, Wu, eps)
    Ba, Bb = deferred_bound(x, Wg, eps), deferred_bound(x, Wu, eps)
    h = oracle.silu(a) * b
    return 1.1 * np.abs(b) * Ba + np.abs(oracle.silu(a)) * Bb + 1.1 * Ba * Bb + 8 * U32 * np.abs(h) + 1e-30


def e4m3_step(v):
    """Spacing of the E4M3 values around |v| (v in code units, |v| <= 448):
    2^(e-3) in the binade [2^e, 2^(e+1)), 2^-9 below 2^-6."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.exp2(e - 3)


def fp8_act_bounds(x, codes_w, q_w, eps):
    """References and elementwise bounds for the fp8-activation product.

    Kernel-only: the deferred form on the oracle's own codes of x (which the
    GPU reproduces bit for bit) with a float32 accumulation bound, (1.5 K +
    8) u times the sum of |product| terms, u = 2^-24, plus a few u of the
    scale products.  Textbook: quantising RMSNorm(x) instead of x resolves
    exact E4M3 ties (frequent for bf16 inputs) by the float32 rounding of a
    different scale, so a code may differ by one step; the bound adds one
    step (times the scale and |w|) for each element whose two codes differ,
    and 2^-22 relative for the two scales' roundings.  Returns (ref_k,
    bound_k, ref_t, bound_t, flips)."""
    xf = f64(x)
    K = xf.shape[1]
    s = 1.0 / oracle.rms(x, eps)
    cx, qx = oracle.quantize_fp8_per_channel(x)
    xn = oracle.rmsnorm(x, np.ones(K), eps)
    cxn, qxn = oracle.quantize_fp8_per_channel(xn)
    Wd = np.abs(oracle.dequantize_fp8(codes_w, q_w))
    dx = np.abs(oracle.dequantize_fp8(cx, qx)) * s[:, None]
    ref_k = oracle.deferred_fp8_act(x, codes_w, q_w, eps)
    bound_k = (1.5 * K + 8) * U32 * (dx @ Wd.T) + 8 * U32 * np.abs(ref_k)
    ref_t = oracle.norm_linear_fp8_act(x, codes_w, q_w, eps)
    flip = cx != cxn
    vals = np.maximum(np.abs(oracle.e4m3_value(cx)), np.abs(oracle.e4m3_value(cxn)))
    step = np.where(flip, e4m3_step(vals) * qxn[:, None].astype(np.float64), 0.0)
    bound_t = bound_k + step @ Wd.T + 2.0 ** -22 * (dx @ Wd.T)
    return ref_k, bound_k, ref_t, bound_t, int(flip.sum())


def fp8_act_glu_bounds(x, cg, qg, cu, qu, eps):
    """The same for SiLU(a) * b, propagated as in ``glu_bound``."""
    a_k, Ba_k, a_t, Ba_t, fa = fp8_act_bounds(x, cg, qg, eps)
    b_k, Bb_k, b_t, Bb_t, _ = fp8_act_bounds(x, cu, qu, eps)

    def prop(a, b, Ba, Bb):
        h = oracle.silu(a) * b
        return h, 1.1 * np.abs(b) * Ba + np.abs(oracle.silu(a)) * Bb + 1.1 * Ba * Bb + 8 * U32 * np.abs(h) + 1e-30

    hk, Bk = prop(a_k, b_k, Ba_k, Bb_k)
    ht, Bt = prop(a_t, b_t, Ba_t, Bb_t)  # ht is oracle.glu_fp8_act
    return hk, Bk, ht, Bt, fa
