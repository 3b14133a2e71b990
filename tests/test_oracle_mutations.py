"""The pins have teeth: plant a plausible mistake in the oracle (on the CPU,
by monkeypatching it) and check that at least one pin in
``test_oracle_pins`` then fails."""

import inspect
import json

import numpy as np
import pytest

import oracle
import oracle.reference as ref
from tests import test_oracle_pins as pins


def _pin_tests():
    return [f for n, f in inspect.getmembers(pins, inspect.isfunction) if n.startswith("test_")]


def _run_all_pins(golden):
    failures = 0
    for f in _pin_tests():
        try:
            if "golden" in inspect.signature(f).parameters:
                f(golden)
            else:
                f()
        except (AssertionError, ValueError, FloatingPointError):
            failures += 1
    return failures


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(ref, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


_orig = {n: getattr(ref, n) for n in ("rms", "rmsnorm", "silu", "head_rmsnorm", "round_to_bf16",
                                      "norm_linear", "norm_glu_ffn", "linear_qknorm", "fold_weights",
                                      "rope", "rope_angles", "linear_qknorm_rope", "layernorm",
                                      "layernorm_linear", "fold_layernorm", "round_to_e4m3", "e4m3_value",
                                      "quantize_fp8_per_channel", "dequantize_fp8", "_latent_epilogue",
                                      "glu_deferred_on_quantized", "deferred_fp8_act", "norm_linear_fp8_act")}


def _m_eps_outside(x, eps):
    x = ref._f64(x)
    return np.sqrt(np.sum(x * x, axis=-1) / x.shape[-1]) + eps


def _m_sum_not_mean(x, eps):
    x = ref._f64(x)
    return np.sqrt(np.sum(x * x, axis=-1) + eps)


def _m_mean_k_minus_1(x, eps):
    x = ref._f64(x)
    return np.sqrt(np.sum(x * x, axis=-1) / (x.shape[-1] - 1 if x.shape[-1] > 1 else 1) + eps)


def _m_gain_divided(x, g, eps):
    x = ref._f64(x)
    return (x / ref.rms(x, eps)[..., None]) / ref._f64(g)


def _m_silu_sign(t):
    t = np.asarray(t, dtype=np.float64)
    with np.errstate(over="ignore"):
        return t / (1.0 + np.exp(t))


def _m_glu_swapped(x, Wg, Wu, g, eps):
    return _orig["norm_glu_ffn"](x, Wu, Wg, g, eps)


def _m_head_no_gain(u, gain, eps_h, head_dim):
    return _orig["head_rmsnorm"](u, None, eps_h, head_dim)


def _m_head_eps_outside(u, gain, eps_h, head_dim):
    y = _orig["head_rmsnorm"](u, gain, 0.0, head_dim)
    return y if eps_h == 0 else y * 0.999


def _m_bf16_double_round(d):
    return _orig["round_to_bf16"](np.asarray(d, dtype=np.float64).astype(np.float32).astype(np.float64))


def _m_fold_via_f32(W, g, out_dtype):
    p = (ref._f64(W) * ref._f64(g)[None, :]).astype(np.float32).astype(np.float64)
    if out_dtype == "f32":
        return p.astype(np.float32)
    return ref._bf16_bits_of_values(_orig["round_to_bf16"](p))


def _m_qk_kgain_is_qgain(x, W_qkv, g1, eps_x, nq, nkv, hd, g_q, g_k, eps_head, v_mode=0):
    return _orig["linear_qknorm"](x, W_qkv, g1, eps_x, nq, nkv, hd, g_q, g_q, eps_head, v_mode)


def _m_qk_v_normed(x, W_qkv, g1, eps_x, nq, nkv, hd, g_q, g_k, eps_head, v_mode=0):
    return _orig["linear_qknorm"](x, W_qkv, g1, eps_x, nq, nkv, hd, g_q, g_k, eps_head, 1 - v_mode)


def _m_rope_sign(u, positions, base, rot_dim, head_dim):
    return _orig["rope"](u, -np.asarray(positions, dtype=np.float64), base, rot_dim, head_dim)


def _m_rope_half_split(u, positions, base, rot_dim, head_dim):
    # pairs (i, i + rot_dim/2) instead of (2i, 2i+1)
    u = ref._f64(u)
    M, C = u.shape
    perm = np.concatenate([np.arange(0, rot_dim, 2), np.arange(1, rot_dim, 2), np.arange(rot_dim, head_dim)])
    inv = np.argsort(perm)
    uh = u.reshape(M, C // head_dim, head_dim)[:, :, inv].reshape(M, C)
    y = _orig["rope"](uh, positions, base, rot_dim, head_dim)
    return y.reshape(M, C // head_dim, head_dim)[:, :, perm].reshape(M, C)


def _m_rope_freq_i_over_d(positions, base, rot_dim):
    p = np.asarray(positions, dtype=np.float64)
    i = np.arange(rot_dim // 2, dtype=np.float64)
    return p[:, None] * (float(base) ** (-i / rot_dim))[None, :]


def _m_rope_rotates_v(x, W_qkv, g1, eps_x, nq, nkv, hd, g_q, g_k, eps_head, v_mode, positions, base, rot_dim):
    y = _orig["linear_qknorm"](x, W_qkv, g1, eps_x, nq, nkv, hd, g_q, g_k, eps_head, v_mode)
    return ref.rope(y, positions, base, rot_dim, hd)


def _m_rope_before_gain(x, W_qkv, g1, eps_x, nq, nkv, hd, g_q, g_k, eps_head, v_mode, positions, base, rot_dim):
    one = np.ones(hd)
    y = _orig["linear_qknorm"](x, W_qkv, g1, eps_x, nq, nkv, hd, one, one, eps_head, v_mode)
    nqk = (nq + nkv) * hd
    y[:, :nqk] = ref.rope(y[:, :nqk], positions, base, rot_dim, hd)
    M = y.shape[0]
    y[:, :nq * hd] = (y[:, :nq * hd].reshape(M, nq, hd) * ref._f64(g_q)).reshape(M, -1)
    y[:, nq * hd:nqk] = (y[:, nq * hd:nqk].reshape(M, nkv, hd) * ref._f64(g_k)).reshape(M, -1)
    return y


def _m_ln_unbiased_var(x, g, beta, eps):
    x = ref._f64(x)
    K = x.shape[-1]
    d = x - x.mean(axis=-1, keepdims=True)
    y = d / np.sqrt((d * d).sum(axis=-1, keepdims=True) / (K - 1) + eps) * ref._f64(g)
    return y if beta is None else y + ref._f64(beta)


def _m_ln_eps_outside(x, g, beta, eps):
    x = ref._f64(x)
    d = x - x.mean(axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = d / (np.sqrt((d * d).mean(axis=-1, keepdims=True)) + eps) * ref._f64(g)
    return y if beta is None else y + ref._f64(beta)


def _m_ln_no_centering(x, g, beta, eps):
    y = ref.rmsnorm(x, g, eps)
    return y if beta is None else y + ref._f64(beta)


def _m_ln_beta_before_gain(x, g, beta, eps):
    y = _orig["layernorm"](x, np.ones_like(ref._f64(g)), beta, eps)
    return y * ref._f64(g)


def _m_ln_linear_drops_bias(x, W, g, beta, bias, eps):
    return _orig["layernorm_linear"](x, W, g, beta, None, eps)


def _m_fold_ln_unrounded_colsum(W, g, beta, bias, out_dtype):
    Ws, _, b = _orig["fold_layernorm"](W, g, beta, bias, out_dtype)
    c = (ref._f64(W) * ref._f64(g)[None, :]).sum(axis=1)
    return Ws, ref.round_to_f32(c).astype(np.float32), b


def _m_e4m3_truncate(d):
    d = np.asarray(d, dtype=np.float64)
    a = np.abs(d)
    out = np.zeros_like(a)
    nz = a > 0
    e = np.floor(np.log2(a[nz]))
    sp = np.exp2(np.maximum(e, -6) - 3)
    out[nz] = np.floor(a[nz] / sp) * sp
    return np.clip(np.sign(d) * out, -448, 448)


def _m_e4m3_bias8(code):
    return _orig["e4m3_value"](code) / 2.0


def _m_fp8_scale_240(W_star):
    Wf = ref._f64(W_star)
    amax = np.max(np.abs(Wf), axis=1)
    q = ref.round_to_f32(np.where(amax > 0, amax / 240.0, 1.0))
    return ref.e4m3_code(ref.round_to_e4m3(Wf / q[:, None])), q.astype(np.float32)


def _m_fp8_dequant_divides(codes, q):
    return ref.e4m3_value(codes) / ref._f64(q)[:, None]


def _m_fp8_glu_swapped(x, codes_g, q_g, codes_u, q_u, eps):
    return _orig["glu_deferred_on_quantized"](x, codes_u, q_u, codes_g, q_g, eps)


def _m_fp8_glu_scales_swapped(x, codes_g, q_g, codes_u, q_u, eps):
    return _orig["glu_deferred_on_quantized"](x, codes_g, q_u, codes_u, q_g, eps)


def _m_fp8_act_scale_from_quantised(x, codes_w, q_w, eps):
    cx, qx = ref.quantize_fp8_per_channel(x)
    xd = ref.dequantize_fp8(cx, qx)
    return (xd @ ref.dequantize_fp8(codes_w, q_w).T) / ref.rms(xd, eps)[:, None]


def _m_fp8_act_columns(x, codes_w, q_w, eps):
    cx, qx = ref.quantize_fp8_per_channel(ref._f64(x).T)
    xd = ref.dequantize_fp8(cx, qx).T
    return (xd @ ref.dequantize_fp8(codes_w, q_w).T) / ref.rms(x, eps)[:, None]


def _m_fp8_act_no_x_scale(x, codes_w, q_w, eps):
    cx, _ = ref.quantize_fp8_per_channel(x)
    return (ref.e4m3_value(cx) @ ref.dequantize_fp8(codes_w, q_w).T) / ref.rms(x, eps)[:, None]


def _m_fp8_text_gain_kept(x, codes_w, q_w, eps):
    # normalises with a gain of 2 instead of the folded unit gain
    xn = ref.rmsnorm(x, 2 * np.ones(ref._f64(x).shape[-1]), eps)
    cx, qx = ref.quantize_fp8_per_channel(xn)
    return ref.dequantize_fp8(cx, qx) @ ref.dequantize_fp8(codes_w, q_w).T


def _m_latent_per_chunk(u, nq, nkv, nr, g_q, g_kv, eps_l, positions, base, rot_dim, s_plain):
    # normalises each latent in chunks of at most 32 columns instead of over its width
    parts = []
    for lo, w, g in ((0, nq, g_q), (nq, nkv, g_kv)):
        if w:
            hd = min(w, 32)
            parts.append(ref.head_rmsnorm(u[:, lo:lo + w], None, eps_l, hd) * ref._f64(g)[None, :])
    if nr:
        p = u[:, nq + nkv:]
        if s_plain is not None:
            p = p * s_plain[:, None]
        if positions is not None:
            p = ref.rope(p, positions, base, rot_dim, nr)
        parts.append(p)
    return np.concatenate(parts, axis=1)


def _m_latent_rope_part_normed(u, nq, nkv, nr, g_q, g_kv, eps_l, positions, base, rot_dim, s_plain):
    y = _orig["_latent_epilogue"](u, nq, nkv, nr, g_q, g_kv, eps_l, positions, base, rot_dim, s_plain)
    if nr:
        y[:, nq + nkv:] = ref.head_rmsnorm(y[:, nq + nkv:], None, eps_l, nr)
    return y


def _m_latent_no_deferred_scale(u, nq, nkv, nr, g_q, g_kv, eps_l, positions, base, rot_dim, s_plain):
    return _orig["_latent_epilogue"](u, nq, nkv, nr, g_q, g_kv, eps_l, positions, base, rot_dim, None)


MUTATIONS = [
    ("rms", _m_eps_outside),
    ("rms", _m_sum_not_mean),
    ("rms", _m_mean_k_minus_1),
    ("rmsnorm", _m_gain_divided),
    ("silu", _m_silu_sign),
    ("norm_glu_ffn", _m_glu_swapped),
    ("head_rmsnorm", _m_head_no_gain),
    ("head_rmsnorm", _m_head_eps_outside),
    ("round_to_bf16", _m_bf16_double_round),
    ("fold_weights", _m_fold_via_f32),
    ("linear_qknorm", _m_qk_kgain_is_qgain),
    ("linear_qknorm", _m_qk_v_normed),
    ("rope", _m_rope_sign),
    ("rope", _m_rope_half_split),
    ("rope_angles", _m_rope_freq_i_over_d),
    ("linear_qknorm_rope", _m_rope_rotates_v),
    ("linear_qknorm_rope", _m_rope_before_gain),
    ("layernorm", _m_ln_unbiased_var),
    ("layernorm", _m_ln_eps_outside),
    ("layernorm", _m_ln_no_centering),
    ("layernorm", _m_ln_beta_before_gain),
    ("layernorm_linear", _m_ln_linear_drops_bias),
    ("fold_layernorm", _m_fold_ln_unrounded_colsum),
    ("round_to_e4m3", _m_e4m3_truncate),
    ("e4m3_value", _m_e4m3_bias8),
    ("quantize_fp8_per_channel", _m_fp8_scale_240),
    ("dequantize_fp8", _m_fp8_dequant_divides),
    ("glu_deferred_on_quantized", _m_fp8_glu_swapped),
    ("glu_deferred_on_quantized", _m_fp8_glu_scales_swapped),
    ("deferred_fp8_act", _m_fp8_act_scale_from_quantised),
    ("deferred_fp8_act", _m_fp8_act_columns),
    ("deferred_fp8_act", _m_fp8_act_no_x_scale),
    ("norm_linear_fp8_act", _m_fp8_text_gain_kept),
    ("_latent_epilogue", _m_latent_per_chunk),
    ("_latent_epilogue", _m_latent_rope_part_normed),
    ("_latent_epilogue", _m_latent_no_deferred_scale),
]


@pytest.fixture(scope="module")
def golden():
    with open(pins.GOLDEN) as f:
        return json.load(f)


def test_unmutated_oracle_passes_every_pin(golden):
    assert _run_all_pins(golden) == 0


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, golden, name, fn):
    _patch(monkeypatch, name, fn)
    with np.errstate(all="ignore"):
        assert _run_all_pins(golden) > 0, f"no pin catches mutation {fn.__name__} of {name}"


def test_transposed_weight_is_caught(monkeypatch, golden):
    def transposed(x, W, g, eps):
        W = ref._f64(W)
        xn = ref.rmsnorm(x, g, eps)
        return xn @ W if W.shape[0] == W.shape[1] else xn @ W.T

    _patch(monkeypatch, "norm_linear", transposed)
    assert _run_all_pins(golden) > 0
