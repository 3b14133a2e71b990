"""Pins of the CPU oracle against things other than itself.

Each test ties an oracle function to a hand-derived golden case, a closed
form, a mathematical invariant, a library routine on a special case or a
brute-force loop on tiny inputs.  Together they are meant to catch a dropped
term, a wrong sign or index, eps in the wrong place, a transposed operand or
a double rounding anywhere in the oracle.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from oracle.reference import _round_to_format  # noqa: F401  (exercised via the public wrappers)
from synth import bf16_bits_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "flashnorm_cases.json")


def _q(s):
    return float(Fraction(s))


def _arr(rows):
    return np.array([[_q(v) for v in r] for r in rows], dtype=np.float64)


def _vec(v):
    return np.array([_q(s) for s in v], dtype=np.float64)


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _close(a, b, rtol=4e-16 * 8, atol=1e-15):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape
    assert np.all(np.abs(a - b) <= atol + rtol * np.abs(b)), (a, b)


# --------------------------------------------------------------------------
# golden, hand-derived cases
# --------------------------------------------------------------------------

def test_golden_rmsnorm(golden):
    for c in golden["rmsnorm"]:
        x = _arr(c["x"])
        g = _vec(c["g"])
        eps = _q(c["eps"])
        _close(oracle.rms(x, eps), _vec(c["rms"]))
        _close(oracle.rmsnorm(x, g, eps), _arr(c["xn"]))


def test_golden_norm_linear(golden):
    for c in golden["norm_linear"]:
        y = oracle.norm_linear(_arr(c["x"]), _arr(c["W"]), _vec(c["g"]), _q(c["eps"]))
        _close(y, _arr(c["y"]))


def test_golden_qknorm(golden):
    for c in golden["linear_qknorm"]:
        y = oracle.linear_qknorm(_arr(c["x"]), _arr(c["W_qkv"]), _vec(c["g1"]), _q(c["eps_x"]),
                                 c["n_q_heads"], c["n_kv_heads"], c["head_dim"],
                                 _vec(c["g_q"]), _vec(c["g_k"]), _q(c["eps_head"]), 0)
        _close(y, _arr(c["y"]))


def _to_bf16_bits_exact(vals):
    f = np.asarray(vals, dtype=np.float64).astype(np.float32)
    assert np.all(f.astype(np.float64) == vals)
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.all(bf16_bits_to_f64(bits) == vals), "golden W must be exactly bf16"
    return bits


def test_golden_fold_bf16(golden):
    for c in golden["fold_bf16"]:
        W = _to_bf16_bits_exact(_arr(c["W"]))
        gv = _vec(c["g"])
        g32 = gv.astype(np.float32)
        assert np.all(g32.astype(np.float64) == gv), "golden g must be exactly float32"
        got = oracle.fold_weights(W, g32, "bf16")
        assert got.dtype == np.uint16
        assert np.array_equal(bf16_bits_to_f64(got), _arr(c["W_star"])), c["name"]


# --------------------------------------------------------------------------
# rounding, against library casts and against the definition
# --------------------------------------------------------------------------

def _random_f32(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


def test_round_bf16_matches_torch_cast_on_float32_inputs():
    f = _random_f32(1 << 20, 1)
    # add the hard spots: ties, subnormals, overflow edge
    extra = np.array([1 + 2 ** -8, 1 + 2 ** -7 + 2 ** -8, -(1 + 2 ** -8), 2 ** -133, 2 ** -134,
                      3 * 2 ** -135, 2 ** -126 * (1 - 2 ** -8), 3.3895313892515355e38,
                      3.3895314e38, 3.4e38, 0.0, -0.0], dtype=np.float32)
    f = np.concatenate([f, extra])
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(f.astype(np.float64))
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert np.all(same), f[~same][:8]
    # signed zeros too
    assert np.array_equal(np.signbit(got[want == 0]), np.signbit(want[want == 0]))


def test_round_f32_matches_numpy_cast_on_float64_inputs():
    rng = np.random.default_rng(2)
    d = rng.standard_normal(1 << 18) * np.exp2(rng.integers(-160, 130, size=1 << 18))
    # exact float32 midpoints (ties) in the normal and subnormal range
    a = np.float32(1.2345).astype(np.float64)
    ties = np.array([a + 2.0 ** -24 * 1.0, 1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 2.0 ** -150, 3 * 2.0 ** -150])
    d = np.concatenate([d, ties, -ties])
    with np.errstate(over="ignore"):  # beyond float32's range the cast gives inf, as it should
        want = d.astype(np.float32).astype(np.float64)
    got = oracle.round_to_f32(d)
    assert np.array_equal(got, want)


def test_round_bf16_single_rounding_from_float64():
    # 1 + 2^-8 is a bf16 tie (goes to even 1.0); anything above it goes up
    assert oracle.round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert oracle.round_to_bf16(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 1 + 2 ** -7
    assert oracle.round_to_bf16(np.array([1 + 2 ** -7 + 2 ** -8]))[0] == 1 + 2 ** -6
    assert oracle.round_to_bf16(np.array([-(1 + 2 ** -8 + 2 ** -40)]))[0] == -(1 + 2 ** -7)


def test_fold_power_of_two_gain_is_exact():
    rng = np.random.default_rng(3)
    W = rng.standard_normal((17, 33)).astype(np.float32)
    g = np.exp2(rng.integers(-3, 4, size=33)).astype(np.float32)
    got = oracle.fold_weights(W, g, "f32")
    assert np.array_equal(got.astype(np.float64), W.astype(np.float64) * g.astype(np.float64))
    Wb = _to_bf16_bits_exact(bf16_bits_to_f64(
        (W.view(np.uint32) >> np.uint32(16)).astype(np.uint16)))
    gotb = oracle.fold_weights(Wb, g, "bf16")
    assert np.array_equal(bf16_bits_to_f64(gotb), bf16_bits_to_f64(Wb) * g.astype(np.float64))


def test_fold_bf16_is_nearest_bf16_of_exact_product():
    """Brute force: the folded value is the bf16 value closest to g*W, with
    ties to an even last bit, checked against the two bf16 neighbours found
    by stepping bit patterns (no rounding arithmetic involved)."""
    rng = np.random.default_rng(4)
    Wbits = rng.integers(0x3000, 0x4800, size=(64, 32), dtype=np.uint64).astype(np.uint16)
    Wbits[::2] |= np.uint16(0x8000)
    g = (1 + 0.1 * rng.standard_normal(32)).astype(np.float32)
    got = oracle.fold_weights(Wbits, g, "bf16")
    p = bf16_bits_to_f64(Wbits) * g.astype(np.float64)
    mag = np.abs(p)
    # candidate magnitudes: truncation of |p| to bf16 and the next bf16 up
    t = (mag.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint32)
    lo = bf16_bits_to_f64(t.astype(np.uint16))
    lo_fix = lo > mag
    t[lo_fix] -= 1
    lo = bf16_bits_to_f64(t.astype(np.uint16))
    hi = bf16_bits_to_f64((t + 1).astype(np.uint16))
    assert np.all((lo <= mag) & (mag < hi))
    dl, dh = mag - lo, hi - mag
    pick_hi = (dh < dl) | ((dh == dl) & (t % 2 == 1))
    want = np.where(pick_hi, hi, lo) * np.sign(p)
    assert np.array_equal(bf16_bits_to_f64(got), want)


# --------------------------------------------------------------------------
# closed forms and invariants
# --------------------------------------------------------------------------

def test_rmsnorm_unit_gain_no_eps_is_scaled_unit_vector():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 13))
    want = math.sqrt(13) * x / np.linalg.norm(x, axis=1, keepdims=True)
    _close(oracle.rmsnorm(x, np.ones(13), 0.0), want, rtol=1e-14)


def test_rmsnorm_scale_invariance():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 16))
    g = 1 + 0.1 * rng.standard_normal(16)
    base = oracle.rmsnorm(x, g, 0.0)
    for k in (-5, 1, 7):
        assert np.array_equal(oracle.rmsnorm(x * 2.0 ** k, g, 0.0), base)
    _close(oracle.rmsnorm(x * 3.7, g, 0.0), base, rtol=1e-15)
    # and with eps > 0 it is not invariant
    assert not np.allclose(oracle.rmsnorm(x * 1e-3, g, 1e-5), base, rtol=1e-3)


def test_constant_row_closed_form():
    for c, eps in [(2.0, 1e-5), (-0.3, 1e-6), (5.0, 0.0)]:
        xn = oracle.rmsnorm(np.full((1, 9), c), np.ones(9), eps)
        _close(xn, np.full((1, 9), c / math.sqrt(c * c + eps)), rtol=1e-15)


def test_degenerate_rows():
    x = np.zeros((2, 4))
    x[1] = [1, 2, 3, 4]
    W = np.arange(12, dtype=np.float64).reshape(3, 4)
    y = oracle.norm_linear(x, W, np.ones(4), 1e-6)
    assert np.all(y[0] == 0.0)
    y0 = oracle.norm_linear(x, W, np.ones(4), 0.0)
    assert np.all(np.isnan(y0[0])) and np.all(np.isfinite(y0[1]))


def test_deferral_identity():
    """(x . (diag(g) W)^T) * s  ==  RMSNorm(x; g) . W^T  (Abstract, (i)+(ii))."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((9, 24)) * np.exp(rng.standard_normal((9, 1)))
    W = rng.standard_normal((11, 24))
    g = 1 + 0.1 * rng.standard_normal(24)
    ref = oracle.norm_linear(x, W, g, 1e-5)
    folded = W * g[None, :]  # unrounded fold
    _close(oracle.deferred_on_folded(x, folded, 1e-5), ref, rtol=1e-13, atol=1e-13)
    a = oracle.glu_deferred_on_folded(x, folded, folded[::-1].copy(), 1e-5)
    b = oracle.norm_glu_ffn(x, W, W[::-1].copy(), g, 1e-5)
    _close(a, b, rtol=1e-12, atol=1e-13)


def test_fold_then_unit_gain_equals_gain():
    rng = np.random.default_rng(8)
    x = rng.integers(-4, 5, size=(6, 8)).astype(np.float64)
    x[:, 0] = 8  # no zero rows
    W = rng.integers(-3, 4, size=(5, 8)).astype(np.float32)
    g = np.exp2(rng.integers(-2, 3, size=8)).astype(np.float32)
    Wstar = oracle.fold_weights(W, g, "f32")
    _close(oracle.norm_linear(x, Wstar, np.ones(8), 1e-3), oracle.norm_linear(x, W, g, 1e-3),
           rtol=1e-15, atol=1e-15)


def test_silu_closed_forms():
    ln3 = math.log(3.0)
    _close(oracle.silu(np.array([0.0, ln3, -ln3])), np.array([0.0, 0.75 * ln3, -0.25 * ln3]), rtol=1e-15)
    t = np.linspace(-30, 30, 601)
    _close(oracle.silu(t) - oracle.silu(-t), t, rtol=1e-14, atol=1e-14)
    _close(oracle.silu(t), t * expit(t), rtol=1e-15, atol=1e-300)
    assert oracle.silu(np.array([-800.0]))[0] == 0.0


def test_glu_gate_and_up_roles():
    """xn = [2/5, 7/5] (x=[1,7], g=[2,1]); gate rows give a = ln3, 0, -ln3;
    up rows give b = 1, 5, 2 -> h = SiLU(a) * b = 3/4 ln3, 0, -1/2 ln3."""
    ln3 = math.log(3.0)
    x = np.array([[1.0, 7.0]])
    g = np.array([2.0, 1.0])
    Wg = np.array([[2.5 * ln3, 0.0], [0.0, 0.0], [-2.5 * ln3, 0.0]])
    Wu = np.array([[0.0, 5.0 / 7.0], [12.5, 0.0], [5.0, 0.0]])
    h = oracle.norm_glu_ffn(x, Wg, Wu, g, 0.0)
    _close(h, np.array([[0.75 * ln3, 0.0, -0.5 * ln3]]), rtol=1e-14, atol=1e-15)
    # swapping the roles gives a different answer
    assert not np.allclose(oracle.norm_glu_ffn(x, Wu, Wg, g, 0.0), h)


def test_head_norm_unit_mean_square():
    rng = np.random.default_rng(9)
    u = rng.standard_normal((4, 6 * 8)) * 3
    y = oracle.head_rmsnorm(u, None, 0.0, 8)
    ms = np.mean(y.reshape(4, 6, 8) ** 2, axis=-1)
    _close(ms, np.ones((4, 6)), rtol=1e-14)
    gh = rng.standard_normal((6, 8))
    yg = oracle.head_rmsnorm(u, gh, 0.0, 8)
    _close(yg, (y.reshape(4, 6, 8) * gh[None]).reshape(4, 48), rtol=1e-15)


def _qk_case(rng, M=5, K=12, nq=2, nkv=1, hd=4):
    x = rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))
    N = (nq + 2 * nkv) * hd
    W = rng.standard_normal((N, K))
    g1 = 1 + 0.1 * rng.standard_normal(K)
    gq = 1 + 0.1 * rng.standard_normal(hd)
    gk = 1 + 0.1 * rng.standard_normal(hd)
    return x, W, g1, gq, gk, nq, nkv, hd


def test_scale_invariance_drops_first_norm():
    """RMSNorm(Linear(RMSNorm(x))) == RMSNorm(Linear(x)) without bias, eps 0
    (Abstract, the first RMSNorm can be eliminated)."""
    rng = np.random.default_rng(10)
    x, W, g1, gq, gk, nq, nkv, hd = _qk_case(rng)
    ref = oracle.linear_qknorm(x, W, g1, 0.0, nq, nkv, hd, gq, gk, 0.0, v_mode=1)
    dropped = oracle.qknorm_dropped_on_folded(x, W * g1[None, :], 0.0, nq, nkv, hd, gq, gk, 0.0, v_mode=1)
    _close(dropped, ref, rtol=1e-13, atol=1e-14)
    # v_mode 0 keeps V = u_v, which needs the deferred row scale
    ref0 = oracle.linear_qknorm(x, W, g1, 1e-6, nq, nkv, hd, gq, gk, 0.0, v_mode=0)
    d0 = oracle.qknorm_dropped_on_folded(x, W * g1[None, :], 1e-6, nq, nkv, hd, gq, gk, 0.0, v_mode=0)
    _close(d0, ref0, rtol=1e-12, atol=1e-13)


def test_eps_head_breaks_invariance_by_closed_form():
    """With eps_h > 0 the dropped form differs from the reference by
    sqrt(mean(z^2) + eps_h r^2) / sqrt(mean(z^2) + eps_h), z = x . W*^T."""
    rng = np.random.default_rng(11)
    x, W, g1, gq, gk, nq, nkv, hd = _qk_case(rng)
    x *= 0.05
    eps_x, eps_h = 1e-6, 1e-3
    ref = oracle.linear_qknorm(x, W, g1, eps_x, nq, nkv, hd, gq, gk, eps_h, 0)
    dropped = oracle.qknorm_dropped_on_folded(x, W * g1[None, :], eps_x, nq, nkv, hd, gq, gk, eps_h, 0)
    z = x @ (W * g1[None, :]).T
    r = oracle.rms(x, eps_x)
    nqk = (nq + nkv) * hd
    zh = z[:, :nqk].reshape(x.shape[0], nq + nkv, hd)
    mz = np.mean(zh ** 2, axis=-1)
    ratio = np.sqrt(mz + eps_h * r[:, None] ** 2) / np.sqrt(mz + eps_h)
    got = dropped[:, :nqk].reshape(zh.shape) / ref[:, :nqk].reshape(zh.shape)
    _close(got, np.repeat(ratio[..., None], hd, axis=-1), rtol=1e-12)
    assert np.max(np.abs(ratio - 1)) > 1e-6
    # V heads are exact in v_mode 0
    _close(dropped[:, nqk:], ref[:, nqk:], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# brute force on tiny inputs: pure-Python loops with exactly rounded sums
# --------------------------------------------------------------------------

def _bf_norm_linear(x, W, g, eps):
    M, K = len(x), len(x[0])
    out = []
    for m in range(M):
        r = math.sqrt(math.fsum(v * v for v in x[m]) / K + eps)
        xn = [x[m][k] / r * g[k] for k in range(K)]
        out.append([math.fsum(xn[k] * W[n][k] for k in range(K)) for n in range(len(W))])
    return out


def test_brute_force_norm_linear_glu_qknorm():
    rng = np.random.default_rng(12)
    for trial in range(20):
        M, K, N = rng.integers(1, 6, size=3)
        x = rng.standard_normal((M, K))
        W = rng.standard_normal((N, K))
        Wu = rng.standard_normal((N, K))
        g = 1 + 0.1 * rng.standard_normal(K)
        eps = float(rng.choice([0.0, 1e-6, 0.5]))
        bf = np.array(_bf_norm_linear(x.tolist(), W.tolist(), g.tolist(), eps))
        _close(oracle.norm_linear(x, W, g, eps), bf, rtol=1e-13, atol=1e-14)
        bu = np.array(_bf_norm_linear(x.tolist(), Wu.tolist(), g.tolist(), eps))
        bh = [[bf[m][n] / (1 + math.exp(-bf[m][n])) * bu[m][n] for n in range(N)] for m in range(M)]
        _close(oracle.norm_glu_ffn(x, W, Wu, g, eps), np.array(bh), rtol=1e-12, atol=1e-14)
    # qknorm: heads of 3, 2 q heads, 1 kv head
    x = rng.standard_normal((3, 5))
    W = rng.standard_normal((12, 5))
    g1 = 1 + 0.1 * rng.standard_normal(5)
    gq = rng.standard_normal(3)
    gk = rng.standard_normal(3)
    u = _bf_norm_linear(x.tolist(), W.tolist(), g1.tolist(), 1e-6)
    want = []
    for m in range(3):
        row = []
        for h in range(4):
            seg = u[m][3 * h:3 * h + 3]
            if h < 3:
                rr = math.sqrt(math.fsum(v * v for v in seg) / 3 + 1e-4)
                gg = gq if h < 2 else gk
                row += [seg[j] / rr * gg[j] for j in range(3)]
            else:
                row += seg
        want.append(row)
    got = oracle.linear_qknorm(x, W, g1, 1e-6, 2, 1, 3, gq, gk, 1e-4, 0)
    _close(got, np.array(want), rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# rotary position embedding (RoFormer, Section 3.2, general form) after the
# head norms
# --------------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(20)
    u = rng.standard_normal((3, 2 * 8))
    _close(oracle.rope(u, [0, 0, 0], 10000.0, 8, 8), u, rtol=0, atol=0)


def test_rope_closed_form_unit_vectors():
    """base 10^4, four rotated columns: theta_0 = 1, theta_1 = 10^4^(-2/4) =
    1/100, so at position 100 pair 0 turns by 100 rad and pair 1 by 1 rad; a
    pair (a, b) goes to (a cos t - b sin t, a sin t + b cos t)."""
    e = np.eye(4)
    y = oracle.rope(e, [100] * 4, 10000.0, 4, 4)
    c100, s100, c1, s1 = math.cos(100), math.sin(100), math.cos(1), math.sin(1)
    _close(y[0], [c100, s100, 0, 0], rtol=1e-14, atol=1e-15)
    _close(y[1], [-s100, c100, 0, 0], rtol=1e-14, atol=1e-15)
    _close(y[2], [0, 0, c1, s1], rtol=1e-14, atol=1e-15)
    _close(y[3], [0, 0, -s1, c1], rtol=1e-14, atol=1e-15)
    # eight rotated columns, base 10^4: theta_i = 10^-i, position 1000
    e8 = np.eye(8)
    y8 = oracle.rope(e8, [1000] * 8, 10000.0, 8, 8)
    for i, t in enumerate([1000.0, 100.0, 10.0, 1.0]):
        _close(y8[2 * i, 2 * i:2 * i + 2], [math.cos(t), math.sin(t)], rtol=1e-13, atol=1e-14)


def test_rope_is_complex_multiplication():
    """Pair (a, b) as a + ib times exp(i t): numpy's complex exponential."""
    rng = np.random.default_rng(21)
    M, hd, rot = 4, 16, 12
    u = rng.standard_normal((M, 3 * hd))
    pos = [0, 5, 77, 4095]
    y = oracle.rope(u, pos, 500000.0, rot, hd)
    t = oracle.rope_angles(pos, 500000.0, rot)
    uh = u.reshape(M, 3, hd)
    z = (uh[:, :, 0:rot:2] + 1j * uh[:, :, 1:rot:2]) * np.exp(1j * t)[:, None, :]
    yh = y.reshape(M, 3, hd)
    _close(yh[:, :, 0:rot:2], z.real, rtol=1e-13, atol=1e-13)
    _close(yh[:, :, 1:rot:2], z.imag, rtol=1e-13, atol=1e-13)
    # columns from rot_dim on are untouched
    _close(yh[:, :, rot:], uh[:, :, rot:], rtol=0, atol=0)


def test_rope_relative_position_and_norm():
    """The rotated dot product of a query at p and a key at p' depends only on
    p - p' (the property the embedding is built for); rotation keeps norms."""
    rng = np.random.default_rng(22)
    hd = 32
    q = rng.standard_normal((1, hd))
    k = rng.standard_normal((1, hd))
    d1 = (oracle.rope(q, [37], 10000.0, hd, hd) @ oracle.rope(k, [12], 10000.0, hd, hd).T).item()
    d2 = (oracle.rope(q, [1025], 10000.0, hd, hd) @ oracle.rope(k, [1000], 10000.0, hd, hd).T).item()
    d3 = (oracle.rope(q, [25], 10000.0, hd, hd) @ k.T).item()
    assert abs(d1 - d2) < 1e-12 and abs(d1 - d3) < 1e-12
    assert abs(d1 - (q @ k.T).item()) > 1e-3
    y = oracle.rope(q, [1025], 10000.0, hd, hd)
    pn = lambda a: np.hypot(a[:, 0::2], a[:, 1::2])  # noqa: E731
    _close(pn(y), pn(q), rtol=1e-14)


def test_qknorm_rope_gain_then_rotation_closed_form():
    """One token, K = 4, x = [1,1,1,1] (rms 1, eps 0), head_dim 4, one q,
    one k and one v head.  u_q = [1,0,0,0] -> head norm 2*[1,0,0,0] -> gain
    [3,5,1,1] -> [6,0,0,0] -> turned by 7 rad (pair 0, position 7):
    [6 cos 7, 6 sin 7, 0, 0].  u_k = [0,0,0,1] -> [0,0,0,2] -> gain [1,1,1,3]
    -> pair 1 (theta_1 = 1/100 at base 10^4) turned by 0.07 rad:
    [0, 0, -6 sin 0.07, 6 cos 0.07].  v = u_v = [1,2,3,4] is not rotated."""
    x = np.ones((1, 4))
    W = np.zeros((12, 4))
    W[0, 0] = 1.0
    W[7, 3] = 1.0
    W[8:12, 0] = [1, 2, 3, 4]
    gq = np.array([3.0, 5.0, 1.0, 1.0])
    gk = np.array([1.0, 1.0, 1.0, 3.0])
    y = oracle.linear_qknorm_rope(x, W, np.ones(4), 0.0, 1, 1, 4, gq, gk, 0.0, 0, [7], 10000.0, 4)
    _close(y[0, 0:4], [6 * math.cos(7), 6 * math.sin(7), 0, 0], rtol=1e-14, atol=1e-14)
    _close(y[0, 4:8], [0, 0, -6 * math.sin(0.07), 6 * math.cos(0.07)], rtol=1e-14, atol=1e-14)
    _close(y[0, 8:12], [1, 2, 3, 4], rtol=1e-15)


# --------------------------------------------------------------------------
# LayerNorm (Layer Normalization, Section 3) and its deferred, folded form
# --------------------------------------------------------------------------

def test_layernorm_golden_cases():
    """Hand-worked rows whose mean and biased variance are exact:
    [0,0,4,4]: mu 2, var 4 -> [-1,-1,1,1]; with eps 5 the root is 3;
    [7,1,1,1,1,1,1,3]: mu 2, var (25 + 6 + 1)/8 = 4 -> d / 2;
    gain and bias: (x - mu)/sigma * g + beta."""
    _close(oracle.layernorm([[0, 0, 4, 4]], np.ones(4), None, 0.0), [[-1, -1, 1, 1]], rtol=0, atol=0)
    _close(oracle.layernorm([[0, 0, 4, 4]], np.ones(4), None, 5.0), [[-2 / 3, -2 / 3, 2 / 3, 2 / 3]], rtol=1e-15)
    _close(oracle.layernorm([[7, 1, 1, 1, 1, 1, 1, 3]], np.ones(8), None, 0.0),
           [[2.5, -0.5, -0.5, -0.5, -0.5, -0.5, -0.5, 0.5]], rtol=0, atol=0)
    g = np.array([2.0, 1.0, 0.5, 1.0])
    beta = np.array([0.25, 0.0, -1.0, 3.0])
    _close(oracle.layernorm([[0, 0, 4, 4]], g, beta, 0.0), [[-1.75, -1.0, -0.5, 4.0]], rtol=0, atol=0)
    # a constant row has zero variance: with eps > 0 the output is beta
    _close(oracle.layernorm([[3, 3, 3, 3]], g, beta, 1e-5), [beta], rtol=0, atol=0)


def test_layernorm_invariances_and_moments():
    """Translation and (eps = 0) scale invariance; unit gain and zero bias
    give mean 0 and mean square var / (var + eps)."""
    rng = np.random.default_rng(30)
    x = rng.standard_normal((5, 24)) * 3 + rng.standard_normal((5, 1)) * 4
    g = 1 + 0.1 * rng.standard_normal(24)
    beta = 0.1 * rng.standard_normal(24)
    y = oracle.layernorm(x, g, beta, 1e-3)
    _close(oracle.layernorm(x + 7.0, g, beta, 1e-3), y, rtol=1e-12, atol=1e-12)
    y0 = oracle.layernorm(x, g, beta, 0.0)
    _close(oracle.layernorm(8.0 * x, g, beta, 0.0), y0, rtol=1e-13, atol=1e-13)
    u = oracle.layernorm(x, np.ones(24), None, 0.5)
    var = np.var(x, axis=1)
    _close(np.mean(u, axis=1), np.zeros(5), rtol=0, atol=1e-14)
    _close(np.mean(u * u, axis=1), var / (var + 0.5), rtol=1e-13)


def test_layernorm_matches_torch_float64():
    """torch's layer_norm on float64 CPU tensors, a library routine."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((6, 40)) * np.exp(rng.standard_normal((6, 1))) + 2.0
    g = 1 + 0.1 * rng.standard_normal(40)
    beta = 0.1 * rng.standard_normal(40)
    t = torch.nn.functional.layer_norm(torch.from_numpy(x), (40,), torch.from_numpy(g), torch.from_numpy(beta),
                                       eps=1e-5).numpy()
    _close(oracle.layernorm(x, g, beta, 1e-5), t, rtol=1e-13, atol=1e-14)
    W = rng.standard_normal((7, 40))
    bias = rng.standard_normal(7)
    tl = torch.nn.functional.linear(torch.from_numpy(t), torch.from_numpy(W), torch.from_numpy(bias)).numpy()
    _close(oracle.layernorm_linear(x, W, g, beta, bias, 1e-5), tl, rtol=1e-12, atol=1e-13)


def test_layernorm_deferral_identity():
    """s (x.W*^T - mu c) + b* == LayerNorm(x) . W^T + bias with the exact
    float64 fold (W* = W diag(g), c = row sums of W*, b* = W beta + bias)."""
    rng = np.random.default_rng(32)
    x = rng.standard_normal((5, 16)) * 2 + 1.5
    W = rng.standard_normal((9, 16))
    g = 1 + 0.1 * rng.standard_normal(16)
    beta = 0.1 * rng.standard_normal(16)
    bias = rng.standard_normal(9)
    Ws = W * g[None, :]
    got = oracle.layernorm_deferred_on_folded(x, Ws, Ws.sum(axis=1), W @ beta + bias, 1e-5)
    _close(got, oracle.layernorm_linear(x, W, g, beta, bias, 1e-5), rtol=1e-12, atol=1e-12)


def test_fold_layernorm_sums_the_stored_weight():
    """c sums the bf16 W* the kernels read (not g W before rounding), b* is
    W beta + bias; small dyadic values make every sum exact."""
    W = np.array([[1.0, 1.0, 0.5, 3.0], [2.0, -1.0, 0.25, 0.0]], dtype=np.float32)
    g = np.array([1.0 + 2.0 ** -9, 1.0, 2.0, 1.0 + 2.0 ** -8], dtype=np.float32)
    beta = np.array([0.5, 0.25, -1.0, 2.0], dtype=np.float32)
    bias = np.array([1.0, -2.0], dtype=np.float32)
    Ws, c, b = oracle.fold_layernorm(W, g, beta, bias, "bf16")
    # 1 + 2^-9 rounds to 1 in bf16 (ties to even), 3 (1 + 2^-8) = 3 + 3/256 rounds to 3 + 2^-6
    stored = bf16_bits_to_f64(Ws)
    _close(stored, [[1.0, 1.0, 1.0, 3.0 + 2.0 ** -6], [2.0, -1.0, 0.5, 0.0]], rtol=0, atol=0)
    _close(c, [6.0 + 2.0 ** -6, 1.5], rtol=0, atol=0)
    _close(b, [0.5 + 0.25 - 0.5 + 6.0 + 1.0, 1.0 - 0.25 - 0.25 + 0.0 - 2.0], rtol=0, atol=0)
    _, c0, b0 = oracle.fold_layernorm(W, g, None, None, "bf16")
    _close(b0, [0.0, 0.0], rtol=0, atol=0)


# --------------------------------------------------------------------------
# fp8 (OCP E4M3) per-channel quantisation of the folded weight
# --------------------------------------------------------------------------

def test_e4m3_golden_codes():
    """Code points fixed by the OCP 8-bit floating point specification's E4M3
    format: 0x38 = 1, 0x3C = 1.5, 0x40 = 2, 0xB8 = -1, 0x7E = 448 (largest),
    0x08 = 2^-6 (smallest normal), 0x01 = 2^-9 (smallest subnormal),
    0x07 = 7 * 2^-9, 0x7F and 0xFF NaN."""
    want = {0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0xB8: -1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
            0x07: 7 * 2.0 ** -9, 0x00: 0.0}
    for c, v in want.items():
        assert oracle.e4m3_value(np.uint8(c)) == v
        assert oracle.e4m3_code(np.float64(v)) == c
    assert np.isnan(oracle.e4m3_value(np.uint8(0x7F))) and np.isnan(oracle.e4m3_value(np.uint8(0xFF)))
    assert oracle.e4m3_code(np.float64(-0.0)) == 0x80


def test_e4m3_matches_torch_float8():
    """torch's float8_e4m3fn, a library routine: decoding of all 256 codes and
    round-to-nearest-even of 2^16 random float32 values within +-448."""
    codes = torch.arange(256, dtype=torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ov = oracle.e4m3_value(codes.numpy())
    assert np.array_equal(np.isnan(tv), np.isnan(ov))
    assert np.array_equal(tv[~np.isnan(tv)], ov[~np.isnan(ov)])
    rng = np.random.default_rng(40)
    f = (rng.standard_normal(1 << 16) * np.exp2(rng.uniform(-12, 8, 1 << 16))).astype(np.float32)
    f = np.clip(f, -448, 448)
    tb = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ob = oracle.e4m3_code(oracle.round_to_e4m3(f.astype(np.float64)))
    assert np.array_equal(tb, ob)


def test_e4m3_ties_and_saturation():
    r = oracle.round_to_e4m3
    _close(r(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 460.0, 1e6, -1e6, 464.0])),
           [1.0, 1.25, 0.0, 2.0 ** -8, 448.0, 448.0, -448.0, 448.0], rtol=0, atol=0)


def test_quantize_fp8_golden_row_and_exact_cases():
    """Row [1, -0.5, 0.25, 0.1]: amax 1, q = float32(1/448), codes
    448 -> 0x7E, -224 -> 0xF6, 112 -> 0x6E, 44.8 -> 44 = 1.375 * 2^5 -> 0x63.
    A zero row gets q = 1 and zero codes.  A row whose values are E4M3 values
    times 2^k with amax = 448 * 2^k quantises exactly, so the deferred product
    on it equals the deferred product on the unquantised weight."""
    W = np.array([[1.0, -0.5, 0.25, 0.1], [0.0, 0.0, 0.0, 0.0]])
    codes, q = oracle.quantize_fp8_per_channel(W)
    assert q.dtype == np.float32 and q[0] == np.float32(np.float64(1.0) / 448.0) and q[1] == 1.0
    assert codes.tolist() == [[0x7E, 0xF6, 0x6E, 0x63], [0, 0, 0, 0]]
    rng = np.random.default_rng(41)
    vals = oracle.e4m3_value(rng.integers(0, 0x7E, size=(6, 32)).astype(np.uint8))
    vals[:, 0] = 448.0
    Wx = vals * np.exp2(rng.integers(-12, -4, size=(6, 1)))
    c2, q2 = oracle.quantize_fp8_per_channel(Wx)
    _close(oracle.dequantize_fp8(c2, q2), Wx, rtol=0, atol=0)
    x = rng.standard_normal((3, 32))
    _close(oracle.deferred_on_quantized(x, c2, q2, 1e-6), oracle.deferred_on_folded(x, Wx, 1e-6), rtol=1e-14,
           atol=1e-15)


def test_glu_on_quantized_hand_worked():
    """The SiLU-GLU on fp8 gate and up weights, worked by hand.  x = [3, -3,
    3, -3] with eps 0 has rms 3, so RMSNorm(x) = [1, -1, 1, -1] (unit gain).
    Gate row W*_g = [3.5, 1.5, 0, 0]: amax 3.5 -> q_g = 3.5/448 = 2^-7, codes
    448 = 1.75 * 2^8 -> 0x7E and 192 = 1.5 * 2^7 -> 0x74 (both exact), a = 3.5 - 1.5 = 2.
    Up row W*_u = [1.75, 0, 0, 0.75]: q_u = 2^-8,
    b = 1.75 - 0.75 = 1 (codes 0x7E and 0x74).  h = SiLU(2) * 1 = 2 / (1 + e^-2) = 1.7615941559...
    Gate and up swapped would give SiLU(1) * 2 = 1.4621171572..., and so
    would the two channel scales swapped."""
    x = np.array([[3.0, -3.0, 3.0, -3.0]])
    cg, qg = oracle.quantize_fp8_per_channel(np.array([[3.5, 1.5, 0.0, 0.0]]))
    cu, qu = oracle.quantize_fp8_per_channel(np.array([[1.75, 0.0, 0.0, 0.75]]))
    assert qg[0] == 2.0 ** -7 and qu[0] == 2.0 ** -8
    assert cg.tolist() == [[0x7E, 0x74, 0, 0]] and cu.tolist() == [[0x7E, 0, 0, 0x74]]
    h = oracle.glu_deferred_on_quantized(x, cg, qg, cu, qu, 0.0)
    _close(h, [[2.0 / (1.0 + math.exp(-2.0))]], rtol=1e-15)


def test_glu_on_quantized_equals_textbook_glu_on_dequantised():
    """The deferred form on fp8 codes and channel scales equals the textbook
    RMSNorm (unit gain, the gain being folded into the quantised weights) ->
    gate and up projections of the dequantised weights -> SiLU(a) * b, to
    float64 rounding.  Gate and up differ in scale (amax differs per row and
    between the two), so a swapped weight or scale does not cancel out."""
    rng = np.random.default_rng(43)
    M, K, N = 5, 48, 7
    x = rng.standard_normal((M, K)) * np.exp(0.5 * rng.standard_normal((M, 1)))
    g = 1 + 0.1 * rng.standard_normal(K)
    Wg = rng.standard_normal((N, K)) / math.sqrt(K)
    Wu = 3.0 * rng.standard_normal((N, K)) / math.sqrt(K)
    cg, qg = oracle.quantize_fp8_per_channel(Wg * g)
    cu, qu = oracle.quantize_fp8_per_channel(Wu * g)
    want = oracle.norm_glu_ffn(x, oracle.dequantize_fp8(cg, qg), oracle.dequantize_fp8(cu, qu), np.ones(K), 1e-6)
    got = oracle.glu_deferred_on_quantized(x, cg, qg, cu, qu, 1e-6)
    _close(got, want, rtol=1e-12, atol=1e-14)


def test_fp8_activations_hand_worked():
    """Both operands in fp8.  x = [3, -3, 3, -3], eps 0: rms 3.  Quantised
    per row, amax 3 gives q_x = float32(3/448) and codes 448 -> 0x7E (3 /
    q_x is within 2^-24 relative of 448, and the E4M3 spacing there is 32),
    so the dequantised row is 448 q_x [1, -1, 1, -1].  Gate row W*_g =
    [3.5, 1.5, 0, 0] (exact codes, q_g = 2^-7), up row W*_u = [1.75, 0, 0,
    0.75] (q_u = 2^-8).  Deferred: a = (448 q_x)(3.5 - 1.5) / 3 = 896 q_x / 3,
    b = 448 q_x / 3.  Textbook: RMSNorm(x) = [1, -1, 1, -1] quantises with
    q = float32(1/448), a = 896 float32(1/448).  Both are 2 up to the float32
    rounding of the scales, which these pins resolve: the row scale must come
    from x, not from its quantised copy (that would give exactly 2)."""
    x = np.array([[3.0, -3.0, 3.0, -3.0]])
    cg, qg = oracle.quantize_fp8_per_channel(np.array([[3.5, 1.5, 0.0, 0.0]]))
    cu, qu = oracle.quantize_fp8_per_channel(np.array([[1.75, 0.0, 0.0, 0.75]]))
    qx = float(np.float32(3.0 / 448.0))
    assert 896.0 * qx / 3.0 != 2.0
    _close(oracle.deferred_fp8_act(x, cg, qg, 0.0), [[896.0 * qx / 3.0]], rtol=1e-15, atol=0)
    _close(oracle.norm_linear_fp8_act(x, cg, qg, 0.0), [[896.0 * float(np.float32(1.0 / 448.0))]], rtol=1e-15,
           atol=0)
    a, b = 896.0 * qx / 3.0, 448.0 * qx / 3.0
    _close(oracle.glu_deferred_fp8_act(x, cg, qg, cu, qu, 0.0), [[a / (1.0 + math.exp(-a)) * b]], rtol=1e-15, atol=0)


def test_fp8_activations_ties_on_bf16_inputs():
    """With bf16 inputs, x / q_x often lands exactly on a midpoint between
    two E4M3 values (both have few significant bits), and quantising x or
    RMSNorm(x) then resolves the tie by the float32 rounding of two
    different scales.  The codes may differ there, by one step, and only
    there: every element whose codes differ has x / q_x within 2^-22
    (relative) of a midpoint, and its two values are adjacent."""
    from synth import bf16_bits_from_f32
    rng = np.random.default_rng(46)
    M, K = 64, 512
    x = bf16_bits_to_f64(bf16_bits_from_f32((rng.standard_normal((M, K)) *
                                             np.exp(0.5 * rng.standard_normal((M, 1)))).astype(np.float32)))
    cx, qx = oracle.quantize_fp8_per_channel(x)
    cxn, _ = oracle.quantize_fp8_per_channel(oracle.rmsnorm(x, np.ones(K), 1e-6))
    flip = cx != cxn
    assert flip.any(), "no tie in the sample (the test needs one)"
    v = np.abs(x / qx[:, None].astype(np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    step = np.exp2(e - 3)
    mid = np.floor(v / step) * step + step / 2
    assert np.all(np.abs(v[flip] - mid[flip]) <= 2.0 ** -22 * v[flip])
    va, vb = np.abs(oracle.e4m3_value(cx[flip])), np.abs(oracle.e4m3_value(cxn[flip]))
    assert np.all(np.abs(va - vb) == step[flip])


def test_fp8_activations_deferred_equals_textbook():
    """Per-row quantisation is invariant to the positive row scale, so the
    codes of x and of RMSNorm(x) coincide (for these float64 inputs at every
    element: a flip needs x / q within float32 rounding of an E4M3 midpoint,
    which random float64 values do not hit), and the deferred form equals
    the textbook one to the float32 rounding of the scales.  The rows differ in scale and the gate and up
    weights in magnitude, so a transposed quantisation axis or swapped
    operands do not cancel."""
    rng = np.random.default_rng(44)
    M, K, N = 6, 64, 9
    x = rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))
    Wg = rng.standard_normal((N, K)) / math.sqrt(K)
    Wu = 2.5 * rng.standard_normal((N, K)) / math.sqrt(K)
    cg, qg = oracle.quantize_fp8_per_channel(Wg)
    cu, qu = oracle.quantize_fp8_per_channel(Wu)
    cx, _ = oracle.quantize_fp8_per_channel(x)
    cxn, _ = oracle.quantize_fp8_per_channel(oracle.rmsnorm(x, np.ones(K), 1e-6))
    assert np.array_equal(cx, cxn)
    _close(oracle.deferred_fp8_act(x, cg, qg, 1e-6), oracle.norm_linear_fp8_act(x, cg, qg, 1e-6), rtol=1e-6,
           atol=1e-12)
    _close(oracle.glu_deferred_fp8_act(x, cg, qg, cu, qu, 1e-6), oracle.glu_fp8_act(x, cg, qg, cu, qu, 1e-6),
           rtol=1e-6, atol=1e-12)


def test_fp8_activations_exact_when_x_is_representable():
    """Rows of x that are E4M3 values times 2^k with amax 448 * 2^k quantise
    exactly, so the fp8-activation forms equal the weight-only fp8 forms."""
    rng = np.random.default_rng(45)
    vals = oracle.e4m3_value(rng.integers(0, 0x7E, size=(4, 32)).astype(np.uint8))
    vals[:, 3] = -448.0
    x = vals * np.exp2(rng.integers(-10, -2, size=(4, 1)))
    W = rng.standard_normal((5, 32)) / math.sqrt(32)
    cw, qw = oracle.quantize_fp8_per_channel(W)
    _close(oracle.deferred_fp8_act(x, cw, qw, 1e-6), oracle.deferred_on_quantized(x, cw, qw, 1e-6), rtol=1e-14,
           atol=1e-15)
    cu, qu = oracle.quantize_fp8_per_channel(2 * W[::-1])
    _close(oracle.glu_deferred_fp8_act(x, cw, qw, cu, qu, 1e-6),
           oracle.glu_deferred_on_quantized(x, cw, qw, cu, qu, 1e-6), rtol=1e-14, atol=1e-15)


def test_quantize_fp8_error_bound():
    """Every dequantised weight is within half an E4M3 spacing (times q) of
    W*: relative 2^-4 for normal values, absolute 2^-10 q below 2^-6 q; each
    row's largest magnitude maps to 448."""
    rng = np.random.default_rng(42)
    W = rng.standard_normal((16, 200)) * np.exp2(rng.integers(-8, 3, size=(16, 1)))
    codes, q = oracle.quantize_fp8_per_channel(W)
    dq = oracle.dequantize_fp8(codes, q)
    v = np.abs(W) / q[:, None].astype(np.float64)
    bound = np.where(v >= 2.0 ** -6, np.abs(W) * 2.0 ** -4, q[:, None] * 2.0 ** -10)
    assert np.all(np.abs(dq - W) <= bound * (1 + 1e-12))
    assert np.all(np.max(np.abs(oracle.e4m3_value(codes)), axis=1) == 448.0)


# --------------------------------------------------------------------------
# MLA attention input with latent normalisation
# --------------------------------------------------------------------------

def test_latent_norm_closed_form():
    """x = [1,1,1,1] (rms 1, eps 0, unit g1).  q latent (width 4): u = [2,0,0,0],
    mean square 1 -> u * g_q with g_q = [0.5,1,1,1] -> [1,0,0,0].  kv latent
    (width 8): u = 3 * ones, rms 3 -> ones * g_kv.  Rope part (width 4):
    u = [1,0,0,0], not normalised, turned at position 3 (theta_0 = 1):
    [cos 3, sin 3, 0, 0]."""
    x = np.ones((1, 4))
    W = np.zeros((16, 4))
    W[0, 0] = 2.0
    W[4:12, :] = 0.75
    W[12, 0] = 1.0
    gq = np.array([0.5, 1.0, 1.0, 1.0])
    gkv = np.linspace(0.5, 1.2, 8)
    y = oracle.linear_latent_norm(x, W, np.ones(4), 0.0, 4, 8, 4, gq, gkv, 0.0, positions=[3], base=10000.0,
                                  rot_dim=4)
    _close(y[0, :4], [1, 0, 0, 0], rtol=0, atol=0)
    _close(y[0, 4:12], gkv, rtol=1e-15)
    _close(y[0, 12:], [math.cos(3), math.sin(3), 0, 0], rtol=1e-15, atol=1e-16)


def test_latent_norm_is_over_the_whole_latent():
    """With unit gains and eps 0 each latent has mean square 1 over its whole
    width, while its two halves (of different scale) do not."""
    rng = np.random.default_rng(50)
    K, nq, nkv = 16, 64, 32
    x = rng.standard_normal((3, K))
    W = rng.standard_normal((nq + nkv, K))
    W[:nq // 2] *= 4.0
    y = oracle.linear_latent_norm(x, W, np.ones(K), 0.0, nq, nkv, 0, np.ones(nq), np.ones(nkv), 0.0)
    _close(np.mean(y[:, :nq] ** 2, axis=1), np.ones(3), rtol=1e-13)
    _close(np.mean(y[:, nq:] ** 2, axis=1), np.ones(3), rtol=1e-13)
    assert np.all(np.abs(np.mean(y[:, :nq // 2] ** 2, axis=1) - 1) > 0.5)


def test_latent_scale_invariance_drops_first_norm():
    """Dropping the pre-attention RMSNorm (folding its gain) leaves the
    latents unchanged for eps_latent = 0; the rope part then needs the
    deferred row scale."""
    rng = np.random.default_rng(51)
    K = 24
    x = rng.standard_normal((5, K)) * np.exp(rng.standard_normal((5, 1)))
    W = rng.standard_normal((32 + 16 + 8, K))
    g1 = 1 + 0.1 * rng.standard_normal(K)
    gq, gkv = 1 + 0.1 * rng.standard_normal(32), 1 + 0.1 * rng.standard_normal(16)
    pos = [0, 7, 100, 4095, 12]
    ref = oracle.linear_latent_norm(x, W, g1, 1e-6, 32, 16, 8, gq, gkv, 0.0, pos, 10000.0, 8)
    got = oracle.latent_dropped_on_folded(x, W * g1[None, :], 1e-6, 32, 16, 8, gq, gkv, 0.0, pos, 10000.0, 8)
    _close(got, ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# the comparison metric itself
# --------------------------------------------------------------------------

def test_check_close_metric():
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])
    y = np.array([[3.0, 4.05], [0.0, 0.001]])
    ok, info = oracle.check_close(y, ref, 1e-2, 0.06)
    assert ok and abs(info["max_rel_l2"] - 0.01) < 1e-12 and abs(info["max_abs"] - 0.05) < 1e-12
    ok, _ = oracle.check_close(y, ref, 5e-3, 0.06)
    assert not ok
    ok, _ = oracle.check_close(y, ref, 1e-2, 0.04)
    assert not ok
    # bf16 output: half an ulp of |ref| is added to the max-abs bound
    ref2 = np.array([[20.0, 1.0]])
    ok, _ = oracle.check_close(np.array([[20.0625, 1.0]]), ref2, 1e-2, 0.0, out_is_bf16=True)
    assert ok
    ok, _ = oracle.check_close(np.array([[20.07, 1.0]]), ref2, 1e-2, 0.0, out_is_bf16=True)
    assert not ok
    nanref = np.array([[np.nan, np.nan], [1.0, 2.0]])
    assert oracle.check_close(nanref.copy(), nanref, 1e-9, 0.0)[0]
    assert not oracle.check_close(np.array([[0.0, 0.0], [1.0, 2.0]]), nanref, 1e-9, 0.0)[0]
