"""Float64 definitions of RMSNorm -> linear, its GLU and QK-norm variants,
and of the offline weight fold.  TEST INFRASTRUCTURE ONLY (see package doc).

Notation (row-major, float64 unless stated):
  x  [M x K]  activations, one token per row
  g  [K]      RMSNorm gain
  W  [N x K]  projection weight in checkpoint layout (out x in); the layer
              computes x . W^T
  eps         added to the mean square inside the root

Every function upcasts its stored inputs exactly (float32 or bf16 bit
patterns, see ``synth.stored_to_f64``) and computes in float64 with numpy;
matrix products use numpy's float64 matmul as a library step.
"""

from __future__ import annotations

import numpy as np

from synth import stored_to_f64


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return stored_to_f64(a)
    return a.astype(np.float64)


# ---------------------------------------------------------------------------
# RMSNorm (Root Mean Square Layer Normalization; FlashNorm Abstract, the
# normalisation that precedes the linear layer)
# ---------------------------------------------------------------------------

def rms(x, eps: float) -> np.ndarray:
    """Per-row root mean square: r[m] = sqrt(mean_k x[m,k]^2 + eps).

    The mean runs over the true row length K.  eps sits inside the root,
    added to the mean square.
    """
    x = _f64(x)
    K = x.shape[-1]
    ms = np.sum(x * x, axis=-1) / K
    return np.sqrt(ms + float(eps))


def rmsnorm(x, g, eps: float) -> np.ndarray:
    """Textbook RMSNorm: divide each row by its RMS, then multiply by g."""
    x = _f64(x)
    r = rms(x, eps)
    with np.errstate(divide="ignore", invalid="ignore"):
        return (x / r[..., None]) * _f64(g)


def norm_linear(x, W, g, eps: float) -> np.ndarray:
    """RMSNorm then a bias-free linear layer: y = RMSNorm(x; g) . W^T.

    This is the unfolded, undeferred norm-then-project operation that
    FlashNorm rewrites (Abstract, first sentence of the method).
    """
    return rmsnorm(x, g, eps) @ _f64(W).T


def silu(t) -> np.ndarray:
    """SiLU(t) = t * sigmoid(t) = t / (1 + exp(-t))."""
    t = np.asarray(t, dtype=np.float64)
    with np.errstate(over="ignore"):
        return t / (1.0 + np.exp(-t))


def norm_glu_ffn(x, W_gate, W_up, g, eps: float) -> np.ndarray:
    """RMSNorm, then the gate and up projections of a SiLU-gated FFN:
    h = SiLU(xn . W_gate^T) * (xn . W_up^T), xn = RMSNorm(x; g).

    The Abstract lists feed-forward networks with GLU variants among the
    layers the technique extends to; SwiGLU is the GLU variant used here.
    """
    xn = rmsnorm(x, g, eps)
    a = xn @ _f64(W_gate).T
    b = xn @ _f64(W_up).T
    return silu(a) * b


def head_rmsnorm(u, gain, eps_h: float, head_dim: int) -> np.ndarray:
    """RMSNorm over each run of ``head_dim`` columns of u.

    ``gain`` is [head_dim] (shared by every head) or [n_heads, head_dim];
    ``None`` means a unit gain.
    """
    u = _f64(u)
    M, C = u.shape
    H = C // head_dim
    uh = u.reshape(M, H, head_dim)
    ms = np.sum(uh * uh, axis=-1) / head_dim
    with np.errstate(divide="ignore", invalid="ignore"):
        y = uh / np.sqrt(ms + float(eps_h))[..., None]
    if gain is not None:
        gg = _f64(gain)
        y = y * (gg[None, None, :] if gg.ndim == 1 else gg[None, :, :])
    return y.reshape(M, C)


def linear_qknorm(x, W_qkv, g1, eps_x: float, n_q_heads: int, n_kv_heads: int,
                  head_dim: int, g_q, g_k, eps_head: float, v_mode: int = 0) -> np.ndarray:
    """Attention input with QK-norm, the pre-attention RMSNorm *present*:

      u = RMSNorm(x; g1, eps_x) . W_qkv^T, columns [q heads | k heads | v heads]
      q and k heads: per-head RMSNorm with gains g_q / g_k and eps_head
      v heads: u itself (v_mode 0) or a unit-gain per-head RMSNorm (v_mode 1)

    The GPU path drops the first RMSNorm for the q and k heads by scale
    invariance (Abstract, the RMSNorm -> linear -> RMSNorm simplification);
    this oracle keeps it, so agreement shows the simplification holds.
    """
    u = norm_linear(x, W_qkv, g1, eps_x)
    nq = n_q_heads * head_dim
    nk = n_kv_heads * head_dim
    q = head_rmsnorm(u[:, :nq], g_q, eps_head, head_dim)
    k = head_rmsnorm(u[:, nq:nq + nk], g_k, eps_head, head_dim)
    v = u[:, nq + nk:]
    if v_mode == 1:
        v = head_rmsnorm(v, None, eps_head, head_dim)
    elif v_mode != 0:
        raise ValueError("v_mode must be 0 or 1")
    return np.concatenate([q, k, v], axis=1)


# ---------------------------------------------------------------------------
# Rounding to a storage dtype, written from the definition of round to
# nearest, ties to even: find the spacing of representable values around d,
# count d in units of that spacing, round that count half-to-even.
# ---------------------------------------------------------------------------

def _round_to_format(d, sig_bits: int, min_exp: int, max_exp: int) -> np.ndarray:
    """Round float64 values once to a binary format with ``sig_bits``
    significant bits, smallest normal 2**min_exp and largest binade
    [2**max_exp, 2**(max_exp+1)).  Out-of-range results become +-inf."""
    d = np.asarray(d, dtype=np.float64)
    out = d.copy()
    fin = np.isfinite(d)
    v = d[fin]
    _, e = np.frexp(v)  # |v| in [2**(e-1), 2**e)
    # spacing inside that binade; never below the subnormal spacing
    q = np.maximum(e - sig_bits, min_exp - (sig_bits - 1))
    n = np.ldexp(v, -q)          # exact: scaling by a power of two
    r = np.rint(n)               # nearest integer, ties to even
    res = np.ldexp(r, q)
    big = np.abs(res) >= np.ldexp(1.0, max_exp + 1)
    res[big] = np.copysign(np.inf, res[big])
    out[fin] = res
    return out


def round_to_bf16(d) -> np.ndarray:
    """float64 -> nearest bf16 value (8 significant bits), as float64."""
    return _round_to_format(d, 8, -126, 127)


def round_to_f32(d) -> np.ndarray:
    """float64 -> nearest float32 value (24 significant bits), as float64."""
    return _round_to_format(d, 24, -126, 127)


def _bf16_bits_of_values(v: np.ndarray) -> np.ndarray:
    """Bit patterns of values that are already exactly bf16 (float64 in)."""
    f = v.astype(np.float32)  # exact, every bf16 value is a float32 value
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def fold_weights(W, g, out_dtype: str) -> np.ndarray:
    """Offline weight fold W*[n,k] = g[k] * W[n,k] (FlashNorm Abstract,
    point (i): the normalisation weights are folded into the next linear
    layer; the summary page's "Weight Folding" bullet: done offline).

    The product is exact in float64 (at most 24 + 24 significant bits) and
    is rounded once to ``out_dtype`` ("f32" -> float32 array, "bf16" ->
    uint16 bit patterns), which is the storage the GPU reads.
    """
    prod = _f64(W) * _f64(g)[None, :]
    if out_dtype == "f32":
        return round_to_f32(prod).astype(np.float32)
    if out_dtype == "bf16":
        return _bf16_bits_of_values(round_to_bf16(prod))
    raise ValueError(out_dtype)


# ---------------------------------------------------------------------------
# The same computations on the *stored folded* weights, in the deferred
# order the method uses: contract first, scale the output rows afterwards
# (Abstract, point (ii)).  They isolate kernel error from fold rounding.
# ---------------------------------------------------------------------------

def deferred_on_folded(x, W_star, eps: float) -> np.ndarray:
    """y = (x . W*^T) * s[m], s[m] = 1 / sqrt(mean_k x[m,k]^2 + eps)."""
    z = _f64(x) @ _f64(W_star).T
    with np.errstate(divide="ignore", invalid="ignore"):
        return z / rms(x, eps)[:, None]


def glu_deferred_on_folded(x, Wg_star, Wu_star, eps: float) -> np.ndarray:
    """h = SiLU(s * (x . Wg*^T)) * (s * (x . Wu*^T)); the row scale goes in
    before the SiLU, which is where RMSNorm puts it."""
    a = deferred_on_folded(x, Wg_star, eps)
    b = deferred_on_folded(x, Wu_star, eps)
    return silu(a) * b


def qknorm_dropped_on_folded(x, Wqkv_star, eps_x: float, n_q_heads: int, n_kv_heads: int,
                             head_dim: int, g_q, g_k, eps_head: float, v_mode: int = 0) -> np.ndarray:
    """QK-norm attention input with the first RMSNorm dropped for q and k:
    z = x . W*^T; q/k heads get per-head RMSNorm of z directly; v heads get
    z * s[m] (v_mode 0) or a unit-gain per-head RMSNorm of z (v_mode 1)."""
    z = _f64(x) @ _f64(Wqkv_star).T
    nq = n_q_heads * head_dim
    nk = n_kv_heads * head_dim
    q = head_rmsnorm(z[:, :nq], g_q, eps_head, head_dim)
    k = head_rmsnorm(z[:, nq:nq + nk], g_k, eps_head, head_dim)
    if v_mode == 0:
        with np.errstate(divide="ignore", invalid="ignore"):
            v = z[:, nq + nk:] / rms(x, eps_x)[:, None]
    elif v_mode == 1:
        v = head_rmsnorm(z[:, nq + nk:], None, eps_head, head_dim)
    else:
        raise ValueError("v_mode must be 0 or 1")
    return np.concatenate([q, k, v], axis=1)


# ---------------------------------------------------------------------------
# Rotary position embedding after the head norms (FlashNorm Abstract: the
# techniques extend to RoPE-based attention).  The rotation itself follows
# its published definition (RoFormer: Enhanced Transformer with Rotary
# Position Embedding, Section 3.2, the general form): the rotated part of a
# head is cut into consecutive pairs (2i, 2i+1), and pair i of the token at
# position p turns by the angle p * theta_i, theta_i = base^(-2i/d), where d
# is the number of rotated columns.
# ---------------------------------------------------------------------------

def rope_angles(positions, base: float, rot_dim: int) -> np.ndarray:
    """[M, rot_dim/2] angles p[m] * base^(-2i/rot_dim), in float64."""
    if rot_dim <= 0 or rot_dim % 2:
        raise ValueError("rot_dim must be a positive even number")
    p = np.asarray(positions, dtype=np.float64)
    i = np.arange(rot_dim // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * i / rot_dim)
    return p[:, None] * theta[None, :]


def rope(u, positions, base: float, rot_dim: int, head_dim: int) -> np.ndarray:
    """Rotate every head of u (columns in runs of ``head_dim``): in each
    head, pair (2i, 2i+1) with i < rot_dim/2 becomes
    (a cos t - b sin t, a sin t + b cos t), t = p[m] * theta_i; the columns
    from rot_dim on are left as they are."""
    u = _f64(u)
    M, C = u.shape
    if rot_dim > head_dim:
        raise ValueError("rot_dim must not exceed head_dim")
    t = rope_angles(positions, base, rot_dim)
    c, s = np.cos(t)[:, None, :], np.sin(t)[:, None, :]
    uh = u.reshape(M, C // head_dim, head_dim).copy()
    a = uh[:, :, 0:rot_dim:2].copy()
    b = uh[:, :, 1:rot_dim:2].copy()
    uh[:, :, 0:rot_dim:2] = a * c - b * s
    uh[:, :, 1:rot_dim:2] = a * s + b * c
    return uh.reshape(M, C)


def linear_qknorm_rope(x, W_qkv, g1, eps_x: float, n_q_heads: int, n_kv_heads: int,
                       head_dim: int, g_q, g_k, eps_head: float, v_mode: int,
                       positions, base: float, rot_dim: int) -> np.ndarray:
    """``linear_qknorm`` (first RMSNorm present), then the rotary embedding
    of every q and k head at the token's position; v heads are not rotated.
    The rotation comes after the head norm's gain, the order of a
    QK-normalised attention block."""
    y = linear_qknorm(x, W_qkv, g1, eps_x, n_q_heads, n_kv_heads, head_dim, g_q, g_k,
                      eps_head, v_mode)
    nqk = (n_q_heads + n_kv_heads) * head_dim
    y[:, :nqk] = rope(y[:, :nqk], positions, base, rot_dim, head_dim)
    return y


# ---------------------------------------------------------------------------
# LayerNorm followed by a linear layer (FlashNorm Abstract: the same
# techniques extend to LayerNorm).  LayerNorm as defined in Layer
# Normalization (Ba, Kiros and Hinton, Section 3): subtract the row mean,
# divide by the root of the (biased) variance plus eps, then gain and bias.
# ---------------------------------------------------------------------------

def layernorm(x, g, beta, eps: float) -> np.ndarray:
    """Textbook LayerNorm: mu = mean_k x, var = mean_k (x - mu)^2,
    (x - mu) / sqrt(var + eps) * g + beta (beta None = 0)."""
    x = _f64(x)
    K = x.shape[-1]
    mu = np.sum(x, axis=-1) / K
    d = x - mu[..., None]
    var = np.sum(d * d, axis=-1) / K
    with np.errstate(divide="ignore", invalid="ignore"):
        y = d / np.sqrt(var + float(eps))[..., None] * _f64(g)
    if beta is not None:
        y = y + _f64(beta)
    return y


def layernorm_linear(x, W, g, beta, bias, eps: float) -> np.ndarray:
    """LayerNorm then a linear layer with optional bias:
    y = LayerNorm(x; g, beta) . W^T + bias (bias None = 0)."""
    y = layernorm(x, g, beta, eps) @ _f64(W).T
    if bias is not None:
        y = y + _f64(bias)
    return y


def fold_layernorm(W, g, beta, bias, out_dtype: str):
    """Offline fold for the deferred LayerNorm form: W* = round(g * W) as in
    ``fold_weights``, c[n] = sum_k W*[n,k] over the *stored* W*, and
    b*[n] = sum_k beta[k] W[n,k] + bias[n], the last two rounded once to
    float32.  Returns (W*, c, b*)."""
    Ws = fold_weights(W, g, out_dtype)
    c = np.sum(_f64(Ws), axis=1)
    b = np.zeros(_f64(W).shape[0]) if beta is None else _f64(W) @ _f64(beta)
    if bias is not None:
        b = b + _f64(bias)
    return Ws, round_to_f32(c).astype(np.float32), round_to_f32(b).astype(np.float32)


def layernorm_deferred_on_folded(x, W_star, c, b_star, eps: float) -> np.ndarray:
    """The deferred form on stored folded operands:
    y = s[m] (z[m,n] - mu[m] c[n]) + b*[n], z = x . W*^T,
    s = 1 / sqrt(var + eps), mu and var the row's mean and biased variance."""
    x = _f64(x)
    K = x.shape[-1]
    mu = np.sum(x, axis=-1) / K
    d = x - mu[:, None]
    var = np.sum(d * d, axis=-1) / K
    z = x @ _f64(W_star).T
    with np.errstate(divide="ignore", invalid="ignore"):
        s = 1.0 / np.sqrt(var + float(eps))
    return s[:, None] * (z - mu[:, None] * _f64(c)[None, :]) + _f64(b_star)[None, :]


# ---------------------------------------------------------------------------
# fp8 folded weights (FlashNorm: the folded checkpoint stays compatible with
# quantized models; the summary page's "Results" bullet).  Fold first, then
# quantize W* per output channel to OCP FP8 E4M3 (1 sign, 4 exponent bits
# with bias 7, 3 mantissa bits, no infinities, largest finite 448, smallest
# normal 2^-6, subnormal spacing 2^-9; the OCP 8-bit floating point
# specification, E4M3 format).  The dequantisation scale of channel n
# multiplies the product's output together with the deferred row scale.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def round_to_e4m3(d) -> np.ndarray:
    """float64 -> nearest E4M3 value (ties to even), as float64; values
    beyond the largest finite one saturate to +-448."""
    r = _round_to_format(d, 4, -6, 8)
    return np.clip(r, -E4M3_MAX, E4M3_MAX)


def e4m3_code(v) -> np.ndarray:
    """Bit patterns (uint8) of values that are exactly E4M3 (float64 in)."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.uint8)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.uint8)  # exact: multiples of 2^-9
    m, e = np.frexp(a[~sub])  # a = m 2^e, m in [0.5, 1)
    exp_field = (e - 1 + 7).astype(np.uint8)
    mant = np.rint((m * 2 - 1) * 8).astype(np.uint8)  # exact: 3 fraction bits
    code[~sub] = (exp_field << 3) | mant
    return code | sign


def e4m3_value(code) -> np.ndarray:
    """float64 values of E4M3 bit patterns (0x7F and 0xFF are NaN)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = c & 0x7
    val = np.where(e == 0, f * 2.0 ** -9, (1 + f / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def quantize_fp8_per_channel(W_star):
    """Per-output-channel E4M3 quantisation of the folded weight:
    amax[n] = max_k |W*[n,k]|, scale q[n] = float32(amax[n] / 448) (the
    quotient formed in float64, then rounded once to float32; q = 1 for an
    all-zero row), code[n,k] = E4M3(W*[n,k] / q[n]) with the quotient in
    float64 (IEEE division) and one round to nearest even.  Returns
    (codes uint8 [N x K], q float32 [N])."""
    Wf = _f64(W_star)
    amax = np.max(np.abs(Wf), axis=1)
    q = round_to_f32(np.where(amax > 0, amax / E4M3_MAX, 1.0))
    codes = e4m3_code(round_to_e4m3(Wf / q[:, None]))
    return codes, q.astype(np.float32)


def dequantize_fp8(codes, q) -> np.ndarray:
    """W8[n,k] = q[n] * value(code[n,k]), float64."""
    return _f64(q)[:, None] * e4m3_value(codes)


def deferred_on_quantized(x, codes, q, eps: float) -> np.ndarray:
    """y = s[m] * sum_k x[m,k] * q[n] value(code[n,k]): the deferred form on
    the stored fp8 weight and its channel scales."""
    return deferred_on_folded(x, dequantize_fp8(codes, q), eps)


def glu_deferred_on_quantized(x, codes_g, q_g, codes_u, q_u, eps: float) -> np.ndarray:
    """The SiLU-GLU epilogue on fp8 gate and up weights."""
    return glu_deferred_on_folded(x, dequantize_fp8(codes_g, q_g), dequantize_fp8(codes_u, q_u), eps)


def norm_linear_fp8_act(x, codes_w, q_w, eps: float) -> np.ndarray:
    """RMSNorm -> linear with both operands in fp8, the textbook order: the
    unit-gain RMSNorm of x (the gain is folded into the quantised weight),
    that normalised activation quantised to E4M3 per row (the per-channel
    rule applied to the rows of the activation), dequantised, then the
    product with the dequantised weight."""
    xn = rmsnorm(x, np.ones(_f64(x).shape[-1]), eps)
    cx, qx = quantize_fp8_per_channel(xn)
    return dequantize_fp8(cx, qx) @ dequantize_fp8(codes_w, q_w).T


def deferred_fp8_act(x, codes_w, q_w, eps: float) -> np.ndarray:
    """The deferred form with fp8 activations: x itself quantised per row
    (codes cx, scales qx), the product of the dequantised operands, then the
    row scale s[m] = 1 / rms(x) of the unquantised x.  Per-row quantisation
    is invariant to a positive row scale (the scale cancels in x / amax(x)),
    so this equals ``norm_linear_fp8_act`` up to the float32 rounding of
    the quantisation scales."""
    with np.errstate(divide="ignore", invalid="ignore"):
        s = 1.0 / rms(x, eps)
    cx, qx = quantize_fp8_per_channel(x)
    return (dequantize_fp8(cx, qx) @ dequantize_fp8(codes_w, q_w).T) * s[:, None]


def glu_fp8_act(x, codes_g, q_g, codes_u, q_u, eps: float) -> np.ndarray:
    """SiLU-GLU with both operands in fp8, the textbook order (as
    ``norm_linear_fp8_act``, for the gate and the up projection)."""
    a = norm_linear_fp8_act(x, codes_g, q_g, eps)
    b = norm_linear_fp8_act(x, codes_u, q_u, eps)
    return silu(a) * b


def glu_deferred_fp8_act(x, codes_g, q_g, codes_u, q_u, eps: float) -> np.ndarray:
    """The deferred SiLU-GLU with fp8 activations: SiLU(s a) * (s b) with a
    and b the products of the per-row quantised x and the dequantised gate
    and up weights."""
    a = deferred_fp8_act(x, codes_g, q_g, eps)
    b = deferred_fp8_act(x, codes_u, q_u, eps)
    return silu(a) * b


# ---------------------------------------------------------------------------
# MLA attention input with latent normalisation (FlashNorm Abstract: the
# first RMSNorm of an RMSNorm -> linear -> RMSNorm chain can be eliminated,
# which removes the pre-attention RMSNorm in MLA models with latent
# normalisation).  One projection of x gives, side by side, the compressed
# query latent, the compressed key/value latent (each followed by its own
# RMSNorm) and the decoupled rotary key part, which no norm follows.
# ---------------------------------------------------------------------------

def linear_latent_norm(x, W, g1, eps_x: float, n_q_latent: int, n_kv_latent: int, n_rope: int,
                       g_q_latent, g_kv_latent, eps_latent: float, positions=None, base: float = 10000.0,
                       rot_dim: int = 0) -> np.ndarray:
    """u = RMSNorm(x; g1, eps_x) . W^T (the first RMSNorm *present*), columns
    [q latent | kv latent | rope part]; each latent gets its own RMSNorm
    (gain, eps_latent) over its whole width; the rope part is u itself,
    turned by the rotary embedding of the row's position when positions are
    given (rot_dim columns, the part as one head)."""
    u = norm_linear(x, W, g1, eps_x)
    return _latent_epilogue(u, n_q_latent, n_kv_latent, n_rope, g_q_latent, g_kv_latent, eps_latent,
                            positions, base, rot_dim, None)


def latent_dropped_on_folded(x, W_star, eps_x: float, n_q_latent: int, n_kv_latent: int, n_rope: int,
                             g_q_latent, g_kv_latent, eps_latent: float, positions=None, base: float = 10000.0,
                             rot_dim: int = 0) -> np.ndarray:
    """The same with the first RMSNorm dropped: z = x . W*^T; latents get
    their RMSNorm of z directly, the rope part z * s[m] (the deferred row
    scale), then the rotation."""
    z = _f64(x) @ _f64(W_star).T
    with np.errstate(divide="ignore", invalid="ignore"):
        s = 1.0 / rms(x, eps_x)
    return _latent_epilogue(z, n_q_latent, n_kv_latent, n_rope, g_q_latent, g_kv_latent, eps_latent,
                            positions, base, rot_dim, s)


def _latent_epilogue(u, nq, nkv, nr, g_q, g_kv, eps_l, positions, base, rot_dim, s_plain):
    if u.shape[1] != nq + nkv + nr:
        raise ValueError("W must have n_q_latent + n_kv_latent + n_rope rows")
    parts = []
    if nq:
        parts.append(head_rmsnorm(u[:, :nq], g_q, eps_l, nq))
    if nkv:
        parts.append(head_rmsnorm(u[:, nq:nq + nkv], g_kv, eps_l, nkv))
    if nr:
        p = u[:, nq + nkv:]
        if s_plain is not None:
            p = p * s_plain[:, None]
        if positions is not None:
            p = rope(p, positions, base, rot_dim, nr)
        parts.append(p)
    return np.concatenate(parts, axis=1)
