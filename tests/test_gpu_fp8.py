"""GPU parity of the fp8-weight path (fn_quantize_fp8, fn_norm_linear_fp8,
fn_norm_glu_ffn_fp8) through the C ABI against the float64 oracle.

The quantiser is integer work: its codes and scales must equal the oracle's
bit for bit.  The ops are compared with the deferred form on the oracle's own
codes and scales (kernel-only tolerance) and with the textbook RMSNorm ->
linear, or gate and up projections then SiLU-GLU, on the dequantised
weights (workload tolerance).  The quantisation
error against the unquantised model is printed, not graded.  Every case
prints its name and shape before it runs.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import KERNEL_REL_L2, assert_parity, assert_within, fp8_act_bounds, fp8_act_glu_bounds, from_dev, to_dev
from oracle.compare import _half_ulp_bf16
from synth import BF16, F32

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _w(M, K, N, name="llama7b_ffn_decode_m4_fp8"):
    return dataclasses.replace(synth.workload(name), M=M, K=K, N=N)


def _vec(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _codes_dev(c):
    return torch.from_numpy(np.ascontiguousarray(c)).cuda()


@pytest.mark.parametrize("dt", [BF16, F32])
@pytest.mark.parametrize("N,K", [(300, 528), (77, 4096), (40, 8208)])  # the last: rows longer than a thread keeps
def test_quantize_fp8_bit_exact(gpu_lib, dt, N, K):
    fn = gpu_lib
    w = dataclasses.replace(_w(1, K, N), dtype=dt)
    _say(f"quantize_fp8 {dt} N={N} K={K}")
    Ws = oracle.fold_weights(w.w(), w.g(), dt)
    codes_ref, q_ref = oracle.quantize_fp8_per_channel(Ws)
    codes, q = fn.quantize_fp8(to_dev(Ws))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy().view(np.uint32), q_ref.view(np.uint32))
    got = codes.cpu().numpy()
    bad = np.argwhere(got != codes_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:4].tolist()}"


def test_quantize_fp8_zero_row_and_full_gate(gpu_lib):
    fn = gpu_lib
    w = _w(1, 4096, 11008)
    _say("quantize_fp8: the folded Llama-7B gate weight 11008x4096, with a zero row")
    Ws = oracle.fold_weights(w.w(), w.g(), BF16)
    Ws[5] = 0
    codes_ref, q_ref = oracle.quantize_fp8_per_channel(Ws)
    codes, q = fn.quantize_fp8(to_dev(Ws))
    torch.cuda.synchronize()
    assert q_ref[5] == 1.0 and np.all(codes_ref[5] == 0)
    assert np.array_equal(q.cpu().numpy().view(np.uint32), q_ref.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), codes_ref)


def _e4m3_grid():
    """The 127 finite non-negative E4M3 values, by code (0 .. 0x7E)."""
    return np.array([float(oracle.e4m3_value(c)) for c in range(0x7F)])


def _bf16_neighbours(f32):
    """bf16 bit patterns of the values and their two bf16 neighbours."""
    b = synth.bf16_bits_from_f32(np.asarray(f32, dtype=np.float32)).astype(np.int64)
    return np.concatenate([b, b + 1, np.maximum(b - 1, 0)]).astype(np.uint16)


@pytest.mark.parametrize("dt", [BF16, F32])
def test_quantize_fp8_rounding_edges(gpu_lib, dt):
    """Rows built to hit the hard cases of the per-channel rounding, against
    the oracle's float64 division bit for bit: every E4M3 value and every
    midpoint between neighbours (exact ties when q is a power of two) with
    their bf16 neighbours, both signs and negative zero; a row whose scale
    is below 2^-96 (the float64 path); a row near the bf16 maximum; a row of
    subnormal bf16 values next to normal ones; a generic row."""
    fn = gpu_lib
    K = 2048  # holds each tie row whole (1518 values)
    grid = _e4m3_grid()
    mids = 0.5 * (grid[:-1] + grid[1:])
    rows = []
    for j in (0, -20, 30):  # q = 2^j exactly: amax = 448 * 2^j
        q = 2.0 ** j
        vals = np.concatenate([grid, mids]) * q
        b = _bf16_neighbours(vals)
        v = synth.bf16_bits_to_f64(b)
        v = v[np.abs(v) <= 448.0 * q]
        row = np.concatenate([v, -v, [448.0 * q, -0.0]])
        rows.append(row)
    rows.append(np.array([2.0 ** -100, 2.0 ** -101, 3 * 2.0 ** -103, -(2.0 ** -100)]))  # q < 2^-96
    rows.append(np.array([3.3895313892515355e38, -1.7e38, 2.5e37, 1e36, -3e30]))     # near the bf16 maximum
    sub = synth.bf16_bits_to_f64(np.arange(1, 128, dtype=np.uint16))                  # subnormal bf16
    rows.append(np.concatenate([sub, [2.0 ** -126, 1.5 * 2.0 ** -126, 2.0 ** -120]]))
    rng = np.random.default_rng(11)
    rows.append(rng.standard_normal(K) * 3.0)
    W = np.zeros((len(rows), K))
    for i, r in enumerate(rows):
        assert len(r) <= K
        W[i, :len(r)] = r
    if dt == BF16:
        Ws = synth.bf16_bits_from_f32(W.astype(np.float32))
    else:
        Ws = W.astype(np.float32)
    _say(f"quantize_fp8 rounding edges, {dt}, {len(rows)} rows of {K}")
    codes_ref, q_ref = oracle.quantize_fp8_per_channel(Ws)
    codes, q = fn.quantize_fp8(to_dev(Ws))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy().view(np.uint32), q_ref.view(np.uint32))
    got = codes.cpu().numpy()
    bad = np.argwhere(got != codes_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first {[(int(i), int(k), int(got[i, k]), int(codes_ref[i, k])) for i, k in bad[:6]]}"


FP8_CASES = [
    # M, K, N
    (1, 4096, 1000),
    (4, 528, 300),    # K not a multiple of the 64-wide step
    (16, 1040, 77),   # ragged N
    (5, 4096, 300),
]


@pytest.mark.parametrize("M,K,N", FP8_CASES)
def test_fp8_fused_parity(gpu_lib, M, K, N):
    fn = gpu_lib
    w = _w(M, K, N)
    _say(f"fp8 fused M={M} K={K} N={N}: linear and glu, f32 and bf16 out")
    Wg = oracle.fold_weights(w.w(), w.g(), BF16)
    Wu = oracle.fold_weights(w.w_up(), w.g(), BF16)
    cg, qg = oracle.quantize_fp8_per_channel(Wg)
    cu, qu = oracle.quantize_fp8_per_channel(Wu)
    x = to_dev(w.x())
    eps = w.eps_f32()
    ref_lin = oracle.deferred_on_quantized(w.x(), cg, qg, eps)
    ref_glu = oracle.glu_deferred_on_quantized(w.x(), cg, qg, cu, qu, eps)
    ones = np.ones(K)
    text_lin = oracle.norm_linear(w.x(), oracle.dequantize_fp8(cg, qg), ones, eps)
    text_glu = oracle.norm_glu_ffn(w.x(), oracle.dequantize_fp8(cg, qg), oracle.dequantize_fp8(cu, qu), ones, eps)
    for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
        y = fn.norm_linear_fp8(x, _codes_dev(cg), _vec(qg), eps, out_dtype=od)
        h = fn.norm_glu_ffn_fp8(x, _codes_dev(cg), _vec(qg), _codes_dev(cu), _vec(qu), eps, out_dtype=od)
        torch.cuda.synchronize()
        if od == torch.float32:
            assert_parity(y, ref_lin, BF16, "fp8 linear kernel-only", rel_l2=KERNEL_REL_L2, max_abs=np.inf)
            assert_parity(h, ref_glu, BF16, "fp8 glu kernel-only", rel_l2=KERNEL_REL_L2, max_abs=np.inf)
        assert_parity(y, text_lin, BF16, f"fp8 linear textbook {od}", out_bf16=ob)
        assert_parity(h, text_glu, BF16, f"fp8 glu textbook {od}", out_bf16=ob)


@pytest.mark.parametrize("M,K,N", [(4, 528, 300), (16, 4096, 300)])
def test_fp8_unfused_parity(gpu_lib, M, K, N):
    """The baseline quantises the unfolded weight and normalises x first."""
    fn = gpu_lib
    w = _w(M, K, N)
    _say(f"fp8 unfused M={M} K={K} N={N}")
    cg, qg = oracle.quantize_fp8_per_channel(w.w())
    cu, qu = oracle.quantize_fp8_per_channel(w.w_up())
    g = _vec(w.g())
    eps = w.eps_f32()
    ref = oracle.norm_glu_ffn(w.x(), oracle.dequantize_fp8(cg, qg), oracle.dequantize_fp8(cu, qu), w.g(), eps)
    h = fn.norm_glu_ffn_fp8(to_dev(w.x()), _codes_dev(cg), _vec(qg), _codes_dev(cu), _vec(qu), eps, g=g,
                            variant=fn.UNFUSED, out_dtype=torch.float32)
    assert_parity(h, ref, BF16, "fp8 glu unfused")
    ref_l = oracle.norm_linear(w.x(), oracle.dequantize_fp8(cg, qg), w.g(), eps)
    y = fn.norm_linear_fp8(to_dev(w.x()), _codes_dev(cg), _vec(qg), eps, g=g, variant=fn.UNFUSED,
                           out_dtype=torch.float32)
    assert_parity(y, ref_l, BF16, "fp8 linear unfused")


@pytest.mark.parametrize("name", ["llama7b_ffn_decode_m1_fp8", "llama7b_ffn_decode_m4_fp8",
                                  "llama7b_ffn_decode_m16_fp8"])
def test_full_fp8_decode_gpu_pipeline(gpu_lib, name):
    """Fold and quantise on the GPU, then the op, against the oracle's fold,
    quantisation and deferred form; the quantisation error against the bf16
    model is printed."""
    fn = gpu_lib
    w = synth.workload(name)
    _say(f"full {name}: GPU fold + quantise + fused op, M={w.M} K=4096 N=11008")
    g = _vec(w.g())
    Wg_d, Wu_d = fn.fold_weights(to_dev(w.w()), g), fn.fold_weights(to_dev(w.w_up()), g)
    cg_d, qg_d = fn.quantize_fp8(Wg_d)
    cu_d, qu_d = fn.quantize_fp8(Wu_d)
    h = fn.norm_glu_ffn_fp8(to_dev(w.x()), cg_d, qg_d, cu_d, qu_d, w.eps_f32(), out_dtype=torch.float32)
    cg, qg = oracle.quantize_fp8_per_channel(oracle.fold_weights(w.w(), w.g(), BF16))
    cu, qu = oracle.quantize_fp8_per_channel(oracle.fold_weights(w.w_up(), w.g(), BF16))
    torch.cuda.synchronize()
    assert np.array_equal(cg_d.cpu().numpy(), cg) and np.array_equal(cu_d.cpu().numpy(), cu)
    ref = oracle.glu_deferred_on_quantized(w.x(), cg, qg, cu, qu, w.eps_f32())
    assert_parity(h, ref, BF16, f"{name} kernel-only", rel_l2=KERNEL_REL_L2, max_abs=np.inf)
    text = oracle.norm_glu_ffn(w.x(), oracle.dequantize_fp8(cg, qg), oracle.dequantize_fp8(cu, qu), np.ones(w.K),
                               w.eps_f32())
    assert_parity(h, text, BF16, f"{name} textbook on the dequantised weights")
    full = oracle.norm_glu_ffn(w.x(), w.w(), w.w_up(), w.g(), w.eps_f32())
    ok, info = oracle.check_close(from_dev(h), full, 1.0, np.inf)
    print(f"[quantisation] {name}: fp8 model against the bf16 model: {info}", flush=True)
    assert info["max_rel_l2"] < 0.1


# ---------------------------------------------------------------------------
# prefill (M > 16): x quantised per row to E4M3 as well, the fp8 matrix cores
# ---------------------------------------------------------------------------

def _fp8_prefill_operands(w):
    Wg = oracle.fold_weights(w.w(), w.g(), BF16)
    cg, qg = oracle.quantize_fp8_per_channel(Wg)
    cu = qu = None
    if w.kind == "glu":
        cu, qu = oracle.quantize_fp8_per_channel(oracle.fold_weights(w.w_up(), w.g(), BF16))
    return cg, qg, cu, qu


FP8_PREFILL_CASES = [
    # M, K, N: several tiles with ragged M and N; K not a multiple of the
    # 128-value step; a single 128-row tile
    (300, 1040, 700),
    (200, 528, 300),
    (129, 4096, 77),
    (17, 272, 260),
]


@pytest.mark.parametrize("M,K,N", FP8_PREFILL_CASES)
@pytest.mark.parametrize("kind", ["linear", "glu"])
def test_fp8_prefill_fused_parity(gpu_lib, M, K, N, kind):
    fn = gpu_lib
    base = "llama7b_qkv_prefill_fp8" if kind == "linear" else "smollm2_ffn_prefill_fp8"
    w = dataclasses.replace(synth.workload(base), M=M, K=K, N=N)
    op = fn.OP_NORM_LINEAR_FP8 if kind == "linear" else fn.OP_NORM_GLU_FFN_FP8
    _say(f"fp8 prefill {kind} M={M} K={K} N={N} -> "
         f"{fn.dispatch_name(op, fn.FUSED, M, K, N, torch.bfloat16, torch.float32)}")
    cg, qg, cu, qu = _fp8_prefill_operands(w)
    x = to_dev(w.x())
    eps = w.eps_f32()
    wsb = fn.workspace_bytes(op, fn.FUSED, M, K, N, torch.bfloat16)
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device="cuda")
    if kind == "linear":
        ref_k, bound_k, ref_t, bound_t, flips = fp8_act_bounds(w.x(), cg, qg, eps)
    else:
        ref_k, bound_k, ref_t, bound_t, flips = fp8_act_glu_bounds(w.x(), cg, qg, cu, qu, eps)
    print(f"[fp8] {flips} of {M * K} x codes differ between quantising x and RMSNorm(x) (exact ties)", flush=True)
    for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
        if kind == "linear":
            y = fn.norm_linear_fp8(x, _codes_dev(cg), _vec(qg), eps, out_dtype=od, ws=ws)
        else:
            y = fn.norm_glu_ffn_fp8(x, _codes_dev(cg), _vec(qg), _codes_dev(cu), _vec(qu), eps, out_dtype=od, ws=ws)
        torch.cuda.synchronize()
        # bf16 output adds the store's rounding: half a bf16 ulp of the result
        half = _half_ulp_bf16(ref_k) if ob else 0.0
        assert_within(y, ref_k, bound_k + half, f"fp8 prefill {kind} kernel-only {od}")
        assert_within(y, ref_t, bound_t + half, f"fp8 prefill {kind} textbook (one-step ties) {od}")
        if od == torch.float32:
            _, info = oracle.check_close(from_dev(y), ref_k, 1.0, np.inf)
            print(f"[fp8] prefill {kind} kernel-only: {info}", flush=True)
    # the quantised rows in the workspace (codes first, then the row
    # factors): integer work, equal to the oracle's codes bit for bit
    cx, qx = oracle.quantize_fp8_per_channel(w.x())
    codes = ws[:M * K].cpu().numpy().reshape(M, K)
    bad = np.argwhere(codes != cx)
    assert bad.size == 0, f"{len(bad)} x codes differ, first {bad[:4].tolist()}"
    off = (M * K + 255) // 256 * 256
    r = ws[off:off + 4 * M].cpu().view(torch.float32).numpy().astype(np.float64)
    want = qx.astype(np.float64) / oracle.rms(w.x(), eps)
    assert np.all(np.abs(r - want) <= 4e-7 * np.abs(want)), "row factors s q_x"


@pytest.mark.parametrize("kind", ["linear", "glu"])
def test_fp8_prefill_unfused_parity(gpu_lib, kind):
    """The baseline: RMSNorm (with the gain) to bf16 xn, xn quantised per
    row, the fp8 product with the quantised unfolded weight.  Checked step by
    step from what it leaves in the workspace: xn within one bf16 rounding
    of the oracle's RMSNorm; the codes and scales of xn equal to the oracle's
    quantisation of that xn (integer work, bit for bit); the output within a
    float32 accumulation bound of the product on those codes."""
    fn = gpu_lib
    M, K, N = 300, 1040, 400
    base = "llama7b_qkv_prefill_fp8" if kind == "linear" else "smollm2_ffn_prefill_fp8"
    w = dataclasses.replace(synth.workload(base), M=M, K=K, N=N)
    op = fn.OP_NORM_LINEAR_FP8 if kind == "linear" else fn.OP_NORM_GLU_FFN_FP8
    _say(f"fp8 prefill unfused {kind} M={M} K={K} N={N}")
    cg, qg = oracle.quantize_fp8_per_channel(w.w())
    cu, qu = oracle.quantize_fp8_per_channel(w.w_up())
    eps = w.eps_f32()
    g = _vec(w.g())
    ws = torch.zeros(fn.workspace_bytes(op, fn.UNFUSED, M, K, N, torch.bfloat16), dtype=torch.uint8, device="cuda")
    if kind == "linear":
        y = fn.norm_linear_fp8(to_dev(w.x()), _codes_dev(cg), _vec(qg), eps, g=g, variant=fn.UNFUSED,
                               out_dtype=torch.float32, ws=ws)
    else:
        y = fn.norm_glu_ffn_fp8(to_dev(w.x()), _codes_dev(cg), _vec(qg), _codes_dev(cu), _vec(qu), eps, g=g,
                                variant=fn.UNFUSED, out_dtype=torch.float32, ws=ws)
    torch.cuda.synchronize()
    rup = lambda v: (v + 255) // 256 * 256  # noqa: E731
    wsn = ws.cpu().numpy()
    xn_bits = wsn[:M * K * 2].view(np.uint16).reshape(M, K)
    xn = synth.stored_to_f64(xn_bits)
    xn_ref = oracle.rmsnorm(w.x(), w.g(), eps)
    assert np.all(np.abs(xn - xn_ref) <= 2.0 ** -8 * np.abs(xn_ref) + 1e-30), "xn off by more than a bf16 rounding"
    cx, qx = oracle.quantize_fp8_per_channel(xn_bits)
    off = rup(M * K * 2)
    assert np.array_equal(wsn[off:off + M * K].reshape(M, K), cx), "codes of xn"
    r = wsn[off + rup(M * K):off + rup(M * K) + 4 * M].view(np.float32)
    assert np.array_equal(r.view(np.uint32), qx.view(np.uint32)), "scales of xn"
    dx = oracle.dequantize_fp8(cx, qx)
    Wg, Wu = oracle.dequantize_fp8(cg, qg), oracle.dequantize_fp8(cu, qu)
    a = dx @ Wg.T
    Ba = (1.5 * K + 8) * 2.0 ** -24 * (np.abs(dx) @ np.abs(Wg).T) + 8 * 2.0 ** -24 * np.abs(a)
    if kind == "linear":
        ref, bound = a, Ba
    else:
        b = dx @ Wu.T
        Bb = (1.5 * K + 8) * 2.0 ** -24 * (np.abs(dx) @ np.abs(Wu).T) + 8 * 2.0 ** -24 * np.abs(b)
        ref = oracle.silu(a) * b
        bound = 1.1 * np.abs(b) * Ba + np.abs(oracle.silu(a)) * Bb + 1.1 * Ba * Bb + 8 * 2.0 ** -24 * np.abs(ref)
    assert_within(y, ref, bound, f"fp8 prefill unfused {kind}, product on its own codes")
    # the textbook fp8 form on the unfolded weights, RMSNorm with the gain in
    # float64, quantised per row (reported: the bf16 xn and ties move codes)
    ct, qt = oracle.quantize_fp8_per_channel(xn_ref)
    dt = oracle.dequantize_fp8(ct, qt)
    text = dt @ Wg.T if kind == "linear" else oracle.silu(dt @ Wg.T) * (dt @ Wu.T)
    _, info = oracle.check_close(from_dev(y), text, 1.0, np.inf)
    print(f"[fp8] prefill unfused {kind} against the textbook fp8 form: {info}", flush=True)


def test_fp8_prefill_every_tile(gpu_lib, monkeypatch):
    fn = gpu_lib
    w = dataclasses.replace(synth.workload("llama7b_qkv_prefill_fp8"), M=300, K=1040, N=520)
    cg, qg, _, _ = _fp8_prefill_operands(w)
    ref, bound, _, _, _ = fp8_act_bounds(w.x(), cg, qg, w.eps_f32())
    for tile in (0, 1, 3, 4):
        monkeypatch.setenv("FN_TILE", str(tile))
        _say(f"fp8 prefill tile {tile}: "
             f"{fn.dispatch_name(fn.OP_NORM_LINEAR_FP8, fn.FUSED, w.M, w.K, w.N, torch.bfloat16, torch.float32)}")
        y = fn.norm_linear_fp8(to_dev(w.x()), _codes_dev(cg), _vec(qg), w.eps_f32(), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_within(y, ref, bound, f"fp8 prefill tile {tile} kernel-only")


def test_fp8_prefill_zero_row_and_eps_zero(gpu_lib):
    fn = gpu_lib
    w = dataclasses.replace(synth.workload("llama7b_qkv_prefill_fp8"), M=40, K=528, N=300)
    x = w.x().copy()
    x[3] = 0
    cg, qg, _, _ = _fp8_prefill_operands(w)
    _say("fp8 prefill: zero row with eps > 0 (exact zeros) and eps = 0 (NaN)")
    y = from_dev(fn.norm_linear_fp8(to_dev(x), _codes_dev(cg), _vec(qg), 1e-6, out_dtype=torch.float32))
    assert np.all(y[3] == 0.0) and np.all(np.isfinite(y))
    y0 = from_dev(fn.norm_linear_fp8(to_dev(x), _codes_dev(cg), _vec(qg), 0.0, out_dtype=torch.float32))
    assert np.all(np.isnan(y0[3])) and np.all(np.isfinite(np.delete(y0, 3, axis=0)))


@pytest.mark.parametrize("name", ["llama7b_qkv_prefill_fp8", "smollm2_ffn_prefill_fp8"])
def test_full_fp8_prefill(gpu_lib, name):
    """The full workload: fold and quantise the weights on the GPU, then the
    op; every output against the oracle's deferred form on its own codes
    (kernel tolerance) and the textbook fp8 form (workload tolerance); the
    error against the bf16 model is printed, not graded."""
    fn = gpu_lib
    w = synth.workload(name)
    _say(f"full {name}: M={w.M} K={w.K} N={w.N} ({w.kind}) fold + quantise on the GPU")
    g = _vec(w.g())
    cg_d, qg_d = fn.quantize_fp8(fn.fold_weights(to_dev(w.w()), g))
    cg, qg, cu, qu = _fp8_prefill_operands(w)
    x = to_dev(w.x())
    if w.kind == "glu":
        cu_d, qu_d = fn.quantize_fp8(fn.fold_weights(to_dev(w.w_up()), g))
        y = fn.norm_glu_ffn_fp8(x, cg_d, qg_d, cu_d, qu_d, w.eps_f32(), out_dtype=torch.float32)
        ref_k, bound_k, ref_t, bound_t, flips = fp8_act_glu_bounds(w.x(), cg, qg, cu, qu, w.eps_f32())
        full = oracle.norm_glu_ffn(w.x(), w.w(), w.w_up(), w.g(), w.eps_f32())
    else:
        y = fn.norm_linear_fp8(x, cg_d, qg_d, w.eps_f32(), out_dtype=torch.float32)
        ref_k, bound_k, ref_t, bound_t, flips = fp8_act_bounds(w.x(), cg, qg, w.eps_f32())
        full = oracle.norm_linear(w.x(), w.w(), w.g(), w.eps_f32())
    torch.cuda.synchronize()
    assert np.array_equal(cg_d.cpu().numpy(), cg)
    print(f"[fp8] {flips} of {w.M * w.K} x codes differ between quantising x and RMSNorm(x)", flush=True)
    assert_within(y, ref_k, bound_k, f"{name} kernel-only")
    _, info = oracle.check_close(from_dev(y), ref_k, 1.0, np.inf)
    print(f"[fp8] {name} kernel-only: {info}", flush=True)
    assert_within(y, ref_t, bound_t, f"{name} textbook fp8 form (one-step ties)")
    ok, info = oracle.check_close(from_dev(y), full, 1.0, np.inf)
    print(f"[quantisation] {name}: fp8 x and weights against the bf16 model: {info}", flush=True)
    assert info["max_rel_l2"] < 0.2
    ok, info = oracle.check_close(from_dev(y), ref_t, 1.0, np.inf)
    print(f"[fp8] {name} against the textbook fp8 form: {info}", flush=True)
