"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Every case prints its name and shape before it runs.  Reduced-size cases
keep each workload's distributions and span several workgroup tiles with
ragged tails; the full-size cases run the exact workload shapes and
compare every output.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (BF16_MAX_ABS, BF16_REL_L2, KERNEL_REL_L2, assert_parity, assert_within, bits_of,
                      deferred_bound, from_dev, glu_bound, to_dev)
from synth import BF16, F32

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _gain(w):
    return torch.from_numpy(w.g()).cuda()


# ---------------------------------------------------------------------------
# runners: one call of the library per variant, plus the oracle reference
# ---------------------------------------------------------------------------

def run_linear(fn, w, variant, out_dtype, aux=None):
    x, W, g = to_dev(w.x()), to_dev(w.w()), _gain(w)
    if variant == fn.UNFUSED:
        return fn.norm_linear(x, W, w.eps_f32(), g=g, variant=variant, out_dtype=out_dtype)
    Ws = fn.fold_weights(W, g)
    return fn.norm_linear(x, Ws, w.eps_f32(), variant=variant, out_dtype=out_dtype, aux_stream=aux)


def ref_linear(w):
    return oracle.norm_linear(w.x(), w.w(), w.g(), w.eps_f32())


def run_glu(fn, w, variant, out_dtype):
    x, Wg, Wu, g = to_dev(w.x()), to_dev(w.w()), to_dev(w.w_up()), _gain(w)
    if variant == fn.UNFUSED:
        return fn.norm_glu_ffn(x, Wg, Wu, w.eps_f32(), g=g, variant=variant, out_dtype=out_dtype)
    return fn.norm_glu_ffn(x, fn.fold_weights(Wg, g), fn.fold_weights(Wu, g), w.eps_f32(), variant=variant,
                           out_dtype=out_dtype)


def ref_glu(w):
    return oracle.norm_glu_ffn(w.x(), w.w(), w.w_up(), w.g(), w.eps_f32())


def run_qk(fn, w, variant, out_dtype, v_mode=0):
    x, W, g1 = to_dev(w.x()), to_dev(w.w()), _gain(w)
    gq = torch.from_numpy(w.g_q()).cuda()
    gk = torch.from_numpy(w.g_k()).cuda()
    if variant == fn.UNFUSED:
        return fn.linear_qknorm(x, W, w.n_q_heads, w.n_kv_heads, w.head_dim, gq, gk, w.eps_f32(),
                                w.eps_head_f32(), v_mode=v_mode, g1=g1, variant=variant, out_dtype=out_dtype)
    return fn.linear_qknorm(x, fn.fold_weights(W, g1), w.n_q_heads, w.n_kv_heads, w.head_dim, gq, gk, w.eps_f32(),
                            w.eps_head_f32(), v_mode=v_mode, variant=variant, out_dtype=out_dtype)


def ref_qk(w, v_mode=0):
    return oracle.linear_qknorm(w.x(), w.w(), w.g(), w.eps_f32(), w.n_q_heads, w.n_kv_heads, w.head_dim,
                                w.g_q(), w.g_k(), w.eps_head_f32(), v_mode)


def _qk_workload(M, K, nq, nkv, hd):
    base = synth.workload("qknorm_attn_in_bf16")
    import dataclasses
    return dataclasses.replace(base, M=M, K=K, N=(nq + 2 * nkv) * hd, n_q_heads=nq, n_kv_heads=nkv, head_dim=hd)


# ---------------------------------------------------------------------------
# fold: bit-exact against the oracle's single rounding
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("w_dt,o_dt", [(F32, F32), (BF16, BF16), (F32, BF16), (BF16, F32)])
def test_fold_bit_exact(gpu_lib, w_dt, o_dt):
    fn = gpu_lib
    _say(f"fold {w_dt}->{o_dt} 96x1040 with edge values")
    rng = np.random.default_rng(20)
    N, K = 96, 1040
    v = rng.standard_normal((N, K)) * np.exp2(rng.integers(-30, 30, size=(N, K)))
    edge = np.array([0.0, -0.0, 1e-40, -1e-40, 3e38, -3e38, 1.0, -1.0, 2 ** -126, 2 ** -133])
    v[0, :edge.size] = edge
    f = v.astype(np.float32)
    W = f if w_dt == F32 else synth.bf16_bits_from_f32(f)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    g[:4] = [1.0, 2.0, 0.5, 1.0 + 2 ** -10]
    want = oracle.fold_weights(W, g, o_dt)
    got = fn.fold_weights(to_dev(W), torch.from_numpy(g).cuda(),
                          out_dtype=torch.float32 if o_dt == F32 else torch.bfloat16)
    torch.cuda.synchronize()
    got_bits = bits_of(got)
    want_bits = want.view(np.uint32) if o_dt == F32 else want
    mism = np.argwhere(got_bits != want_bits)
    assert mism.size == 0, f"{len(mism)} mismatches, first at {mism[:4].tolist()}"


def test_fold_golden_and_in_place(gpu_lib):
    fn = gpu_lib
    _say("fold golden double-rounding cases, in place")
    # bf16 W = 177/128 and 171/128, g = 13886227/2^23 and 12484800/2^23 (see golden file)
    W = np.zeros((2, 8), dtype=np.float64)
    W[0, 0], W[1, 0] = 177 / 128, 171 / 128
    g = np.ones(8, dtype=np.float64)
    Wb = synth.bf16_bits_from_f32(W.astype(np.float32))
    gA = g.copy(); gA[0] = 13886227 / 2 ** 23
    gB = g.copy(); gB[0] = 12484800 / 2 ** 23
    for gg, row, want in [(gA, 0, 147 / 64), (gB, 1, 255 / 128)]:
        t = to_dev(Wb.copy())
        fn.fold_weights(t, torch.from_numpy(gg.astype(np.float32)).cuda(), out=t)
        torch.cuda.synchronize()
        assert from_dev(t)[row, 0] == want


# ---------------------------------------------------------------------------
# reduced-size parity, every op and variant
# ---------------------------------------------------------------------------

LINEAR_CASES = [
    ("smollm2_qkv_f32", 200, 576, 330),
    ("llama7b_qkv_prefill_bf16", 300, 520, 700),
    ("llama7b_qkv_prefill_bf16", 64, 4096, 512),
]


@pytest.mark.parametrize("name,M,K,N", LINEAR_CASES)
@pytest.mark.parametrize("variant", ["fused", "unfused", "two_stream"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_norm_linear_parity(gpu_lib, name, M, K, N, variant, out):
    fn = gpu_lib
    w = synth.workload(name).with_shape(M, K, N)
    if w.dtype == F32 and (out == "bf16" or variant == "two_stream"):
        pytest.skip("float32 workloads run fused/unfused with float32 output")
    v = {"fused": fn.FUSED, "unfused": fn.UNFUSED, "two_stream": fn.TWO_STREAM}[variant]
    od = torch.float32 if out == "f32" else torch.bfloat16
    _say(f"norm_linear {name} M={M} K={K} N={N} {variant} out={out} -> "
         f"{fn.dispatch_name(fn.OP_NORM_LINEAR, v, M, K, N, torch.float32 if w.dtype == F32 else torch.bfloat16, od)}")
    aux = torch.cuda.Stream() if v == fn.TWO_STREAM else None
    y = run_linear(fn, w, v, od, aux)
    torch.cuda.synchronize()
    assert_parity(y, ref_linear(w), w.dtype, f"{name} {variant} {out}", out_bf16=(out == "bf16"))


GLU_CASES = [(300, 576, 400), (70, 264, 1000), (1, 520, 300), (4, 4096, 1100), (16, 1032, 700), (17, 576, 96)]


@pytest.mark.parametrize("M,K,N", GLU_CASES)
@pytest.mark.parametrize("variant", ["fused", "unfused"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_norm_glu_ffn_parity(gpu_lib, M, K, N, variant, out):
    fn = gpu_lib
    base = "smollm2_ffn_prefill_bf16" if K <= 600 else "llama7b_ffn_decode_m16_bf16"
    w = synth.workload(base).with_shape(M, K, N)
    v = fn.FUSED if variant == "fused" else fn.UNFUSED
    od = torch.float32 if out == "f32" else torch.bfloat16
    _say(f"glu M={M} K={K} N={N} {variant} out={out} -> "
         f"{fn.dispatch_name(fn.OP_NORM_GLU_FFN, v, M, K, N, torch.bfloat16, od)}")
    y = run_glu(fn, w, v, od)
    torch.cuda.synchronize()
    assert_parity(y, ref_glu(w), BF16, f"glu {M}x{K}x{N} {variant} {out}", out_bf16=(out == "bf16"))


QK_CASES = [(130, 2560, 8, 4, 256), (300, 520, 3, 2, 64), (200, 264, 2, 1, 128), (5, 512, 4, 2, 256)]


@pytest.mark.parametrize("M,K,nq,nkv,hd", QK_CASES)
@pytest.mark.parametrize("variant", ["fused", "unfused"])
@pytest.mark.parametrize("v_mode", [0, 1])
def test_linear_qknorm_parity(gpu_lib, M, K, nq, nkv, hd, variant, v_mode):
    fn = gpu_lib
    w = _qk_workload(M, K, nq, nkv, hd)
    v = fn.FUSED if variant == "fused" else fn.UNFUSED
    _say(f"qknorm M={M} K={K} heads q{nq} kv{nkv} hd{hd} {variant} v_mode={v_mode} -> "
         f"{fn.dispatch_name(fn.OP_LINEAR_QKNORM, v, M, K, w.N, torch.bfloat16, torch.float32)}")
    y = run_qk(fn, w, v, torch.float32, v_mode)
    torch.cuda.synchronize()
    assert_parity(y, ref_qk(w, v_mode), BF16, f"qknorm {variant} v{v_mode}")


# ---------------------------------------------------------------------------
# every prefill tile configuration (FN_TILE overrides the library's choice):
# ragged M, N and K tails, interior tiles with staged bf16 stores, all three
# epilogues
# ---------------------------------------------------------------------------

TILE_IDS = list(range(10))


@pytest.mark.parametrize("tile", TILE_IDS)
def test_every_tile_config(gpu_lib, tile, monkeypatch):
    fn = gpu_lib
    monkeypatch.setenv("FN_TILE", str(tile))
    bf = torch.bfloat16
    wl = synth.workload("llama7b_qkv_prefill_bf16").with_shape(300, 1032, 700)
    wg = synth.workload("smollm2_ffn_prefill_bf16").with_shape(300, 576, 400)
    wq = _qk_workload(260, 520, 3, 2, 64)
    _say(f"tile {tile}: " + ", ".join(fn.dispatch_name(op, fn.FUSED, M, K, N, bf, bf) for op, M, K, N in
                                        [(fn.OP_NORM_LINEAR, wl.M, wl.K, wl.N), (fn.OP_NORM_GLU_FFN, wg.M, wg.K, wg.N),
                                         (fn.OP_LINEAR_QKNORM, wq.M, wq.K, wq.N)]))
    for od, out_bf16 in ((torch.float32, False), (bf, True)):
        y = run_linear(fn, wl, fn.FUSED, od)
        h = run_glu(fn, wg, fn.FUSED, od)
        q = run_qk(fn, wq, fn.FUSED, od)
        torch.cuda.synchronize()
        assert_parity(y, ref_linear(wl), BF16, f"tile {tile} linear", out_bf16=out_bf16)
        assert_parity(h, ref_glu(wg), BF16, f"tile {tile} glu", out_bf16=out_bf16)
        assert_parity(q, ref_qk(wq), BF16, f"tile {tile} qknorm", out_bf16=out_bf16)


# ---------------------------------------------------------------------------
# kernel-only pin: fused kernels against the deferred form on the oracle's
# own folded weights (isolates kernel arithmetic from fold rounding)
# ---------------------------------------------------------------------------

def test_kernel_only_pin_linear_glu_qk(gpu_lib):
    fn = gpu_lib
    _say("kernel-only pins: linear 300x1032x700, glu 200x576x300, glu decode 4x4096x300, qk 130x520")
    w = synth.workload("llama7b_qkv_prefill_bf16").with_shape(300, 1032, 700)
    Ws = oracle.fold_weights(w.w(), w.g(), BF16)
    y = fn.norm_linear(to_dev(w.x()), to_dev(Ws), w.eps_f32(), out_dtype=torch.float32)
    assert_parity(y, oracle.deferred_on_folded(w.x(), Ws, w.eps_f32()), BF16, "kernel linear",
                  rel_l2=KERNEL_REL_L2, max_abs=np.inf)
    for M, K, N in [(200, 576, 300), (4, 4096, 300)]:
        w = synth.workload("smollm2_ffn_prefill_bf16").with_shape(M, K, N)
        Wg, Wu = oracle.fold_weights(w.w(), w.g(), BF16), oracle.fold_weights(w.w_up(), w.g(), BF16)
        h = fn.norm_glu_ffn(to_dev(w.x()), to_dev(Wg), to_dev(Wu), w.eps_f32(), out_dtype=torch.float32)
        assert_parity(h, oracle.glu_deferred_on_folded(w.x(), Wg, Wu, w.eps_f32()), BF16, f"kernel glu M={M}",
                      rel_l2=KERNEL_REL_L2, max_abs=np.inf)
    w = _qk_workload(130, 520, 8, 4, 256)
    Wq = oracle.fold_weights(w.w(), w.g(), BF16)
    gq, gk = torch.from_numpy(w.g_q()).cuda(), torch.from_numpy(w.g_k()).cuda()
    for vm in (0, 1):
        y = fn.linear_qknorm(to_dev(w.x()), to_dev(Wq), 8, 4, 256, gq, gk, w.eps_f32(), w.eps_head_f32(),
                             v_mode=vm, out_dtype=torch.float32)
        ref = oracle.qknorm_dropped_on_folded(w.x(), Wq, w.eps_f32(), 8, 4, 256, w.g_q(), w.g_k(),
                                              w.eps_head_f32(), vm)
        assert_parity(y, ref, BF16, f"kernel qk v{vm}", rel_l2=KERNEL_REL_L2, max_abs=np.inf)


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------

def test_full_smollm2_qkv_f32(gpu_lib):
    fn = gpu_lib
    w = synth.workload("smollm2_qkv_f32")
    for variant in (fn.FUSED, fn.UNFUSED):
        _say(f"full smollm2_qkv_f32 128x576x960 variant={variant}")
        y = run_linear(fn, w, variant, torch.float32)
        assert_parity(y, ref_linear(w), F32, f"smollm2_qkv_f32 v{variant}")


def test_full_smollm2_ffn_prefill(gpu_lib):
    fn = gpu_lib
    w = synth.workload("smollm2_ffn_prefill_bf16")
    ref = ref_glu(w)
    for variant in (fn.FUSED, fn.UNFUSED):
        for od in (torch.float32, torch.bfloat16):
            _say(f"full smollm2_ffn_prefill 2048x576x2x1536 variant={variant} out={od}")
            y = run_glu(fn, w, variant, od)
            assert_parity(y, ref, BF16, f"smollm2_ffn v{variant} {od}", out_bf16=(od == torch.bfloat16))


@pytest.mark.parametrize("name", ["llama7b_ffn_decode_m1_bf16", "llama7b_ffn_decode_m4_bf16",
                                  "llama7b_ffn_decode_m16_bf16"])
def test_full_llama7b_ffn_decode(gpu_lib, name):
    fn = gpu_lib
    w = synth.workload(name)
    ref = ref_glu(w)
    for variant in (fn.FUSED, fn.UNFUSED):
        _say(f"full {name} M={w.M}x4096x2x11008 variant={variant}")
        y = run_glu(fn, w, variant, torch.float32)
        assert_parity(y, ref, BF16, f"{name} v{variant}")


def test_full_qknorm_attn_in(gpu_lib):
    fn = gpu_lib
    w = synth.workload("qknorm_attn_in_bf16")
    for vm in (0, 1):
        ref = ref_qk(w, vm)
        for variant in (fn.FUSED, fn.UNFUSED):
            _say(f"full qknorm_attn_in 1024x2560x4096 variant={variant} v_mode={vm}")
            y = run_qk(fn, w, variant, torch.float32, vm)
            assert_parity(y, ref, BF16, f"qknorm v{variant} vm{vm}")


@pytest.fixture(scope="module")
def llama7b_qkv_full():
    """The Llama-7B QKV prefill workload and the oracle on all 4096 rows
    (412 GFLOP in float64: a few seconds on the host's cores)."""
    w = synth.workload("llama7b_qkv_prefill_bf16")
    return w, ref_linear(w)


FULL_LLAMA7B_VARIANTS = [
    # label, variant, output dtype, FN_PRESTATS and FN_TILE (None: the library's choice)
    ("fused f32", "fused", "f32", None, None),
    ("fused bf16", "fused", "bf16", None, None),
    ("fused bf16, sums of squares inside the GEMM", "fused", "bf16", "0", None),
    ("fused f32, sums of squares inside the GEMM", "fused", "f32", "0", None),
    ("fused bf16, sums inside the GEMM, three x stages", "fused", "bf16", "0", "9"),
    ("fused bf16, row-statistics pass", "fused", "bf16", "1", None),
    ("fused bf16, row-statistics pass, three x stages", "fused", "bf16", "1", "9"),
    ("unfused f32", "unfused", "f32", None, None),
    ("unfused bf16", "unfused", "bf16", None, None),
    ("two_stream f32", "two_stream", "f32", None, None),
    ("two_stream bf16", "two_stream", "bf16", None, None),
]


@pytest.mark.parametrize("label,variant,out,prestats,tile", FULL_LLAMA7B_VARIANTS,
                         ids=[c[0].replace(" ", "_").replace(",", "") for c in FULL_LLAMA7B_VARIANTS])
def test_full_llama7b_qkv_prefill(gpu_lib, llama7b_qkv_full, label, variant, out, prestats, tile, monkeypatch):
    """Every output of the 4096 x 4096 x 12288 workload against the oracle."""
    fn = gpu_lib
    w, ref = llama7b_qkv_full
    if prestats is not None:
        monkeypatch.setenv("FN_PRESTATS", prestats)
    if tile is not None:
        monkeypatch.setenv("FN_TILE", tile)
    v = {"fused": fn.FUSED, "unfused": fn.UNFUSED, "two_stream": fn.TWO_STREAM}[variant]
    od = torch.float32 if out == "f32" else torch.bfloat16
    _say(f"full llama7b_qkv_prefill 4096x4096x12288 {label} -> "
         f"{fn.dispatch_name(fn.OP_NORM_LINEAR, v, w.M, w.K, w.N, torch.bfloat16, od)}")
    aux = torch.cuda.Stream() if v == fn.TWO_STREAM else None
    y = run_linear(fn, w, v, od, aux)
    torch.cuda.synchronize()
    assert_parity(y, ref, BF16, f"llama7b_qkv {label}", out_bf16=(out == "bf16"))


# ---------------------------------------------------------------------------
# shape sweep: ragged tails in M, N and K (K a multiple of 8)
# ---------------------------------------------------------------------------

SWEEP = [(1, 8, 1), (3, 24, 5), (17, 72, 17), (63, 136, 130), (65, 200, 257), (127, 64, 511), (129, 8, 33),
         (257, 520, 300), (33, 4104, 40)]


@pytest.mark.parametrize("M,K,N", SWEEP)
def test_shape_sweep_linear_and_glu(gpu_lib, M, K, N):
    """Every shape against the deferred form on the oracle's folded weights
    within a derived float32 error bound; shapes with K >= 64 also against
    the unfolded oracle at the workload tolerance (with fewer terms the
    bf16 fold rounding does not average out and that tolerance does not
    apply)."""
    fn = gpu_lib
    _say(f"sweep M={M} K={K} N={N}")
    w = synth.workload("llama7b_qkv_prefill_bf16").with_shape(M, K, N)
    Ws = oracle.fold_weights(w.w(), w.g(), BF16)
    y = fn.norm_linear(to_dev(w.x()), to_dev(Ws), w.eps_f32(), out_dtype=torch.float32)
    assert_within(y, oracle.deferred_on_folded(w.x(), Ws, w.eps_f32()), deferred_bound(w.x(), Ws, w.eps_f32()),
                  "sweep linear kernel")
    wg = synth.workload("smollm2_ffn_prefill_bf16").with_shape(M, K, N)
    Wg, Wu = oracle.fold_weights(wg.w(), wg.g(), BF16), oracle.fold_weights(wg.w_up(), wg.g(), BF16)
    h = fn.norm_glu_ffn(to_dev(wg.x()), to_dev(Wg), to_dev(Wu), wg.eps_f32(), out_dtype=torch.float32)
    assert_within(h, oracle.glu_deferred_on_folded(wg.x(), Wg, Wu, wg.eps_f32()),
                  glu_bound(wg.x(), Wg, Wu, wg.eps_f32()), "sweep glu kernel")
    wf = synth.workload("smollm2_qkv_f32").with_shape(M, K, N)
    Wf = oracle.fold_weights(wf.w(), wf.g(), F32)
    yf = fn.norm_linear(to_dev(wf.x()), to_dev(Wf), wf.eps_f32(), out_dtype=torch.float32)
    assert_within(yf, oracle.deferred_on_folded(wf.x(), Wf, wf.eps_f32()), deferred_bound(wf.x(), Wf, wf.eps_f32()),
                  "sweep f32 kernel")
    if K >= 64:
        assert_parity(run_linear(fn, w, fn.FUSED, torch.float32), ref_linear(w), BF16, "sweep linear")
        assert_parity(run_glu(fn, wg, fn.FUSED, torch.float32), ref_glu(wg), BF16, "sweep glu")
        assert_parity(run_linear(fn, wf, fn.FUSED, torch.float32), ref_linear(wf), F32, "sweep f32")


# ---------------------------------------------------------------------------
# the row-statistics pass of the fused variant (FN_PRESTATS forces it on
# small, ragged shapes; full size it is the default)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N", [(300, 1032, 700), (17, 72, 17), (600, 4096, 520)])
def test_prestats_pass_linear(gpu_lib, M, K, N, monkeypatch):
    fn = gpu_lib
    monkeypatch.setenv("FN_PRESTATS", "1")
    w = synth.workload("llama7b_qkv_prefill_bf16").with_shape(M, K, N)
    _say(f"row-statistics pass: linear {M}x{K}x{N} -> "
         f"{fn.dispatch_name(fn.OP_NORM_LINEAR, fn.FUSED, M, K, N, torch.bfloat16, torch.float32)}")
    assert "row_scale+" in fn.dispatch_name(fn.OP_NORM_LINEAR, fn.FUSED, M, K, N, torch.bfloat16, torch.float32)
    for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
        y = run_linear(fn, w, fn.FUSED, od)
        torch.cuda.synchronize()
        assert_parity(y, ref_linear(w), BF16, f"prestats linear {od}", out_bf16=ob)
    Ws = oracle.fold_weights(w.w(), w.g(), BF16)
    y = fn.norm_linear(to_dev(w.x()), to_dev(Ws), w.eps_f32(), out_dtype=torch.float32)
    assert_parity(y, oracle.deferred_on_folded(w.x(), Ws, w.eps_f32()), BF16, "prestats kernel-only",
                  rel_l2=KERNEL_REL_L2, max_abs=np.inf)


# ---------------------------------------------------------------------------
# degenerate and extreme rows
# ---------------------------------------------------------------------------

def test_zero_rows_and_eps_zero(gpu_lib):
    fn = gpu_lib
    _say("zero rows: eps>0 -> exact 0, eps=0 -> NaN (prefill and decode)")
    for M in (40, 3):
        w = synth.workload("llama7b_qkv_prefill_bf16").with_shape(M, 264, 300)
        x = w.x().copy()
        x[1] = 0
        Ws = oracle.fold_weights(w.w(), w.g(), BF16)
        xd, Wd = to_dev(x), to_dev(Ws)
        y = from_dev(fn.norm_linear(xd, Wd, 1e-6, out_dtype=torch.float32))
        assert np.all(y[1] == 0.0) and np.all(np.isfinite(y))
        y0 = from_dev(fn.norm_linear(xd, Wd, 0.0, out_dtype=torch.float32))
        assert np.all(np.isnan(y0[1])) and np.all(np.isfinite(np.delete(y0, 1, axis=0)))
        h = from_dev(fn.norm_glu_ffn(xd, Wd, Wd, 1e-6, out_dtype=torch.float32))
        assert np.all(h[1] == 0.0)
        ref = oracle.norm_linear(x, w.w(), w.g(), 0.0)
        ok, info = oracle.check_close(y0, ref, BF16_REL_L2, BF16_MAX_ABS)
        assert ok, info


def test_extreme_row_scales(gpu_lib):
    fn = gpu_lib
    _say("rows scaled by 2^-50 .. 2^50")
    w = synth.workload("llama7b_qkv_prefill_bf16").with_shape(64, 1024, 300)
    x = synth.stored_to_f64(w.x())
    x *= np.exp2(np.linspace(-50, 50, 64))[:, None]
    xb = synth.bf16_bits_from_f32(x.astype(np.float32))
    Ws = oracle.fold_weights(w.w(), w.g(), BF16)
    y = fn.norm_linear(to_dev(xb), to_dev(Ws), w.eps_f32(), out_dtype=torch.float32)
    assert_parity(y, oracle.norm_linear(xb, w.w(), w.g(), w.eps_f32()), BF16, "extreme row scales")


# ---------------------------------------------------------------------------
# invalid arguments: an error code, nothing launched, output untouched
# ---------------------------------------------------------------------------

def test_invalid_arguments_write_nothing(gpu_lib):
    fn = gpu_lib
    _say("invalid arguments")
    lib = fn.load()
    M, K, N = 32, 64, 48
    x = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    W = torch.randn(N, K, device="cuda").to(torch.bfloat16)
    g = torch.ones(K, device="cuda")
    y = torch.full((M, N), 7.0, device="cuda")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # a non-null stream handle
    st = ctypes.c_void_p(side.cuda_stream)
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)  # noqa: E731
    cases = [
        ("eps < 0", lib.fn_norm_linear(P(x), 1, M, K, P(W), 1, N, None, -1.0, P(y), 0, 0, None, 0, st, None), 8),
        ("g with fused", lib.fn_norm_linear(P(x), 1, M, K, P(W), 1, N, P(g), 1e-6, P(y), 0, 0, None, 0, st, None), 8),
        ("no g unfused", lib.fn_norm_linear(P(x), 1, M, K, P(W), 1, N, None, 1e-6, P(y), 0, 1, None, 0, st, None), 1),
        ("no workspace", lib.fn_norm_linear(P(x), 1, M, K, P(W), 1, N, P(g), 1e-6, P(y), 0, 1, None, 0, st, None), 5),
        ("small workspace", lib.fn_norm_linear(P(x), 1, M, K, P(W), 1, N, P(g), 1e-6, P(y), 0, 1, P(y), 64, st, None), 5),
        ("misaligned x", lib.fn_norm_linear(P(x, 2), 1, M, K, P(W), 1, N, None, 1e-6, P(y), 0, 0, None, 0, st, None), 4),
        ("K % 8", lib.fn_norm_linear(P(x), 1, M, 60, P(W), 1, N, None, 1e-6, P(y), 0, 0, None, 0, st, None), 4),
        ("dtype mix", lib.fn_norm_linear(P(x), 1, M, K, P(W), 0, N, None, 1e-6, P(y), 0, 0, None, 0, st, None), 3),
        ("bad variant", lib.fn_norm_linear(P(x), 1, M, K, P(W), 1, N, None, 1e-6, P(y), 0, 7, None, 0, st, None), 8),
        ("aux == stream", lib.fn_norm_linear(P(x), 1, M, K, P(W), 1, N, None, 1e-6, P(y), 0, 2, P(y), 1 << 20, st, st), 8),
        ("null x", lib.fn_norm_linear(None, 1, M, K, P(W), 1, N, None, 1e-6, P(y), 0, 0, None, 0, st, None), 1),
        ("negative M", lib.fn_norm_linear(P(x), 1, -1, K, P(W), 1, N, None, 1e-6, P(y), 0, 0, None, 0, st, None), 2),
        ("glu two-stream", lib.fn_norm_glu_ffn(P(x), 1, M, K, P(W), P(W), 1, N, None, 1e-6, P(y), 0, 2, None, 0, st), 6),
        ("qk head_dim", lib.fn_linear_qknorm(P(x), 1, M, K, P(W), 1, 1, 1, 16, P(g), P(g), 0, 1e-6, 1e-6, 0, None,
                                             P(y), 0, 0, None, 0, st), 2),
        ("qk v_mode", lib.fn_linear_qknorm(P(x), 1, M, K, P(W), 1, 1, 1, 64, P(g), P(g), 0, 1e-6, 1e-6, 3, None,
                                           P(y), 0, 0, None, 0, st), 8),
    ]
    torch.cuda.synchronize()
    for name, status, want in cases:
        assert status == want, f"{name}: got {status} ({lib.fn_last_error().decode()}), want {want}"
        assert lib.fn_last_error().decode() != ""
    assert torch.all(y == 7.0)
    # M == 0 is a valid no-op
    assert lib.fn_norm_linear(P(x), 1, 0, K, P(W), 1, N, None, 1e-6, P(y), 0, 0, None, 0, st, None) == 0
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ---------------------------------------------------------------------------
# re-entrancy: host threads calling at once, each on its own streams
# ---------------------------------------------------------------------------

def test_concurrent_threads_and_streams(gpu_lib):
    import threading

    fn = gpu_lib
    T, iters = 4, 24
    _say(f"{T} host threads x {iters} calls, fused / two-stream / unfused on their own streams")
    base = synth.workload("llama7b_qkv_prefill_bf16").with_shape(128, 512, 384)
    # distinct x per thread (a new seed also redraws W and g: the references
    # use the shared base weight and gain, as the calls do)
    cases = [base.with_rows(128, seed=base.seed + 500 + t) for t in range(T)]
    refs = [oracle.norm_linear(w.x(), base.w(), base.g(), base.eps_f32()) for w in cases]
    Wd, gd = to_dev(base.w()), _gain(base)
    Ws = fn.fold_weights(Wd, gd)
    xs = [to_dev(w.x()) for w in cases]
    torch.cuda.synchronize()
    outs = [[None] * iters for _ in range(T)]
    errors = []

    def worker(t):
        try:
            s, aux = torch.cuda.Stream(), torch.cuda.Stream()
            with torch.cuda.stream(s):
                for i in range(iters):
                    v = (fn.FUSED, fn.TWO_STREAM, fn.UNFUSED)[i % 3]
                    if v == fn.UNFUSED:
                        outs[t][i] = fn.norm_linear(xs[t], Wd, base.eps_f32(), g=gd, variant=v,
                                                    out_dtype=torch.float32)
                    else:
                        outs[t][i] = fn.norm_linear(xs[t], Ws, base.eps_f32(), variant=v,
                                                    out_dtype=torch.float32, aux_stream=aux if v == fn.TWO_STREAM else None)
            s.synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(T)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(T):
        for i in range(iters):
            assert_parity(outs[t][i], refs[t], BF16, f"thread {t} call {i}")


# ---------------------------------------------------------------------------
# the two-stream join (the pages' stale-buffer lesson): many steps with
# different inputs, the aux stream held back by queued work every step
# ---------------------------------------------------------------------------

def _join_stress(fn, steps, poison=False):
    """`steps` two-stream calls over 16 distinct inputs through one
    workspace, the aux stream held back by queued work every step; returns
    the steps whose output is not their own input's (classified as a
    one-step lag, a read of the poison, or wrong).  With `poison` the
    workspace is filled with NaN on the main stream before every call (the
    fork orders the aux stream's GEMM after the fill)."""
    M, K, N, P = 64, 256, 512, 16
    base = synth.workload("llama7b_qkv_prefill_bf16").with_shape(M, K, N)
    xs, refs = [], []
    Wfold = oracle.fold_weights(base.w(), base.g(), BF16)
    for p in range(P):
        w = base.with_rows(M, seed=base.seed + 1000 + p)
        xs.append(to_dev(w.x()))
        refs.append(oracle.deferred_on_folded(w.x(), Wfold, base.eps_f32()))
    Ws = to_dev(Wfold)
    aux = torch.cuda.Stream()
    ys = torch.empty((steps, M, N), device="cuda")
    ws = torch.empty(fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.TWO_STREAM, M, K, N, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    ws.record_stream(aux)
    da = torch.randn(1024, 1024, device="cuda")
    db = torch.randn(1024, 1024, device="cuda")
    dc = torch.empty(1024, 1024, device="cuda")
    torch.cuda.synchronize()
    for t in range(steps):
        with torch.cuda.stream(aux):
            torch.mm(da, db, out=dc)  # keeps the aux stream busy so its GEMM starts late
        if poison:
            ws.fill_(255)  # float32 NaN in the product and the row scales: an early read shows
        fn.norm_linear(xs[t % P], Ws, base.eps_f32(), variant=fn.TWO_STREAM, out=ys[t], ws=ws, aux_stream=aux)
    torch.cuda.synchronize()
    got = ys.cpu().numpy().astype(np.float64)
    bad = []
    for t in range(steps):
        ok, _ = oracle.check_close(got[t], refs[t % P], KERNEL_REL_L2 * 10, np.inf)
        if not ok:
            lag, _ = oracle.check_close(got[t], refs[(t - 1) % P], KERNEL_REL_L2 * 10, np.inf)
            kind = "one-step lag" if lag else ("poison read" if np.isnan(got[t]).any() else "wrong")
            bad.append((t, kind))
    return bad


def test_two_stream_join_long_run(gpu_lib):
    fn = gpu_lib
    steps = 1500
    _say(f"two-stream join: {steps} steps over 16 distinct inputs, delayed aux stream")
    bad = _join_stress(fn, steps)
    assert not bad, f"{len(bad)} bad steps, first {bad[:5]}"
    bad = _join_stress(fn, 300, poison=True)
    assert not bad, f"poisoned workspace: {len(bad)} bad steps, first {bad[:5]}"


def test_two_stream_stress_catches_a_missing_join(gpu_lib):
    """The same stress with the join taken out (the test-only switch): the
    post-scale then reads the product before the delayed GEMM has written
    it, and the checker must flag steps as lagging or wrong.  This is what
    shows the stress test above can fail."""
    fn = gpu_lib
    lib = fn.load()
    steps = 300
    _say(f"two-stream stress with the join removed: {steps} steps, expecting stale reads")
    assert lib.fn_testing_skip_join(1) == 0
    try:
        bad = _join_stress(fn, steps) + _join_stress(fn, steps, poison=True)
    finally:
        assert lib.fn_testing_skip_join(0) == 1
    kinds = {k for _, k in bad}
    print(f"[join removed] {len(bad)} of {2 * steps} steps flagged: {sorted(kinds)}", flush=True)
    assert len(bad) > 0, "the stress test did not notice the missing join"


@pytest.mark.parametrize("op", ["linear_prestats", "fp8_linear"])
def test_gemm_timing_hook_brackets_each_gemm(gpu_lib, monkeypatch, op):
    """The measurement hook records one event pair around each prefill GEMM
    launch, on the launch stream, and changes nothing in the results: the
    outputs with the hook on equal those with it off bit for bit, every
    pair measures a positive time no longer than the whole call's, and the
    hook is off again afterwards."""
    fn = gpu_lib
    lib = fn.load()
    monkeypatch.setenv("FN_PRESTATS", "1")
    w = synth.workload("llama7b_qkv_prefill_bf16").with_shape(640, 1040, 700)  # K: a multiple of 16 for fp8
    x = to_dev(w.x())
    g = torch.from_numpy(w.g()).cuda()
    Ws = fn.fold_weights(to_dev(w.w()), g)
    if op == "fp8_linear":
        codes, q = fn.quantize_fp8(Ws)
        call = lambda: fn.norm_linear_fp8(x, codes, q, w.eps_f32(), out_dtype=torch.bfloat16)  # noqa: E731
    else:
        call = lambda: fn.norm_linear(x, Ws, w.eps_f32(), out_dtype=torch.bfloat16)  # noqa: E731
    _say(f"gemm timing hook, {op}: "
         f"{fn.dispatch_name(fn.OP_NORM_LINEAR_FP8 if op == 'fp8_linear' else fn.OP_NORM_LINEAR, fn.FUSED, 640, 1040, 700, torch.bfloat16, torch.bfloat16)}")
    ref = call()
    torch.cuda.synchronize()
    n = 3
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    whole = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    stream = torch.cuda.current_stream()
    for a, b in ev:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    arr = ctypes.c_void_p * n
    starts = arr(*[a.cuda_event for a, _ in ev])
    stops = arr(*[b.cuda_event for _, b in ev])
    assert lib.fn_testing_gemm_events(starts, stops, n) == 0
    outs = []
    try:
        for i in range(n):
            whole[i][0].record(stream)
            outs.append(call())
            whole[i][1].record(stream)
        torch.cuda.synchronize()
    finally:
        assert lib.fn_testing_gemm_events(None, None, 0) == 0
    for i in range(n):
        assert torch.equal(outs[i], ref)
        t_gemm = ev[i][0].elapsed_time(ev[i][1])
        t_call = whole[i][0].elapsed_time(whole[i][1])
        assert 0.0 < t_gemm <= t_call, (i, t_gemm, t_call)
    # off again: a further call leaves the events where they were
    before = [a.elapsed_time(b) for a, b in ev]
    call()
    torch.cuda.synchronize()
    assert [a.elapsed_time(b) for a, b in ev] == before
