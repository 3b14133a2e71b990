"""GPU parity of the LayerNorm variant (fn_fold_layernorm,
fn_layernorm_linear) through the C ABI against the float64 oracle.

The oracle is the textbook LayerNorm followed by a biased linear layer,
unfolded and undeferred; the kernel-only pin compares against the deferred
form on the oracle's own folded, stored operands.  Every case prints its name
and shape before it runs.
"""

import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import KERNEL_REL_L2, assert_parity, bits_of, from_dev, to_dev
from synth import BF16, F32

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _ln_workload(M, K, N, dtype=BF16, mean_sigma=1.0, name="ln_qkv_prefill_bf16"):
    w = synth.workload(name)
    return dataclasses.replace(w, M=M, K=K, N=N, dtype=dtype, mean_sigma=mean_sigma)


def _vec(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def run_ln(fn, w, variant, out_dtype, with_beta=True, with_bias=True, x=None):
    xd = to_dev(w.x() if x is None else x)
    W, g = to_dev(w.w()), _vec(w.g())
    beta = _vec(w.beta()) if with_beta else None
    bias = _vec(w.bias()) if with_bias else None
    if variant == fn.UNFUSED:
        return fn.layernorm_linear(xd, W, w.eps_f32(), g=g, beta=beta, bias=bias, variant=variant,
                                   out_dtype=out_dtype)
    Ws, c, b = fn.fold_layernorm(W, g, beta, bias)
    return fn.layernorm_linear(xd, Ws, w.eps_f32(), colsum=c, b_star=b, variant=variant, out_dtype=out_dtype)


def ref_ln(w, with_beta=True, with_bias=True, x=None):
    return oracle.layernorm_linear(w.x() if x is None else x, w.w(), w.g(), w.beta() if with_beta else None,
                                   w.bias() if with_bias else None, w.eps_f32())


# ---------------------------------------------------------------------------
# the fold: W* bit-exact, column sums and folded bias as the oracle rounds them
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", [BF16, F32])
def test_fold_layernorm_matches_oracle(gpu_lib, dt):
    fn = gpu_lib
    w = _ln_workload(1, 1032, 300, dtype=dt)
    _say(f"fold_layernorm N=300 K=1032 {dt} (and in place)")
    Wn, g, beta, bias = w.w(), w.g(), w.beta(), w.bias()
    Ws_ref, c_ref, b_ref = oracle.fold_layernorm(Wn, g, beta, bias, dt)
    W = to_dev(Wn)
    Ws, c, b = fn.fold_layernorm(W, _vec(g), _vec(beta), _vec(bias))
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(Ws), Ws_ref.view(np.uint16) if dt == BF16 else Ws_ref.view(np.uint32))
    # float64 sums rounded once: equal to the oracle's unless a sum sits on a
    # float32 rounding boundary to within float64 error (then one ulp)
    for got, want in ((c, c_ref), (b, b_ref)):
        g32 = got.cpu().numpy()
        assert np.all(np.abs(g32.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64)) <= 1)
        assert np.mean(g32 == want) > 0.99
    # in place, no beta or bias
    Wi = W.clone()
    lib = fn.load()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    cc = torch.empty(300, device="cuda")
    bb = torch.full((300,), 5.0, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.fn_fold_layernorm(P(Wi), fn._dt(Wi), P(_vec(g)), None, None, 300, 1032, P(Wi), fn._dt(Wi), P(cc),
                                 P(bb), st) == 0
    torch.cuda.synchronize()
    Ws_ref0, c_ref0, _ = oracle.fold_layernorm(Wn, g, None, None, dt)
    assert np.array_equal(bits_of(Wi), Ws_ref0.view(np.uint16) if dt == BF16 else Ws_ref0.view(np.uint32))
    assert torch.all(bb == 0.0)


# ---------------------------------------------------------------------------
# the op on reduced shapes: several tiles, ragged M / N / K tails, decode rows
# ---------------------------------------------------------------------------

LN_CASES = [
    # M, K, N
    (300, 1032, 700),  # K tail of 8: the statistics see 56 zero columns
    (130, 576, 300),
    (600, 1024, 520),
    (16, 4096, 300),   # decode kernel
    (4, 520, 77),      # decode kernel, ragged N
    (1, 4096, 1000),
]


@pytest.mark.parametrize("M,K,N", LN_CASES)
@pytest.mark.parametrize("variant", ["fused", "unfused"])
def test_layernorm_linear_parity(gpu_lib, M, K, N, variant):
    fn = gpu_lib
    w = _ln_workload(M, K, N)
    v = fn.FUSED if variant == "fused" else fn.UNFUSED
    _say(f"layernorm_linear M={M} K={K} N={N} {variant} -> "
         f"{fn.dispatch_name(fn.OP_LAYERNORM_LINEAR, v, M, K, N, torch.bfloat16, torch.float32)}")
    ref = ref_ln(w)
    for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
        y = run_ln(fn, w, v, od)
        torch.cuda.synchronize()
        assert_parity(y, ref, BF16, f"layernorm {variant} {od}", out_bf16=ob)
    # no LayerNorm bias, no linear bias
    y = run_ln(fn, w, v, torch.float32, with_beta=False, with_bias=False)
    assert_parity(y, ref_ln(w, False, False), BF16, f"layernorm {variant} no biases")


@pytest.mark.parametrize("M,K,N", [(128, 576, 960), (37, 100, 50)])
@pytest.mark.parametrize("variant", ["fused", "unfused"])
def test_layernorm_linear_f32(gpu_lib, M, K, N, variant):
    fn = gpu_lib
    w = _ln_workload(M, K, N, dtype=F32)
    v = fn.FUSED if variant == "fused" else fn.UNFUSED
    _say(f"layernorm_linear f32 M={M} K={K} N={N} {variant}")
    y = run_ln(fn, w, v, torch.float32)
    torch.cuda.synchronize()
    assert_parity(y, ref_ln(w), F32, f"layernorm f32 {variant}")


@pytest.mark.parametrize("tile", list(range(9)))
def test_layernorm_every_tile_config(gpu_lib, tile, monkeypatch):
    fn = gpu_lib
    monkeypatch.setenv("FN_TILE", str(tile))
    w = _ln_workload(300, 1032, 700)
    _say(f"layernorm tile {tile}: "
         f"{fn.dispatch_name(fn.OP_LAYERNORM_LINEAR, fn.FUSED, w.M, w.K, w.N, torch.bfloat16, torch.bfloat16)}")
    ref = ref_ln(w)
    for v in (fn.FUSED, fn.UNFUSED):
        for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
            y = run_ln(fn, w, v, od)
            torch.cuda.synchronize()
            assert_parity(y, ref, BF16, f"tile {tile} layernorm v{v} {od}", out_bf16=ob)


def test_layernorm_kernel_only_pin(gpu_lib):
    """Against the deferred form on the oracle's own folded, stored operands
    (W*, column sums, folded bias): only float32 arithmetic differs."""
    fn = gpu_lib
    _say("kernel-only pins: layernorm 300x1032x700 (prefill), 8x1032x300 (decode)")
    for M, K, N in [(300, 1032, 700), (8, 1032, 300)]:
        w = _ln_workload(M, K, N)
        Ws, c, b = oracle.fold_layernorm(w.w(), w.g(), w.beta(), w.bias(), BF16)
        y = fn.layernorm_linear(to_dev(w.x()), to_dev(Ws), w.eps_f32(), colsum=_vec(c), b_star=_vec(b),
                                out_dtype=torch.float32)
        ref = oracle.layernorm_deferred_on_folded(w.x(), Ws, c, b, w.eps_f32())
        assert_parity(y, ref, BF16, f"kernel layernorm M={M}", rel_l2=KERNEL_REL_L2, max_abs=np.inf)


@pytest.mark.parametrize("M,K,N", [(300, 1032, 700), (17, 72, 17)])
@pytest.mark.parametrize("prestats", ["0", "1"])
def test_layernorm_prestats_switch(gpu_lib, M, K, N, prestats, monkeypatch):
    """The fused variant with the row statistics taken inside the GEMM (0) or
    in a pass before it (1), on ragged shapes, against the oracle and the
    kernel-only reference."""
    fn = gpu_lib
    monkeypatch.setenv("FN_PRESTATS", prestats)
    w = _ln_workload(M, K, N)
    name = fn.dispatch_name(fn.OP_LAYERNORM_LINEAR, fn.FUSED, M, K, N, torch.bfloat16, torch.bfloat16)
    _say(f"layernorm FN_PRESTATS={prestats} {M}x{K}x{N} -> {name}")
    assert ("ln_stats+" in name) == (prestats == "1")
    for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
        y = run_ln(fn, w, fn.FUSED, od)
        torch.cuda.synchronize()
        assert_parity(y, ref_ln(w), BF16, f"layernorm prestats={prestats} {od}", out_bf16=ob)
    Ws, c, b = oracle.fold_layernorm(w.w(), w.g(), w.beta(), w.bias(), BF16)
    y = fn.layernorm_linear(to_dev(w.x()), to_dev(Ws), w.eps_f32(), colsum=_vec(c), b_star=_vec(b),
                            out_dtype=torch.float32)
    assert_parity(y, oracle.layernorm_deferred_on_folded(w.x(), Ws, c, b, w.eps_f32()), BF16,
                  f"kernel layernorm prestats={prestats}", rel_l2=KERNEL_REL_L2, max_abs=np.inf)


@pytest.mark.parametrize("offset", [10.0, 30.0, 100.0])
def test_layernorm_large_row_means(gpu_lib, offset):
    """Rows whose mean is `offset` standard deviations away from zero: the
    shifted statistics keep the variance accurate; the deferred product keeps
    a relative error of about 2^-24 sqrt(K) offset."""
    fn = gpu_lib
    w = _ln_workload(200, 1032, 300, mean_sigma=0.0)
    _say(f"layernorm row means {offset} x std, prefill and decode")
    x = synth.stored_to_f64(w.x())
    x = x + offset * np.abs(x).std(axis=1, keepdims=True) * np.sign(np.arange(200) % 3 - 1 + 0.5)[:, None]
    xb = synth.bf16_bits_from_f32(x.astype(np.float32))
    ref = ref_ln(w, x=xb)
    y = run_ln(fn, w, fn.FUSED, torch.float32, x=xb)
    assert_parity(y, ref, BF16, f"layernorm offset {offset} prefill")
    import os
    os.environ["FN_PRESTATS"] = "1"
    try:
        y = run_ln(fn, w, fn.FUSED, torch.float32, x=xb)
        assert_parity(y, ref, BF16, f"layernorm offset {offset} prefill, statistics pass")
    finally:
        del os.environ["FN_PRESTATS"]
    y16 = run_ln(fn, dataclasses.replace(w, M=16), fn.FUSED, torch.float32, x=xb[:16])
    assert_parity(y16, ref[:16], BF16, f"layernorm offset {offset} decode")


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------

def test_full_ln_qkv_prefill(gpu_lib):
    """Every output of the 4096 x 4096 x 12288 LayerNorm workload."""
    fn = gpu_lib
    w = synth.workload("ln_qkv_prefill_bf16")
    _say("full ln_qkv_prefill 4096x4096x12288 (fused, unfused; every row)")
    ref = oracle.layernorm_linear(w.x(), w.w(), w.g(), w.beta(), w.bias(), w.eps_f32())
    for v in (fn.FUSED, fn.UNFUSED):
        for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
            y = run_ln(fn, w, v, od)
            assert_parity(y, ref, BF16, f"ln_qkv v{v} {od}", out_bf16=ob)
            del y


@pytest.mark.parametrize("name", ["ln_fc1_decode_m1_bf16", "ln_fc1_decode_m16_bf16"])
def test_full_ln_fc1_decode(gpu_lib, name):
    fn = gpu_lib
    w = synth.workload(name)
    ref = ref_ln(w)
    for v in (fn.FUSED, fn.UNFUSED):
        _say(f"full {name} M={w.M}x4096x16384 variant={v}")
        y = run_ln(fn, w, v, torch.float32)
        assert_parity(y, ref, BF16, f"{name} v{v}")
