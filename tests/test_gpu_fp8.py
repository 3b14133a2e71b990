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
from gpu_util import KERNEL_REL_L2, assert_parity, from_dev, to_dev
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
@pytest.mark.parametrize("N,K", [(300, 528), (77, 4096)])
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
