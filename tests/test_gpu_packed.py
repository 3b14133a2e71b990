"""GPU tests of the decode-packed weight layout (fn_pack_decode_weights and
the FUSED_PACKED variant) through the C ABI.

The layout is integer work: the packed bytes must equal, bit for bit, a
numpy re-layout written from the layout's definition (16-row slabs; each
64-byte K step of a slab stored as 64 pieces of 16 bytes, piece p holding
row p mod 16 and bytes 16 floor(p / 16) .. + 15 of the step; zero padding).
The ops on packed weights are compared with the float64 oracle on the
oracle's own folded (and quantised) operands, with the workload tolerance on
the full decode workloads, and with the row-major fused result: bit for bit
where the two walk K in the same order (every fp8 call; bf16 glu calls with
M > 4 and single-weight calls with M <= 4), else within the kernel-only
tolerance.  Every case prints its name
and shape before it runs.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import KERNEL_REL_L2, assert_parity, bits_of, from_dev, to_dev
from synth import BF16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _vec(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _pack_ref(row_bytes: np.ndarray) -> np.ndarray:
    """The decode-packed layout of a row-major [N x B] byte matrix."""
    N, B = row_bytes.shape
    J, S = -(-N // 16), -(-B // 64)
    pad = np.zeros((J * 16, S * 64), np.uint8)
    pad[:N, :B] = row_bytes
    # [slab j, row r, step st, chunk c, byte] -> [j, st, piece c * 16 + r, byte]
    return pad.reshape(J, 16, S, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)


def _bytes_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


@pytest.mark.parametrize("kind,N,K", [("bf16", 77, 520), ("bf16", 16, 64), ("bf16", 33, 72), ("fp8", 300, 528),
                                      ("fp8", 1, 16)])
def test_pack_layout_bit_exact(gpu_lib, kind, N, K):
    fn = gpu_lib
    _say(f"pack_decode_weights {kind} N={N} K={K}")
    gen = torch.Generator().manual_seed(N * 1000 + K)
    if kind == "bf16":
        W = torch.randn(N, K, generator=gen).to(torch.bfloat16).cuda()
    else:
        W = torch.randint(0, 256, (N, K), generator=gen, dtype=torch.uint8).cuda()
    guard = torch.full((fn.decode_packed_bytes(N, K, W.dtype) + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    P = fn.pack_decode_weights(W, out=guard)
    torch.cuda.synchronize()
    want = _pack_ref(_bytes_of(W))
    got = guard.cpu().numpy()
    assert P.N == N and P.K == K and want.size == fn.decode_packed_bytes(N, K, W.dtype)
    assert np.array_equal(got[:want.size], want)
    assert np.all(got[want.size:] == 0xA5), "wrote past the packed size"


def _glu_w(M, K, N, name="llama7b_ffn_decode_m4_bf16"):
    return dataclasses.replace(synth.workload(name), M=M, K=K, N=N)


CASES = [
    # M, K, N
    (1, 4096, 1000),
    (3, 520, 77),     # ragged N and a K tail inside the last 32-wide step
    (5, 1040, 300),
    (16, 4096, 300),
    (16, 72, 33),
]


def _same_order(M, glu):
    """bf16 row-major calls take consecutive K steps per wave for M <= 4 and
    round-robin ones above; packed calls take round-robin steps for the glu
    epilogue and consecutive ones for a single weight, at every M."""
    return M > 4 if glu else M <= 4


def _compare_to_rowmajor(y_pk, y_rm, exact, label):
    if exact:
        assert np.array_equal(bits_of(y_pk), bits_of(y_rm)), f"{label}: packed differs from row-major"
    else:
        ok, info = oracle.check_close(from_dev(y_pk), from_dev(y_rm), KERNEL_REL_L2, np.inf)
        print(f"[rowmajor] {label}: {info}", flush=True)
        assert ok, f"{label}: {info}"


@pytest.mark.parametrize("M,K,N", CASES)
def test_packed_bf16_ops(gpu_lib, M, K, N):
    fn = gpu_lib
    w = _glu_w(M, K, N)
    _say(f"packed bf16 linear / glu M={M} K={K} N={N}")
    eps = w.eps_f32()
    x = to_dev(w.x())
    Wg = oracle.fold_weights(w.w(), w.g(), BF16)
    Wu = oracle.fold_weights(w.w_up(), w.g(), BF16)
    Wg_d, Wu_d = to_dev(Wg), to_dev(Wu)
    Pg, Pu = fn.pack_decode_weights(Wg_d), fn.pack_decode_weights(Wu_d)
    for od in (torch.float32, torch.bfloat16):
        y = fn.norm_linear(x, Pg, eps, out_dtype=od)
        h = fn.norm_glu_ffn(x, Pg, Pu, eps, out_dtype=od)
        y_rm = fn.norm_linear(x, Wg_d, eps, out_dtype=od)
        h_rm = fn.norm_glu_ffn(x, Wg_d, Wu_d, eps, out_dtype=od)
        torch.cuda.synchronize()
        if od == torch.float32:
            assert_parity(y, oracle.deferred_on_folded(w.x(), Wg, eps), BF16, "packed linear kernel-only",
                          rel_l2=KERNEL_REL_L2, max_abs=np.inf)
            assert_parity(h, oracle.glu_deferred_on_folded(w.x(), Wg, Wu, eps), BF16, "packed glu kernel-only",
                          rel_l2=KERNEL_REL_L2, max_abs=np.inf)
        _compare_to_rowmajor(y, y_rm, _same_order(M, False), f"linear {od}")
        _compare_to_rowmajor(h, h_rm, _same_order(M, True), f"glu {od}")


@pytest.mark.parametrize("M,K,N", [(1, 4096, 1000), (3, 520, 77), (16, 1040, 300)])
def test_packed_layernorm(gpu_lib, M, K, N):
    fn = gpu_lib
    w = dataclasses.replace(synth.workload("ln_fc1_decode_m16_bf16"), M=M, K=K, N=N)
    _say(f"packed layernorm M={M} K={K} N={N}")
    eps = w.eps_f32()
    Ws, c, b = oracle.fold_layernorm(w.w(), w.g(), w.beta(), w.bias(), BF16)
    Ws_d = to_dev(Ws)
    P = fn.pack_decode_weights(Ws_d)
    x = to_dev(w.x())
    y = fn.layernorm_linear(x, P, eps, colsum=_vec(c), b_star=_vec(b), out_dtype=torch.float32)
    y_rm = fn.layernorm_linear(x, Ws_d, eps, colsum=_vec(c), b_star=_vec(b), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_parity(y, oracle.layernorm_deferred_on_folded(w.x(), Ws, c, b, eps), BF16, "packed ln kernel-only",
                  rel_l2=KERNEL_REL_L2, max_abs=np.inf)
    _compare_to_rowmajor(y, y_rm, _same_order(M, False), "layernorm")


@pytest.mark.parametrize("M,K,N", [(1, 4096, 1000), (4, 528, 300), (16, 1040, 77)])
def test_packed_fp8_ops(gpu_lib, M, K, N):
    fn = gpu_lib
    w = _glu_w(M, K, N, "llama7b_ffn_decode_m4_fp8")
    _say(f"packed fp8 linear / glu M={M} K={K} N={N}")
    eps = w.eps_f32()
    cg, qg = oracle.quantize_fp8_per_channel(oracle.fold_weights(w.w(), w.g(), BF16))
    cu, qu = oracle.quantize_fp8_per_channel(oracle.fold_weights(w.w_up(), w.g(), BF16))
    cg_d, cu_d = torch.from_numpy(cg).cuda(), torch.from_numpy(cu).cuda()
    Pg, Pu = fn.pack_decode_weights(cg_d), fn.pack_decode_weights(cu_d)
    x = to_dev(w.x())
    y = fn.norm_linear_fp8(x, Pg, _vec(qg), eps, out_dtype=torch.float32)
    h = fn.norm_glu_ffn_fp8(x, Pg, _vec(qg), Pu, _vec(qu), eps, out_dtype=torch.float32)
    y_rm = fn.norm_linear_fp8(x, cg_d, _vec(qg), eps, out_dtype=torch.float32)
    h_rm = fn.norm_glu_ffn_fp8(x, cg_d, _vec(qg), cu_d, _vec(qu), eps, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_parity(y, oracle.deferred_on_quantized(w.x(), cg, qg, eps), BF16, "packed fp8 linear kernel-only",
                  rel_l2=KERNEL_REL_L2, max_abs=np.inf)
    assert_parity(h, oracle.glu_deferred_on_quantized(w.x(), cg, qg, cu, qu, eps), BF16,
                  "packed fp8 glu kernel-only", rel_l2=KERNEL_REL_L2, max_abs=np.inf)
    _compare_to_rowmajor(y, y_rm, True, "fp8 linear")
    _compare_to_rowmajor(h, h_rm, True, "fp8 glu")


@pytest.mark.parametrize("name", ["llama7b_ffn_decode_m1_bf16", "llama7b_ffn_decode_m4_bf16",
                                  "llama7b_ffn_decode_m16_bf16"])
def test_full_decode_packed(gpu_lib, name):
    """The full Llama-7B FFN decode step: fold and pack on the GPU, then the
    packed op, against the textbook oracle (workload tolerance) and the
    deferred form on the oracle's folded weights."""
    fn = gpu_lib
    w = synth.workload(name)
    _say(f"full {name} packed: M={w.M} K=4096 N=11008")
    g = _vec(w.g())
    Pg = fn.pack_decode_weights(fn.fold_weights(to_dev(w.w()), g))
    Pu = fn.pack_decode_weights(fn.fold_weights(to_dev(w.w_up()), g))
    h = fn.norm_glu_ffn(to_dev(w.x()), Pg, Pu, w.eps_f32(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_parity(h, oracle.norm_glu_ffn(w.x(), w.w(), w.w_up(), w.g(), w.eps_f32()), BF16, f"{name} packed")
    Wg = oracle.fold_weights(w.w(), w.g(), BF16)
    Wu = oracle.fold_weights(w.w_up(), w.g(), BF16)
    assert_parity(h, oracle.glu_deferred_on_folded(w.x(), Wg, Wu, w.eps_f32()), BF16, f"{name} packed kernel-only",
                  rel_l2=KERNEL_REL_L2, max_abs=np.inf)


@pytest.mark.parametrize("name", ["llama7b_ffn_decode_m1_fp8", "llama7b_ffn_decode_m16_fp8"])
def test_full_decode_packed_fp8(gpu_lib, name):
    fn = gpu_lib
    w = synth.workload(name)
    _say(f"full {name} packed: M={w.M} K=4096 N=11008, fold + quantise + pack on the GPU")
    g = _vec(w.g())
    cg_d, qg_d = fn.quantize_fp8(fn.fold_weights(to_dev(w.w()), g))
    cu_d, qu_d = fn.quantize_fp8(fn.fold_weights(to_dev(w.w_up()), g))
    h = fn.norm_glu_ffn_fp8(to_dev(w.x()), fn.pack_decode_weights(cg_d), qg_d, fn.pack_decode_weights(cu_d), qu_d,
                            w.eps_f32(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    cg, qg = oracle.quantize_fp8_per_channel(oracle.fold_weights(w.w(), w.g(), BF16))
    cu, qu = oracle.quantize_fp8_per_channel(oracle.fold_weights(w.w_up(), w.g(), BF16))
    assert_parity(h, oracle.glu_deferred_on_quantized(w.x(), cg, qg, cu, qu, w.eps_f32()), BF16,
                  f"{name} packed kernel-only", rel_l2=KERNEL_REL_L2, max_abs=np.inf)
    assert_parity(h, oracle.norm_glu_ffn(w.x(), oracle.dequantize_fp8(cg, qg), oracle.dequantize_fp8(cu, qu),
                                         np.ones(w.K), w.eps_f32()), BF16, f"{name} packed textbook")


def test_full_ln_decode_packed(gpu_lib):
    fn = gpu_lib
    w = synth.workload("ln_fc1_decode_m16_bf16")
    _say(f"full ln_fc1_decode_m16_bf16 packed: M={w.M} K={w.K} N={w.N}")
    Ws, c, b = fn.fold_layernorm(to_dev(w.w()), _vec(w.g()), _vec(w.beta()), _vec(w.bias()))
    y = fn.layernorm_linear(to_dev(w.x()), fn.pack_decode_weights(Ws), w.eps_f32(), colsum=c, b_star=b,
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_parity(y, oracle.layernorm_linear(w.x(), w.w(), w.g(), w.beta(), w.bias(), w.eps_f32()), BF16,
                  "ln decode packed")


def test_packed_rejections_write_nothing(gpu_lib):
    """Packed weights with more than 16 rows, or on an op without the
    weight-streaming kernel, fail before launching anything."""
    fn = gpu_lib
    _say("packed weights: M = 17 and the qknorm op are rejected")
    W = torch.randn(64, 128, device="cuda").to(torch.bfloat16)
    P = fn.pack_decode_weights(W)
    x = torch.randn(17, 128, device="cuda").to(torch.bfloat16)
    y = torch.full((17, 64), 7.0, device="cuda")
    with pytest.raises(fn.FlashNormError, match="UNSUPPORTED"):
        fn.norm_linear(x, P, 1e-6, out=y)
    with pytest.raises(ValueError):
        fn.norm_linear(x[:4], P, 1e-6, g=torch.ones(128, device="cuda"), variant=fn.UNFUSED, out=y[:4])
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ---------------------------------------------------------------------------
# the gate/up pair layout (fn_pack_decode_weights_glu)
# ---------------------------------------------------------------------------

def _pair_ref(gate_bytes: np.ndarray, up_bytes: np.ndarray) -> np.ndarray:
    """Each K step of a slab: the gate slab's 1 KB, then the up slab's."""
    N, B = gate_bytes.shape
    J, S = -(-N // 16), -(-B // 64)
    g = _pack_ref(gate_bytes).reshape(J, S, 1024)
    u = _pack_ref(up_bytes).reshape(J, S, 1024)
    return np.stack([g, u], axis=2).reshape(-1)


@pytest.mark.parametrize("kind,N,K", [("bf16", 77, 520), ("fp8", 300, 528), ("bf16", 16, 64)])
def test_pack_pair_layout_bit_exact(gpu_lib, kind, N, K):
    fn = gpu_lib
    _say(f"pack_decode_weights_glu {kind} N={N} K={K}")
    gen = torch.Generator().manual_seed(N * 7 + K)
    if kind == "bf16":
        Wg = torch.randn(N, K, generator=gen).to(torch.bfloat16).cuda()
        Wu = torch.randn(N, K, generator=gen).to(torch.bfloat16).cuda()
    else:
        Wg = torch.randint(0, 256, (N, K), generator=gen, dtype=torch.uint8).cuda()
        Wu = torch.randint(0, 256, (N, K), generator=gen, dtype=torch.uint8).cuda()
    size = 2 * fn.decode_packed_bytes(N, K, Wg.dtype)
    guard = torch.full((size + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    P = fn.pack_decode_weights_glu(Wg, Wu, out=guard)
    torch.cuda.synchronize()
    want = _pair_ref(_bytes_of(Wg), _bytes_of(Wu))
    got = guard.cpu().numpy()
    assert P.pair and want.size == size
    assert np.array_equal(got[:size], want)
    assert np.all(got[size:] == 0xA5), "wrote past the packed size"


@pytest.mark.parametrize("M,K,N", [(1, 4096, 1000), (3, 520, 77), (16, 1040, 300)])
def test_pair_layout_matches_two_buffers(gpu_lib, M, K, N):
    """The pair layout changes only where the kernel reads: bit for bit the
    result of the two packed buffers, and the oracle's deferred form."""
    fn = gpu_lib
    _say(f"gate/up pair layout, bf16 and fp8, M={M} K={K} N={N}")
    w = _glu_w(M, K, N)
    eps = w.eps_f32()
    x = to_dev(w.x())
    Wg = oracle.fold_weights(w.w(), w.g(), BF16)
    Wu = oracle.fold_weights(w.w_up(), w.g(), BF16)
    Wg_d, Wu_d = to_dev(Wg), to_dev(Wu)
    for od in (torch.float32, torch.bfloat16):
        h_pair = fn.norm_glu_ffn(x, fn.pack_decode_weights_glu(Wg_d, Wu_d), None, eps, out_dtype=od)
        h_two = fn.norm_glu_ffn(x, fn.pack_decode_weights(Wg_d), fn.pack_decode_weights(Wu_d), eps, out_dtype=od)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(h_pair), bits_of(h_two)), f"bf16 pair differs from two buffers ({od})"
        if od == torch.float32:
            assert_parity(h_pair, oracle.glu_deferred_on_folded(w.x(), Wg, Wu, eps), BF16, "pair glu kernel-only",
                          rel_l2=KERNEL_REL_L2, max_abs=np.inf)
    if K % 16 == 0:
        cg, qg = oracle.quantize_fp8_per_channel(Wg)
        cu, qu = oracle.quantize_fp8_per_channel(Wu)
        cg_d, cu_d = torch.from_numpy(cg).cuda(), torch.from_numpy(cu).cuda()
        h8_pair = fn.norm_glu_ffn_fp8(x, fn.pack_decode_weights_glu(cg_d, cu_d), _vec(qg), None, _vec(qu), eps,
                                      out_dtype=torch.float32)
        h8_two = fn.norm_glu_ffn_fp8(x, fn.pack_decode_weights(cg_d), _vec(qg), fn.pack_decode_weights(cu_d),
                                     _vec(qu), eps, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(h8_pair), bits_of(h8_two)), "fp8 pair differs from two buffers"
        assert_parity(h8_pair, oracle.glu_deferred_on_quantized(w.x(), cg, qg, cu, qu, eps), BF16,
                      "fp8 pair glu kernel-only", rel_l2=KERNEL_REL_L2, max_abs=np.inf)


@pytest.mark.parametrize("name", ["llama7b_ffn_decode_m1_bf16", "llama7b_ffn_decode_m16_bf16",
                                  "llama7b_ffn_decode_m4_fp8"])
def test_full_decode_pair(gpu_lib, name):
    fn = gpu_lib
    w = synth.workload(name)
    _say(f"full {name} on the gate/up pair layout: M={w.M} K=4096 N=11008")
    g = _vec(w.g())
    Wg_d, Wu_d = fn.fold_weights(to_dev(w.w()), g), fn.fold_weights(to_dev(w.w_up()), g)
    if w.fp8:
        cg_d, qg_d = fn.quantize_fp8(Wg_d)
        cu_d, qu_d = fn.quantize_fp8(Wu_d)
        h = fn.norm_glu_ffn_fp8(to_dev(w.x()), fn.pack_decode_weights_glu(cg_d, cu_d), qg_d, None, qu_d, w.eps_f32(),
                                out_dtype=torch.float32)
        cg, qg = oracle.quantize_fp8_per_channel(oracle.fold_weights(w.w(), w.g(), BF16))
        cu, qu = oracle.quantize_fp8_per_channel(oracle.fold_weights(w.w_up(), w.g(), BF16))
        ref = oracle.glu_deferred_on_quantized(w.x(), cg, qg, cu, qu, w.eps_f32())
        torch.cuda.synchronize()
        assert_parity(h, ref, BF16, f"{name} pair kernel-only", rel_l2=KERNEL_REL_L2, max_abs=np.inf)
        assert_parity(h, oracle.norm_glu_ffn(w.x(), oracle.dequantize_fp8(cg, qg), oracle.dequantize_fp8(cu, qu),
                                             np.ones(w.K), w.eps_f32()), BF16, f"{name} pair textbook")
    else:
        h = fn.norm_glu_ffn(to_dev(w.x()), fn.pack_decode_weights_glu(Wg_d, Wu_d), None, w.eps_f32(),
                            out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_parity(h, oracle.norm_glu_ffn(w.x(), w.w(), w.w_up(), w.g(), w.eps_f32()), BF16, f"{name} pair")
