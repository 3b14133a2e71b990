"""Edge cases of the later entry points on the GPU: empty inputs (M = 0
launches nothing and writes nothing), the smallest legal shapes and ragged
ones, against the float64 oracle.  Every case prints its name and shape
before it runs."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, to_dev
from synth import BF16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _vec(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _ln_bound(w, c, b, K):
    """Elementwise bound on |float32 result - the deferred form on the oracle's
    folded operands| for the LayerNorm path.  The kernels zero-pad K up to
    their step (at most 64 columns) and take the row statistics shifted by
    the row's first element sh, so every float32 sum runs over Kp = K + 64
    terms that include up to 64 copies of sh; each such sum errs by at most
    Kp u times the sum of its terms' magnitudes (u = 2^-24).  The fold's
    column sums and folded bias are within one float32 ulp of the oracle's."""
    u, Kp = 2.0 ** -24, K + 64
    xf = synth.stored_to_f64(w.x())
    Wn = synth.stored_to_f64(oracle.fold_layernorm(w.w(), w.g(), w.beta(), w.bias(), BF16)[0])
    sh = np.abs(xf[:, 0])
    d = xf - xf[:, :1]
    mu = xf.mean(axis=1)
    var = xf.var(axis=1)
    s = 1.0 / np.sqrt(var + w.eps_f32())
    ds1 = Kp * u * (np.abs(d).sum(axis=1) + 64 * sh)
    ds2 = Kp * u * ((d * d).sum(axis=1) + 64 * sh * sh)
    dvar = ds2 / K + 2 * np.abs(d.mean(axis=1)) * ds1 / K + (ds1 / K) ** 2 + 4 * u * (var + d.mean(axis=1) ** 2)
    rel_s = 0.5 * dvar / (var + w.eps_f32()) + 4 * u
    dmu = ds1 / K + 2 * u * np.abs(mu)
    aW = np.abs(Wn).sum(axis=1)
    core = s[:, None] * np.abs(xf @ Wn.T - mu[:, None] * np.asarray(c, np.float64)[None, :])
    z_err = Kp * u * (np.abs(xf) @ np.abs(Wn).T)
    c_err = dmu[:, None] * aW[None, :] + np.abs(mu)[:, None] * (2 * u * np.abs(c) + Kp * u * aW)[None, :]
    bb = np.abs(np.asarray(b, np.float64))[None, :]
    return s[:, None] * (z_err + c_err) + rel_s[:, None] * core + 4 * u * (core + bb) + 2 * u * bb


@pytest.mark.parametrize("M,K,N", [(1, 8, 1), (3, 24, 5), (17, 72, 33), (2, 4104, 3)])
def test_layernorm_small_and_ragged(gpu_lib, M, K, N):
    """K >= 64: the workload tolerance against the textbook oracle.  Tiny K
    leaves a row of one or a few outputs with no averaging, so (as for the
    RMSNorm shape sweep) the fused result is held to a float32 error bound
    against the deferred form on the oracle's own folded operands, and the
    unfused one against the textbook form with its bf16-stored xn."""
    from gpu_util import assert_within

    fn = gpu_lib
    w = dataclasses.replace(synth.workload("ln_qkv_prefill_bf16"), M=M, K=K, N=N)
    _say(f"layernorm {M}x{K}x{N} fused and unfused")
    W, g = to_dev(w.w()), _vec(w.g())
    Ws, c, b = fn.fold_layernorm(W, g, _vec(w.beta()), _vec(w.bias()))
    y = fn.layernorm_linear(to_dev(w.x()), Ws, w.eps_f32(), colsum=c, b_star=b, out_dtype=torch.float32)
    yu = fn.layernorm_linear(to_dev(w.x()), W, w.eps_f32(), g=g, beta=_vec(w.beta()), bias=_vec(w.bias()),
                             variant=fn.UNFUSED, out_dtype=torch.float32)
    if K >= 64:
        ref = oracle.layernorm_linear(w.x(), w.w(), w.g(), w.beta(), w.bias(), w.eps_f32())
        assert_parity(y, ref, BF16, f"layernorm fused {M}x{K}x{N}")
        assert_parity(yu, ref, BF16, f"layernorm unfused {M}x{K}x{N}")
        return
    Wso, co, bo = oracle.fold_layernorm(w.w(), w.g(), w.beta(), w.bias(), BF16)
    ref_k = oracle.layernorm_deferred_on_folded(w.x(), Wso, co, bo, w.eps_f32())
    assert_within(y, ref_k, _ln_bound(w, co, bo, K), f"layernorm fused {M}x{K}x{N}")
    xn = oracle.round_to_bf16(oracle.layernorm(w.x(), w.g(), w.beta(), w.eps_f32()))
    Wd = synth.stored_to_f64(w.w())
    ref_u = xn @ Wd.T + w.bias()
    # a float32 LayerNorm may round xn one bf16 ulp (2^-7 relative) away
    # from the float64 one; then the float32 product of K terms
    mag_u = np.abs(xn) @ np.abs(Wd).T
    bound_u = 2.0 ** -7 * mag_u + (K + 64) * 2.0 ** -24 * (1 + 2.0 ** -7) * mag_u + 2.0 ** -22 * np.abs(w.bias())
    assert_within(yu, ref_u, bound_u, f"layernorm unfused {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(1, 16, 1), (16, 16, 7), (2, 48, 17)])
def test_fp8_smallest_shapes(gpu_lib, M, K, N):
    fn = gpu_lib
    w = dataclasses.replace(synth.workload("llama7b_ffn_decode_m4_fp8"), M=M, K=K, N=N)
    _say(f"fp8 {M}x{K}x{N}")
    Wg = oracle.fold_weights(w.w(), w.g(), BF16)
    Wu = oracle.fold_weights(w.w_up(), w.g(), BF16)
    cg, qg = oracle.quantize_fp8_per_channel(Wg)
    cu, qu = oracle.quantize_fp8_per_channel(Wu)
    c_dev, q_dev = fn.quantize_fp8(to_dev(Wg))
    torch.cuda.synchronize()
    assert np.array_equal(c_dev.cpu().numpy(), cg)
    h = fn.norm_glu_ffn_fp8(to_dev(w.x()), torch.from_numpy(cg).cuda(), _vec(qg), torch.from_numpy(cu).cuda(),
                            _vec(qu), w.eps_f32(), out_dtype=torch.float32)
    assert_parity(h, oracle.glu_deferred_on_quantized(w.x(), cg, qg, cu, qu, w.eps_f32()), BF16,
                  f"fp8 glu {M}x{K}x{N}", rel_l2=2e-5, max_abs=np.inf)


@pytest.mark.parametrize("M,K,nq,nkv,nr,rot", [(1, 8, 32, 0, 4, 4), (3, 24, 0, 32, 8, 4), (33, 40, 64, 32, 0, 0)])
def test_latent_small(gpu_lib, M, K, nq, nkv, nr, rot):
    fn = gpu_lib
    w = dataclasses.replace(synth.workload("mla_latent_attn_in_bf16"), M=M, K=K, N=nq + nkv + nr, n_q_latent=nq,
                            n_kv_latent=nkv, n_rope=nr, rot_dim=rot, n_pos=64)
    _say(f"latent {M}x{K} q{nq} kv{nkv} rope{nr} rot{rot}")
    pos = w.positions() if nr else None
    ref = oracle.linear_latent_norm(w.x(), w.w(), w.g(), w.eps_f32(), nq, nkv, nr,
                                    w.g_q_latent() if nq else None, w.g_kv_latent() if nkv else None,
                                    w.eps_head_f32(), pos, w.rope_base, rot)
    g1 = _vec(w.g())
    y = fn.linear_latent_norm(to_dev(w.x()), fn.fold_weights(to_dev(w.w()), g1), nq, nkv, nr,
                              _vec(w.g_q_latent()) if nq else None, _vec(w.g_kv_latent()) if nkv else None,
                              w.eps_f32(), w.eps_head_f32(),
                              torch.from_numpy(pos).cuda() if nr else None,
                              fn.rope_table(w.rope_base, rot, 64) if nr else None, out_dtype=torch.float32)
    assert_parity(y, ref, BF16, f"latent {M}x{K}")


def test_rope_minimal_rotation(gpu_lib):
    """rot_dim 4: only the first two pairs of each q / k head turn."""
    fn = gpu_lib
    w = dataclasses.replace(synth.workload("qknorm_rope_attn_in_bf16"), M=9, K=64, N=4 * 64, n_q_heads=2,
                            n_kv_heads=1, head_dim=64, rot_dim=4, n_pos=100)
    _say("rope rot_dim 4, 9x64, heads of 64")
    ref = oracle.linear_qknorm_rope(w.x(), w.w(), w.g(), w.eps_f32(), 2, 1, 64, w.g_q(), w.g_k(),
                                    w.eps_head_f32(), 0, w.positions(), w.rope_base, 4)
    g1 = _vec(w.g())
    y = fn.linear_qknorm_rope(to_dev(w.x()), fn.fold_weights(to_dev(w.w()), g1), 2, 1, 64, _vec(w.g_q()),
                              _vec(w.g_k()), w.eps_f32(), w.eps_head_f32(), torch.from_numpy(w.positions()).cuda(),
                              fn.rope_table(w.rope_base, 4, 100), out_dtype=torch.float32)
    assert_parity(y, ref, BF16, "rope rot 4")


def test_empty_inputs_write_nothing(gpu_lib):
    """M = 0 is valid for every op: status OK, nothing launched or written."""
    fn = gpu_lib
    _say("M = 0 for the LayerNorm, fp8, RoPE and latent ops")
    K, N = 64, 96
    x = torch.empty(0, K, dtype=torch.bfloat16, device="cuda")
    W = torch.randn(N, K, device="cuda").to(torch.bfloat16)
    W8 = torch.zeros(N, K, dtype=torch.uint8, device="cuda")
    v = torch.ones(N, device="cuda")
    sentinel = torch.full((4, N), 7.0, device="cuda")
    y = sentinel[:0]
    torch.cuda.synchronize()
    fn.layernorm_linear(x, W, 1e-5, colsum=v, out=y)
    fn.norm_linear_fp8(x, W8, v, 1e-6, out=y)
    fn.norm_glu_ffn_fp8(x, W8, v, W8, v, 1e-6, out=y)
    gq = torch.ones(64, device="cuda")
    Wr = torch.randn(3 * 64, K, device="cuda").to(torch.bfloat16)  # one q, one k, one v head of 64
    sentinel_r = torch.full((4, 3 * 64), 7.0, device="cuda")
    fn.linear_qknorm_rope(x, Wr, 1, 1, 64, gq, gq, 1e-6, 1e-6, torch.zeros(1, dtype=torch.int32, device="cuda"),
                          torch.ones(8, 64, device="cuda"), out=sentinel_r[:0])
    ws = torch.empty(fn.workspace_bytes(fn.OP_LINEAR_LATENT_NORM, fn.FUSED, 0, K, N, torch.bfloat16) + 256,
                     dtype=torch.uint8, device="cuda")
    fn.linear_latent_norm(x, W, 64, 32, 0, gq, gq[:32], 1e-6, 1e-6, out=y, ws=ws)
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0) and torch.all(sentinel_r == 7.0)
