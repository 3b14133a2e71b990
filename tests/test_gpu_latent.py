"""GPU parity of the MLA latent-norm op (fn_linear_latent_norm) through the C
ABI against the float64 oracle, which keeps the pre-attention RMSNorm that
the GPU path drops.  Every case prints its name and shape before it runs.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import KERNEL_REL_L2, assert_parity, from_dev, to_dev
from synth import BF16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _lat(M, K, nq, nkv, nr, rot=None, n_pos=4096):
    w = synth.workload("mla_latent_attn_in_bf16")
    return dataclasses.replace(w, M=M, K=K, N=nq + nkv + nr, n_q_latent=nq, n_kv_latent=nkv, n_rope=nr,
                               rot_dim=nr if rot is None else rot, n_pos=n_pos)


def _vec(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def run_lat(fn, w, variant, out_dtype, rope=True, positions=None):
    x, W, g1 = to_dev(w.x()), to_dev(w.w()), _vec(w.g())
    gq = _vec(w.g_q_latent()) if w.n_q_latent else None
    gkv = _vec(w.g_kv_latent()) if w.n_kv_latent else None
    pos = table = None
    if rope and w.n_rope:
        p = w.positions() if positions is None else np.asarray(positions, dtype=np.int32)
        pos = torch.from_numpy(p).cuda()
        table = fn.rope_table(w.rope_base, w.rot_dim, w.n_pos)
    if variant == fn.UNFUSED:
        return fn.linear_latent_norm(x, W, w.n_q_latent, w.n_kv_latent, w.n_rope, gq, gkv, w.eps_f32(),
                                     w.eps_head_f32(), pos, table, g1=g1, variant=variant, out_dtype=out_dtype)
    return fn.linear_latent_norm(x, fn.fold_weights(W, g1), w.n_q_latent, w.n_kv_latent, w.n_rope, gq, gkv,
                                 w.eps_f32(), w.eps_head_f32(), pos, table, variant=variant, out_dtype=out_dtype)


def ref_lat(w, rope=True, positions=None):
    pos = None
    if rope and w.n_rope:
        pos = w.positions() if positions is None else positions
    return oracle.linear_latent_norm(w.x(), w.w(), w.g(), w.eps_f32(), w.n_q_latent, w.n_kv_latent, w.n_rope,
                                     w.g_q_latent() if w.n_q_latent else None,
                                     w.g_kv_latent() if w.n_kv_latent else None, w.eps_head_f32(), pos,
                                     w.rope_base, w.rot_dim)


LAT_CASES = [
    # M, K, nq, nkv, n_rope
    (130, 520, 96, 64, 16),
    (300, 1032, 1536, 512, 64),
    (5, 512, 0, 512, 64),     # kv latent only (no q compression), few rows
    (64, 256, 128, 0, 0),     # one latent, no rope part
    (260, 776, 256, 256, 32),
]


@pytest.mark.parametrize("M,K,nq,nkv,nr", LAT_CASES)
@pytest.mark.parametrize("variant", ["fused", "unfused"])
def test_latent_norm_parity(gpu_lib, M, K, nq, nkv, nr, variant):
    fn = gpu_lib
    w = _lat(M, K, nq, nkv, nr)
    v = fn.FUSED if variant == "fused" else fn.UNFUSED
    _say(f"latent M={M} K={K} q{nq} kv{nkv} rope{nr} {variant} -> "
         f"{fn.dispatch_name(fn.OP_LINEAR_LATENT_NORM, v, M, K, w.N, torch.bfloat16, torch.float32)}")
    for rope in (True, False):
        ref = ref_lat(w, rope)
        for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
            y = run_lat(fn, w, v, od, rope)
            torch.cuda.synchronize()
            assert_parity(y, ref, BF16, f"latent {variant} rope={rope} {od}", out_bf16=ob)


@pytest.mark.parametrize("tile", list(range(9)))
def test_latent_every_tile_config(gpu_lib, tile, monkeypatch):
    fn = gpu_lib
    monkeypatch.setenv("FN_TILE", str(tile))
    w = _lat(260, 776, 256, 256, 32)
    _say(f"latent tile {tile}: "
         f"{fn.dispatch_name(fn.OP_LINEAR_LATENT_NORM, fn.FUSED, w.M, w.K, w.N, torch.bfloat16, torch.bfloat16)}")
    ref = ref_lat(w)
    for v in (fn.FUSED, fn.UNFUSED):
        y = run_lat(fn, w, v, torch.bfloat16)
        torch.cuda.synchronize()
        assert_parity(y, ref, BF16, f"tile {tile} latent v{v}", out_bf16=True)


def test_latent_kernel_only_pin(gpu_lib):
    """Against the dropped-norm form on the oracle's own folded weight."""
    fn = gpu_lib
    w = _lat(300, 1032, 1536, 512, 64)
    _say("kernel-only pin: latent 300x1032, q1536 kv512 rope64")
    Ws = oracle.fold_weights(w.w(), w.g(), BF16)
    pos = w.positions()
    y = fn.linear_latent_norm(to_dev(w.x()), to_dev(Ws), 1536, 512, 64, _vec(w.g_q_latent()),
                              _vec(w.g_kv_latent()), w.eps_f32(), w.eps_head_f32(), torch.from_numpy(pos).cuda(),
                              fn.rope_table(w.rope_base, 64, w.n_pos), out_dtype=torch.float32)
    ref = oracle.latent_dropped_on_folded(w.x(), Ws, w.eps_f32(), 1536, 512, 64, w.g_q_latent(), w.g_kv_latent(),
                                          w.eps_head_f32(), pos, w.rope_base, 64)
    assert_parity(y, ref, BF16, "kernel latent", rel_l2=KERNEL_REL_L2, max_abs=np.inf)


@pytest.mark.parametrize("prestats", ["0", "1"])
def test_latent_prestats_switch(gpu_lib, prestats, monkeypatch):
    """The deferred row scale of the rope part taken inside the GEMM (0) or
    in a pass before it (1)."""
    fn = gpu_lib
    monkeypatch.setenv("FN_PRESTATS", prestats)
    w = _lat(260, 776, 256, 256, 32)
    name = fn.dispatch_name(fn.OP_LINEAR_LATENT_NORM, fn.FUSED, w.M, w.K, w.N, torch.bfloat16, torch.bfloat16)
    _say(f"latent FN_PRESTATS={prestats}: {name}")
    assert ("row_scale+" in name) == (prestats == "1")
    y = run_lat(fn, w, fn.FUSED, torch.float32)
    assert_parity(y, ref_lat(w), BF16, f"latent prestats={prestats}")


def test_latent_bad_positions(gpu_lib):
    """A position outside the table turns that row's rope part into NaN and
    leaves its latents and the other rows alone."""
    fn = gpu_lib
    w = _lat(40, 264, 64, 64, 32, n_pos=50)
    _say("latent: positions -1 and n_pos")
    pos = (np.arange(40) % 50).astype(np.int32)
    pos[3], pos[20] = -1, 50
    y = from_dev(run_lat(fn, w, fn.FUSED, torch.float32, positions=pos))
    assert np.all(np.isnan(y[[3, 20], 128:])) and np.all(np.isfinite(y[:, :128]))
    good = np.delete(np.arange(40), [3, 20])
    ref = ref_lat(w, positions=np.clip(pos, 0, 49))
    ok, info = oracle.check_close(y[good], ref[good], 5e-3, 3e-2)
    assert ok, info


def test_full_mla_latent_attn_in(gpu_lib):
    fn = gpu_lib
    w = synth.workload("mla_latent_attn_in_bf16")
    ref = ref_lat(w)
    for v in (fn.FUSED, fn.UNFUSED):
        for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
            _say(f"full mla_latent_attn_in 2048x5120x2112 variant={v} out={od}")
            y = run_lat(fn, w, v, od)
            assert_parity(y, ref, BF16, f"mla latent v{v} {od}", out_bf16=ob)


def test_later_entry_points_reject_without_writing(gpu_lib):
    """Invalid calls of the LayerNorm, fp8 and latent entry points return
    their status and leave a sentinel-filled output untouched."""
    import ctypes

    fn = gpu_lib
    _say("invalid arguments: layernorm, fp8, latent")
    lib = fn.load()
    M, K, N = 16, 64, 96
    x = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    W = torch.randn(N, K, device="cuda").to(torch.bfloat16)
    W8 = torch.zeros(N, K, dtype=torch.uint8, device="cuda")
    v = torch.ones(max(N, K), device="cuda")
    y = torch.full((M, N), 7.0, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)  # noqa: E731
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cases = [
        ("ln fused without colsum", lib.fn_layernorm_linear(P(x), 1, M, K, P(W), 1, N, None, None, None, None, None,
                                                            1e-5, P(y), 0, 0, None, 0, st), 1),
        ("ln eps < 0", lib.fn_layernorm_linear(P(x), 1, M, K, P(W), 1, N, P(v), None, None, None, None, -1.0, P(y), 0,
                                               0, None, 0, st), 8),
        ("ln misaligned bias", lib.fn_layernorm_linear(P(x), 1, M, K, P(W), 1, N, None, None, P(v), None, P(v, 4),
                                                       1e-5, P(y), 0, 1, P(ws), 1 << 20, st), 4),
        # above 16 rows the fp8 ops quantise x into a workspace
        ("fp8 M > 16 no ws", lib.fn_norm_linear_fp8(P(x), 1, 17, K, P(W8), P(v), N, None, 1e-6, P(y), 0, 0, None, 0,
                                                     st), 5),
        ("fp8 M > 16 packed", lib.fn_norm_linear_fp8(P(x), 1, 17, K, P(W8), P(v), N, None, 1e-6, P(y), 0, 3, P(ws),
                                                      1 << 20, st), 6),
        ("fp8 K % 16", lib.fn_norm_linear_fp8(P(x), 1, M, 56, P(W8), P(v), N, None, 1e-6, P(y), 0, 0, None, 0, st), 4),
        ("glu fp8 no up", lib.fn_norm_glu_ffn_fp8(P(x), 1, M, K, P(W8), P(v), None, None, N, None, 1e-6, P(y), 0, 0,
                                                  None, 0, st), 1),
        ("latent width", lib.fn_linear_latent_norm(P(x), 1, M, K, P(W), 1, 48, 32, 16, P(v), P(v), 1e-6, 1e-6, None,
                                                   None, 0, 0, None, P(y), 0, 0, P(ws), 1 << 20, st), 2),
        ("latent no ws", lib.fn_linear_latent_norm(P(x), 1, M, K, P(W), 1, 64, 32, 0, P(v), P(v), 1e-6, 1e-6, None,
                                                   None, 0, 0, None, P(y), 0, 0, None, 0, st), 5),
        ("latent rot_dim", lib.fn_linear_latent_norm(P(x), 1, M, K, P(W), 1, 32, 32, 32, P(v), P(v), 1e-6, 1e-6,
                                                     P(v), P(v), 8, 64, None, P(y), 0, 0, P(ws), 1 << 20, st), 2),
    ]
    torch.cuda.synchronize()
    for name, status, want in cases:
        assert status == want, f"{name}: got {status} ({lib.fn_last_error().decode()}), want {want}"
    assert torch.all(y == 7.0)
