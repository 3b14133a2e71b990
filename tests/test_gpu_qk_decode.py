"""GPU parity of the head-norm ops (fn_linear_qknorm, fn_linear_qknorm_rope)
at decode batch sizes (M <= 16), where the weight-streaming kernel writes
the float32 product and a second kernel applies the head norms and the
rotation, against the float64 oracle.  Every case prints its name and shape
before it runs.
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


def _w(M, K, nq, nkv, hd, rot_dim=None, n_pos=4096):
    base = synth.workload("qknorm_rope_attn_in_bf16")
    return dataclasses.replace(base, M=M, K=K, N=(nq + 2 * nkv) * hd, n_q_heads=nq, n_kv_heads=nkv, head_dim=hd,
                               rot_dim=rot_dim if rot_dim else hd, n_pos=n_pos)


def _run(fn, w, variant, od, v_mode, rope, positions=None):
    gq, gk = torch.from_numpy(w.g_q()).cuda(), torch.from_numpy(w.g_k()).cuda()
    if variant == fn.FUSED:
        W, g1 = fn.fold_weights(to_dev(w.w()), torch.from_numpy(w.g()).cuda()), None
    else:
        W, g1 = to_dev(w.w()), torch.from_numpy(w.g()).cuda()
    x = to_dev(w.x())
    if rope:
        pos = torch.from_numpy(w.positions() if positions is None else positions).cuda()
        table = fn.rope_table(w.rope_base, w.rot_dim, w.n_pos)
        return fn.linear_qknorm_rope(x, W, w.n_q_heads, w.n_kv_heads, w.head_dim, gq, gk, w.eps_f32(),
                                     w.eps_head_f32(), pos, table, v_mode=v_mode, g1=g1, variant=variant,
                                     out_dtype=od)
    return fn.linear_qknorm(x, W, w.n_q_heads, w.n_kv_heads, w.head_dim, gq, gk, w.eps_f32(), w.eps_head_f32(),
                            v_mode=v_mode, g1=g1, variant=variant, out_dtype=od)


def _ref(w, v_mode, rope):
    if rope:
        return oracle.linear_qknorm_rope(w.x(), w.w(), w.g(), w.eps_f32(), w.n_q_heads, w.n_kv_heads, w.head_dim,
                                         w.g_q(), w.g_k(), w.eps_head_f32(), v_mode, w.positions(), w.rope_base,
                                         w.rot_dim)
    return oracle.linear_qknorm(w.x(), w.w(), w.g(), w.eps_f32(), w.n_q_heads, w.n_kv_heads, w.head_dim, w.g_q(),
                                w.g_k(), w.eps_head_f32(), v_mode)


SHAPES = [
    # K, n_q, n_kv, head_dim
    (2560, 8, 4, 256),  # the attention-input widths
    (520, 3, 2, 128),   # K tail inside the last 32-wide step
    (136, 2, 1, 64),    # heads of 64: 32 lanes per head
]


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("K,nq,nkv,hd", SHAPES)
@pytest.mark.parametrize("rope", [False, True])
def test_qk_decode_parity(gpu_lib, M, K, nq, nkv, hd, rope):
    fn = gpu_lib
    w = _w(M, K, nq, nkv, hd, rot_dim=hd // 2 if rope else None)
    name = fn.dispatch_name(fn.OP_LINEAR_QKNORM, fn.FUSED, M, K, w.N, torch.bfloat16, torch.bfloat16)
    assert "qk_finish" in name, name
    for variant in (fn.FUSED, fn.UNFUSED):
        for v_mode in (0, 1):
            ref = _ref(w, v_mode, rope)
            for od in (torch.float32, torch.bfloat16):
                _say(f"qk decode M={M} K={K} {nq}q/{nkv}kv x{hd} rope={rope} variant={variant} v_mode={v_mode} {od}")
                y = _run(fn, w, variant, od, v_mode, rope)
                torch.cuda.synchronize()
                assert_parity(y, ref, BF16, f"qk decode v{variant} vm{v_mode} {od}", out_bf16=(od == torch.bfloat16))


@pytest.mark.parametrize("rope", [False, True])
def test_qk_decode_kernel_only_pin(gpu_lib, rope):
    """Against the dropped-norm form on the oracle's own folded weights (and
    the oracle's rotation): only float32 arithmetic differs."""
    fn = gpu_lib
    w = _w(5, 1040, 4, 2, 128, rot_dim=128)
    _say(f"qk decode kernel-only pin M=5 K=1040 4q/2kv x128 rope={rope}")
    Wq = oracle.fold_weights(w.w(), w.g(), BF16)
    gq, gk = torch.from_numpy(w.g_q()).cuda(), torch.from_numpy(w.g_k()).cuda()
    nqk = (w.n_q_heads + w.n_kv_heads) * w.head_dim
    for vm in (0, 1):
        if rope:
            y = fn.linear_qknorm_rope(to_dev(w.x()), to_dev(Wq), 4, 2, 128, gq, gk, w.eps_f32(), w.eps_head_f32(),
                                      torch.from_numpy(w.positions()).cuda(),
                                      fn.rope_table(w.rope_base, w.rot_dim, w.n_pos), v_mode=vm,
                                      out_dtype=torch.float32)
        else:
            y = fn.linear_qknorm(to_dev(w.x()), to_dev(Wq), 4, 2, 128, gq, gk, w.eps_f32(), w.eps_head_f32(),
                                 v_mode=vm, out_dtype=torch.float32)
        ref = oracle.qknorm_dropped_on_folded(w.x(), Wq, w.eps_f32(), 4, 2, 128, w.g_q(), w.g_k(),
                                              w.eps_head_f32(), vm)
        if rope:
            ref[:, :nqk] = oracle.rope(ref[:, :nqk], w.positions(), w.rope_base, w.rot_dim, w.head_dim)
        assert_parity(y, ref, BF16, f"qk decode kernel-only v{vm} rope={rope}", rel_l2=KERNEL_REL_L2,
                      max_abs=np.inf)


def test_qk_decode_positions_out_of_range(gpu_lib):
    """A position outside the table gives NaN in that row's rotated q/k
    columns only; the other rows, the unrotated columns and v are exact."""
    fn = gpu_lib
    w = _w(6, 520, 2, 1, 128, rot_dim=64, n_pos=100)
    _say("qk decode: positions -1 and 100 in rows 1 and 4 of 6, rot_dim 64 of 128, table of 100")
    pos = w.positions() % 100
    pos[1], pos[4] = -1, 100
    y = from_dev(_run(fn, w, fn.FUSED, torch.float32, 0, True, positions=pos.astype(np.int32)))
    ref = _ref(dataclasses.replace(w), 0, False)  # no rotation: the columns past rot_dim and v
    hd, nqk = 128, 3 * 128
    for m in range(6):
        bad = m in (1, 4)
        for c in range(w.N):
            rotated = c < nqk and (c % hd) < 64
            if bad and rotated:
                assert np.isnan(y[m, c]), (m, c)
            else:
                assert np.isfinite(y[m, c]), (m, c)
    good = [0, 2, 3, 5]
    cols = [c for c in range(w.N) if not (c < nqk and (c % hd) < 64)]
    ok, info = oracle.check_close(y[np.ix_(good, cols)], ref[np.ix_(good, cols)], 5e-3, 3e-2)
    assert ok, info
