"""GPU parity of the rotary embedding fused into the QK-norm epilogue
(fn_linear_qknorm_rope) and of its table (fn_rope_table), through the C ABI,
against the float64 oracle.

The oracle computes the angles and their cosines and sines itself, in
float64, from (positions, base, rot_dim); the GPU gets a float32 table from
fn_rope_table.  Every case prints its name and shape before it runs.
"""

import ctypes
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


def _rope_workload(M, K, nq, nkv, hd, rot_dim, n_pos=4096, base=10000.0):
    w = synth.workload("qknorm_rope_attn_in_bf16")
    return dataclasses.replace(w, M=M, K=K, N=(nq + 2 * nkv) * hd, n_q_heads=nq, n_kv_heads=nkv, head_dim=hd,
                               rot_dim=rot_dim, n_pos=n_pos, rope_base=base)


def _dev_args(fn, w):
    gq = torch.from_numpy(w.g_q()).cuda()
    gk = torch.from_numpy(w.g_k()).cuda()
    pos = torch.from_numpy(w.positions()).cuda()
    table = fn.rope_table(w.rope_base, w.rot_dim, w.n_pos)
    return gq, gk, pos, table


def run_rope(fn, w, variant, out_dtype, v_mode=0, positions=None):
    x, W, g1 = to_dev(w.x()), to_dev(w.w()), torch.from_numpy(w.g()).cuda()
    gq, gk, pos, table = _dev_args(fn, w)
    if positions is not None:
        pos = torch.from_numpy(np.asarray(positions, dtype=np.int32)).cuda()
    if variant == fn.UNFUSED:
        return fn.linear_qknorm_rope(x, W, w.n_q_heads, w.n_kv_heads, w.head_dim, gq, gk, w.eps_f32(),
                                     w.eps_head_f32(), pos, table, v_mode=v_mode, g1=g1, variant=variant,
                                     out_dtype=out_dtype)
    return fn.linear_qknorm_rope(x, fn.fold_weights(W, g1), w.n_q_heads, w.n_kv_heads, w.head_dim, gq, gk,
                                 w.eps_f32(), w.eps_head_f32(), pos, table, v_mode=v_mode, variant=variant,
                                 out_dtype=out_dtype)


def ref_rope(w, v_mode=0, positions=None):
    pos = w.positions() if positions is None else positions
    return oracle.linear_qknorm_rope(w.x(), w.w(), w.g(), w.eps_f32(), w.n_q_heads, w.n_kv_heads, w.head_dim,
                                     w.g_q(), w.g_k(), w.eps_head_f32(), v_mode, pos, w.rope_base, w.rot_dim)


# ---------------------------------------------------------------------------
# the table: float64 angle, cosine and sine, one rounding to float32
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("base,rot_dim,n_pos", [(10000.0, 256, 32768), (1e6, 64, 1000), (500000.0, 6, 17)])
def test_rope_table_is_rounded_definition(gpu_lib, base, rot_dim, n_pos):
    fn = gpu_lib
    _say(f"rope table base={base} rot_dim={rot_dim} n_pos={n_pos}")
    t = from_dev(fn.rope_table(base, rot_dim, n_pos)).reshape(n_pos, rot_dim // 2, 2)
    ang = oracle.rope_angles(np.arange(n_pos), base, rot_dim)
    c, s = np.cos(ang), np.sin(ang)
    # half a float32 ulp of the value, plus the float64 error of the angle
    # (|p theta| up to 3.3e4 rad: a few 1e-12)
    tol = lambda v: np.maximum(np.abs(v), 2.0 ** -126) * 2.0 ** -24 + 1e-11  # noqa: E731
    assert np.all(np.abs(t[..., 0] - c) <= tol(c))
    assert np.all(np.abs(t[..., 1] - s) <= tol(s))


# ---------------------------------------------------------------------------
# the op: reduced shapes spanning several tiles with ragged tails
# ---------------------------------------------------------------------------

ROPE_CASES = [
    # M, K, nq, nkv, hd, rot_dim
    (130, 2560, 8, 4, 256, 256),
    (300, 520, 3, 2, 64, 64),
    (200, 264, 2, 1, 128, 32),   # partial rotation: a quarter of each head
    (5, 512, 4, 2, 256, 128),
    (600, 1024, 4, 2, 128, 128),  # 256-row tiles
]


@pytest.mark.parametrize("M,K,nq,nkv,hd,rot", ROPE_CASES)
@pytest.mark.parametrize("variant", ["fused", "unfused"])
@pytest.mark.parametrize("v_mode", [0, 1])
def test_linear_qknorm_rope_parity(gpu_lib, M, K, nq, nkv, hd, rot, variant, v_mode):
    fn = gpu_lib
    w = _rope_workload(M, K, nq, nkv, hd, rot)
    v = fn.FUSED if variant == "fused" else fn.UNFUSED
    _say(f"qknorm_rope M={M} K={K} heads q{nq} kv{nkv} hd{hd} rot{rot} {variant} v_mode={v_mode} -> "
         f"{fn.dispatch_name(fn.OP_LINEAR_QKNORM_ROPE, v, M, K, w.N, torch.bfloat16, torch.float32)}")
    ref = ref_rope(w, v_mode)
    for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
        y = run_rope(fn, w, v, od, v_mode)
        torch.cuda.synchronize()
        assert_parity(y, ref, BF16, f"qknorm_rope {variant} v{v_mode} {od}", out_bf16=ob)


@pytest.mark.parametrize("tile", [0, 1, 2, 4, 5, 6, 8])
def test_rope_every_tile_config(gpu_lib, tile, monkeypatch):
    fn = gpu_lib
    monkeypatch.setenv("FN_TILE", str(tile))
    w = _rope_workload(260, 520, 3, 2, 64, 64)
    _say(f"qknorm_rope tile {tile}: "
         f"{fn.dispatch_name(fn.OP_LINEAR_QKNORM_ROPE, fn.FUSED, w.M, w.K, w.N, torch.bfloat16, torch.bfloat16)}")
    ref = ref_rope(w)
    for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
        y = run_rope(fn, w, fn.FUSED, od)
        torch.cuda.synchronize()
        assert_parity(y, ref, BF16, f"tile {tile} qknorm_rope {od}", out_bf16=ob)


def test_rope_kernel_only_pin(gpu_lib):
    """Against the dropped-norm form on the oracle's own folded weights, then
    the oracle's rotation: only float32 arithmetic and the float32 table
    differ."""
    fn = gpu_lib
    w = _rope_workload(130, 520, 8, 4, 256, 256, n_pos=32768)
    _say("kernel-only pin: qknorm_rope 130x520, 8q/4kv heads of 256, positions up to 32767")
    Wq = oracle.fold_weights(w.w(), w.g(), BF16)
    gq, gk, pos, table = _dev_args(fn, w)
    nqk = (w.n_q_heads + w.n_kv_heads) * w.head_dim
    for vm in (0, 1):
        y = fn.linear_qknorm_rope(to_dev(w.x()), to_dev(Wq), 8, 4, 256, gq, gk, w.eps_f32(), w.eps_head_f32(),
                                  pos, table, v_mode=vm, out_dtype=torch.float32)
        ref = oracle.qknorm_dropped_on_folded(w.x(), Wq, w.eps_f32(), 8, 4, 256, w.g_q(), w.g_k(),
                                              w.eps_head_f32(), vm)
        ref[:, :nqk] = oracle.rope(ref[:, :nqk], w.positions(), w.rope_base, w.rot_dim, w.head_dim)
        assert_parity(y, ref, BF16, f"kernel qk rope v{vm}", rel_l2=KERNEL_REL_L2, max_abs=np.inf)


def test_rope_positions_edge_cases(gpu_lib):
    """Position 0 leaves q and k as the plain qknorm op gives them; the last
    table row is used; a position outside the table turns that row's q and k
    into NaN and touches nothing else."""
    fn = gpu_lib
    w = _rope_workload(70, 264, 2, 1, 64, 64, n_pos=100)
    _say("rope positions: zeros, n_pos-1, out of range (-1, n_pos)")
    x, Wf = to_dev(w.x()), None
    g1 = torch.from_numpy(w.g()).cuda()
    Wf = fn.fold_weights(to_dev(w.w()), g1)
    gq, gk, _, table = _dev_args(fn, w)
    zeros = torch.zeros(w.M, dtype=torch.int32, device="cuda")
    y0 = fn.linear_qknorm_rope(x, Wf, 2, 1, 64, gq, gk, w.eps_f32(), w.eps_head_f32(), zeros, table,
                               out_dtype=torch.float32)
    yq = fn.linear_qknorm(x, Wf, 2, 1, 64, gq, gk, w.eps_f32(), w.eps_head_f32(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y0, yq)
    pos = np.full(w.M, w.n_pos - 1, dtype=np.int32)
    pos[3], pos[40] = -1, w.n_pos
    y = from_dev(fn.linear_qknorm_rope(x, Wf, 2, 1, 64, gq, gk, w.eps_f32(), w.eps_head_f32(),
                                       torch.from_numpy(pos).cuda(), table, out_dtype=torch.float32))
    nqk = 3 * 64
    bad = [3, 40]
    assert np.all(np.isnan(y[bad, :nqk])) and np.all(np.isfinite(y[bad, nqk:]))
    good = np.delete(np.arange(w.M), bad)
    ref = ref_rope(w, 0, positions=pos.clip(0, w.n_pos - 1))
    ok, info = oracle.check_close(y[good], ref[good], 5e-3, 3e-2)
    assert ok, info
    ok, info = oracle.check_close(y[bad, nqk:], ref[bad, nqk:], 5e-3, 3e-2)
    assert ok, info


def test_rope_invalid_arguments_write_nothing(gpu_lib):
    fn = gpu_lib
    _say("rope invalid arguments")
    lib = fn.load()
    M, K, hd = 16, 64, 64
    x = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    W = torch.randn(3 * hd, K, device="cuda").to(torch.bfloat16)
    g = torch.ones(hd, device="cuda")
    pos = torch.zeros(M, dtype=torch.int32, device="cuda")
    tab = torch.zeros(8, hd, device="cuda")
    y = torch.full((M, 3 * hd), 7.0, device="cuda")
    torch.cuda.synchronize()
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)  # noqa: E731

    def call(p_pos, p_tab, n_pos, rot):
        return lib.fn_linear_qknorm_rope(P(x), 1, M, K, P(W), 1, 1, 1, hd, P(g), P(g), 0, 1e-6, 1e-6, 0, p_pos,
                                         p_tab, n_pos, rot, None, P(y), 0, 0, None, 0, None)

    assert call(None, P(tab), 8, hd) == 1
    assert call(P(pos), P(tab, 4), 8, hd) == 4
    assert call(P(pos), P(tab), 8, 66) == 2
    assert call(P(pos), P(tab), 8, 2) == 2
    assert call(P(pos), P(tab), 0, hd) == 2
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ---------------------------------------------------------------------------
# full size: the QK-norm attention input with the rotary embedding
# ---------------------------------------------------------------------------

def test_full_qknorm_rope_attn_in(gpu_lib):
    fn = gpu_lib
    w = synth.workload("qknorm_rope_attn_in_bf16")
    for vm in (0, 1):
        ref = ref_rope(w, vm)
        for variant in (fn.FUSED, fn.UNFUSED):
            for od, ob in ((torch.float32, False), (torch.bfloat16, True)):
                _say(f"full qknorm_rope_attn_in 1024x2560x4096 variant={variant} v_mode={vm} out={od}")
                y = run_rope(fn, w, variant, od, vm)
                assert_parity(y, ref, BF16, f"qknorm_rope v{variant} vm{vm} {od}", out_bf16=ob)
