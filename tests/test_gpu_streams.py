"""Calls enqueued on a side stream (``stream=``) with workspaces and outputs
the binding allocates itself.

The binding takes those buffers from the caching-allocator pool of the
stream the call runs on.  Were they taken from the current stream's pool
instead, the workspace freed when the wrapper returns could be handed to the
next allocation on the current stream while the side stream's kernels still
use it.  Each case holds the side stream back with queued work, calls the op
there, then at once allocates buffers of the workspace's size on the current
stream and keeps overwriting them with NaN while the side stream catches up;
the op's result must still match the oracle.  Every case prints its name
before it runs.
"""

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


def _hammer_after(side, ws_bytes, call):
    """Hold `side` back, enqueue `call()` on it, then overwrite freshly
    allocated current-stream buffers of the workspace's size with NaN until
    `side` has drained."""
    a = torch.randn(2048, 2048, device="cuda")
    b = torch.randn(2048, 2048, device="cuda")
    c = torch.empty(2048, 2048, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for _ in range(8):
            torch.mm(a, b, out=c)
    out = call()
    n = max(1, ws_bytes // 4)
    bufs = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(4)]
    for _ in range(200):
        for t in bufs:
            t.fill_(float("nan"))
    torch.cuda.synchronize()
    return out


def test_side_stream_norm_linear_unfused_and_prestats(gpu_lib, monkeypatch):
    fn = gpu_lib
    w = synth.workload("llama7b_qkv_prefill_bf16").with_shape(640, 1032, 700)
    x, W, g = to_dev(w.x()), to_dev(w.w()), _vec(w.g())
    Ws = fn.fold_weights(W, g)
    ref = oracle.norm_linear(w.x(), w.w(), w.g(), w.eps_f32())
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    _say("side stream: norm_linear unfused (xn workspace) 640x1032x700")
    wsb = fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.UNFUSED, w.M, w.K, w.N, torch.bfloat16)
    y = _hammer_after(side, wsb, lambda: fn.norm_linear(x, W, w.eps_f32(), g=g, variant=fn.UNFUSED,
                                                        out_dtype=torch.float32, stream=side))
    assert_parity(y, ref, BF16, "side stream unfused")
    _say("side stream: norm_linear fused with the row-statistics pass (row-scale workspace)")
    monkeypatch.setenv("FN_PRESTATS", "1")
    wsb = fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.FUSED, w.M, w.K, w.N, torch.bfloat16)
    assert wsb > 0
    y = _hammer_after(side, wsb, lambda: fn.norm_linear(x, Ws, w.eps_f32(), out_dtype=torch.float32, stream=side))
    assert_parity(y, ref, BF16, "side stream fused, statistics pass")


def test_side_stream_glu_unfused(gpu_lib):
    fn = gpu_lib
    w = synth.workload("smollm2_ffn_prefill_bf16").with_shape(300, 576, 400)
    x, Wg, Wu, g = to_dev(w.x()), to_dev(w.w()), to_dev(w.w_up()), _vec(w.g())
    side = torch.cuda.Stream()
    _say("side stream: norm_glu_ffn unfused 300x576x400")
    wsb = fn.workspace_bytes(fn.OP_NORM_GLU_FFN, fn.UNFUSED, w.M, w.K, w.N, torch.bfloat16)
    h = _hammer_after(side, wsb, lambda: fn.norm_glu_ffn(x, Wg, Wu, w.eps_f32(), g=g, variant=fn.UNFUSED,
                                                         out_dtype=torch.float32, stream=side))
    assert_parity(h, oracle.norm_glu_ffn(w.x(), w.w(), w.w_up(), w.g(), w.eps_f32()), BF16, "side stream glu")


def test_side_stream_qknorm_decode(gpu_lib):
    fn = gpu_lib
    base = synth.workload("qknorm_attn_in_bf16")
    w = dataclasses.replace(base, M=4)
    x, W, g1 = to_dev(w.x()), to_dev(w.w()), _vec(w.g())
    gq, gk = _vec(w.g_q()), _vec(w.g_k())
    Ws = fn.fold_weights(W, g1)
    side = torch.cuda.Stream()
    _say("side stream: linear_qknorm at M=4 (float32 product workspace)")
    wsb = fn.workspace_bytes(fn.OP_LINEAR_QKNORM, fn.FUSED, w.M, w.K, w.N, torch.bfloat16)
    assert wsb > 0
    y = _hammer_after(side, wsb, lambda: fn.linear_qknorm(x, Ws, w.n_q_heads, w.n_kv_heads, w.head_dim, gq, gk,
                                                          w.eps_f32(), w.eps_head_f32(), out_dtype=torch.float32,
                                                          stream=side))
    ref = oracle.linear_qknorm(w.x(), w.w(), w.g(), w.eps_f32(), w.n_q_heads, w.n_kv_heads, w.head_dim, w.g_q(),
                               w.g_k(), w.eps_head_f32(), 0)
    assert_parity(y, ref, BF16, "side stream qknorm decode")


def test_side_stream_latent(gpu_lib):
    fn = gpu_lib
    base = synth.workload("mla_latent_attn_in_bf16")
    w = dataclasses.replace(base, M=300, K=1040, N=640, n_q_latent=384, n_kv_latent=192, n_rope=64, rot_dim=64,
                            n_pos=4096)
    x, W, g1 = to_dev(w.x()), to_dev(w.w()), _vec(w.g())
    gq, gkv = _vec(w.g_q_latent()), _vec(w.g_kv_latent())
    pos = torch.from_numpy(w.positions()).cuda()
    table = fn.rope_table(w.rope_base, w.rot_dim, w.n_pos)
    Ws = fn.fold_weights(W, g1)
    side = torch.cuda.Stream()
    _say("side stream: linear_latent_norm 300x1040 -> 384+192+64 (float32 latent workspace)")
    wsb = fn.workspace_bytes(fn.OP_LINEAR_LATENT_NORM, fn.FUSED, w.M, w.K, w.N, torch.bfloat16)
    y = _hammer_after(side, wsb, lambda: fn.linear_latent_norm(x, Ws, 384, 192, 64, gq, gkv, w.eps_f32(),
                                                               w.eps_head_f32(), pos, table, out_dtype=torch.float32,
                                                               stream=side))
    ref = oracle.linear_latent_norm(w.x(), w.w(), w.g(), w.eps_f32(), 384, 192, 64, w.g_q_latent(),
                                    w.g_kv_latent(), w.eps_head_f32(), w.positions(), w.rope_base, w.rot_dim)
    assert_parity(y, ref, BF16, "side stream latent")
