"""HIP graph capture of the ops (torch.cuda.CUDAGraph): with preallocated
outputs and workspaces a call launches kernels only (no allocation, no
memset), so a captured call replays correctly.  Each graph is replayed
several times, with other eager work and synchronisations between the
replays, and every replay must equal the eager result bit for bit.  Every
case prints its name before it runs.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, bits_of, to_dev
from synth import BF16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _vec(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _ws(fn, op, variant, M, K, N):
    n = fn.workspace_bytes(op, variant, M, K, N, torch.bfloat16)
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") if n else None


def _cases(fn):
    """(name, call(out), out) for each op family; call writes into out."""
    cases = []
    # prefill: fused linear (ragged tiles)
    w = synth.workload("llama7b_qkv_prefill_bf16").with_shape(300, 1032, 700)
    x, Ws = to_dev(w.x()), fn.fold_weights(to_dev(w.w()), _vec(w.g()))
    ws = _ws(fn, fn.OP_NORM_LINEAR, fn.FUSED, 300, 1032, 700)
    y = torch.empty(300, 700, device="cuda", dtype=torch.bfloat16)
    cases.append(("prefill linear 300x1032x700", lambda o, x=x, Ws=Ws, ws=ws: fn.norm_linear(x, Ws, w.eps_f32(), out=o,
                                                                                               ws=ws), y))
    # the unfused baseline: the RMSNorm pass writes xn into the workspace, then the product
    Wr, gr = to_dev(w.w()), _vec(w.g())
    wsu = _ws(fn, fn.OP_NORM_LINEAR, fn.UNFUSED, 300, 1032, 700)
    yu = torch.empty(300, 700, device="cuda", dtype=torch.bfloat16)
    cases.append(("prefill linear unfused 300x1032x700",
                  lambda o, x=x, Wr=Wr, gr=gr, wsu=wsu: fn.norm_linear(x, Wr, w.eps_f32(), g=gr, variant=fn.UNFUSED,
                                                                        out=o, ws=wsu), yu))
    # decode: GLU on the packed gate/up pair, bf16 and fp8 codes
    g = dataclasses.replace(synth.workload("llama7b_ffn_decode_m4_bf16"), M=4, K=4096, N=1000)
    Wg, Wu = oracle.fold_weights(g.w(), g.g(), BF16), oracle.fold_weights(g.w_up(), g.g(), BF16)
    xg = to_dev(g.x())
    P = fn.pack_decode_weights_glu(to_dev(Wg), to_dev(Wu))
    h = torch.empty(4, 1000, device="cuda")
    cases.append(("decode glu, packed pair, M=4", lambda o, xg=xg, P=P: fn.norm_glu_ffn(xg, P, None, g.eps_f32(), out=o), h))
    cg, qg = oracle.quantize_fp8_per_channel(Wg)
    cu, qu = oracle.quantize_fp8_per_channel(Wu)
    P8 = fn.pack_decode_weights_glu(torch.from_numpy(cg).cuda(), torch.from_numpy(cu).cuda())
    qg_d, qu_d = _vec(qg), _vec(qu)
    h8 = torch.empty(4, 1000, device="cuda", dtype=torch.bfloat16)
    cases.append(("decode fp8 glu, packed pair, M=4",
                  lambda o, xg=xg: fn.norm_glu_ffn_fp8(xg, P8, qg_d, None, qu_d, g.eps_f32(), out=o), h8))
    # head norms with RoPE: the decode path (two kernels) and the prefill tile
    for M in (3, 40):
        q = dataclasses.replace(synth.workload("qknorm_rope_attn_in_bf16"), M=M, K=520, N=5 * 128, n_q_heads=3,
                                n_kv_heads=1, head_dim=128, rot_dim=64, n_pos=4096)
        xq, Wq = to_dev(q.x()), fn.fold_weights(to_dev(q.w()), _vec(q.g()))
        gq, gk = torch.from_numpy(q.g_q()).cuda(), torch.from_numpy(q.g_k()).cuda()
        pos, table = torch.from_numpy(q.positions()).cuda(), fn.rope_table(q.rope_base, 64, 4096)
        wsq = _ws(fn, fn.OP_LINEAR_QKNORM_ROPE, fn.FUSED, M, 520, 5 * 128)
        yq = torch.empty(M, 5 * 128, device="cuda", dtype=torch.bfloat16)
        cases.append((f"qknorm rope M={M}",
                      lambda o, xq=xq, Wq=Wq, gq=gq, gk=gk, pos=pos, table=table, wsq=wsq, q=q: fn.linear_qknorm_rope(
                          xq, Wq, 3, 1, 128, gq, gk, q.eps_f32(), q.eps_head_f32(), pos, table, out=o, ws=wsq), yq))
        Wqr, g1 = to_dev(q.w()), _vec(q.g())
        wsqu = _ws(fn, fn.OP_LINEAR_QKNORM_ROPE, fn.UNFUSED, M, 520, 5 * 128)
        yqu = torch.empty(M, 5 * 128, device="cuda", dtype=torch.bfloat16)
        cases.append((f"qknorm rope unfused M={M}",
                      lambda o, xq=xq, Wqr=Wqr, g1=g1, gq=gq, gk=gk, pos=pos, table=table, wsqu=wsqu, q=q:
                      fn.linear_qknorm_rope(xq, Wqr, 3, 1, 128, gq, gk, q.eps_f32(), q.eps_head_f32(), pos, table,
                                            g1=g1, variant=fn.UNFUSED, out=o, ws=wsqu), yqu))
    # LayerNorm on packed weights, M=1
    ln = dataclasses.replace(synth.workload("ln_fc1_decode_m1_bf16"), M=1, K=1040, N=300)
    Wl, c, b = fn.fold_layernorm(to_dev(ln.w()), _vec(ln.g()), _vec(ln.beta()), _vec(ln.bias()))
    Pl, xl = fn.pack_decode_weights(Wl), to_dev(ln.x())
    yl = torch.empty(1, 300, device="cuda")
    cases.append(("layernorm decode packed M=1",
                  lambda o, xl=xl, Pl=Pl, c=c, b=b: fn.layernorm_linear(xl, Pl, ln.eps_f32(), colsum=c, b_star=b,
                                                                        out=o), yl))
    return cases


def test_graph_replays_equal_eager(gpu_lib):
    fn = gpu_lib
    cases = _cases(fn)
    side = torch.randn(2048, 2048, device="cuda")
    for name, call, out in cases:
        _say(f"graph capture and replay: {name}")
        call(out)
        torch.cuda.synchronize()
        eager = out.clone()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call(out)  # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call(out)
        for rep in range(4):
            out.fill_(float("nan"))
            side = side @ side.T * 1e-3  # other eager work between the replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(bits_of(out), bits_of(eager)), f"{name}: replay {rep} differs from eager"
        del graph


def test_graph_two_stream_fork_join(gpu_lib):
    """The two-stream variant under capture: its event fork and join bring
    the auxiliary stream into the graph, and the replays equal eager."""
    fn = gpu_lib
    w = synth.workload("llama7b_qkv_prefill_bf16").with_shape(300, 1032, 700)
    x, Ws = to_dev(w.x()), fn.fold_weights(to_dev(w.w()), _vec(w.g()))
    ws = _ws(fn, fn.OP_NORM_LINEAR, fn.TWO_STREAM, 300, 1032, 700)
    out = torch.empty(300, 700, device="cuda", dtype=torch.bfloat16)
    aux = torch.cuda.Stream()
    _say("graph capture and replay: prefill linear two-stream 300x1032x700")

    def call():
        fn.norm_linear(x, Ws, w.eps_f32(), variant=fn.TWO_STREAM, out=out, ws=ws, aux_stream=aux)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    ref = oracle.norm_linear(w.x(), w.w(), w.g(), w.eps_f32())
    assert_parity(eager, ref, BF16, "two-stream eager", out_bf16=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    side = torch.randn(1024, 1024, device="cuda")
    for rep in range(4):
        out.fill_(float("nan"))
        side = side @ side.T * 1e-3
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), bits_of(eager)), f"two-stream replay {rep} differs from eager"
    del graph
