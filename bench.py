#!/usr/bin/env python3
"""Benchmark of the FlashNorm norm-then-project hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--out-dtype bf16|f32]

One step is one call of the fused op (fold done offline, before timing) on
one batch of seeded synthetic input already resident in HBM.  Untimed
warm-up runs first: at least W steps of each variant and at least
--warmup-seconds of wall time, so the timed region does not start on a cold
clock.  Then exactly K steps are timed between two stream synchronisations
with HIP events (`value`, `ms_per_step`); a second pass brackets every call
with its own event pair for the per-launch distribution.  Inputs rotate over
several copies whose total exceeds the 256 MB Infinity Cache, so weights
come from HBM.  The unfused baseline (RMSNorm kernel, then the GEMM on the
unfolded weight) and the fused step are then timed in alternating blocks of
exactly K steps each (the order flipped every block, cold and hot), and the
speedup is the ratio of their medians.  One JSON line is printed.

`roofline.achieved` is the dominant kernel's rate: over the timed region
for a step of one launch; for a step that also launches a pass (row
statistics, x quantisation, latent norms), over the median of the GEMM's
own launch durations, which the library's timing hook brackets with HIP
events on the launch stream (flashnorm_testing.h).

With --graph every timed region is one replay of a captured HIP graph of
its steps (the ops allocate nothing and launch kernels only), for steps
short enough that the host's cost per call, not the GPU, would set the pace
(the float32 workload: about 10 us per eager call).  The line then says
"launch": "hip graph replay".

The default workload is the Llama-7B-shaped QKV prefill
(x 4096 x 4096, W 12288 x 4096, bf16), the largest single-GPU workload.
For the QK-norm workload with the rotary embedding, the positions and the
(cos, sin) table are built once before timing, like the fold.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "norm+projection TFLOP/s (prefill) / GB/s (decode), % roofline, speedup vs unfused"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default 200; 2000 for the short float32 and decode workloads)")
    p.add_argument("--warmup", type=int, default=20,
                   help="untimed warm-up steps before the timed region (at least; see --warmup-seconds)")
    p.add_argument("--warmup-seconds", type=float, default=1.0,
                   help="the untimed warm-up also runs until this much wall time has passed, so the first "
                        "timed region does not start on a cold clock")
    p.add_argument("--blocks", type=int, default=5,
                   help="alternating blocks of the fused and the unfused step (each exactly --steps steps) "
                        "for the speedup, taken from the medians")
    p.add_argument("--workload", default="llama7b_qkv_prefill_bf16")
    p.add_argument("--out-dtype", default=None, choices=[None, "bf16", "f32"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-unfused", action="store_true")
    p.add_argument("--no-rowmajor", action="store_true",
                   help="with packed weights, skip timing the fused step on the row-major weights")
    p.add_argument("--layout", default="auto", choices=["auto", "rowmajor", "packed"],
                   help="weight layout of the fused variant; auto: decode-packed for the weight-streaming "
                        "(M <= 16) workloads, row-major otherwise")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    p.add_argument("--mark-regions", action="store_true",
                   help="launch a short torch sleep kernel right before and after the timed region, so a "
                        "kernel trace can find the region's dispatches")
    p.add_argument("--graph", action="store_true",
                   help="time every region by replaying a HIP graph that holds its steps (captured once and "
                        "replayed once untimed before timing), so the host's cost per call (about 10 us "
                        "through the Python binding) is not part of a short step")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="after timing, run a plain device copy of this many MiB (3 times) so a counter "
                        "profile holds a copy kernel of known size to scale FETCH_SIZE / WRITE_SIZE by")
    return p.parse_args()


# Every source that decides what runs: the kernels and the C ABI layer that
# picks tiles, passes and the decode/prefill split.
KERNEL_SOURCES = ("api.cpp", "common.hpp", "decode.hip", "gemm_bf16.hip", "gemm_f32.hip", "kernels.hpp",
                  "rowwise.hip")


def kernel_source_sha() -> str:
    """Hash of the library sources with comments and whitespace removed,
    so that a counter record stays valid across edits that cannot change
    the compiled kernels or the dispatch, and goes stale with any that can."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rmsnorm_linear_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def profile_record(workload: str, out_dtype: str, sha: str):
    """The committed rocprofv3 counter record of this workload's fused
    kernel, or None if there is none for this exact kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{out_dtype}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != sha:
        return None
    return t


def traffic_from_profiles(workload: str, out_dtype: str, sha: str):
    """Measured HBM bytes per launch from committed rocprofv3 counter runs,
    or None if none exist for this exact kernel source."""
    t = profile_record(workload, out_dtype, sha)
    return None if t is None else t.get("hbm_bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(rows are independent; sharding is described in the design notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rmsnorm_linear_amd as fn
    import synth

    fn.load()
    OPS = {"linear": fn.OP_NORM_LINEAR, "glu": fn.OP_NORM_GLU_FFN, "qknorm": fn.OP_LINEAR_QKNORM,
           "qknorm_rope": fn.OP_LINEAR_QKNORM_ROPE, "layernorm": fn.OP_LAYERNORM_LINEAR,
           "latent": fn.OP_LINEAR_LATENT_NORM}
    w0 = synth.workload(args.workload)
    if w0.fp8:
        OPS.update({"linear": fn.OP_NORM_LINEAR_FP8, "glu": fn.OP_NORM_GLU_FFN_FP8})
    dev = torch.device("cuda:0")
    w = synth.workload(args.workload)
    if args.steps is None:
        args.steps = 2000 if (w.dtype == synth.F32 or w.M <= 16) else 200
    if w.dtype == synth.F32:
        out_dtype = "f32"
    else:
        out_dtype = args.out_dtype or "bf16"
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    xdt = torch.float32 if w.dtype == synth.F32 else torch.bfloat16

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---- inputs (seeded, synthetic), folded offline ------------------------
    t0 = time.time()
    x_np = w.x()
    g = torch.from_numpy(w.g()).to(dev)
    W0 = up(w.w())
    W1 = up(w.w_up()) if w.kind == "glu" else None
    gen_s = time.time() - t0

    out_bytes = 4 if out_dtype == "f32" else 2
    set_bytes = w.algo_bytes(out_bytes)
    copies = max(2, math.ceil(3 * MALL_BYTES / set_bytes))
    copies = min(copies, 64)
    xs, Ws0, Ws1, Wu0, Wu1, ys, gq, gk = [], [], [], [], [], [], None, None
    x0 = up(x_np)
    ln_beta = ln_bias = ln_c = ln_b = None
    if w.kind == "layernorm":
        ln_beta = torch.from_numpy(w.beta()).to(dev)
        ln_bias = torch.from_numpy(w.bias()).to(dev)
        Wf0, ln_c, ln_b = fn.fold_layernorm(W0, g, ln_beta, ln_bias)
    else:
        Wf0 = fn.fold_weights(W0, g)
    Wf1 = fn.fold_weights(W1, g) if W1 is not None else None
    if w.fp8:
        # offline: fold, then quantise per channel (the unfused baseline
        # quantises the unfolded weights)
        Wf0, Wf1 = fn.quantize_fp8(Wf0), (fn.quantize_fp8(Wf1) if Wf1 is not None else None)
        W0, W1 = fn.quantize_fp8(W0), (fn.quantize_fp8(W1) if W1 is not None else None)
    def clone(t):
        return None if t is None else (tuple(u.clone() for u in t) if isinstance(t, tuple) else t.clone())

    for c in range(copies):
        xs.append(x0.clone())
        Ws0.append(clone(Wf0))
        Ws1.append(clone(Wf1))
        ys.append(torch.empty((w.M, w.N), dtype=tdt, device=dev))
    # decode-packed copies of the folded weights (offline, like the fold)
    streaming = w.kind in ("glu", "layernorm", "linear") and w.M <= 16 and w.dtype == synth.BF16
    packed = streaming if args.layout == "auto" else args.layout == "packed"
    if packed and not streaming:
        raise SystemExit("--layout packed applies to the weight-streaming workloads (M <= 16, bf16)")

    def pack(t):
        if t is None:
            return None
        if isinstance(t, tuple):  # fp8: (codes, scales)
            return (fn.pack_decode_weights(t[0]), t[1])
        return fn.pack_decode_weights(t)

    Ps0 = [pack(t) for t in Ws0] if packed else Ws0
    Ps1 = [pack(t) for t in Ws1] if packed else Ws1
    if packed and w.kind == "glu":
        # gate and up in one buffer, each K step holding the gate slab's
        # pieces then the up slab's; the up weight argument is then None
        if w.fp8:
            Ps0 = [(fn.pack_decode_weights_glu(a[0], b[0]), a[1]) for a, b in zip(Ws0, Ws1)]
            Ps1 = [(None, b[1]) for b in Ws1]
        else:
            Ps0 = [fn.pack_decode_weights_glu(a, b) for a, b in zip(Ws0, Ws1)]
            Ps1 = [None] * len(Ws1)
    pos = table = None
    if w.kind in ("qknorm", "qknorm_rope"):
        gq = torch.from_numpy(w.g_q()).to(dev)
        gk = torch.from_numpy(w.g_k()).to(dev)
    if w.kind == "qknorm_rope" or (w.kind == "latent" and w.n_rope):
        pos = torch.from_numpy(w.positions()).to(dev)
        table = fn.rope_table(w.rope_base, w.rot_dim, w.n_pos, device=dev)  # set-up, like the fold
    if w.kind == "latent":
        gq = torch.from_numpy(w.g_q_latent()).to(dev) if w.n_q_latent else None
        gk = torch.from_numpy(w.g_kv_latent()).to(dev) if w.n_kv_latent else None
    torch.cuda.synchronize()

    def call(c, variant, Wa, Wb, ws=None):
        gg = g if variant == fn.UNFUSED else None
        if w.fp8 and w.kind == "linear":
            fn.norm_linear_fp8(xs[c], Wa[0], Wa[1], w.eps_f32(), g=gg, variant=variant, out=ys[c], ws=ws)
        elif w.fp8 and w.kind == "glu":
            fn.norm_glu_ffn_fp8(xs[c], Wa[0], Wa[1], Wb[0], Wb[1], w.eps_f32(), g=gg, variant=variant, out=ys[c],
                                ws=ws)
        elif w.kind == "linear":
            fn.norm_linear(xs[c], Wa, w.eps_f32(), g=gg, variant=variant, out=ys[c], ws=ws)
        elif w.kind == "layernorm":
            if variant == fn.UNFUSED:
                fn.layernorm_linear(xs[c], Wa, w.eps_f32(), g=g, beta=ln_beta, bias=ln_bias, variant=variant,
                                    out=ys[c], ws=ws)
            else:
                fn.layernorm_linear(xs[c], Wa, w.eps_f32(), colsum=ln_c, b_star=ln_b, variant=variant, out=ys[c],
                                    ws=ws)
        elif w.kind == "glu":
            fn.norm_glu_ffn(xs[c], Wa, Wb, w.eps_f32(), g=gg, variant=variant, out=ys[c], ws=ws)
        elif w.kind == "qknorm":
            fn.linear_qknorm(xs[c], Wa, w.n_q_heads, w.n_kv_heads, w.head_dim, gq, gk, w.eps_f32(),
                             w.eps_head_f32(), v_mode=0, g1=gg, variant=variant, out=ys[c], ws=ws)
        elif w.kind == "latent":
            fn.linear_latent_norm(xs[c], Wa, w.n_q_latent, w.n_kv_latent, w.n_rope, gq, gk, w.eps_f32(),
                                  w.eps_head_f32(), pos, table, g1=gg, variant=variant, out=ys[c], ws=ws)
        else:
            fn.linear_qknorm_rope(xs[c], Wa, w.n_q_heads, w.n_kv_heads, w.head_dim, gq, gk, w.eps_f32(),
                                  w.eps_head_f32(), pos, table, v_mode=0, g1=gg, variant=variant, out=ys[c], ws=ws)

    stream = torch.cuda.current_stream()
    decode_step = w.kind in ("glu", "layernorm", "linear") and w.M <= 16
    # "fresh x": in a model, x is the previous layer's output, written just
    # before this step.  Prefill only (a decode step's x is a few KB).
    srcx = xs[0].clone() if not decode_step else None

    def run(variant, Wa_list, Wb_list, ws, n, i0=0, hot=False, fresh=False, with_step=True):
        for i in range(i0, i0 + n):
            c = 0 if hot else i % copies
            if fresh:
                xs[c].copy_(srcx)
            if with_step:
                call(c, variant, Wa_list[c], Wb_list[c], ws)

    graphs = {}

    def region(variant, Wa_list, Wb_list, ws, **kw):
        """Exactly `steps` back-to-back steps between two HIP events on the
        launch stream, synchronised on both sides; milliseconds per step.  A
        step of one kernel launch gives that kernel's average launch
        duration (dispatch gaps included).  With --graph the steps are one
        replay of a graph that holds them all."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.graph:
            key = (variant, id(Wa_list), id(Wb_list), tuple(sorted(kw.items())), os.environ.get("FN_PRESTATS"))
            gr = graphs.get(key)
            if gr is None:
                torch.cuda.synchronize()
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    run(variant, Wa_list, Wb_list, ws, args.steps, **kw)
                gr.replay()  # untimed: the first replay uploads the graph
                torch.cuda.synchronize()
                graphs[key] = gr
            torch.cuda.synchronize()
            e0.record(stream)
            gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps
        torch.cuda.synchronize()
        e0.record(stream)
        run(variant, Wa_list, Wb_list, ws, args.steps, **kw)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def event_pairs(variant, Wa_list, Wb_list, ws):
        """Every launch bracketed by its own event pair (never feeds
        `value`: events between launches add dispatch gaps)."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            c = i % copies
            ev[i][0].record(stream)
            call(c, variant, Wa_list[c], Wb_list[c], ws)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) for a, b in ev])
        return {"mean": float(per.mean()), "p10": float(np.percentile(per, 10)), "median": float(np.median(per)),
                "p90": float(np.percentile(per, 90))}

    # the fused variant's workspace (row statistics of large shapes), allocated once
    fws = None
    fwsb = fn.workspace_bytes(OPS[w.kind], fn.FUSED, w.M, w.K, w.N, xdt)
    if fwsb:
        fws = torch.empty(fwsb, dtype=torch.uint8, device=dev)
    fused = (fn.FUSED, Ps0, Ps1, fws)

    # ---- unfused baseline: the unfolded weights and the RMSNorm kernel -----
    unfused = None
    if not args.no_unfused:
        Wu0 = [W0] + [clone(W0) for _ in range(copies - 1)]
        Wu1 = ([W1] + [clone(W1) for _ in range(copies - 1)]) if W1 is not None else [None] * copies
        wsb = fn.workspace_bytes(OPS[w.kind], fn.UNFUSED, w.M, w.K, w.N, xdt)
        uws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        unfused = (fn.UNFUSED, Wu0, Wu1, uws)

    # ---- warm-up: untimed, at least `warmup` steps of each variant and at
    # least `warmup_seconds` of wall time, ending on the fused step ----------
    t_w = time.perf_counter()
    n_warm = 0
    chunk = max(1, min(args.warmup, 50))
    while n_warm < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        if unfused is not None:
            run(*unfused, chunk, i0=n_warm)
        run(*fused, chunk, i0=n_warm)
        n_warm += chunk
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w

    # ---- the timed region: exactly `steps` fused steps ----------------------
    if args.mark_regions:
        torch.cuda._sleep(1)
    t_wall = time.perf_counter()
    ms_step = region(*fused)
    wall = time.perf_counter() - t_wall
    if args.mark_regions:
        torch.cuda._sleep(1)
    k_pct = event_pairs(*fused)

    # ---- the GEMM's own launch duration, where a step launches more than
    # the GEMM (a statistics or quantisation pass before it, a latent-norm
    # kernel after it): the library records an event pair around each GEMM
    # launch on the launch stream (flashnorm_testing.h) ------------------------
    def gemm_event_ms():
        lib = fn.load()
        ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        for e in ev_s + ev_e:
            e.record(stream)  # creates the event
        torch.cuda.synchronize()
        arr = ctypes.c_void_p * args.steps
        starts = arr(*[e.cuda_event for e in ev_s])
        stops = arr(*[e.cuda_event for e in ev_e])
        if lib.fn_testing_gemm_events(starts, stops, args.steps) != 0:
            return None
        try:
            run(*fused, args.steps)
            torch.cuda.synchronize()
        finally:
            lib.fn_testing_gemm_events(None, None, 0)
        per = np.array([a.elapsed_time(b) for a, b in zip(ev_s, ev_e)])
        return {"mean": float(per.mean()), "p10": float(np.percentile(per, 10)), "median": float(np.median(per)),
                "p90": float(np.percentile(per, 90))}

    n_launch = fn.dispatch_name(OPS[w.kind], fn.FUSED_PACKED if packed else fn.FUSED, w.M, w.K, w.N, xdt,
                                tdt).split(":", 1)[1].count("+") + 1
    gemm_ms = gemm_event_ms() if n_launch > 1 else None

    # ---- fused against unfused in alternating blocks (each exactly `steps`
    # steps, the order flipped every block), cold and hot; medians --------
    def blocks(hot=False, fresh=False):
        f, u, cp = [], [], []
        for b in range(args.blocks):
            order = (fused, unfused) if b % 2 == 0 else (unfused, fused)
            for v in order:
                if v is None:
                    continue
                t = region(*v, hot=hot, fresh=fresh)
                (f if v is fused else u).append(t)
            if fresh:
                cp.append(region(*fused, fresh=True, with_step=False))
        return f, u, cp

    med = lambda a: float(np.median(a)) if a else None  # noqa: E731
    f_cold, u_cold, _ = blocks()
    # Where the fused step runs a row-statistics pass before the GEMM, the
    # same step with the sums of squares taken inside the GEMM instead (one
    # launch; FN_PRESTATS=0), timed in blocks alternating with the default
    one_launch = None
    if "row_scale+" in fn.dispatch_name(OPS[w.kind], fn.FUSED, w.M, w.K, w.N, xdt, tdt):
        old = os.environ.get("FN_PRESTATS")
        d_ms, o_ms = [], []
        for b in range(args.blocks):
            for v in (("default", "one") if b % 2 == 0 else ("one", "default")):
                if v == "one":
                    os.environ["FN_PRESTATS"] = "0"
                    o_ms.append(region(fn.FUSED, Ps0, Ps1, fws))
                    name = fn.dispatch_name(OPS[w.kind], fn.FUSED, w.M, w.K, w.N, xdt, tdt)
                    if old is None:
                        del os.environ["FN_PRESTATS"]
                    else:
                        os.environ["FN_PRESTATS"] = old
                else:
                    d_ms.append(region(*fused))
        one_launch = {"kernel": name, "block_ms": o_ms, "median_ms": med(o_ms), "default_block_ms": d_ms,
                      "default_median_ms": med(d_ms), "one_launch_over_default": med(o_ms) / med(d_ms),
                      "speedup_vs_unfused": (med(u_cold) / med(o_ms)) if u_cold else None}
    f_hot, u_hot, _ = blocks(hot=True) if copies > 1 else ([], [], [])
    fresh = None
    if srcx is not None and unfused is not None:
        f_fr, u_fr, cp = blocks(fresh=True)
        fresh = {"copy_ms": med(cp), "fused_ms": med(f_fr) - med(cp), "unfused_ms": med(u_fr) - med(cp),
                 "block_ms": {"copy": cp, "fused_with_copy": f_fr, "unfused_with_copy": u_fr}}
        fresh["speedup_vs_unfused"] = fresh["unfused_ms"] / fresh["fused_ms"]
    hot_ms = med(f_hot)

    # the fused step on the row-major weights, for comparison
    rowmajor = None
    if packed and not args.no_rowmajor:
        run(fn.FUSED, Ws0, Ws1, fws, args.warmup)
        rm_ms = region(fn.FUSED, Ws0, Ws1, fws)
        rowmajor = {"ms_per_step": rm_ms, "packed_speedup": rm_ms / ms_step}

    unf = None
    if unfused is not None:
        unf = {"ms_per_step": med(u_cold), "block_ms": u_cold, "event_pair_ms": event_pairs(*unfused),
               "hot_ms_per_step": med(u_hot), "hot_block_ms": u_hot}

    # ---- the pages' own design: GEMM and row statistics on two streams,
    # explicit join, post-scale (plain bf16 linear workloads) ------------
    two = None
    if not args.no_unfused and w.kind == "linear" and w.dtype == synth.BF16 and not w.fp8 and w.M > 16:
        aux = torch.cuda.Stream()
        tws = torch.empty(fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.TWO_STREAM, w.M, w.K, w.N, xdt),
                          dtype=torch.uint8, device=dev)
        tws.record_stream(aux)
        Wt = [Ws0[0]] + [Ws0[0].clone() for _ in range(copies - 1)]

        def call2(c):
            fn.norm_linear(xs[c], Wt[c], w.eps_f32(), variant=fn.TWO_STREAM, out=ys[c], ws=tws, aux_stream=aux)

        for i in range(args.warmup):
            call2(i % copies)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            call2(i % copies)
        e1.record(stream)
        torch.cuda.synchronize()
        two = {"ms_per_step": e0.elapsed_time(e1) / args.steps}
        del Wt

    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flops = w.flops()
    algo_bytes = w.algo_bytes(out_bytes)
    decode = w.kind in ("glu", "layernorm", "linear") and w.M <= 16
    tflops = flops / (ms_step * 1e-3) / 1e12
    gbs = algo_bytes / (ms_step * 1e-3) / 1e9
    # achieved: algorithmic work of one step over the timed region's time per step
    if decode:
        value, unit = gbs, "GB/s"
        roof = {"bound": "hbm", "achieved": algo_bytes / (ms_step * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        peak = PEAK_F32_TFLOPS if w.dtype == synth.F32 else PEAK_FP8_TFLOPS if w.fp8 else PEAK_BF16_TFLOPS
        value, unit = tflops, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": flops / (ms_step * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    sha = kernel_source_sha()
    roof["traffic"] = traffic_from_profiles(args.workload, out_dtype, sha)
    rec = profile_record(args.workload, out_dtype, sha)
    core = rec.get("core") if rec else None
    if core and not decode:
        # the clock the counters saw during the profiled dispatch, and the
        # dense peak at that clock (the chip cannot reach 2.4 GHz under this load)
        roof["clock_adjusted"] = {"effective_clock_ghz": core["effective_clock_ghz"],
                                  "peak": core["clock_adjusted_peak"],
                                  "frac": roof["achieved"] / core["clock_adjusted_peak"],
                                  "mfma_busy": core["mfma_busy"]}
    roof["kernel"] = fn.dispatch_name(OPS[w.kind], fn.FUSED_PACKED if packed else fn.FUSED, w.M, w.K, w.N, xdt, tdt)
    # launches per fused step: "<variant>:<kernel>+<kernel>..."
    launches = roof["kernel"].split(":", 1)[1].count("+") + 1
    roof["launches_per_step"] = launches
    # the dominant kernel's average launch duration: the timed region's per
    # step time when the step is that one launch; for a step of several
    # launches, the GEMM's own event pairs (recorded by the library around
    # each GEMM launch) over `steps` more fused steps
    roof["kernel_ms"] = ms_step if launches == 1 else None
    roof["step_ms"] = ms_step
    roof["kernel_ms_basis"] = "timed region / steps" if launches == 1 else "step: timed region / steps"
    if launches > 1 and gemm_ms is not None:
        # an event pair around one launch adds several microseconds to a
        # few of them (the mean sits above the timed region's whole step
        # on the Llama-7B shape); the median is the typical launch
        roof["kernel_ms"] = gemm_ms["median"]
        roof["kernel_ms_basis"] = "median of per-launch GEMM event pairs"
        roof["kernel_event_pair_ms"] = gemm_ms
        roof["step_achieved"] = roof["achieved"]
        work = algo_bytes / 1e9 if decode else flops / 1e12
        roof["achieved"] = work / (gemm_ms["median"] * 1e-3)
        roof["frac"] = roof["achieved"] / roof["peak"]
    roof["event_pair_ms"] = k_pct
    roof["hot_ms_per_step"] = hot_ms

    # ---- CPU baseline: the float64 oracle on a bounded row sample -----------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info

        Wn = w.w()
        Wun = w.w_up() if w.kind == "glu" else None
        gn = w.g()
        pos_np = w.positions() if w.kind in ("qknorm_rope", "latent") else None
        ln_beta_np = w.beta() if w.kind == "layernorm" else None
        if w.fp8:  # the oracle's own fold and quantisation, outside the timed sample
            q8g = oracle.quantize_fp8_per_channel(oracle.fold_weights(Wn, gn, synth.BF16))
            q8u = oracle.quantize_fp8_per_channel(oracle.fold_weights(Wun, gn, synth.BF16)) if Wun is not None else None
        ln_bias_np = w.bias() if w.kind == "layernorm" else None
        # whole passes over the rows (restarting at row 0) until the time is spent
        rows_total, t_cpu = 0, 0.0
        chunk = max(1, min(w.M, 64))
        while t_cpu < args.cpu_seconds:
            rows_done = rows_total % w.M
            r1 = min(w.M, rows_done + chunk)
            xr = x_np[rows_done:r1]
            ts = time.perf_counter()
            if w.kind == "glu" and w.fp8 and w.M > 16:
                oracle.glu_fp8_act(xr, *q8g, *q8u, w.eps_f32())
            elif w.kind == "linear" and w.fp8 and w.M > 16:
                oracle.norm_linear_fp8_act(xr, *q8g, w.eps_f32())
            elif w.kind == "linear":
                oracle.norm_linear(xr, Wn, gn, w.eps_f32())
            elif w.kind == "layernorm":
                oracle.layernorm_linear(xr, Wn, gn, ln_beta_np, ln_bias_np, w.eps_f32())
            elif w.kind == "glu" and w.fp8:
                oracle.glu_deferred_on_quantized(xr, *q8g, *q8u, w.eps_f32())
            elif w.kind == "glu":
                oracle.norm_glu_ffn(xr, Wn, Wun, gn, w.eps_f32())
            elif w.kind == "qknorm":
                oracle.linear_qknorm(xr, Wn, gn, w.eps_f32(), w.n_q_heads, w.n_kv_heads, w.head_dim, w.g_q(),
                                     w.g_k(), w.eps_head_f32(), 0)
            elif w.kind == "latent":
                oracle.linear_latent_norm(xr, Wn, gn, w.eps_f32(), w.n_q_latent, w.n_kv_latent, w.n_rope,
                                          w.g_q_latent() if w.n_q_latent else None,
                                          w.g_kv_latent() if w.n_kv_latent else None, w.eps_head_f32(),
                                          pos_np[rows_done:r1] if w.n_rope else None, w.rope_base, w.rot_dim)
            else:
                oracle.linear_qknorm_rope(xr, Wn, gn, w.eps_f32(), w.n_q_heads, w.n_kv_heads, w.head_dim,
                                          w.g_q(), w.g_k(), w.eps_head_f32(), 0, pos_np[rows_done:r1],
                                          w.rope_base, w.rot_dim)
            t_cpu += time.perf_counter() - ts
            rows_total += r1 - rows_done
        frac_rows = rows_total / w.M
        if decode:
            cval = algo_bytes * frac_rows / t_cpu / 1e9
        else:
            cval = flops * frac_rows / t_cpu / 1e12
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        cpu = {"value": cval, "unit": unit, "cores": threads, "kind": "oracle",
               "sample": f"float64 oracle on {rows_total} rows ({frac_rows:.2f} passes over the {w.M} rows, "
                         f"full weights), {t_cpu:.1f} s"}

    res = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == synth.F32 else ("fp8 e4m3" if (w.fp8 and not decode) else "bf16"),
        "data": "synthetic (seeded SplitMix64/Box-Muller, workload distributions)",
        "config": {"workload": args.workload, "M": w.M, "K": w.K, "N": w.N,
                   "projections": 2 if w.kind == "glu" else 1, "out_dtype": out_dtype,
                   "weights": ("e4m3 per output channel, widened to bf16 for the MFMAs" if decode else
                               "e4m3 per output channel; x quantised per row to e4m3 in the op") if w.fp8 else "bf16",
                   "layout": ("decode-packed, gate/up pair" if w.kind == "glu" else "decode-packed") if packed
                   else "row-major", "rotated_copies": copies},
        "tflops": tflops,
        "gbs": gbs,
        "roofline": roof,
        "cpu_baseline": cpu,
        "unfused": unf,
        "fused_rowmajor": rowmajor,
        "two_stream": two,
        "fused_blocks": {"block_ms": f_cold, "median_ms": med(f_cold), "hot_block_ms": f_hot,
                         "hot_median_ms": hot_ms},
        # medians over the alternating blocks (each exactly `steps` steps)
        "speedup_vs_unfused": (unf["ms_per_step"] / med(f_cold)) if unf else None,
        "speedup_vs_unfused_hot": (unf["hot_ms_per_step"] / hot_ms) if (unf and hot_ms and unf["hot_ms_per_step"])
        else None,
        "latency_reduction_vs_unfused": (1 - med(f_cold) / unf["ms_per_step"]) if unf else None,
        # decode on packed weights: the unfused baseline reads row-major
        # weights, so speedup_vs_unfused includes the layout; this is the
        # fusion alone (both on row-major weights)
        "speedup_vs_unfused_same_layout": (unf["ms_per_step"] / rowmajor["ms_per_step"]) if (unf and rowmajor)
        else None,
        "fresh_x": fresh,
        "one_launch": one_launch,
        "speedup_vs_unfused_fresh_x": fresh["speedup_vs_unfused"] if fresh else None,
        "launch": "hip graph replay" if args.graph else "eager",
        "kernel_src_sha": sha,
        "input_gen_s": gen_s,
        "timed_wall_s": wall,
        "warmup_steps_run": n_warm,
        "warmup_seconds": warm_s,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
