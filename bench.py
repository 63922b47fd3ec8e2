#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 linear layer on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over the layer4096 workload
(W0 4096 x 4096 fp32 ~ N(0, 0.02^2); x: M = 4096 tokens = batch 4 x sequence
1024; r = 8, alpha = 16; synthetic, seeded):
    qlora_nf4_quantize(W0)           NF4 codes + double-quantized constants
    qlora_linear_fwd                 Y = X What^T + s (X A^T) B^T
    qlora_linear_bwd                 dX, dA, dB
All inputs are resident in HBM before the timed region.  `value` is the
forward + backward algorithmic flops per step (4 M d k + 6 M r (d + k)) over
the measured time of the whole step (quantization included), in TFLOP/s.
`roofline` is the forward dequant-GEMM kernel, its duration averaged over the
timed steps (each launch stamps its own execution span when asked,
qlora_time_next_kernel); the same kernel launched alone is reported beside it.

The same run measures the decode-shaped forward (decode workload: W0 4096 x
4096 and 14336 x 4096, M in {1, 4, 16}, r = 16, alpha = 32) as GB/s of packed
NF4 bytes and of all algorithmic bytes, from the decode kernel's own
execution span (calls rotating over weight copies totalling more than 512 MB
so that neither the 256 MB Infinity Cache nor L2 serves them), with the time
per call of the same calls replayed from a HIP graph beside it; and the 7B- and
65B-shaped layers (all seven projections, forward + backward, and the quantize
of every weight of the layer).  Calls short enough for the binding's host work
to matter (quantize of one projection, merge, dropout, the other formats'
quantize and decode) are timed as captured calls replayed from a HIP graph;
forward + backward pairs as back-to-back calls between two events.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "QLoRA linear fwd+bwd TFLOP/s at M=4096; NF4 weight GB/s at M=16 forward"
PROFILES = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fwd_flops(m, d, k, r):
    return 2 * m * d * k + 2 * m * r * (d + k)


def bwd_flops(m, d, k, r):
    return 2 * m * d * k + 4 * m * r * (d + k)


def source_sha(name: str) -> str:
    path = os.path.join(ROOT, "bit_nf4_quantized_13_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profiles(key: str, source: str):
    """HBM bytes per launch of one kernel from the committed rocprofv3 --pmc
    summary (profiles/hbm_traffic.txt): FETCH_SIZE + WRITE_SIZE per dispatch,
    scaled by the factor a plain copy of known size gives.  None when the
    summary was taken on another version of the kernel's source."""
    path = os.path.join(PROFILES, "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    for ln in open(path):
        f = ln.split()
        if not f or f[0] != key:
            continue
        kv = dict(x.split("=", 1) for x in f[1:] if "=" in x)
        if kv.get("source_sha") != source_sha(source):
            return None
        return round(float(kv["hbm_bytes_per_launch"]))
    return None


class Timer:
    """HIP events on torch's current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((e0, e1))

    def total_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs)


def run_layer_bench(q, torch, steps, warmup):
    from workloads import WORKLOADS, workload_layer
    from tests.helpers import to_dev_bf16, to_dev_f32
    wl = WORKLOADS["layer4096"]
    p = wl.projections[0]
    m, d, k, r, alpha = wl.m[0], p.d, p.k, wl.r, wl.alpha
    log(f"layer4096: generating inputs d={d} k={k} M={m} r={r}")
    inp = workload_layer("layer4096")
    w0 = to_dev_f32(inp.w0)
    x, a, b, dy = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b, inp.dy))
    wq = q.NF4Weight.empty(d, k)
    qws = torch.empty(q.quantize_workspace_bytes(d, k), dtype=torch.uint8, device="cuda")
    lws = torch.empty(q.linear_workspace_bytes(m, d, k, r), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, d), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((m, r), dtype=torch.float32, device="cuda")
    dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    da = torch.empty((r, k), dtype=torch.float32, device="cuda")
    db = torch.empty((d, r), dtype=torch.float32, device="cuda")

    tq, tf, tb = Timer(torch), Timer(torch), Timer(torch)

    def step(timed):
        e = tq.start() if timed else None
        q.qlora_nf4_quantize(w0, out=wq, workspace=qws)
        if timed:
            tq.stop(e)
            e = tf.start()
        q.qlora_linear_fwd(wq, x, a, b, alpha, out=y, u_out=u, workspace=lws)
        if timed:
            tf.stop(e)
            e = tb.start()
        q.qlora_linear_bwd(wq, x, dy, a, b, alpha, u=u, workspace=lws, outs=(dx, da, db))
        if timed:
            tb.stop(e)

    for _ in range(warmup):
        step(False)
    # execution spans of each timed step's two dequant-GEMM launches
    # (qlora_time_next_kernel: the kernels stamp them themselves)
    spans = torch.tensor([[-1, 0]] * (2 * steps), dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    log(f"layer4096: timing {steps} steps")
    # the timed region: K whole steps, events only at its two ends
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        q.qlora_time_next_kernel("fwd_gemm", spans[2 * i])
        q.qlora_time_next_kernel("dx_gemm", spans[2 * i + 1])
        step(False)
    ev1.record()
    torch.cuda.synchronize()
    khz = q.wall_clock_khz()
    dur = q.span_duration_us(spans, khz)
    gemm_fwd_ms = sum(dur[0::2]) / steps * 1e-3
    gemm_dx_ms = sum(dur[1::2]) / steps * 1e-3
    wall_ms = (time.perf_counter() - t0) * 1e3
    total_ms = ev0.elapsed_time(ev1)
    ms_step = total_ms / steps
    flops = fwd_flops(m, d, k, r) + bwd_flops(m, d, k, r)
    # per-call breakdown in a separate pass (its events stall the queue briefly
    # between calls, so it is not part of the timed region)
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    phases = {"quantize_ms": tq.total_ms() / steps, "fwd_ms": tf.total_ms() / steps,
              "bwd_ms": tb.total_ms() / steps}

    fb_ms = phases["fwd_ms"] + phases["bwd_ms"]
    ctx = (wq, x, a, b, alpha, y, u, lws, r)
    return ctx, {
        "m": m, "d": d, "k": k, "r": r, "alpha": alpha, "ms_per_step": ms_step,
        "wall_ms_per_step": wall_ms / steps,
        "tflops_step": flops / (ms_step * 1e-3) / 1e12,
        "tflops_fwd_bwd": flops / (fb_ms * 1e-3) / 1e12,
        "phases": phases, "flops": flops, "gemm_fwd_ms": gemm_fwd_ms, "gemm_dx_ms": gemm_dx_ms,
        "quantize_gbs": (d * k * 4 + d * k // 2 + d * k // 64) / (phases["quantize_ms"] * 1e-3) / 1e9,
    }


def run_decode_bench(q, torch, iters=50, graph_replays=10):
    """Per decode shape: the decode kernel's duration (its execution span, which
    the kernel stamps itself when asked, qlora_time_next_kernel; averaged over
    `iters` ordinary calls on rotating weight copies; one kernel per call, so
    this is the per-call sum of kernel durations) and, beside it, the time
    per call of the same calls captured in a HIP graph and replayed (no host
    launch gaps)."""
    khz = q.wall_clock_khz()
    from workloads import WORKLOADS, workload_layer
    from tests.helpers import to_dev_bf16, to_dev_f32
    wl = WORKLOADS["decode"]
    out = {}
    for pi, p in enumerate(wl.projections):
        inp = workload_layer("decode", pi)
        packed = p.d * p.k // 2
        copies = max(2, -(-512 * 2**20 // packed) + 1)
        log(f"decode {p.name}: quantizing {copies} weight copies ({copies * packed / 2**20:.0f} MiB packed)")
        w0 = to_dev_f32(inp.w0)
        ws = [q.qlora_nf4_quantize(w0) for _ in range(copies)]
        del w0
        a, b = to_dev_bf16(inp.a), to_dev_bf16(inp.b)
        for m in wl.m:
            x = to_dev_bf16(inp.x[:m])
            y = torch.empty((m, p.d), dtype=torch.bfloat16, device="cuda")
            lws = torch.empty(q.linear_workspace_bytes(m, p.d, p.k, wl.r), dtype=torch.uint8,
                              device="cuda")

            def call(it):
                q.qlora_linear_fwd(ws[it % copies], x, a, b, wl.alpha, save_u=False, out=y, workspace=lws)
            for i in range(copies):
                call(i)
            spans = torch.tensor([[-1, 0]] * iters, dtype=torch.int64, device="cuda")
            torch.cuda.synchronize()
            for it in range(iters):
                q.qlora_time_next_kernel("decode", spans[it])
                call(it)
            torch.cuda.synchronize()
            kern_us = sum(q.span_duration_us(spans, khz)) / iters
            # the same calls captured once and replayed
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for it in range(iters):
                    call(it)
            torch.cuda.current_stream().wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for it in range(iters):
                    call(it)
            graph.replay()
            torch.cuda.synchronize()
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            g0.record()
            for _ in range(graph_replays):
                graph.replay()
            g1.record()
            torch.cuda.synchronize()
            graph_us = g0.elapsed_time(g1) * 1e3 / (graph_replays * iters)
            del graph
            alg = decode_bytes(m, p.d, p.k, wl.r)
            gbs = packed / (kern_us * 1e-6) / 1e9
            out[f"{p.name}_m{m}"] = {"kernel_us": round(kern_us, 3), "kernels_per_call": 1,
                                     "graph_us_per_call": round(graph_us, 3),
                                     "packed_gbs": round(gbs, 1),
                                     "hbm_frac_packed": round(gbs / HBM_PEAK_GBS, 4),
                                     "algorithmic_bytes": alg,
                                     "algorithmic_gbs": round(alg / (kern_us * 1e-6) / 1e9, 1),
                                     "algorithmic_gbs_graph": round(alg / (graph_us * 1e-6) / 1e9, 1)}
            log(f"decode {p.name} M={m}: kernel {kern_us:.2f} us, graph {graph_us:.2f} us/call, "
                f"{gbs:.0f} GB/s packed")
        del ws
        torch.cuda.empty_cache()
    return out


def run_model_bench(q, torch, name, reps=5, warm=2):
    """All projections of a model-shaped layer (llama7b: q, k, v, o 4096x4096,
    gate, up 11008x4096, down 4096x11008, M = 2048, r = 64; llama65b: 8192 and
    22016 wide, M = 4096, r = 64; alpha = 16): per projection, the quantize of
    its W0 and forward + backward (event-timed, `reps` calls after `warm`).
    Inputs with the workload's distributions (W0 ~ N(0, 0.02^2), A ~ N(0,
    1/r), B ~ N(0, 0.01^2), x, dY ~ N(0, 1)), drawn on the device by torch's
    seeded generator: these sizes take too long to draw on the host."""
    from workloads import WORKLOADS, device_normal
    wl = WORKLOADS[name]
    m, r, alpha = wl.m[0], wl.r, wl.alpha
    per, tot_flops, tot_ms, q_ms, n_w = {}, 0, 0.0, 0.0, 0
    for pi, p in enumerate(wl.projections):
        d, k = p.d, p.k
        seed = 1000 * wl.seed + 10 * pi
        w0 = device_normal(seed, (d, k))
        a = device_normal(seed + 1, (r, k), std=1.0 / r ** 0.5).to(torch.bfloat16)
        b = device_normal(seed + 2, (d, r), std=0.01).to(torch.bfloat16)
        x = device_normal(seed + 3, (m, k), std=1.0).to(torch.bfloat16)
        dy = device_normal(seed + 4, (m, d), std=1.0).to(torch.bfloat16)
        wq = q.NF4Weight.empty(d, k)
        qws = torch.empty(q.quantize_workspace_bytes(d, k), dtype=torch.uint8, device="cuda")
        lws = torch.empty(q.linear_workspace_bytes(m, d, k, r), dtype=torch.uint8, device="cuda")
        y = torch.empty((m, d), dtype=torch.bfloat16, device="cuda")
        u = torch.empty((m, r), dtype=torch.float32, device="cuda")
        outs = (torch.empty((m, k), dtype=torch.bfloat16, device="cuda"),
                torch.empty((r, k), dtype=torch.float32, device="cuda"),
                torch.empty((d, r), dtype=torch.float32, device="cuda"))
        # quantize: the calls captured in a HIP graph and replayed (a single call is
        # about as short as the binding's host work per call, which back-to-back
        # eager calls would measure instead)
        qm = time_graph(torch, lambda: q.qlora_nf4_quantize(w0, out=wq, workspace=qws), reps)
        del w0

        def fwd_bwd():
            q.qlora_linear_fwd(wq, x, a, b, alpha, out=y, u_out=u, workspace=lws)
            q.qlora_linear_bwd(wq, x, dy, a, b, alpha, u=u, workspace=lws, outs=outs)
        for _ in range(warm):
            fwd_bwd()
        fb = time_calls(torch, fwd_bwd, reps)
        fl = fwd_flops(m, d, k, r) + bwd_flops(m, d, k, r)
        per[p.name] = {"d": d, "k": k, "fwd_bwd_ms": round(fb, 4),
                       "fwd_bwd_tflops": round(fl / (fb * 1e-3) / 1e12, 2), "quantize_us": round(qm * 1e3, 2)}
        tot_flops += fl
        tot_ms += fb
        q_ms += qm
        n_w += d * k
        log(f"{name} {p.name} {d}x{k}: fwd+bwd {fb:.3f} ms = {fl / (fb * 1e-3) / 1e12:.0f} TFLOP/s, "
            f"quantize {qm * 1e3:.1f} us")
        del wq, qws, lws, y, u, outs, x, dy, a, b
        torch.cuda.empty_cache()
    # quantize bytes: fp32 W0 read, packed codes + c2 bytes + c1 and the mean written
    nb = n_w // 64
    q_bytes = 4 * n_w + n_w // 2 + nb + 4 * (nb // 256) + 4 * len(wl.projections)
    return {"workload": f"{name}: {len(wl.projections)} projections, M={m}, r={r}, alpha={alpha}",
            "fwd_bwd_ms": round(tot_ms, 4), "fwd_bwd_tflops": round(tot_flops / (tot_ms * 1e-3) / 1e12, 2),
            "fwd_bwd_frac": round(tot_flops / (tot_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "flops": tot_flops, "quantize_weights": n_w, "quantize_ms": round(q_ms, 4),
            "quantize_gbs": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
            "quantize_hbm_frac": round(q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "per_projection": per}


def gemm_flops(m, d, k, r):
    """Algorithmic flops of the forward dequant-GEMM kernel: X What^T plus the
    adapter's up-projection (s U) B^T that its epilogue k-columns carry."""
    return 2 * m * d * k + 2 * m * d * r


def time_gemm_only(q, torch, ctx, iters):
    """The forward's GEMM kernel alone (qlora_linear_gemm_only on the workspace
    the preceding forward prepared), timed with HIP events on torch's current
    stream -- the stream the library launches on."""
    w, x, a, b, alpha, y, u, lws, r = ctx
    q.qlora_linear_fwd(w, x, a, b, alpha, out=y, u_out=u, workspace=lws)
    for _ in range(3):
        q.qlora_linear_gemm_only(w, False, x, r, y, lws)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        q.qlora_linear_gemm_only(w, False, x, r, y, lws)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def run_vendor_gemm_context(torch, n=4096, iters=20):
    """Context only (not part of the layer's path): torch's bf16 GEMM (hipBLASLt
    on ROCm) on the forward GEMM's shape, M = N = K = 4096, random N(0, 1)
    operands, event-timed back to back -- the rate a vendor dense bf16 GEMM
    reaches on this machine, beside the fused dequant-GEMM's."""
    g = torch.Generator(device="cuda").manual_seed(5)
    a = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    ms = time_calls(torch, lambda: torch.mm(a, b, out=c), iters)
    tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
    return {"shape": f"{n}x{n}x{n} bf16", "us": round(ms * 1e3, 2), "tflops": round(tf, 1),
            "frac": round(tf / BF16_PEAK_TFLOPS, 4)}


def run_merge_bench(q, torch, ctx, iters=20):
    """qlora_adapter_merge on the layer4096 weight (4096 x 4096, r = 8): the
    merged bf16 weight What + (alpha/r) B A, r fp64 FMAs per weight.  Reported
    with its algorithmic HBM bytes (codes, c2, c1, A, B read; bf16 written) and
    fp64 flops."""
    w, x, a, b, alpha, y, u, lws, r = ctx
    d, k = w.d, w.k
    out = torch.empty((d, k), dtype=torch.bfloat16, device="cuda")
    ms = time_graph(torch, lambda: q.qlora_adapter_merge(w, a, b, alpha, out=out), iters)
    nb = d * k // 64
    nbytes = d * k // 2 + nb + 4 * ((nb + 255) // 256) + 4 + 2 * r * k + 2 * d * r + 2 * d * k
    return {"us_per_call": round(ms * 1e3, 3), "algorithmic_bytes": nbytes,
            "algorithmic_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "fp64_tflops": round(2 * r * d * k / (ms * 1e-3) / 1e12, 2),
            "workload": f"layer4096 weight {d}x{k}, r={r}"}


def time_calls(torch, fn, iters):
    """Average ms of fn() over iters calls on torch's current stream (after 3 warm calls)."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def time_graph(torch, fn, iters, replays=4):
    """Average ms of fn() per call: `iters` calls captured once in a HIP graph
    (after warm-up calls on a side stream), then the graph replayed `replays`
    times between two events on torch's current stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(iters):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / (replays * iters)


def run_format_bench(q, torch, ctx, fmt, iters=20):
    """A further storage format of the block constants -- "no_dq" (one fp32
    absmax per block) or "fp8" (double quantization with c2 in OCP FP8 e4m3):
    quantize, forward + backward on the layer4096 inputs, and the decode
    forward of the 14336 x 4096 projection at M = 16."""
    from workloads import WORKLOADS, workload_layer
    from tests.helpers import to_dev_bf16, to_dev_f32
    kw = {"double_quant": False} if fmt == "no_dq" else {"c2_fp8": True}
    _, x, a, b, alpha, y, u, lws, r = ctx
    inp = workload_layer("layer4096")
    m, d, k = inp.x.shape[0], inp.w0.shape[0], inp.w0.shape[1]
    w0 = to_dev_f32(inp.w0)
    dy = to_dev_bf16(inp.dy)
    wq = q.NF4Weight.empty(d, k, **kw)
    qws = torch.empty(q.quantize_workspace_bytes(d, k, wq.dq_block), dtype=torch.uint8, device="cuda")
    dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    da = torch.empty((r, k), dtype=torch.float32, device="cuda")
    db = torch.empty((d, r), dtype=torch.float32, device="cuda")
    log(f"{fmt}: layer4096 quantize / fwd+bwd")
    q_ms = time_graph(torch, lambda: q.qlora_nf4_quantize(w0, out=wq, workspace=qws), iters)

    def fwd_bwd():
        q.qlora_linear_fwd(wq, x, a, b, alpha, out=y, u_out=u, workspace=lws)
        q.qlora_linear_bwd(wq, x, dy, a, b, alpha, u=u, workspace=lws, outs=(dx, da, db))
    fb_ms = time_calls(torch, fwd_bwd, iters)
    flops = fwd_flops(m, d, k, r) + bwd_flops(m, d, k, r)
    const_bytes = wq.nbytes() - d * k // 2   # block constants of the stored weight
    del w0, wq, qws
    wl = WORKLOADS["decode"]
    pi = max(range(len(wl.projections)), key=lambda i: wl.projections[i].d * wl.projections[i].k)
    p = wl.projections[pi]
    dinp = workload_layer("decode", pi)
    dm = max(wl.m)
    packed = p.d * p.k // 2
    copies = max(2, -(-512 * 2**20 // packed) + 1)
    log(f"{fmt}: decode {p.name} M={dm} over {copies} weight copies")
    dw0 = to_dev_f32(dinp.w0)
    ws = [q.qlora_nf4_quantize(dw0, **kw) for _ in range(copies)]
    dconst = ws[0].nbytes() - packed
    del dw0
    da_, db_, dx_ = to_dev_bf16(dinp.a), to_dev_bf16(dinp.b), to_dev_bf16(dinp.x[:dm])
    dy_ = torch.empty((dm, p.d), dtype=torch.bfloat16, device="cuda")
    dws = torch.empty(q.linear_workspace_bytes(dm, p.d, p.k, wl.r), dtype=torch.uint8, device="cuda")
    it = [0]

    def dec():
        q.qlora_linear_fwd(ws[it[0] % copies], dx_, da_, db_, wl.alpha, save_u=False, out=dy_, workspace=dws)
        it[0] += 1
    dec_us = time_graph(torch, dec, 50) * 1e3
    alg = packed + dconst + 2 * dm * p.k + 2 * wl.r * p.k + 2 * p.d * wl.r + 2 * dm * p.d
    del ws
    torch.cuda.empty_cache()
    desc = {"no_dq": "NF4 codes + fp32 absmax per 64-block (4.5 bits/weight)",
            "fp8": "NF4 codes + double quantization with c2 in OCP FP8 e4m3 (4.127 bits/weight)"}[fmt]
    return {"format": desc,
            "quantize_us": round(q_ms * 1e3, 2),
            "quantize_gbs": round((d * k * 4 + d * k // 2 + const_bytes) / (q_ms * 1e-3) / 1e9, 1),
            "fwd_bwd_ms": round(fb_ms, 4), "fwd_bwd_tflops": round(flops / (fb_ms * 1e-3) / 1e12, 3),
            f"decode_{p.name}_m{dm}": {"us_per_call": round(dec_us, 3), "algorithmic_bytes": alg,
                                        "algorithmic_gbs": round(alg / (dec_us * 1e-6) / 1e9, 1),
                                        "hbm_frac": round(alg / (dec_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}


def run_dropout_bench(q, torch, ctx, p=0.05, iters=20):
    """Forward + backward of the layer4096 inputs with adapter dropout (rate p,
    as in the pages' training configuration), and qlora_lora_dropout alone."""
    from workloads import workload_layer
    from tests.helpers import to_dev_bf16
    w, x, a, b, alpha, y, u, lws, r = ctx
    inp = workload_layer("layer4096")
    m, d, k = inp.x.shape[0], w.d, w.k
    dy = to_dev_bf16(inp.dy)
    ws = torch.empty(q.linear_workspace_bytes(m, d, k, r, dropout=True), dtype=torch.uint8, device="cuda")
    dx = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    da = torch.empty((r, k), dtype=torch.float32, device="cuda")
    db = torch.empty((d, r), dtype=torch.float32, device="cuda")
    xd = torch.empty_like(x)
    log(f"dropout p={p}: layer4096 fwd+bwd")

    def fwd_bwd():
        q.qlora_linear_fwd(w, x, a, b, alpha, out=y, u_out=u, workspace=ws, dropout=p, seed=1234)
        q.qlora_linear_bwd(w, x, dy, a, b, alpha, u=u, workspace=ws, outs=(dx, da, db), dropout=p, seed=1234)
    fb_ms = time_calls(torch, fwd_bwd, iters)
    drop_ms = time_graph(torch, lambda: q.qlora_lora_dropout(x, p, 1234, out=xd), iters)
    flops = fwd_flops(m, d, k, r) + bwd_flops(m, d, k, r)
    return {"p": p, "fwd_bwd_ms": round(fb_ms, 4), "fwd_bwd_tflops": round(flops / (fb_ms * 1e-3) / 1e12, 3),
            "lora_dropout_us": round(drop_ms * 1e3, 2),
            "lora_dropout_gbs": round(4 * m * k / (drop_ms * 1e-3) / 1e9, 1),
            "workload": f"layer4096, M={m}, r={r}"}


def decode_bytes(m, d, k, r):
    """Algorithmic HBM bytes of one decode forward: packed codes, 8-bit block
    constants, fp32 group constants and mean, x, A, B, Y."""
    nb = d * k // 64
    return d * k // 2 + nb + 4 * ((nb + 255) // 256) + 4 + 2 * m * k + 2 * r * k + 2 * d * r + 2 * m * d


def decode_roofline(decode):
    """The decode forward at M = 16 on the 14336 x 4096 projection: one kernel
    per call, bound by HBM; algorithmic bytes over its event-timed duration."""
    e = decode.get("14336x4096_m16") or next(iter(decode.values()))
    out = {"bound": "hbm", "achieved": e["algorithmic_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(e["algorithmic_gbs"] / HBM_PEAK_GBS, 4),
           "traffic": traffic_from_profiles("nf4_decode_kernel_w14336x4096_m16", "decode.hip"),
           "kernel": "nf4_decode_kernel (decode forward, 14336 x 4096, M = 16)",
           "kernel_us": e["kernel_us"], "graph_us_per_call": e["graph_us_per_call"],
           "work_per_launch": f"{e['algorithmic_bytes']} bytes"}
    e1 = decode.get("14336x4096_m1")
    if e1:  # one token: the dot-product kernel
        out["m1"] = {"kernel": "nf4_decode_dot_kernel (decode forward, 14336 x 4096, M = 1)",
                     "kernel_us": e1["kernel_us"], "graph_us_per_call": e1["graph_us_per_call"],
                     "achieved": e1["algorithmic_gbs"],
                     "frac": round(e1["algorithmic_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles("nf4_decode_dot_kernel_w14336x4096_m1", "decode_dot.hip"),
                     "work_per_launch": f"{e1['algorithmic_bytes']} bytes"}
    return out


def run_gemm_ab(q, torch, reps=20):
    """The two ways of feeding the weights to the layer4096 GEMMs (M = 4096),
    interleaved call by call so that clock drift hits both alike: the calls as
    they run (a bf16 copy of What / What^T written by the preparation launch,
    then the GEMM that streams it) and, right after each call, the same GEMM
    work done by the kernel that expands the NF4 codes tile by tile
    (qlora_linear_gemm_only(expand=True): block scales, then the expanding
    kernel, on the adapter operands the call prepared).  Event-timed per call;
    a kernel trace of this run splits each into its launches."""
    from workloads import WORKLOADS, workload_layer
    from tests.helpers import to_dev_bf16, to_dev_f32
    wl = WORKLOADS["layer4096"]
    m, r, alpha = wl.m[0], wl.r, wl.alpha
    inp = workload_layer("layer4096")
    d, k = inp.w0.shape
    w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
    x, a, b, dy = (to_dev_bf16(t) for t in (inp.x, inp.a, inp.b, inp.dy))
    lws = torch.empty(q.linear_workspace_bytes(m, d, k, r), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, d), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y)
    u = torch.empty((m, r), dtype=torch.float32, device="cuda")
    outs = (torch.empty((m, k), dtype=torch.bfloat16, device="cuda"), torch.empty((r, k), device="cuda"),
            torch.empty((d, r), device="cuda"))
    dx2 = torch.empty_like(outs[0])
    t = {kk: Timer(torch) for kk in ("fwd_call", "fwd_expand", "bwd_call", "dx_expand")}
    same = True
    for it in range(reps + 2):
        timed = it >= 2
        e = t["fwd_call"].start()
        q.qlora_linear_fwd(w, x, a, b, alpha, out=y, u_out=u, workspace=lws)
        t["fwd_call"].stop(e) if timed else None
        e = t["fwd_expand"].start()
        q.qlora_linear_gemm_only(w, False, x, r, y2, lws, expand=True)
        t["fwd_expand"].stop(e) if timed else None
        e = t["bwd_call"].start()
        q.qlora_linear_bwd(w, x, dy, a, b, alpha, u=u, workspace=lws, outs=outs)
        t["bwd_call"].stop(e) if timed else None
        e = t["dx_expand"].start()
        q.qlora_linear_gemm_only(w, True, dy, r, dx2, lws, expand=True)
        t["dx_expand"].stop(e) if timed else None
        same = same and bool(torch.equal(y, y2)) and bool(torch.equal(outs[0], dx2))
    torch.cuda.synchronize()
    res = {kk: round(v.total_ms() / reps, 4) for kk, v in t.items()}
    res.update({"same_bits": same, "reps": reps,
                "workload": f"layer4096: W0 {d}x{k}, M={m}, r={r}; *_call: the whole call (U or G, dA/dB "
                            "for bwd, the bf16 copy, the GEMM); *_expand: block scales + expanding GEMM"})
    return res


def pmc_run(q, torch, which):
    """A short, fixed sequence of launches for rocprofv3 --pmc counter passes:
    a plain device copy of 256 MiB (the calibration of FETCH_SIZE/WRITE_SIZE),
    then three launches of the kernel under study."""
    from workloads import WORKLOADS, workload_layer
    from tests.helpers import to_dev_bf16, to_dev_f32
    n = 256 * 2**20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    if which == "gemm":
        ctx, _ = run_layer_bench(q, torch, 1, 0)
        w, x, a, b, alpha, y, u, lws, r = ctx
        for _ in range(3):
            q.qlora_linear_gemm_only(w, False, x, r, y, lws)
    else:
        wl = WORKLOADS["decode"]
        for pi, p in enumerate(wl.projections):
            inp = workload_layer("decode", pi)
            w = q.qlora_nf4_quantize(to_dev_f32(inp.w0))
            a, b = to_dev_bf16(inp.a), to_dev_bf16(inp.b)
            x = to_dev_bf16(inp.x[:16])
            y = torch.empty((16, p.d), dtype=torch.bfloat16, device="cuda")
            lws = torch.empty(q.linear_workspace_bytes(16, p.d, p.k, wl.r), dtype=torch.uint8, device="cuda")
            for _ in range(3):
                q.qlora_linear_fwd(w, x, a, b, wl.alpha, save_u=False, out=y, workspace=lws)
            if p.d >= 8192:  # one token: the dot-product decode kernel
                x1, y1 = x[:1].contiguous(), y[:1].contiguous()
                for _ in range(3):
                    q.qlora_linear_fwd(w, x1, a, b, wl.alpha, save_u=False, out=y1, workspace=lws)
    torch.cuda.synchronize()
    log(f"pmc run ({which}) done")


def run_cpu_baseline(target_s=15.0):
    """The oracle as it stands, on a bounded sample of the layer4096 step:
    quantize + doubleDequant of the full W0 and fp64 forward + backward for
    the first `ms` tokens; reported as fp64 TFLOP/s of those tokens' flops."""
    import numpy as np
    from oracle import nf4, qlora
    from workloads import WORKLOADS, bf16_bits_as_f32, workload_layer
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = 1
    wl = WORKLOADS["layer4096"]
    p = wl.projections[0]
    inp = workload_layer("layer4096")
    ms = 256
    x = bf16_bits_as_f32(inp.x[:ms])
    dy = bf16_bits_as_f32(inp.dy[:ms])
    a, b = bf16_bits_as_f32(inp.a), bf16_bits_as_f32(inp.b)
    t0 = time.perf_counter()
    reps = 0
    while True:
        qd = nf4.quantize(inp.w0)
        w_hat = nf4.bf16_bits_to_f32(nf4.dequantize(qd, inp.w0.shape))
        qlora.forward(w_hat, x, a, b, wl.alpha)
        qlora.backward(w_hat, x, dy, a, b, wl.alpha)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 50:
            break
    flops = (fwd_flops(ms, p.d, p.k, wl.r) + bwd_flops(ms, p.d, p.k, wl.r)) * reps
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"layer4096 step on the first {ms} of 4096 tokens (oracle quantize + "
                      f"doubleDequant of the full 4096x4096 W0, fp64 fwd+bwd), {reps} reps, "
                      f"{el:.1f} s; numpy/OpenBLAS threads={threads}, "
                      f"host cpus={len(os.sched_getaffinity(0))}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-models", action="store_true")
    ap.add_argument("--pmc-run", choices=["gemm", "decode"],
                    help="only a short fixed launch sequence for rocprofv3 --pmc passes")
    ap.add_argument("--gemm-ab", action="store_true",
                    help="only the A/B of the bf16-copy GEMM path against the expanding kernel at M = 4096")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is a design note only)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_nf4_quantized_13_amd as q
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.pmc_run:
        pmc_run(q, torch, args.pmc_run)
        return
    if args.gemm_ab:
        print(json.dumps({"gemm_ab": run_gemm_ab(q, torch)}), flush=True)
        return

    ctx, lay = run_layer_bench(q, torch, args.steps, args.warmup)
    m, d, k, r = lay["m"], lay["d"], lay["k"], lay["r"]
    # dominant kernel: the forward dequant-GEMM (nf4_gemm_kernel), its average
    # duration inside the timed steps; the same kernel launched alone beside it
    gemm_ms = lay["gemm_fwd_ms"]
    log("layer4096: timing the forward GEMM kernel alone")
    alone_ms = time_gemm_only(q, torch, ctx, max(args.steps, 10))
    gf = gemm_flops(m, d, k, r)
    achieved = gf / (gemm_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_from_profiles("nf4_gemm_kernel_fwd_layer4096", "gemm_nf4.hip"),
                "kernel": "nf4_gemm_kernel<fwd> (layer4096 forward), average inside the timed steps",
                "kernel_us": round(gemm_ms * 1e3, 2),
                "work_per_launch": f"2*M*d*k + 2*M*d*r = {gf} flop",
                "alone_kernel_us": round(alone_ms * 1e3, 2),
                "alone_frac": round(gf / (alone_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "dx_kernel_us": round(lay["gemm_dx_ms"] * 1e3, 2),
                "dx_frac": round((2 * m * d * k + 2 * m * k * r) / (lay["gemm_dx_ms"] * 1e-3) / 1e12
                                 / BF16_PEAK_TFLOPS, 4)}
    roofline["vendor_bf16_gemm_context"] = run_vendor_gemm_context(torch)
    log("layer4096: timing the adapter merge")
    merge = run_merge_bench(q, torch, ctx)
    decode = None if args.skip_decode else run_decode_bench(q, torch)
    formats = None if args.skip_decode else {f: run_format_bench(q, torch, ctx, f) for f in ("no_dq", "fp8")}
    dropout = None if args.skip_decode else run_dropout_bench(q, torch, ctx)
    models = None if args.skip_models else {n: run_model_bench(q, torch, n) for n in ("llama7b", "llama65b")}
    cpu = None
    if not args.skip_cpu_baseline:
        log("cpu baseline: timing the oracle on a bounded sample")
        cpu = run_cpu_baseline()
    line = {
        "metric": METRIC, "value": round(lay["tflops_step"], 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(lay["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "layer4096: W0 4096x4096 NF4 (block 64, DQ block 256), M=4096 "
                               "(batch 4 x seq 1024), r=8, alpha=16; step = quantize + fwd + bwd",
                   "global_batch": 4, "seq_len": 1024, "parallelism": "none (1 GPU)"},
        "fwd_bwd_tflops": round(lay["tflops_fwd_bwd"], 3),
        "phases_ms": {kk: round(v, 4) for kk, v in lay["phases"].items()},
        "quantize_gbs": round(lay["quantize_gbs"], 1),
        "roofline": roofline,
        "decode_fwd": decode,
        "decode_roofline": None if decode is None else decode_roofline(decode),
        "adapter_merge": merge,
        "other_formats": formats,
        "adapter_dropout": dropout,
        "model_layers": models,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
