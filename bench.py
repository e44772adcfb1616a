#!/usr/bin/env python3
"""Benchmark of one pass of the windowed joint-attention layer on one MI355X.

A step is one pass of the whole hot path over the 1080p-shaped workload
(T=21, H=68, W=120 latent grid, 171360 video tokens; windows from
nt,nh,nw = 4,3,3; 20 heads x 128; 256 text tokens; bf16): q, k, v in
canonical token order enter the regular-layout window attention + text mean,
then the shifted-layout window attention + text mean, and the video output
leaves in canonical order.  The headline step runs the layout permutations
inside the attention kernels (canonical-order I/O: each layer reads its
layout's rows through the plan's ids table and scatters its output back);
the same pass with explicit relayout kernels (entry relayout of q, k, v,
relayout between the layers, exit relayout of the output) is timed beside it
and reported as `explicit_pass`, with the relayout's HBM rate.  Both give
bit-identical outputs.
Inputs are synthetic (seeded normal samples, N(0,1)/sqrt(128)) and resident in
HBM before the timed region.  The JSON line reports window-attention TFLOP/s
over the whole step, video tokens/s/layer, the roofline of the attention
kernel and the CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import wsp_inputs as I  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
METRIC = "window-attn TFLOP/s + video tokens/s/layer at 1080p grid; % MFMA peak"

# HBM bytes per attention launch from rocprofv3 FETCH_SIZE / WRITE_SIZE passes over this
# benchmark, scaled by what the same counters read for a plain 2 GiB device copy
# (FETCH_SIZE x2.0, WRITE_SIZE x1.0); the committed summary under profiles/ holds the
# figures and commands.  Keyed by the sha256 prefix of the attention kernel source the
# counters were taken on: any later change to the kernel reports null.
# QK^T at the fp8 rate and PV at the bf16 rate, equal FLOPs each.
MIXED_FP8_PEAK_TFLOPS = 1.0 / (0.5 / 5000.0 + 0.5 / 2500.0)
MEASURED_TRAFFIC = {"50aefd175428a106": {"1080p_bf16": {"layout": 4.6333e9, "canonical": 4.9037e9}}}
ATTN_SRCS = [os.path.join(ROOT, "video_dit_window_amd", "csrc", f)
             for f in ("attn_bf16.hip", "attn_bf16_common.h")]


def attn_source_hash():
    return hashlib.sha256(b"".join(open(f, "rb").read() for f in ATTN_SRCS)).hexdigest()[:16]


def measured_traffic(workload, io):
    """HBM bytes per launch for io = "canonical" or "layout" I/O, or None."""
    return MEASURED_TRAFFIC.get(attn_source_hash(), {}).get(workload, {}).get(io)


def attn_flops(lengths, heads, head_dim, text_len):
    """Algorithmic FLOPs: QK^T and PV of every video and text query,
    4 * D * H * sum_w (L_w + Lt)^2."""
    L = np.asarray(lengths, dtype=np.int64) + text_len
    return 4 * head_dim * heads * int((L * L).sum())


def cpu_baseline(w, budget_s):
    """The oracle, as it stands, on the host cores: its joint_attention in
    float32 (numpy BLAS), one (window, head) pair per host thread (one BLAS
    thread each), over the regular layer of the workload, largest windows
    first.  The whole layer runs unless the time budget ends first; the
    result is FLOPs done / wall time either way, and the sample says which."""
    import oracle as O
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    op = O.plan(*geo, O.REGULAR)
    inp = I.qkv(w, bits_only=True)
    f32 = {n: I.bf16_bits_to_f32(b) for n, (_, b) in inp.items()}      # canonical order
    del inp
    threads = min(os.cpu_count() or 1, 64)
    pairs = [(int(win), h) for win in op.lpt for h in range(w.heads)]
    deadline = [None]

    def one(pair):
        win, h = pair
        if time.perf_counter() > deadline[0]:
            return 0
        ids = op.ids[op.offsets[win]:op.offsets[win + 1]]
        O.joint_attention(f32["q"][ids, h], f32["k"][ids, h], f32["v"][ids, h], f32["txt_q"][:, h],
                          f32["txt_k"][:, h], f32["txt_v"][:, h], dtype=np.float32)
        return 4 * w.head_dim * (len(ids) + w.text_len) ** 2

    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        deadline[0] = t0 + budget_s
        done = list(ex.map(one, pairs))
        el = time.perf_counter() - t0
    flops, n_done = sum(done), sum(1 for d in done if d)
    total = attn_flops(np.diff(op.offsets), w.heads, w.head_dim, w.text_len)
    full = n_done == len(pairs)
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"the whole {w.name} regular layer ({len(pairs)} (window, head) pairs, "
                       f"{total:.4e} FLOP) in {el:.1f} s" if full else
                       f"{n_done} of {len(pairs)} (window, head) pairs of the {w.name} regular layer, "
                       f"largest windows first, in {el:.1f} s (whole layer extrapolated: "
                       f"{total / (flops / el):.1f} s)")
                      + f"; float32 numpy oracle, one pair per host thread",
            "layer_seconds": round(el if full else total / (flops / el), 2),
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def stack_measure(w, n_layers, attn_flops_per_layer, reps=2):
    """The multi-layer stack workload on the same grid: per layer q/k/v and
    output projections (wsp_linear) and window attention with canonical-order
    I/O, layers alternating regular / shifted.  Synthetic inputs from torch's
    seeded device generator: hidden state N(0,1), weights N(0, 0.02)."""
    import torch
    import video_dit_window_amd as W
    from video_dit_window_amd.stack import Stack
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    N, Lt, E = w.n_tokens, w.text_len, w.heads * w.head_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    bf = torch.bfloat16
    xv = torch.randn((N, E), device="cuda", generator=g).to(bf)
    xt = torch.randn((Lt, E), device="cuda", generator=g).to(bf)
    wts = [tuple((torch.randn((E, E), device="cuda", generator=g) * 0.02).to(bf) for _ in range(4))
           for _ in range(n_layers)]
    st = Stack(*geo, n_layers, w.heads, w.head_dim, Lt, canonical_io=True)
    ov, ot = torch.empty_like(xv), torch.empty_like(xt)
    stream = torch.cuda.current_stream()
    # one projection launch on the stack's own buffers, timed alone; beside
    # it the q / k projection with the window-local rotation in its epilogue
    # (wsp_linear_rope: canonical rows, layer 0's layout), plain - rotated -
    # plain so that both see the same minutes of the box
    plain = lambda: W.linear(st.X[0], wts[0][0], out=st.q)
    rot = lambda: W.linear_rope(st.X[0], wts[0][0], st.canon, st.layout(0), Lt, out=st.q)
    for _ in range(3):
        plain()
        rot()
    marks = []
    for fn in (plain, rot, plain):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(10):
            fn()
        b.record(stream)
        marks.append((a, b))
    # the same passes with rotated q / k (the q and k projections rotate as
    # they store; attention unchanged), alternating with the plain passes
    st_r = Stack(*geo, n_layers, w.heads, w.head_dim, Lt, canonical_io=True, rope_theta=10000.0)
    st.forward(xv, xt, wts, out_vid=ov, out_txt=ot)      # warm-up passes
    st_r.forward(xv, xt, wts, out_vid=ov, out_txt=ot)
    torch.cuda.synchronize()
    lin_ms = (marks[0][0].elapsed_time(marks[0][1]) + marks[2][0].elapsed_time(marks[2][1])) / 20
    lin_rope_ms = marks[1][0].elapsed_time(marks[1][1]) / 10
    lin_flops = 2 * (N + Lt) * E * E
    passes = {"plain": [], "rope": []}
    for _ in range(reps):
        for name, s_ in (("plain", st), ("rope", st_r)):
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            s_.forward(xv, xt, wts, out_vid=ov, out_txt=ot)
            s1.record(stream)
            passes[name].append((s0, s1))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in passes["plain"]]))
    ms_rope = float(np.mean([a.elapsed_time(b) for a, b in passes["rope"]]))
    layer_flops = 4 * lin_flops + attn_flops_per_layer
    return {"note": f"{n_layers}-layer stack: q/k/v/out projections (wsp_linear) + window attention + "
                    "regular/shifted alternating; the stream stays in canonical order and each layer's attention reads "
                    "and writes through its layout's ids table",
            "layers": n_layers, "hidden": E, "ms_per_pass": round(ms, 3),
            "ms_per_layer": round(ms / n_layers, 4),
            "video_tokens_per_s_per_layer": round(n_layers * N / (ms * 1e-3), 1),
            "tflops_per_pass": round(n_layers * layer_flops / (ms * 1e-3) / 1e12, 2),
            "linear_avg_ms": round(lin_ms, 4),
            "linear_kernel_tflops": round(lin_flops / (lin_ms * 1e-3) / 1e12, 2),
            "linear_rope_avg_ms": round(lin_rope_ms, 4),
            "rope_ms_per_pass": round(ms_rope, 3), "rope_ms_per_layer": round(ms_rope / n_layers, 4),
            "flop_per_layer": {"projections": 4 * lin_flops, "attention": attn_flops_per_layer}}


def config_launches(names, warmup=3, reps=10):
    """The other workload grids on the same kernel and launch (canonical-order
    I/O): the 720p-shaped regular layer and the 4K-shaped shifted layer
    (inputs N(0,1)/sqrt(128) from torch's seeded device generator, rounded
    to bf16).  Per grid: average launch time by HIP events on the launch
    stream (attention kernel + text-mean combine of one call), TFLOP/s,
    fraction of the bf16 MFMA peak and video tokens/s/layer."""
    import torch
    import video_dit_window_amd as W
    stream = torch.cuda.current_stream()
    res = {}
    for name, method in names:
        w = I.WORKLOADS[name]
        geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
        p = W.Plan(*geo, W.REGULAR if method == "regular" else W.SHIFTED)
        g = torch.Generator(device="cuda")
        g.manual_seed(w.index)

        def rnd(rows):
            t = torch.empty((rows, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
            for lo in range(0, rows, 1 << 16):   # bounded float32 temporaries
                hi = min(rows, lo + (1 << 16))
                t[lo:hi] = (torch.randn((hi - lo, w.heads, w.head_dim), device="cuda", generator=g)
                            * w.std).to(torch.bfloat16)
            return t
        q, k, v = (rnd(w.n_tokens) for _ in range(3))
        tq, tk, tv = (rnd(w.text_len) for _ in range(3))
        out, txt = torch.empty_like(q), torch.empty_like(tq)
        ws = torch.empty(max(W.window_attn_workspace(p, w.heads, w.head_dim, w.text_len, W.BF16, per_window=True), 16),
                         dtype=torch.uint8, device="cuda")
        call = lambda: W.window_attn(p, q, k, v, tq, tk, tv, out=out, txt_out=txt, workspace=ws, canonical=True)
        r = max(2, reps if w.n_tokens < 500000 else reps // 2)
        for _ in range(warmup):
            call()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(r):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / r
        flops = attn_flops(np.diff(p.tables()["offsets"]), w.heads, w.head_dim, w.text_len)
        tf = flops / (ms * 1e-3) / 1e12
        res[f"{name}_{method}"] = {
            "grid_thw": [w.T, w.H, w.W], "windows": p.n_windows, "text_len": w.text_len,
            "avg_launch_ms": round(ms, 4), "flop_per_launch": flops, "attn_kernel_tflops": round(tf, 2),
            "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "video_tokens_per_s_per_layer": round(w.n_tokens / (ms * 1e-3), 1), "launches": r}
        del q, k, v, out, ws
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="1080p_bf16", choices=["720p_bf16", "1080p_bf16", "4k_bf16"])
    ap.add_argument("--cpu-budget", type=float, default=40.0,
                    help="seconds of oracle timing at most (the whole regular layer if it fits)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fused", action="store_true",
                    help="headline = the pass with explicit relayout kernels (skip the fused pass)")
    ap.add_argument("--stack-layers", type=int, default=32,
                    help="layers of the multi-layer stack side measurement")
    ap.add_argument("--no-stack", action="store_true", help="skip the multi-layer stack side measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 720p regular / 4K shifted attention launches")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (a known-size "
                         "reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (got --gpus {args.gpus}); "
              "the multi-GPU window-parallel path is not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import video_dit_window_amd as W

    w = I.WORKLOADS[args.workload]
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    layouts = [W.REGULAR if m == "regular" else W.SHIFTED for m in w.layouts]
    plans = [W.Plan(*geo, m) for m in layouts]
    canon = W.canonical(w.T, w.H, w.W)
    inp = I.qkv(w, bits_only=True)
    dev = {n: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda() for n, (_, b) in inp.items()}
    del inp
    N, Hh, D, Lt = w.n_tokens, w.heads, w.head_dim, w.text_len
    bufs = {n: torch.empty_like(dev["q"]) for n in ("q", "k", "v")}
    outs = [torch.empty_like(dev["q"]) for _ in plans]
    out_c = torch.empty_like(dev["q"])
    txts = [torch.empty_like(dev["txt_q"]) for _ in plans]
    # one text partial per window (the faster text reduction); the minimum
    # workspace (16 chunks of windows) is timed beside it as `text_chunked`
    ws_bytes = max(W.window_attn_workspace(p, Hh, D, Lt, W.BF16, per_window=True) for p in plans)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    ws_min_bytes = max(W.window_attn_workspace(p, Hh, D, Lt, W.BF16) for p in plans)
    ws_min = torch.empty(max(ws_min_bytes, 16), dtype=torch.uint8, device="cuda")
    flops = [attn_flops(np.diff(p.tables()["offsets"]), Hh, D, Lt) for p in plans]
    row_bytes = Hh * D * 2
    stream = torch.cuda.current_stream()

    ev = {"attn": [], "relayout": [], "fused_attn": [], "rope": [], "qk8_attn": [], "chunked_attn": [],
          "rope_attn": [], "rope_chain": [], "plain_near": []}

    def timed(kind, fn, record):
        if record:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev[kind].append((a, b))
        else:
            fn()

    # q,k,v of consecutive layouts need distinct source/destination buffers.
    bufs2 = {n: torch.empty_like(dev["q"]) for n in ("q", "k", "v")}

    def step(record):
        src, cur = canon, {"q": dev["q"], "k": dev["k"], "v": dev["v"]}
        for li, p in enumerate(plans):
            dst = bufs if li % 2 == 0 else bufs2
            for n in ("q", "k", "v"):
                timed("relayout", lambda n=n, dst=dst, src=src, p=p: W.relayout(cur[n], src, p, out=dst[n]), record)
            cur, src = {n: dst[n] for n in ("q", "k", "v")}, p
            timed("attn", lambda li=li, p=p, cur=cur: W.window_attn(
                p, cur["q"], cur["k"], cur["v"], dev["txt_q"], dev["txt_k"], dev["txt_v"],
                out=outs[li], txt_out=txts[li], workspace=ws), record)
        timed("relayout", lambda: W.relayout(outs[-1], plans[-1], canon, out=out_c), record)

    def step_fused(record):
        # The same pass with the layout permutations fused into the attention
        # kernels: q, k, v and outputs stay in canonical order (wsp_window_attn_ex).
        for li, p in enumerate(plans):
            timed("fused_attn", lambda li=li, p=p: W.window_attn(
                p, dev["q"], dev["k"], dev["v"], dev["txt_q"], dev["txt_k"], dev["txt_v"],
                out=outs[li], txt_out=txts[li], workspace=ws, canonical=True), record)

    def step_rope(record):
        # Window-local RoPE of q and k fused with the entry move (canonical ->
        # each layer's layout, that layout's positions).
        for li, p in enumerate(plans):
            dst = bufs if li % 2 == 0 else bufs2
            for n in ("q", "k"):
                timed("rope", lambda n=n, p=p, dst=dst: W.rope_relayout(dev[n], canon, p, p, Lt, out=dst[n]),
                      record)

    # E4M3 q / k codes (per-head scales), moved into each layout once, outside the timing.
    amax_q, amax_k = W.fp8_amax(dev["q"], dev["txt_q"]), W.fp8_amax(dev["k"], dev["txt_k"])
    tq8, tk8 = W.fp8_quantize(dev["txt_q"], amax_q), W.fp8_quantize(dev["txt_k"], amax_k)
    q8c, k8c = W.fp8_quantize(dev["q"], amax_q), W.fp8_quantize(dev["k"], amax_k)
    codes = [(W.relayout(q8c, canon, p), W.relayout(k8c, canon, p)) for p in plans]
    del q8c, k8c

    def step_qk8(record):
        # The two layers on the FP8 q/k path (v, softmax and outputs bf16).
        for li, p in enumerate(plans):
            vv = bufs["v"] if li % 2 == 0 else bufs2["v"]
            timed("qk8_attn", lambda li=li, p=p, vv=vv: W.window_attn_qk8(
                p, codes[li][0], codes[li][1], vv, tq8, tk8, dev["txt_v"], amax_q, amax_k,
                out=outs[li], txt_out=txts[li], workspace=ws), record)

    def run(fn):
        for _ in range(args.warmup):
            fn(False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            fn(True)
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps, time.perf_counter() - t0

    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ms_step, wall = run(step)
    ms_fused, wall_f = (None, None) if args.no_fused else run(step_fused)
    run(step_rope)
    run(step_qk8)
    attn_ms = [a.elapsed_time(b) for a, b in ev["attn"]]
    rel_ms = [a.elapsed_time(b) for a, b in ev["relayout"]]
    step_flops = sum(flops)
    # dominant kernel: window attention (per call = attention kernel + text mean)
    per_call_flops = step_flops / len(plans)
    attn_avg_ms = float(np.mean(attn_ms))
    rel_bytes = 2 * N * row_bytes + 4 * N
    rel_avg_ms = float(np.mean(rel_ms))
    rel_gbps = rel_bytes / (rel_avg_ms * 1e-3) / 1e9
    explicit = {
        "note": "same pass with explicit relayout kernels (entry relayout of q,k,v, relayout between the "
                "layers, exit relayout of the output) and layout-order attention I/O",
        "ms_per_step": round(ms_step, 4),
        "attn_tflops_per_step": round(step_flops / (ms_step * 1e-3) / 1e12, 3),
        "attn_kernel_tflops": round(per_call_flops / (attn_avg_ms * 1e-3) / 1e12, 2),
        "avg_launch_ms": round(attn_avg_ms, 4),
        "breakdown_ms_per_step": {"attention+text_mean": round(sum(attn_ms) / args.steps, 4),
                                  "relayout": round(sum(rel_ms) / args.steps, 4)},
        "traffic_bytes_per_launch": measured_traffic(w.name, "layout")}
    if ms_fused is not None:
        f_ms = [a.elapsed_time(b) for a, b in ev["fused_attn"]]
        head_ms, head_avg, io = ms_fused, float(np.mean(f_ms)), "canonical"
        kernel = "attn_bf16_kernel<128, 8, true> (canonical-order I/O, resident work groups taking items from per-XCD queues; + " \
                 "text_mean_kernel in the same call)"
        breakdown = {"attention+text_mean": round(sum(f_ms) / args.steps, 4)}
    else:
        head_ms, head_avg, io = ms_step, attn_avg_ms, "layout"
        kernel = "attn_bf16_kernel<128, 8, false> (resident work groups taking items from per-XCD queues; + text_mean_kernel in the same call)"
        breakdown = explicit["breakdown_ms_per_step"]
    value = step_flops / (head_ms * 1e-3) / 1e12
    attn_tflops = per_call_flops / (head_avg * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "grid_thw": [w.T, w.H, w.W], "n_thw": [w.nt, w.nh, w.nw],
                   "video_tokens": N, "heads": Hh, "head_dim": D, "text_len": Lt,
                   "layers": list(w.layouts), "windows": [p.n_windows for p in plans],
                   "io": "canonical order, layout permutations inside the attention kernels"
                         if io == "canonical" else "explicit relayout kernels"},
        "video_tokens_per_s_per_layer": round(N / (head_avg * 1e-3), 1),
        "attn_kernel_tflops": round(attn_tflops, 2),
        "attn_mfma_frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "relayout_gbps": round(rel_gbps, 1),
        "relayout_hbm_frac": round(rel_gbps / HBM_PEAK_GBPS, 4),
        "breakdown_ms_per_step": breakdown,
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(w.name, io), "traffic_unit": "B/launch",
                     "kernel": kernel, "flop_per_launch": per_call_flops, "avg_launch_ms": round(head_avg, 4)},
        "wall_s_timed": round(wall if ms_fused is None else wall_f, 3),
    }
    if ms_fused is not None:
        res["explicit_pass"] = explicit
    if ms_fused is not None:
        # Dispatch-order A/B on the headline pass: window-id order, largest
        # first, largest first with (window, head) groups kept on one XCD.
        orders = {}
        for name, o in (("window_id", W.ORDER_ID), ("lpt", W.ORDER_LPT), ("lpt_xcd", W.ORDER_LPT_XCD)):
            W.set_attn_order(o)
            orders[name] = round(run(step_fused)[0], 4)
        W.set_attn_order(W.ORDER_LPT_XCD)
        res["dispatch_order_ms_per_step"] = orders
        # The same pass with the minimum workspace: the text mean from 16
        # chunks of windows (text items over whole chunks) instead of one
        # partial per window.
        def step_chunked(record):
            for li, p in enumerate(plans):
                timed("chunked_attn", lambda li=li, p=p: W.window_attn(
                    p, dev["q"], dev["k"], dev["v"], dev["txt_q"], dev["txt_k"], dev["txt_v"],
                    out=outs[li], txt_out=txts[li], workspace=ws_min, canonical=True), record)
        ms_ch = run(step_chunked)[0]
        ch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["chunked_attn"]]))
        res["text_chunked"] = {
            "note": "headline pass with the minimum workspace (text mean from min(windows, 16) chunk sums)",
            "workspace_bytes": ws_min_bytes, "headline_workspace_bytes": ws_bytes,
            "ms_per_step": round(ms_ch, 4), "avg_launch_ms": round(ch_ms, 4),
            "attn_kernel_tflops": round(per_call_flops / (ch_ms * 1e-3) / 1e12, 2)}
        # The headline pass with window-local RoPE of q and k: queries rotated
        # inside the attention kernel, keys and text rows by the stand-alone
        # rotation kernel (wsp_window_attn_rope); beside it the unfused chain
        # (rotation of q, k and text rows, then the plain launch).
        ws_rope = torch.empty(max(W.window_attn_rope_workspace(p, Hh, Lt) for p in plans), dtype=torch.uint8,
                              device="cuda")
        rtq, rtk = torch.empty_like(dev["txt_q"]), torch.empty_like(dev["txt_k"])

        def step_rope_attn(record):
            for li, p in enumerate(plans):
                timed("rope_attn", lambda li=li, p=p: W.window_attn_rope(
                    p, dev["q"], dev["k"], dev["v"], dev["txt_q"], dev["txt_k"], dev["txt_v"],
                    out=outs[li], txt_out=txts[li], workspace=ws_rope, canonical=True), record)

        def step_rope_chain(record):
            for li, p in enumerate(plans):
                def chain(li=li, p=p):
                    W.rope_relayout(dev["q"], canon, canon, p, Lt, out=bufs["q"])
                    W.rope_relayout(dev["k"], canon, canon, p, Lt, out=bufs["k"])
                    W.rope_text(dev["txt_q"], out=rtq)
                    W.rope_text(dev["txt_k"], out=rtk)
                    W.window_attn(p, bufs["q"], bufs["k"], dev["v"], rtq, rtk, dev["txt_v"], out=outs[li],
                                  txt_out=txts[li], workspace=ws, canonical=True)
                timed("rope_chain", chain, record)
        def step_plain_near(record):
            for li, p in enumerate(plans):
                timed("plain_near", lambda li=li, p=p: W.window_attn(
                    p, dev["q"], dev["k"], dev["v"], dev["txt_q"], dev["txt_k"], dev["txt_v"],
                    out=outs[li], txt_out=txts[li], workspace=ws, canonical=True), record)
        # the plain launch timed right before and after, so that the ratios
        # compare launches of the same minutes on the box
        run(step_plain_near)
        ms_ra = run(step_rope_attn)[0]
        ms_rc = run(step_rope_chain)[0]
        run(step_plain_near)
        del ws_rope
        head_launch = float(np.mean([a.elapsed_time(b) for a, b in ev["plain_near"]]))
        ra_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["rope_attn"]]))
        rc_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["rope_chain"]]))
        res["rope_attention"] = {
            "note": "headline pass with window-local RoPE of q and k: queries rotated inside the attention "
                    "kernel, keys and text rows by the rotation kernel (wsp_window_attn_rope); 'chain' = "
                    "rotation of q, k and text rows by the rotation kernel, then the plain launch; ratios against "
                    "the plain launch timed just before and after",
            "ms_per_step": round(ms_ra, 4), "avg_layer_ms": round(ra_ms, 4),
            "plain_layer_ms": round(head_launch, 4),
            "ratio_vs_plain_layer": round(ra_ms / head_launch, 4),
            "chain_ms_per_step": round(ms_rc, 4), "chain_avg_layer_ms": round(rc_ms, 4),
            "chain_ratio_vs_plain_layer": round(rc_ms / head_launch, 4)}
    rope_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["rope"]]))
    rope_bytes = 2 * N * row_bytes + 12 * N   # rows in + out, perm + id + position per row
    res["rope_relayout"] = {"note": "q or k moved canonical -> layout with window-local 3D RoPE",
                            "avg_launch_ms": round(rope_ms, 4),
                            "gbps": round(rope_bytes / (rope_ms * 1e-3) / 1e9, 1),
                            "hbm_frac": round(rope_bytes / (rope_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    q8_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["qk8_attn"]]))
    q8_tflops = per_call_flops / (q8_ms * 1e-3) / 1e12
    res["fp8_qk_attention"] = {
        "note": "q, k as OCP E4M3 codes (per-head scales) on the FP8 matrix cores; v, P, outputs bf16. "
                "Roofline: half the FLOPs (QK^T) at the fp8 peak, half (PV) at the bf16 peak",
        "avg_launch_ms": round(q8_ms, 4),
        "attn_kernel_tflops": round(q8_tflops, 2),
        "mixed_peak_tflops": round(MIXED_FP8_PEAK_TFLOPS, 1),
        "frac": round(q8_tflops / MIXED_FP8_PEAK_TFLOPS, 4)}
    if not args.no_configs:
        res["configs"] = config_launches([("720p_bf16", "regular"), ("4k_bf16", "shifted")])
    if not args.no_stack:
        res["stack"] = stack_measure(w, args.stack_layers, per_call_flops)
        if "rope_attention" in res:
            # RoPE where the real block has it: the q and k projections rotate
            # as they store (wsp_linear_rope) and attention runs unchanged, so
            # the layer's extra cost is what the two rotating epilogues add
            sm, ra = res["stack"], res["rope_attention"]
            extra = 2.0 * (sm["linear_rope_avg_ms"] - sm["linear_avg_ms"])
            ra["fused_projection"] = {
                "note": "q / k rotated in the epilogue of their projections (wsp_linear_rope), plain attention "
                        "launch: extra ms per layer = 2 x (rotating - plain projection launch); ratio = (plain "
                        "attention launch + extra) / plain attention launch; per layer of the stack passes too",
                "qk_projection_extra_ms": round(extra, 4),
                "ratio_vs_plain_layer": round((ra["plain_layer_ms"] + extra) / ra["plain_layer_ms"], 4),
                "stack_layer_extra_ms": round(sm["rope_ms_per_layer"] - sm["ms_per_layer"], 4)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
