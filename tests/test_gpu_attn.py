"""GPU parity of wsp_window_attn against the CPU oracle.

Small and mid-size grids are compared element by element in full (they span
many 128-row query tiles and 64-key tiles, with ragged tails, tiny edge
windows, D = 64 and 128, text lengths 0, 1 and odd).  The full-size 720p
regular and 1080p regular and shifted layers (canonical-order I/O, the
benchmark's launch) are compared element by element over every window and
head, and on the complete text mean; the 720p shifted, 1080p layout-order and
4K layers on sampled (window, head) pairs and the complete text mean of one
head.
"""
import numpy as np
import pytest

import oracle as O
import video_dit_window_amd as W
import wsp_inputs as I
from helpers import BF16_ATOL, BF16_REL_L2, BF16_RTOL, check_bf16, check_f32, dev_bits, from_dev, log, to_dev

pytestmark = pytest.mark.gpu
METH = {"regular": (O.REGULAR, W.REGULAR), "shifted": (O.SHIFTED, W.SHIFTED)}


def upload(inp, dtype):
    return {k: to_dev(v, b, dtype) for k, (v, b) in inp.items()}


def host_f64(inp, name):
    v, b = inp[name]
    return (v if v is not None else I.bf16_bits_to_f32(b)).astype(np.float64)


def run_full(w, method, dtype_check, order=None, scale=None, per_window=True):
    """Whole-grid comparison for a small workload: canonical inputs are
    relayouted to the method's layout on the GPU, attended, and compared with
    the oracle over every output element.  per_window=False runs the text
    mean from min(windows, 16) chunk sums (the minimum workspace)."""
    import torch
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    om, wm = METH[method]
    op, wp = O.plan(*geo, om), W.Plan(*geo, wm)
    oc, wc = O.canonical_plan(*geo[:3]), W.canonical(*geo[:3])
    inp = I.qkv(w)
    d = upload(inp, w.dtype)
    q, k, v = (W.relayout(d[n], wc, wp) for n in ("q", "k", "v"))
    if order is not None:
        W.set_attn_order(order)
    try:
        out, txt = W.window_attn(wp, q, k, v, d["txt_q"], d["txt_k"], d["txt_v"], scale=scale,
                                 per_window=per_window)
    finally:
        W.set_attn_order(W.ORDER_LPT_XCD)
    out_c = W.relayout(out, wp, wc)
    torch.cuda.synchronize()
    h = {n: host_f64(inp, n) for n in I.QKV_NAMES}
    ref_out, ref_txt = O.window_attn(op, *(O.relayout(h[n], oc, op) for n in ("q", "k", "v")),
                                     h["txt_q"], h["txt_k"], h["txt_v"], scale=scale)
    dtype_check(from_dev(out), ref_out, f"{w.name} {method} video")
    dtype_check(from_dev(out_c), O.relayout(ref_out, op, oc), f"{w.name} {method} video (canonical)")
    if w.text_len:
        dtype_check(from_dev(txt), ref_txt, f"{w.name} {method} text mean")
    return out, txt


# ------------------------------------------------------------------ float32
@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_tiny_f32_workload(gpu, method):
    """The tiny float32 workload: 5x20x36 grid, 2x2x2 ragged windows, 4 heads
    x 64, 16 text tokens, max |err| <= 1e-5 against the float64 oracle."""
    run_full(I.WORKLOADS["tiny_f32"], method, check_f32)


def test_tiny_f32_layer_pair_flow(gpu):
    """Canonical -> regular layer -> relayout q,k,v -> shifted layer -> outputs
    back to canonical order, as one pass of the tiny workload."""
    import torch
    w = I.WORKLOADS["tiny_f32"]
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    oc, orr, osh = O.canonical_plan(*geo[:3]), O.plan(*geo, O.REGULAR), O.plan(*geo, O.SHIFTED)
    wc, wr, ws = W.canonical(*geo[:3]), W.Plan(*geo, W.REGULAR), W.Plan(*geo, W.SHIFTED)
    inp = I.qkv(w)
    d = upload(inp, "f32")
    qr, kr, vr = (W.relayout(d[n], wc, wr) for n in "qkv")
    out_r, txt_r = W.window_attn(wr, qr, kr, vr, d["txt_q"], d["txt_k"], d["txt_v"])
    qs, ks, vs = (W.relayout(t, wr, ws) for t in (qr, kr, vr))
    out_s, txt_s = W.window_attn(ws, qs, ks, vs, d["txt_q"], d["txt_k"], d["txt_v"])
    out_s_c = W.relayout(out_s, ws, wc)
    torch.cuda.synchronize()
    h = {n: host_f64(inp, n) for n in I.QKV_NAMES}
    t = (h["txt_q"], h["txt_k"], h["txt_v"])
    ref_r, ref_tr = O.window_attn(orr, *(O.relayout(h[n], oc, orr) for n in "qkv"), *t)
    ref_s, ref_ts = O.window_attn(osh, *(O.relayout(h[n], oc, osh) for n in "qkv"), *t)
    check_f32(from_dev(out_r), ref_r, "regular video")
    check_f32(from_dev(txt_r), ref_tr, "regular text")
    check_f32(from_dev(out_s_c), O.relayout(ref_s, osh, oc), "shifted video (canonical)")
    check_f32(from_dev(txt_s), ref_ts, "shifted text")


@pytest.mark.parametrize("D", [64, 128])
def test_mid_f32(gpu, D):
    w = I.custom("mid_f32", 6, 30, 52, 2, 3, 3, 2, D, 37, "f32", index=201)
    run_full(w, "shifted", check_f32)


# ------------------------------------------------------------------ bfloat16
# bf16 work distributions (same per-wavefront arithmetic in each)
SCHEDS = {"per_item": W.SCHED_PER_ITEM, "per_item_128": W.SCHED_PER_ITEM_128,
          "queue": W.SCHED_QUEUE, "queue_128": W.SCHED_QUEUE_128}

MID = [  # (name, T, H, W, nt, nh, nw, heads, D, Lt)
    ("mid_bf16", 6, 30, 52, 2, 3, 3, 3, 128, 40),
    ("mid_bf16_d64", 6, 30, 52, 2, 3, 3, 3, 64, 40),
    ("mid_bf16_notext", 6, 30, 52, 2, 3, 3, 2, 128, 0),
    ("mid_bf16_text1", 6, 30, 52, 2, 3, 3, 2, 128, 1),
    ("small_windows_bf16", 5, 24, 40, 3, 9, 12, 2, 128, 19),
    ("one_window_bf16", 3, 12, 20, 1, 1, 1, 2, 128, 77),
    # windows of at most 45 tokens: a joint sequence of one 64-key tile
    ("tiny_windows_bf16", 4, 20, 36, 4, 9, 9, 2, 128, 0),
    ("tiny_windows_text_d64", 4, 20, 36, 4, 9, 9, 2, 64, 19),
    # 300 text rows: more than one query tile of text (joint tiles whose text
    # rows span several tiles with one partial per window; multi-tile text
    # items over chunks of windows otherwise)
    ("long_text_bf16", 6, 30, 52, 2, 3, 3, 2, 128, 300),
]


@pytest.mark.parametrize("case", MID, ids=[c[0] for c in MID])
@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_mid_bf16(gpu, case, method):
    w = I.custom(*case, "bf16", index=300 + MID.index(case))
    run_full(w, method, check_bf16)


@pytest.mark.parametrize("case", MID, ids=[c[0] for c in MID])
@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_mid_bf16_chunked_text(gpu, case, method):
    """The minimum workspace: text items over chunks of consecutive windows
    (16 chunks, or one per window when there are fewer)."""
    w = I.custom(*case, "bf16", index=300 + MID.index(case))
    run_full(w, method, check_bf16, per_window=False)


@pytest.mark.parametrize("D", [64, 128])
def test_mid_f32_chunked_text(gpu, D):
    w = I.custom("mid_f32", 6, 30, 52, 2, 3, 3, 2, D, 37, "f32", index=201)
    run_full(w, "regular", check_f32, per_window=False)


def test_bf16_unscaled_inputs(gpu):
    """N(0,1) inputs give logits of standard deviation ~1 (the default
    N(0,1)/sqrt(D) inputs give ~0.008, a nearly uniform softmax), which
    stresses the running max and the exponentials."""
    w = I.custom("mid_unscaled", 6, 30, 52, 2, 3, 3, 2, 128, 40, "bf16", std=1.0, index=320)
    run_full(w, "regular", check_bf16)


@pytest.mark.parametrize("std", [4.0, 8.0])
@pytest.mark.parametrize("sched", ["per_item", "per_item_128", "queue", "queue_128"])
def test_bf16_large_scores(gpu, std, sched):
    """q, k, v of standard deviation 4 or 8: logits of standard deviation
    ~16 or ~64 (nearly one-hot softmax with near-tied keys in some rows).
    A work item's first tile overflows float32 before its maximum is known
    (std 8), and later tiles raise the maximum often (the exact path of the
    lazy online softmax).  Every schedule, element by element against the
    oracle; canonical-order I/O gives the same bits."""
    import torch
    w = I.custom(f"mid_large_{int(std)}", 6, 30, 52, 2, 3, 3, 2, 128, 40, "bf16", std=std,
                 index=340 + int(std))
    W.set_attn_schedule(SCHEDS[sched])
    try:
        out, txt = run_full(w, "shifted", check_bf16)
        geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
        wp, wc = W.Plan(*geo, W.SHIFTED), W.canonical(*geo[:3])
        d = upload(I.qkv(w), "bf16")
        oc, tc = W.window_attn(wp, d["q"], d["k"], d["v"], d["txt_q"], d["txt_k"], d["txt_v"],
                               canonical=True)
    finally:
        W.set_attn_schedule(W.SCHED_AUTO)
    torch.cuda.synchronize()
    assert torch.equal(oc.view(torch.int16), W.relayout(out, wp, wc).view(torch.int16))
    assert torch.equal(tc.view(torch.int16), txt.view(torch.int16))


def test_bf16_explicit_scale(gpu):
    w = I.custom("mid_scale", 6, 30, 52, 2, 3, 3, 2, 128, 40, "bf16", std=1.0, index=321)
    run_full(w, "shifted", check_bf16, scale=0.05)


@pytest.mark.parametrize("per_window", [True, False], ids=["per_window_text", "chunked_text"])
@pytest.mark.parametrize("sched", ["per_item", "queue"])
def test_bf16_order_independent_and_deterministic(gpu, per_window, sched):
    """Results do not depend on the dispatch order, and repeat bit for bit
    (for either text reduction; the grid has 27 shifted windows, so the
    minimum workspace gives 16 chunks of one or two windows).  In queue mode
    the order decides which list (one per XCD, or a single one) an item is
    taken from."""
    import torch
    w = I.custom("mid_order", 6, 30, 52, 2, 3, 3, 3, 128, 40, "bf16", index=330)
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    p = W.Plan(*geo, W.SHIFTED)
    d = upload(I.qkv(w), "bf16")
    outs = []
    W.set_attn_schedule(SCHEDS[sched])
    try:
        for order in (W.ORDER_LPT_XCD, W.ORDER_LPT, W.ORDER_ID, W.ORDER_LPT_XCD):
            W.set_attn_order(order)
            o, t = W.window_attn(p, d["q"], d["k"], d["v"], d["txt_q"], d["txt_k"], d["txt_v"],
                                 per_window=per_window)
            outs.append((o.clone(), t.clone()))
    finally:
        W.set_attn_order(W.ORDER_LPT_XCD)
        W.set_attn_schedule(W.SCHED_AUTO)
    torch.cuda.synchronize()
    for o, t in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(t.view(torch.int16), outs[0][1].view(torch.int16))


@pytest.mark.parametrize("case", MID, ids=[c[0] for c in MID])
@pytest.mark.parametrize("canonical", [False, True], ids=["layout_io", "canonical_io"])
@pytest.mark.parametrize("per_window", [True, False], ids=["per_window_text", "chunked_text"])
def test_bf16_schedules_bit_identical(gpu, case, canonical, per_window):
    """One work group per 256-row item, one per 128-row item, and resident
    work groups taking either from a queue run the same per-wavefront
    arithmetic in the same order: identical bits, for both I/O orders."""
    import torch
    w = I.custom(*case, "bf16", index=300 + MID.index(case))
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    d = upload(I.qkv(w), "bf16")
    res = {}
    for method in (W.REGULAR, W.SHIFTED):
        p = W.Plan(*geo, method)
        for sched in SCHEDS.values():
            W.set_attn_schedule(sched)
            try:
                # outputs start as NaN: a row no item wrote cannot match
                o, t = W.window_attn(p, d["q"], d["k"], d["v"], d["txt_q"], d["txt_k"], d["txt_v"],
                                     out=torch.full_like(d["q"], float("nan")),
                                     txt_out=torch.full_like(d["txt_q"], float("nan")),
                                     canonical=canonical, per_window=per_window)
            finally:
                W.set_attn_schedule(W.SCHED_AUTO)
            res[(method, sched)] = (o, t)
    torch.cuda.synchronize()
    for method in (W.REGULAR, W.SHIFTED):
        o1, t1 = res[(method, W.SCHED_PER_ITEM)]
        for sched in (W.SCHED_PER_ITEM_128, W.SCHED_QUEUE, W.SCHED_QUEUE_128):
            o2, t2 = res[(method, sched)]
            assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"{w.name} {method} {sched}: video"
            if w.text_len:
                assert torch.equal(t1.view(torch.int16), t2.view(torch.int16)), f"{w.name} {method} {sched}: text"


@pytest.mark.parametrize("canonical", [False, True], ids=["layout_io", "canonical_io"])
def test_1080p_schedules_bit_identical(gpu, canonical):
    """256-row and 128-row items, one work group each or taken from a queue
    by resident work groups, agree bit for bit on the full 1080p grid (both
    layouts), in the launch configuration the benchmark times."""
    import torch
    w = I.WORKLOADS["1080p_bf16"]
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    g = torch.Generator(device="cuda")
    g.manual_seed(1080)

    def rnd(rows):
        return (torch.randn((rows, w.heads, w.head_dim), device="cuda", generator=g) / 11.3).to(torch.bfloat16)
    q, k, v = (rnd(w.n_tokens) for _ in range(3))
    tq, tk, tv = (rnd(w.text_len) for _ in range(3))
    for method in (W.REGULAR, W.SHIFTED):
        p = W.Plan(*geo, method)
        outs = []
        for sched in SCHEDS.values():
            W.set_attn_schedule(sched)
            try:
                outs.append(W.window_attn(p, q, k, v, tq, tk, tv, out=torch.full_like(q, float("nan")),
                                          txt_out=torch.full_like(tq, float("nan")), canonical=canonical))
            finally:
                W.set_attn_schedule(W.SCHED_AUTO)
        torch.cuda.synchronize()
        log(f"  1080p method {method} canonical={canonical}: comparing schedules")
        for o, t in outs[1:]:
            assert torch.equal(outs[0][0].view(torch.int16), o.view(torch.int16))
            assert torch.equal(outs[0][1].view(torch.int16), t.view(torch.int16))


# ------------------------------------------------------------------ full-size, sampled
def sampled_check(w, method, heads_full_text, n_samples=3, text_dtype=np.float64, q=None, canonical=False):
    """Run the whole layer of workload w on the GPU; compare sampled
    (window, head) video outputs and the complete text mean of the given
    heads with the oracle computed window by window.  canonical: q, k, v
    and out stay in canonical token order (the layout permutation inside
    the attention kernel)."""
    import torch
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    om, wm = METH[method]
    op, wp = O.plan(*geo, om), W.Plan(*geo, wm)
    wc = W.canonical(*geo[:3])
    log(f"  generating {w.name} inputs")
    inp = I.qkv(w, bits_only=True)
    d = upload(inp, "bf16")
    if canonical:
        out, txt = W.window_attn(wp, d["q"], d["k"], d["v"], d["txt_q"], d["txt_k"], d["txt_v"],
                                 canonical=True)
    else:
        qq, kk, vv = (W.relayout(d[n], wc, wp) for n in "qkv")
        del d["q"], d["k"], d["v"]
        out, txt = W.window_attn(wp, qq, kk, vv, d["txt_q"], d["txt_k"], d["txt_v"])
    torch.cuda.synchronize()
    bits = {n: inp[n][1] for n in I.QKV_NAMES}

    def rows(name, idx, h):
        return I.bf16_bits_to_f32(bits[name][idx, h]).astype(np.float64)

    lpt = op.lpt
    wins = sorted({int(lpt[0]), int(lpt[len(lpt) // 2]), int(lpt[-1])})[:n_samples]
    heads = sorted({0, w.heads - 1})
    for win in wins:
        a, b = int(op.offsets[win]), int(op.offsets[win + 1])
        ids = op.ids[a:b]
        for h in heads:
            ov, _ = O.joint_attention(rows("q", ids, h), rows("k", ids, h), rows("v", ids, h),
                                      rows("txt_q", slice(None), h), rows("txt_k", slice(None), h),
                                      rows("txt_v", slice(None), h))
            got = out[torch.from_numpy(ids.astype(np.int64)).cuda(), h] if canonical else out[a:b, h]
            check_bf16(from_dev(got), ov, f"{w.name} {method} window {win} (L={b - a}) head {h}"
                       + (" canonical I/O" if canonical else ""))
    for h in heads_full_text:
        acc = np.zeros((w.text_len, w.head_dim), dtype=text_dtype)
        tq, tk, tv = (rows(n, slice(None), h) for n in ("txt_q", "txt_k", "txt_v"))
        for win in range(op.n_windows):
            ids = op.ids[op.offsets[win]:op.offsets[win + 1]]
            _, ot = O.joint_attention(None, rows("k", ids, h), rows("v", ids, h), tq, tk, tv,
                                      dtype=text_dtype, text_only=True)
            acc += ot
        check_bf16(from_dev(txt[:, h]), O.text_mean(acc, op.n_windows).astype(np.float64),
                   f"{w.name} {method} text mean head {h} ({op.n_windows} windows)")
    return out, txt


def test_720p_shifted_sampled(gpu):
    """The 720p grid in the shifted layout (64 windows, edge windows of 252
    rows) -- the workload names the regular layout only; shifted is the
    other layer kind of the same grid."""
    sampled_check(I.WORKLOADS["720p_bf16"], "shifted", heads_full_text=[5])


@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_1080p_sampled(gpu, method):
    sampled_check(I.WORKLOADS["1080p_bf16"], method, heads_full_text=[7])


# ------------------------------------------------------------------ full-size, every element
def full_layer_check(w, method, workers=16, per_window=True):
    """The whole layer of workload w on the GPU with canonical-order I/O (the
    launch the benchmark times), compared with the oracle over EVERY window
    and head, element by element at the bf16 bar, and the complete text mean
    of every head.  The oracle runs window by window on host threads (one
    BLAS thread each)."""
    import time
    from concurrent.futures import ThreadPoolExecutor

    import torch
    from threadpoolctl import threadpool_limits
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    om, wm = METH[method]
    op, wp = O.plan(*geo, om), W.Plan(*geo, wm)
    log(f"  generating {w.name} inputs")
    inp = I.qkv(w, bits_only=True)
    d = upload(inp, "bf16")
    out, txt = W.window_attn(wp, d["q"], d["k"], d["v"], d["txt_q"], d["txt_k"], d["txt_v"], canonical=True,
                             per_window=per_window)
    torch.cuda.synchronize()
    got = dev_bits(out).reshape(w.n_tokens, w.heads, w.head_dim)
    got_txt = from_dev(txt)
    del d, out, txt
    bits = {n: inp[n][1] for n in I.QKV_NAMES}
    txt64 = {n: I.bf16_bits_to_f32(bits[n]).astype(np.float64) for n in ("txt_q", "txt_k", "txt_v")}
    t0 = time.time()

    def one(win):
        a, b = int(op.offsets[win]), int(op.offsets[win + 1])
        ids = op.ids[a:b]
        q, k, v = (I.bf16_bits_to_f32(bits[n][ids]).astype(np.float64) for n in ("q", "k", "v"))
        g = I.bf16_bits_to_f32(got[ids]).astype(np.float64)
        tw = np.empty((w.text_len, w.heads, w.head_dim))
        ratio, rel = 0.0, 0.0
        for h in range(w.heads):
            ov, ot = O.joint_attention(q[:, h], k[:, h], v[:, h], txt64["txt_q"][:, h], txt64["txt_k"][:, h],
                                       txt64["txt_v"][:, h])
            gh = g[:, h]
            assert np.isfinite(gh).all(), f"window {win} head {h}: non-finite output"
            ratio = max(ratio, float(np.max(np.abs(gh - ov) / (BF16_ATOL + BF16_RTOL * np.abs(ov)))))
            rel = max(rel, float(np.linalg.norm(gh - ov) / max(np.linalg.norm(ov), 1e-30)))
            tw[:, h] = ot
        return ratio, rel, tw

    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(one, range(op.n_windows)))
    worst = max(r[0] for r in res)
    worst_rel = max(r[1] for r in res)
    tsum = np.zeros((w.text_len, w.heads, w.head_dim))
    for r in res:       # window order
        tsum += r[2]
    log(f"  {w.name} {method} ({'per-window' if per_window else 'chunked'} text): "
        f"{op.n_windows} windows x {w.heads} heads, worst element ratio {worst:.3f} "
        f"(bar 1), worst rel-L2 {worst_rel:.3e} (bar {BF16_REL_L2}); oracle {time.time() - t0:.1f} s")
    assert worst <= 1.0, f"element error exceeds 3e-2 + 2e-2*|ref| (ratio {worst})"
    assert worst_rel <= BF16_REL_L2, f"relative L2 error {worst_rel}"
    check_bf16(got_txt, O.text_mean(tsum, op.n_windows), f"{w.name} {method} text mean (all heads)")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("per_window", [False, True], ids=["chunked_text", "per_window_text"])
def test_720p_regular_full(gpu, per_window):
    """Minimum workspace: 36 windows in 16 chunks of two or three; one
    partial per window: each window's 128 text rows follow its video rows in
    the same query tiles."""
    full_layer_check(I.WORKLOADS["720p_bf16"], "regular", per_window=per_window)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("method,per_window", [("regular", True), ("shifted", True), ("regular", False)],
                         ids=["regular", "shifted", "regular_chunked_text"])
def test_1080p_full(gpu, method, per_window):
    """Both layers of the benchmark's step, every output element (and the
    regular layer again with the minimum workspace)."""
    full_layer_check(I.WORKLOADS["1080p_bf16"], method, per_window=per_window)


@pytest.mark.timeout(900)
def test_4k_shifted_sampled(gpu):
    sampled_check(I.WORKLOADS["4k_bf16"], "shifted", heads_full_text=[3], text_dtype=np.float32)


@pytest.mark.timeout(900)
def test_4k_regular_sampled(gpu):
    """4K grid, regular layout (324 windows of 2520-3240 rows; the last
    temporal window is 7 of the 31 frames deep)."""
    sampled_check(I.WORKLOADS["4k_bf16"], "regular", heads_full_text=[11], text_dtype=np.float32)


def test_xcd_placement_probe(gpu):
    """The XCD-grouped work list assumes work group b runs on XCD b mod 8;
    the library probes that once per device (XCC_ID of each work group) and
    uses the grouping only where it holds.  On an MI355X the probe must find
    the 8 dies of the device in round-robin order."""
    info = W.device_info()
    log(f"  device: {info}")
    assert info == {"n_xcds": 8, "xcd_round_robin": True}, info

