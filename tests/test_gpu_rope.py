"""GPU parity of the window-local 3D rotary embedding (wsp_rope_relayout,
wsp_rope_text) against the oracle, and of attention on rotated q / k.

Rotation runs in float32 from float32-rounded (cos, sin) tables and rounds
once to the tensor dtype, so against the float64 oracle (same inputs):
bfloat16 outputs within one bf16 rounding (|err| <= 2^-8 |ref| + 1e-6),
float32 outputs within 2e-6 absolute on N(0, 1) inputs.  Parity is pinned
for positions, span and rotation structure; the frequency base, pair layout
and text positions are readings (see the oracle's header).
"""
import numpy as np
import pytest

import oracle as O
import video_dit_window_amd as W
import wsp_inputs as I
from helpers import check_bf16, from_dev, log, to_dev

pytestmark = pytest.mark.gpu
METH = {"regular": (O.REGULAR, W.REGULAR), "shifted": (O.SHIFTED, W.SHIFTED)}


def check_rot(gpu, ref, dtype, what):
    err = np.abs(gpu - ref)
    if dtype == "bf16":
        bad = err > 2.0 ** -8 * np.abs(ref) + 1e-6
    else:
        bad = err > 2e-6
    log(f"  {what}: max|err| = {err.max():.3e}, {int(bad.sum())} outside the bar")
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside the rounding bar"


def plans(w):
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    o = {"canonical": O.canonical_plan(*geo[:3]), "regular": O.plan(*geo, O.REGULAR),
         "shifted": O.plan(*geo, O.SHIFTED)}
    g = {"canonical": W.canonical(*geo[:3]), "regular": W.Plan(*geo, W.REGULAR),
         "shifted": W.Plan(*geo, W.SHIFTED)}
    return o, g


CASES = [("canonical", "regular", "regular"), ("canonical", "shifted", "shifted"),
         ("regular", "shifted", "shifted"), ("canonical", "canonical", "regular"),
         ("shifted", "canonical", "shifted"), ("canonical", "canonical", "canonical")]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=["-".join(c) for c in CASES])
def test_rope_relayout_mid(gpu, dtype, case):
    """Mid grid 6x30x52 (ragged windows), 3 heads, text_len 40."""
    import torch
    src, dst, pos = case
    w = I.custom("rope_mid", 6, 30, 52, 2, 3, 3, 3, 128, 40, dtype, std=1.0, index=500)
    o, g = plans(w)
    vals, bits = I.tensor(w, 0, (w.n_tokens, w.heads, w.head_dim))
    x_src = O.relayout(vals, o["canonical"], o[src])           # source rows in layout src
    xb = I.f32_to_bf16_bits(x_src) if dtype == "bf16" else None
    xd = to_dev(x_src, xb, dtype)
    y = W.rope_relayout(xd, g[src], g[dst], g[pos], w.text_len)
    torch.cuda.synchronize()
    host = I.bf16_bits_to_f32(xb) if dtype == "bf16" else x_src
    ref = O.rope_relayout(host.astype(np.float64), o[src], o[dst], o[pos], w.text_len)
    check_rot(from_dev(y), ref, dtype, f"{dtype} {src}->{dst} positions of {pos}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("text_len", [1, 77, 256])
def test_rope_text(gpu, dtype, text_len):
    import torch
    w = I.custom("rope_txt", 2, 4, 4, 1, 1, 1, 2, 128, text_len, dtype, std=1.0, index=510)
    vals, bits = I.tensor(w, 3, (text_len, 2, 128))
    y = W.rope_text(to_dev(vals, bits, dtype))
    torch.cuda.synchronize()
    host = I.bf16_bits_to_f32(bits) if dtype == "bf16" else vals
    ref = O.rope(host.astype(np.float64), O.text_positions(text_len))
    check_rot(from_dev(y), ref, dtype, f"{dtype} text rows, text_len {text_len}")


def test_rope_theta_argument(gpu):
    """An explicit base reaches the table; 10000 and the default agree bit for bit."""
    import torch
    w = I.custom("rope_theta", 3, 12, 20, 1, 1, 1, 2, 128, 5, "f32", std=1.0, index=520)
    o, g = plans(w)
    vals, _ = I.tensor(w, 0, (w.n_tokens, 2, 128))
    xd = to_dev(vals, None, "f32")
    a = W.rope_relayout(xd, g["canonical"], g["regular"], g["regular"], 5)
    b = W.rope_relayout(xd, g["canonical"], g["regular"], g["regular"], 5, theta=10000.0)
    c = W.rope_relayout(xd, g["canonical"], g["regular"], g["regular"], 5, theta=500.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = O.rope_relayout(vals.astype(np.float64), o["canonical"], o["regular"], o["regular"], 5, theta=500.0)
    check_rot(from_dev(c), ref, "f32", "theta 500")


@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_attention_on_rotated_qk(gpu, method):
    """Layer flow with RoPE: canonical q, k rotated into the layout, v moved,
    text q, k rotated; window attention; compared with the oracle doing the
    same steps in float64."""
    import torch
    w = I.custom("rope_attn", 6, 30, 52, 2, 3, 3, 3, 128, 40, "bf16", std=1.0, index=530)
    o, g = plans(w)
    inp = I.qkv(w)
    d = {n: to_dev(v, b, "bf16") for n, (v, b) in inp.items()}
    lay = method
    q = W.rope_relayout(d["q"], g["canonical"], g[lay], g[lay], w.text_len)
    k = W.rope_relayout(d["k"], g["canonical"], g[lay], g[lay], w.text_len)
    v = W.relayout(d["v"], g["canonical"], g[lay])
    tq, tk = W.rope_text(d["txt_q"]), W.rope_text(d["txt_k"])
    out, txt = W.window_attn(g[lay], q, k, v, tq, tk, d["txt_v"])
    torch.cuda.synchronize()
    h = {n: I.bf16_bits_to_f32(inp[n][1]).astype(np.float64) for n in I.QKV_NAMES}
    c, p = o["canonical"], o[lay]
    # the device rounds rotated q / k to bf16 before attention; the oracle does the same
    rq = I.bf16_bits_to_f32(I.f32_to_bf16_bits(O.rope_relayout(h["q"], c, p, p, w.text_len))).astype(np.float64)
    rk = I.bf16_bits_to_f32(I.f32_to_bf16_bits(O.rope_relayout(h["k"], c, p, p, w.text_len))).astype(np.float64)
    tp = O.text_positions(w.text_len)
    rtq = I.bf16_bits_to_f32(I.f32_to_bf16_bits(O.rope(h["txt_q"], tp))).astype(np.float64)
    rtk = I.bf16_bits_to_f32(I.f32_to_bf16_bits(O.rope(h["txt_k"], tp))).astype(np.float64)
    ref_out, ref_txt = O.window_attn(p, rq, rk, O.relayout(h["v"], c, p), rtq, rtk, h["txt_v"])
    check_bf16(from_dev(out), ref_out, f"rope attention {method} video")
    check_bf16(from_dev(txt), ref_txt, f"rope attention {method} text mean")


def test_rope_relayout_1080p_sampled(gpu):
    """Full 1080p q tensor, canonical -> shifted with shifted positions:
    sampled rows against the oracle."""
    import torch
    w = I.WORKLOADS["1080p_bf16"]
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    oc, osh = O.canonical_plan(*geo[:3]), O.plan(*geo, O.SHIFTED)
    gc, gsh = W.canonical(*geo[:3]), W.Plan(*geo, W.SHIFTED)
    log("  generating 1080p q")
    _, bits = I.tensor(w, 0, (w.n_tokens, w.heads, w.head_dim), bits_only=True)
    y = W.rope_relayout(to_dev(None, bits, "bf16"), gc, gsh, gsh, w.text_len)
    torch.cuda.synchronize()
    rows = np.random.default_rng([7, 1080]).integers(0, w.n_tokens, size=400)
    pos = O.window_positions(osh, w.text_len)
    cids = osh.ids[rows]
    ref = O.rope(I.bf16_bits_to_f32(bits[cids]).astype(np.float64), pos[cids])
    check_rot(from_dev(y[torch.from_numpy(rows).cuda()]), ref, "bf16", "1080p sampled rows")


# ---- rotation inside the attention kernel (wsp_window_attn_rope) -----------

def rope_chain(g, lay, d, Lt, canonical, theta=None, per_window=True):
    """The unfused reference path on the device: stand-alone rotation of
    q, k (into the layout, or in canonical order for layout `lay`) and of the
    text q, k, then window attention with the same I/O order."""
    src = g["canonical"] if canonical else g[lay]
    q = W.rope_relayout(d["q"], src, src, g[lay], Lt, theta=theta)
    k = W.rope_relayout(d["k"], src, src, g[lay], Lt, theta=theta)
    tq, tk = W.rope_text(d["txt_q"], theta=theta), W.rope_text(d["txt_k"], theta=theta)
    return W.window_attn(g[lay], q, k, d["v"], tq, tk, d["txt_v"], canonical=canonical, per_window=per_window)


FUSED = [("rope_fused_mid", 6, 30, 52, 2, 3, 3, 3, 40), ("rope_fused_notext", 5, 20, 36, 2, 3, 3, 2, 0),
         ("rope_fused_ragged", 7, 33, 41, 3, 2, 3, 2, 77), ("rope_fused_onewin", 3, 12, 20, 1, 1, 1, 2, 19)]


@pytest.mark.parametrize("case", FUSED, ids=[c[0] for c in FUSED])
@pytest.mark.parametrize("method", ["regular", "shifted"])
@pytest.mark.parametrize("canonical", [True, False], ids=["canonical_io", "layout_io"])
def test_fused_rope_attention_bit_identical(gpu, case, method, canonical):
    """wsp_window_attn_rope equals rope_relayout / rope_text followed by
    window attention bit for bit: the kernel rotates with the same table,
    the same float32 steps and one bf16 rounding, and runs the same
    per-wavefront attention arithmetic."""
    import torch
    name, T, H, Wd, nt, nh, nw, heads, Lt = case
    w = I.custom(name, T, H, Wd, nt, nh, nw, heads, 128, Lt, "bf16", std=1.0, index=540 + FUSED.index(case))
    o, g = plans(w)
    inp = I.qkv(w)
    d = {n: to_dev(v, b, "bf16") for n, (v, b) in inp.items()}
    if not canonical:  # layout-order inputs
        d = {n: (W.relayout(t, g["canonical"], g[method]) if n in ("q", "k", "v") else t) for n, t in d.items()}
    out, txt = W.window_attn_rope(g[method], d["q"], d["k"], d["v"], d["txt_q"], d["txt_k"], d["txt_v"],
                                  canonical=canonical)
    ref, rtxt = rope_chain(g, method, d, Lt, canonical)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{name} {method}: video"
    if Lt:
        assert torch.equal(txt.view(torch.int16), rtxt.view(torch.int16)), f"{name} {method}: text mean"


@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_fused_rope_attention_oracle(gpu, method):
    """Canonical-order layer with RoPE in the kernel against the oracle's
    rotation (float64, window-local positions, rounded to bf16 as the device
    rounds rotated q / k) and float64 attention, element by element."""
    import torch
    w = I.custom("rope_fused_oracle", 6, 30, 52, 2, 3, 3, 3, 128, 40, "bf16", std=1.0, index=550)
    o, g = plans(w)
    inp = I.qkv(w)
    d = {n: to_dev(v, b, "bf16") for n, (v, b) in inp.items()}
    out, txt = W.window_attn_rope(g[method], d["q"], d["k"], d["v"], d["txt_q"], d["txt_k"], d["txt_v"])
    torch.cuda.synchronize()
    h = {n: I.bf16_bits_to_f32(inp[n][1]).astype(np.float64) for n in I.QKV_NAMES}
    c, p = o["canonical"], o[method]
    r16 = lambda x: I.bf16_bits_to_f32(I.f32_to_bf16_bits(x)).astype(np.float64)
    rq = r16(O.rope_relayout(h["q"], c, p, p, w.text_len))
    rk = r16(O.rope_relayout(h["k"], c, p, p, w.text_len))
    tp = O.text_positions(w.text_len)
    ref_out, ref_txt = O.window_attn(p, rq, rk, O.relayout(h["v"], c, p), r16(O.rope(h["txt_q"], tp)),
                                     r16(O.rope(h["txt_k"], tp)), h["txt_v"])
    check_bf16(from_dev(out), O.relayout(ref_out, p, c), f"fused rope attention {method} video")
    check_bf16(from_dev(txt), ref_txt, f"fused rope attention {method} text mean")


def test_fused_rope_theta_and_workspace(gpu):
    """A non-default rotary base reaches the kernel's table (fused == chain
    with theta 500, != the default), and with the minimum workspace (text
    sums in 16 chunks) the fused call still equals the chain run with the
    same text reduction."""
    import torch
    w = I.custom("rope_fused_theta", 6, 30, 52, 2, 3, 3, 2, 128, 40, "bf16", std=1.0, index=560)
    o, g = plans(w)
    d = {n: to_dev(v, b, "bf16") for n, (v, b) in I.qkv(w).items()}
    args = (g["shifted"], d["q"], d["k"], d["v"], d["txt_q"], d["txt_k"], d["txt_v"])
    a, ta = W.window_attn_rope(*args, theta=500.0)
    b, tb = rope_chain(g, "shifted", d, w.text_len, True, theta=500.0)
    c, tc = W.window_attn_rope(*args)
    e, te = W.window_attn_rope(*args, theta=500.0, per_window=False)
    f, tf = rope_chain(g, "shifted", d, w.text_len, True, theta=500.0, per_window=False)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(ta.view(torch.int16), tb.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert torch.equal(e.view(torch.int16), f.view(torch.int16))
    assert torch.equal(te.view(torch.int16), tf.view(torch.int16))


@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_fused_rope_attention_1080p(gpu, method):
    """Full 1080p canonical-order layer in the benchmark's configuration:
    fused rotation bit-identical to the stand-alone rotation + attention."""
    import torch
    w = I.WORKLOADS["1080p_bf16"]
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    g = {"canonical": W.canonical(*geo[:3]), method: W.Plan(*geo, METH[method][1])}
    log(f"  generating 1080p q, k, v ({method})")
    d = {n: to_dev(None, b, "bf16") for n, (_, b) in I.qkv(w, bits_only=True).items()}
    out, txt = W.window_attn_rope(g[method], d["q"], d["k"], d["v"], d["txt_q"], d["txt_k"], d["txt_v"])
    ref, rtxt = rope_chain(g, method, d, w.text_len, True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"1080p {method}: video"
    assert torch.equal(txt.view(torch.int16), rtxt.view(torch.int16)), f"1080p {method}: text mean"
