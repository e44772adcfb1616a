"""GPU parity of the FP8 (E4M3) q/k path: per-head amax, quantisation codes
(bit-exact against the oracle: the scale and the product are float32 on both
sides), and attention on the codes (wsp_window_attn_qk8) against the oracle
attention on the dequantised q/k at the bf16 tolerance -- the quantisation is
modelled exactly, so the remaining error is the bf16 path's own.  The error
the quantisation itself adds (against unquantised q/k) is measured in
test_fp8_quantisation_error and bounded there.
"""
import numpy as np
import pytest

import oracle as O
import video_dit_window_amd as W
import wsp_inputs as I
from helpers import check_bf16, dev_bits, from_dev, log, to_dev

pytestmark = pytest.mark.gpu
METH = {"regular": (O.REGULAR, W.REGULAR), "shifted": (O.SHIFTED, W.SHIFTED)}


def codes(t):
    return t.cpu().numpy().astype(np.uint8)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_amax_and_codes_bit_exact(gpu, dtype):
    import torch
    w = I.custom("fp8_codes", 4, 10, 12, 1, 1, 1, 5, 128, 33, dtype, std=1.0, index=600)
    a, ab = I.tensor(w, 0, (w.n_tokens, 5, 128))
    b, bb = I.tensor(w, 1, (33, 5, 128))
    scale = np.array([1.0, 1e-3, 37.0, 0.0, 1.0], np.float32)   # head 3 all zeros
    a = (a * scale[None, :, None]).astype(np.float32)
    b = (b * scale[None, :, None]).astype(np.float32)
    if dtype == "bf16":
        ab, bb = I.f32_to_bf16_bits(a), I.f32_to_bf16_bits(b)
        a, b = I.bf16_bits_to_f32(ab), I.bf16_bits_to_f32(bb)
    da, db = to_dev(a, ab, dtype), to_dev(b, bb, dtype)
    amax = W.fp8_amax(da, db)
    ca, cb = W.fp8_quantize(da, amax), W.fp8_quantize(db, amax)
    torch.cuda.synchronize()
    ref_amax = O.fp8_amax(a, b).astype(np.float32)
    assert np.array_equal(amax.cpu().numpy(), ref_amax)
    assert np.array_equal(codes(ca), O.fp8_quantize(a, ref_amax))
    assert np.array_equal(codes(cb), O.fp8_quantize(b, ref_amax))


def run_qk8(w, method, canonical=False):
    """GPU fp8 path and the oracle on the same codes; returns device outputs,
    the oracle outputs and the unquantised-q/k oracle outputs."""
    import torch
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    om, wm = METH[method]
    op, wp, oc, wc = O.plan(*geo, om), W.Plan(*geo, wm), O.canonical_plan(*geo[:3]), W.canonical(*geo[:3])
    inp = I.qkv(w)
    d = {n: to_dev(v, b, "bf16") for n, (v, b) in inp.items()}
    aq, ak = W.fp8_amax(d["q"], d["txt_q"]), W.fp8_amax(d["k"], d["txt_k"])
    q8, k8 = W.fp8_quantize(d["q"], aq), W.fp8_quantize(d["k"], ak)
    tq8, tk8 = W.fp8_quantize(d["txt_q"], aq), W.fp8_quantize(d["txt_k"], ak)
    if canonical:
        out, txt = W.window_attn_qk8(wp, q8, k8, d["v"], tq8, tk8, d["txt_v"], aq, ak, canonical=True)
    else:
        ql, kl, vl = W.relayout(q8, wc, wp), W.relayout(k8, wc, wp), W.relayout(d["v"], wc, wp)
        out_l, txt = W.window_attn_qk8(wp, ql, kl, vl, tq8, tk8, d["txt_v"], aq, ak)
        out = W.relayout(out_l, wp, wc)
    torch.cuda.synchronize()
    h = {n: I.bf16_bits_to_f32(inp[n][1]) for n in I.QKV_NAMES}
    raq, rak = O.fp8_amax(h["q"], h["txt_q"]).astype(np.float32), O.fp8_amax(h["k"], h["txt_k"]).astype(np.float32)
    assert np.array_equal(aq.cpu().numpy(), raq) and np.array_equal(ak.cpu().numpy(), rak)
    cq, ck = O.fp8_quantize(h["q"], raq), O.fp8_quantize(h["k"], rak)
    assert np.array_equal(codes(q8), cq) and np.array_equal(codes(k8), ck)
    deq = {"q": O.fp8_dequantize(cq, raq), "k": O.fp8_dequantize(ck, rak),
           "txt_q": O.fp8_dequantize(O.fp8_quantize(h["txt_q"], raq), raq),
           "txt_k": O.fp8_dequantize(O.fp8_quantize(h["txt_k"], rak), rak)}
    f64 = {n: h[n].astype(np.float64) for n in I.QKV_NAMES}
    lay = lambda x: O.relayout(x, oc, op)
    ref_out, ref_txt = O.window_attn(op, lay(deq["q"]), lay(deq["k"]), lay(f64["v"]),
                                     deq["txt_q"], deq["txt_k"], f64["txt_v"])
    ex_out, ex_txt = O.window_attn(op, lay(f64["q"]), lay(f64["k"]), lay(f64["v"]),
                                   f64["txt_q"], f64["txt_k"], f64["txt_v"])
    back = lambda x: O.relayout(x, op, oc)
    return out, txt, back(ref_out), ref_txt, back(ex_out), ex_txt


CASES = [  # (name, T, H, W, nt, nh, nw, heads, D, Lt)
    ("q8_mid", 6, 30, 52, 2, 3, 3, 3, 128, 40),
    ("q8_notext", 6, 30, 52, 2, 3, 3, 2, 128, 0),
    ("q8_text1", 6, 30, 52, 2, 3, 3, 2, 128, 1),
    ("q8_small_windows", 5, 24, 40, 3, 9, 12, 2, 128, 19),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_qk8_attention_mid(gpu, case, method):
    w = I.custom(*case, "bf16", std=1.0, index=610 + CASES.index(case))
    out, txt, ref, ref_t, _, _ = run_qk8(w, method)
    check_bf16(from_dev(out), ref, f"{w.name} {method} video (codes modelled)")
    if w.text_len:
        check_bf16(from_dev(txt), ref_t, f"{w.name} {method} text mean (codes modelled)")


@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_qk8_canonical_io_bit_identical(gpu, method):
    import torch
    w = I.custom("q8_canon", 6, 30, 52, 2, 3, 3, 3, 128, 40, "bf16", std=1.0, index=620)
    a = run_qk8(w, method, canonical=False)
    b = run_qk8(w, method, canonical=True)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))


@pytest.mark.parametrize("std", [None, 1.0])
def test_fp8_quantisation_error(gpu, std):
    """What quantising q and k costs against the unquantised float64 oracle:
    inputs N(0,1)/sqrt(128) (nearly uniform attention) and N(0,1) (logits of
    standard deviation ~1).  Bound: rel-L2 <= 6e-2 on the video output."""
    w = I.custom("q8_err", 6, 30, 52, 2, 3, 3, 3, 128, 40, "bf16", std=std, index=630)
    out, txt, _, _, ex, ex_t = run_qk8(w, "shifted")
    g = from_dev(out)
    rel = float(np.linalg.norm(g - ex) / np.linalg.norm(ex))
    rel_t = float(np.linalg.norm(from_dev(txt) - ex_t) / np.linalg.norm(ex_t))
    log(f"  fp8 q/k vs unquantised oracle (std {std}): video rel-L2 {rel:.3e}, text rel-L2 {rel_t:.3e}")
    assert rel <= 6e-2 and rel_t <= 6e-2


def host_amax(bits, heads, rows_per_chunk=1 << 14):
    """Per-head max |x| of a bf16 [rows, heads, D] tensor, from its bits on
    the host (the oracle's amax over row chunks, then the max of those)."""
    amax = np.zeros(heads)
    for lo in range(0, bits.shape[0], rows_per_chunk):
        amax = np.maximum(amax, O.fp8_amax(I.bf16_bits_to_f32(bits[lo:lo + rows_per_chunk])))
    return amax


@pytest.mark.parametrize("canonical", [False, True], ids=["layout_io", "canonical_io"])
def test_qk8_1080p_sampled(gpu, canonical):
    """Full 1080p shifted layer on the fp8 path.  The per-head amax of the
    whole q and k (video and text rows) and the codes of the sampled rows are
    computed on the host from the input bits and must equal the GPU's; the
    sampled (window, head) outputs are compared with the oracle run on those
    host codes."""
    import torch
    w = I.WORKLOADS["1080p_bf16"]
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    op, wp, wc = O.plan(*geo, O.SHIFTED), W.Plan(*geo, W.SHIFTED), W.canonical(*geo[:3])
    log("  generating 1080p inputs")
    inp = I.qkv(w, bits_only=True)
    d = {n: to_dev(None, b, "bf16") for n, (_, b) in inp.items()}
    aq, ak = W.fp8_amax(d["q"], d["txt_q"]), W.fp8_amax(d["k"], d["txt_k"])
    q8c, k8c = W.fp8_quantize(d["q"], aq), W.fp8_quantize(d["k"], ak)
    tq8, tk8 = W.fp8_quantize(d["txt_q"], aq), W.fp8_quantize(d["txt_k"], ak)
    if canonical:
        out, _ = W.window_attn_qk8(wp, q8c, k8c, d["v"], tq8, tk8, d["txt_v"], aq, ak, canonical=True)
    else:
        v = W.relayout(d["v"], wc, wp)
        out_l, _ = W.window_attn_qk8(wp, W.relayout(q8c, wc, wp), W.relayout(k8c, wc, wp), v, tq8, tk8,
                                     d["txt_v"], aq, ak)
        out = W.relayout(out_l, wp, wc)
    torch.cuda.synchronize()
    bits = {n: inp[n][1] for n in I.QKV_NAMES}
    log("  host amax of q and k (171360 + 256 rows each)")
    raq = np.maximum(host_amax(bits["q"], w.heads), host_amax(bits["txt_q"], w.heads)).astype(np.float32)
    rak = np.maximum(host_amax(bits["k"], w.heads), host_amax(bits["txt_k"], w.heads)).astype(np.float32)
    assert np.array_equal(aq.cpu().numpy(), raq), "per-head amax of q differs from the host's"
    assert np.array_equal(ak.cpu().numpy(), rak), "per-head amax of k differs from the host's"
    gq, gk = codes(q8c), codes(k8c)                    # canonical row order
    for win in sorted({int(op.lpt[0]), int(op.lpt[len(op.lpt) // 2]), int(op.lpt[-1])}):
        a, b = int(op.offsets[win]), int(op.offsets[win + 1])
        ids = op.ids[a:b]
        for h in (0, 7, w.heads - 1):
            f32 = lambda n, rows, hh=h: I.bf16_bits_to_f32(bits[n][rows, hh:hh + 1])
            cq = O.fp8_quantize(f32("q", ids), raq[h:h + 1])
            ck = O.fp8_quantize(f32("k", ids), rak[h:h + 1])
            assert np.array_equal(gq[ids, h:h + 1], cq), f"q codes of window {win} head {h}"
            assert np.array_equal(gk[ids, h:h + 1], ck), f"k codes of window {win} head {h}"
            tq = O.fp8_quantize(f32("txt_q", slice(None)), raq[h:h + 1])
            tk = O.fp8_quantize(f32("txt_k", slice(None)), rak[h:h + 1])
            assert np.array_equal(codes(tq8)[:, h:h + 1], tq) and np.array_equal(codes(tk8)[:, h:h + 1], tk)
            deq = lambda c, am: O.fp8_dequantize(c, am)[:, 0]
            ov, _ = O.joint_attention(deq(cq, raq[h:h + 1]), deq(ck, rak[h:h + 1]),
                                      f32("v", ids)[:, 0].astype(np.float64),
                                      deq(tq, raq[h:h + 1]), deq(tk, rak[h:h + 1]),
                                      f32("txt_v", slice(None))[:, 0].astype(np.float64))
            got = out[torch.from_numpy(ids.astype(np.int64)).cuda(), h]
            check_bf16(from_dev(got), ov, f"1080p fp8 window {win} head {h}"
                       + (" canonical I/O" if canonical else ""))
