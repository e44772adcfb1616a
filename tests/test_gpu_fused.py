"""GPU parity of wsp_window_attn_ex with canonical-order I/O (the layout
permutation fused into the attention kernels).

The fused call must equal, bit for bit, the unfused sequence
relayout(canonical -> layout) -> wsp_window_attn -> relayout(layout ->
canonical): both read the same rows in the same order and run the same
arithmetic.  It is also compared with the oracle element by element on small
grids (ragged windows, D = 64 and 128, text lengths 0, 1 and odd), and bit for
bit against the unfused path at the full 1080p size.
"""
import numpy as np
import pytest

import oracle as O
import video_dit_window_amd as W
import wsp_inputs as I
from helpers import check_bf16, check_f32, from_dev, log, to_dev

pytestmark = pytest.mark.gpu
METH = {"regular": (O.REGULAR, W.REGULAR), "shifted": (O.SHIFTED, W.SHIFTED)}


def bits_equal(a, b):
    import torch
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def fused_vs_unfused(w, method, d):
    """(fused out, fused text, unfused out in canonical order, unfused text)."""
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    wp, wc = W.Plan(*geo, METH[method][1]), W.canonical(*geo[:3])
    txt = (d["txt_q"], d["txt_k"], d["txt_v"])
    out_f, txt_f = W.window_attn(wp, d["q"], d["k"], d["v"], *txt, canonical=True)
    q, k, v = (W.relayout(d[n], wc, wp) for n in "qkv")
    out_u, txt_u = W.window_attn(wp, q, k, v, *txt)
    return out_f, txt_f, W.relayout(out_u, wp, wc), txt_u


def run_small(w, method, check):
    import torch
    inp = I.qkv(w)
    d = {n: to_dev(v, b, w.dtype) for n, (v, b) in inp.items()}
    out_f, txt_f, out_u, txt_u = fused_vs_unfused(w, method, d)
    torch.cuda.synchronize()
    assert bits_equal(out_f, out_u), f"{w.name} {method}: fused video output differs from unfused"
    if w.text_len:
        assert bits_equal(txt_f, txt_u), f"{w.name} {method}: fused text output differs"
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    op, oc = O.plan(*geo, METH[method][0]), O.canonical_plan(*geo[:3])
    h = {}
    for n in I.QKV_NAMES:
        v, b = inp[n]
        h[n] = (v if v is not None else I.bf16_bits_to_f32(b)).astype(np.float64)
    ref_out, ref_txt = O.window_attn(op, *(O.relayout(h[n], oc, op) for n in "qkv"),
                                     h["txt_q"], h["txt_k"], h["txt_v"])
    check(from_dev(out_f), O.relayout(ref_out, op, oc), f"{w.name} {method} fused video")
    if w.text_len:
        check(from_dev(txt_f), ref_txt, f"{w.name} {method} fused text mean")


@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_fused_tiny_f32(gpu, method):
    run_small(I.WORKLOADS["tiny_f32"], method, check_f32)


def test_fused_mid_f32_d128(gpu):
    run_small(I.custom("fmid_f32", 6, 30, 52, 2, 3, 3, 2, 128, 37, "f32", index=401), "shifted",
              check_f32)


FUSED_BF16 = [  # (name, T, H, W, nt, nh, nw, heads, D, Lt)
    ("fmid_bf16", 6, 30, 52, 2, 3, 3, 3, 128, 40),
    ("fmid_bf16_d64", 6, 30, 52, 2, 3, 3, 3, 64, 40),
    ("fmid_bf16_notext", 6, 30, 52, 2, 3, 3, 2, 128, 0),
    ("fmid_bf16_text1", 6, 30, 52, 2, 3, 3, 2, 128, 1),
    ("fsmall_windows_bf16", 5, 24, 40, 3, 9, 12, 2, 128, 19),
    ("fone_window_bf16", 3, 12, 20, 1, 1, 1, 2, 128, 77),
    ("ftiny_windows_bf16", 4, 20, 36, 4, 9, 9, 2, 128, 0),
    ("ftiny_windows_text_d64", 4, 20, 36, 4, 9, 9, 2, 64, 19),
]


@pytest.mark.parametrize("case", FUSED_BF16, ids=[c[0] for c in FUSED_BF16])
@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_fused_mid_bf16(gpu, case, method):
    run_small(I.custom(*case, "bf16", index=410 + FUSED_BF16.index(case)), method, check_bf16)


def test_fused_canonical_plan_is_identity(gpu):
    """With the one-window canonical plan the ids table is the identity, so
    the fused and plain calls read and write the same rows."""
    import torch
    w = I.custom("fcanon", 2, 10, 14, 1, 1, 1, 2, 128, 9, "bf16", index=430)
    d = {n: to_dev(v, b, "bf16") for n, (v, b) in I.qkv(w).items()}
    wc = W.canonical(w.T, w.H, w.W)
    txt = (d["txt_q"], d["txt_k"], d["txt_v"])
    a, ta = W.window_attn(wc, d["q"], d["k"], d["v"], *txt, canonical=True)
    b, tb = W.window_attn(wc, d["q"], d["k"], d["v"], *txt)
    torch.cuda.synchronize()
    assert bits_equal(a, b) and bits_equal(ta, tb)


@pytest.mark.parametrize("method", ["regular", "shifted"])
def test_fused_1080p_bit_identical(gpu, method):
    """Full 1080p workload: the fused path equals the unfused one bit for bit
    (the unfused path is checked against the oracle by the sampled tests)."""
    import torch
    w = I.WORKLOADS["1080p_bf16"]
    log(f"  generating {w.name} inputs")
    d = {n: to_dev(v, b, "bf16") for n, (v, b) in I.qkv(w, bits_only=True).items()}
    out_f, txt_f, out_u, txt_u = fused_vs_unfused(w, method, d)
    torch.cuda.synchronize()
    assert bits_equal(out_f, out_u)
    assert bits_equal(txt_f, txt_u)
