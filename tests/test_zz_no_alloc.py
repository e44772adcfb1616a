"""wsp_window_attn_noalloc (the entry point for callers that cannot allocate
device memory) against wsp_window_attn_ex, through the C ABI: same kernels,
so the outputs must be identical bit for bit, on two calls in a row (the
second on a smaller input, over the scratch contents the first one left),
in both I/O orders and both dtypes; and its two extra errors."""
import ctypes

import numpy as np
import pytest

import video_dit_window_amd as W
import wsp_inputs as I
from helpers import log, to_dev

pytestmark = pytest.mark.gpu

CASES = [  # (name, T, H, W, nt, nh, nw, heads, D, Lt): a larger call, then a smaller one
    ("noalloc_a", 6, 30, 52, 2, 3, 3, 3, 128, 40),
    ("noalloc_b", 4, 20, 36, 2, 3, 3, 2, 128, 19),
]


def run_pair(case, dtype, canonical, method):
    import torch
    w = I.custom(*case, dtype, index=700 + CASES.index(case))
    if dtype == "f32":
        w = I.custom(*case[:8], 64, case[9], dtype, index=700 + CASES.index(case))
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    p = W.Plan(*geo, method)
    d = {n: to_dev(v, b, dtype) for n, (v, b) in I.qkv(w).items()}
    if not canonical:
        c = W.canonical(*geo[:3])
        for n in ("q", "k", "v"):
            d[n] = W.relayout(d[n], c, p)
    # the reference call uploads the tables, with the text reduction the
    # no-allocation call will choose
    pw = W.noalloc_per_window(p, w.heads, w.head_dim, w.text_len)
    ref, ref_t = W.window_attn(p, d["q"], d["k"], d["v"], d["txt_q"], d["txt_k"], d["txt_v"], canonical=canonical,
                               per_window=pw)
    out, txt = torch.full_like(ref, float("nan")), torch.full_like(ref_t, float("nan"))
    W.window_attn_noalloc(p, d["q"], d["k"], d["v"], d["txt_q"], d["txt_k"], d["txt_v"], out, txt,
                          canonical=canonical)
    torch.cuda.synchronize()
    view = torch.int16 if dtype == "bf16" else torch.int32
    log(f"  {w.name} {dtype} canonical={canonical} method={method} per_window={pw}: comparing")
    assert torch.equal(out.view(view), ref.view(view)), f"{w.name}: video outputs differ"
    assert torch.equal(txt.view(view), ref_t.view(view)), f"{w.name}: text mean differs"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("canonical", [False, True], ids=["layout_io", "canonical_io"])
def test_noalloc_matches_workspace_call(gpu, dtype, canonical):
    for case, method in zip(CASES, (W.SHIFTED, W.REGULAR)):
        run_pair(case, dtype, canonical, method)


def test_noalloc_1080p_then_smaller(gpu):
    """The 1080p layer (its 100 per-window partials would exceed the scratch,
    so 16 chunk partials), then a mid-size layer (one partial per window)
    over what the first left in the scratch."""
    import torch
    w = I.WORKLOADS["1080p_bf16"]
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    p = W.Plan(*geo, W.SHIFTED)
    assert not W.noalloc_per_window(p, w.heads, w.head_dim, w.text_len)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    mk = lambda r: (torch.randn((r, w.heads, w.head_dim), device="cuda", generator=g) / 11.3).to(torch.bfloat16)
    q, k, v, tq, tk, tv = mk(w.n_tokens), mk(w.n_tokens), mk(w.n_tokens), mk(256), mk(256), mk(256)
    ref, ref_t = W.window_attn(p, q, k, v, tq, tk, tv, canonical=True, per_window=False)
    out, txt = torch.empty_like(ref), torch.empty_like(ref_t)
    W.window_attn_noalloc(p, q, k, v, tq, tk, tv, out, txt, canonical=True)
    torch.cuda.synchronize()
    log("  1080p shifted, canonical I/O, 16 chunks: comparing")
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(txt.view(torch.int16), ref_t.view(torch.int16))
    del q, k, v, out, ref
    run_pair(CASES[1], "bf16", True, W.REGULAR)


def test_noalloc_errors(gpu):
    import torch
    L = W.lib()
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    a = ctypes.c_void_p(buf.data_ptr())
    f0 = ctypes.c_float(0)
    # tables of this plan never uploaded: refused, nothing launched
    p = W.Plan(5, 20, 36, 2, 3, 3, W.SHIFTED)
    rc = L.wsp_window_attn_noalloc(p.handle, a, a, a, a, a, a, 2, 128, 16, W.BF16, f0, 0,
                                   ctypes.c_void_p(buf.data_ptr() + 4096), a, None)
    assert rc == -1 and b"wsp_window_attn_ex once" in L.wsp_last_error()
    # a text mean needing more scratch than the fixed array: 16 chunks x 4096
    # text rows x 4 heads x 128 x 4 B = 128 MiB > 96 MiB
    big = W.Plan(21, 68, 120, 4, 3, 3, W.REGULAR)
    rc = L.wsp_window_attn_noalloc(big.handle, a, a, a, a, a, a, 4, 128, 4096, W.BF16, f0, 0,
                                   ctypes.c_void_p(buf.data_ptr() + 4096), a, None)
    assert rc == -2 and b"scratch" in L.wsp_last_error()
