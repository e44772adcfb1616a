"""Host side of libwsp, no GPU needed: the C++ planner against the oracle
(bit-exact tables), argument validation of the device entry points (all
rejected before any HIP call), and the exported symbol set."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O
import video_dit_window_amd as W
import wsp_inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wsp.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wsp_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"wsp_plan", "wsp_relayout", "wsp_window_attn"} <= set(names)
    lib = ctypes.CDLL(W.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    header = open(os.path.join(ROOT, "include", "wsp.h")).read()
    assert W.version() == int(re.search(r"#define WSP_VERSION (\d+)", header).group(1))


def compare(geo, method):
    o = O.plan(*geo, method) if method != O.CANONICAL else O.canonical_plan(*geo[:3])
    p = W.Plan(*geo, method)
    t = p.tables()
    assert p.n_tokens == o.n_tokens and p.n_windows == o.n_windows
    assert tuple(p.win_size) == tuple(o.win)
    for name in ("offsets", "ids", "inv", "lpt"):
        assert np.array_equal(t[name], getattr(o, name)), name
    assert np.array_equal(t["boxes"], o.boxes)


@pytest.mark.parametrize("name", list(I.WORKLOADS))
@pytest.mark.parametrize("method", [O.REGULAR, O.SHIFTED])
def test_planner_matches_oracle_on_workloads(name, method):
    w = I.WORKLOADS[name]
    compare((w.T, w.H, w.W, w.nt, w.nh, w.nw), method)


@pytest.mark.parametrize("geo", [(5, 20, 36, 1, 1, 1), (31, 45, 80, 1, 3, 3), (40, 45, 80, 1, 3, 3),
                                 (1, 75, 192, 1, 1, 1), (1, 25, 576, 1, 1, 1), (3, 9, 16, 2, 9, 16),
                                 (12, 8, 12, 4, 60, 60), (1, 1, 1, 1, 1, 1), (2, 1, 300, 1, 1, 7)])
@pytest.mark.parametrize("method", [O.REGULAR, O.SHIFTED, O.CANONICAL])
def test_planner_matches_oracle_edge_geometries(geo, method):
    compare(geo, method)


@settings(max_examples=60, deadline=None)
@given(T=st.integers(1, 40), H=st.integers(1, 80), Wd=st.integers(1, 80),
       nt=st.integers(1, 8), nh=st.integers(1, 60), nw=st.integers(1, 60),
       method=st.sampled_from([O.REGULAR, O.SHIFTED]))
def test_planner_matches_oracle_random(T, H, Wd, nt, nh, nw, method):
    try:
        O.window_size(T, H, Wd, nt, nh, nw)
    except ValueError:
        with pytest.raises(W.WspError):
            W.Plan(T, H, Wd, nt, nh, nw, method)
        return
    compare((T, H, Wd, nt, nh, nw), method)


@pytest.mark.parametrize("bad", [(0, 4, 4, 1, 1, 1, 0), (2, -1, 4, 1, 1, 1, 0), (2, 4, 4, 0, 1, 1, 0),
                                 (1, 1, 20000, 1, 1, 1, 0), (2, 4, 4, 1, 1, 1, 7)])
def test_planner_rejects_invalid(bad):
    with pytest.raises(W.WspError) as e:
        W.Plan(*bad)
    assert e.value.code == -1


def test_planner_rejects_int32_overflow():
    with pytest.raises(W.WspError) as e:
        W.Plan(2048, 1024, 1024, 1, 1, 1, W.REGULAR)
    assert e.value.code == -2


# ------------------------------------------------ validation without a GPU
def raw():
    return W.lib()


def test_relayout_argument_errors():
    a = W.Plan(5, 20, 36, 2, 3, 3, W.REGULAR)
    b = W.Plan(5, 20, 36, 2, 3, 3, W.SHIFTED)
    c = W.Plan(5, 20, 35, 2, 3, 3, W.SHIFTED)
    x, y = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000)
    L = raw()
    assert L.wsp_relayout(x, y, 256, a.handle, c.handle, None) == -1   # grids differ
    assert L.wsp_relayout(x, y, 24, a.handle, b.handle, None) == -1    # row_bytes % 16
    assert L.wsp_relayout(x, y, 0, a.handle, b.handle, None) == -1
    assert L.wsp_relayout(None, y, 256, a.handle, b.handle, None) == -1
    assert L.wsp_relayout(ctypes.c_void_p(0x1004), y, 256, a.handle, b.handle, None) == -1
    assert L.wsp_relayout(x, x, 256, a.handle, b.handle, None) == -1
    assert L.wsp_relayout(x, y, 256, None, b.handle, None) == -1
    assert b"align" in L.wsp_last_error() or len(L.wsp_last_error()) > 0


def test_window_attn_argument_errors():
    p = W.Plan(5, 20, 36, 2, 3, 3, W.REGULAR)
    L = raw()
    a, b, c, o, t, ws = (ctypes.c_void_p(0x1000 * i) for i in range(1, 7))
    args = dict(q=a, k=b, v=c, tq=a, tk=b, tv=c, H=4, D=64, Lt=16, dt=W.F32, sc=ctypes.c_float(0),
                out=o, to=t, ws=ws, wsb=1 << 30)

    def call(**kw):
        d = dict(args, **kw)
        return L.wsp_window_attn(p.handle, d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"], d["H"],
                                 d["D"], d["Lt"], d["dt"], d["sc"], d["out"], d["to"], d["ws"],
                                 d["wsb"], None)

    assert call(D=96) == -1
    assert call(H=0) == -1
    assert call(H=40000) == -1
    assert call(dt=5) == -1
    assert call(Lt=-1) == -1
    assert call(q=None) == -1
    assert call(k=ctypes.c_void_p(0x1008)) == -1
    assert call(out=a) == -1                       # aliasing
    assert call(tq=None) == -1                     # text needed when Lt > 0
    assert call(wsb=16) == -4                      # workspace too small
    assert call(ws=None) == -4
    def call_ex(flags, **kw):
        d = dict(args, **kw)
        return L.wsp_window_attn_ex(p.handle, d["q"], d["k"], d["v"], d["tq"], d["tk"], d["tv"],
                                    d["H"], d["D"], d["Lt"], d["dt"], d["sc"], flags, d["out"],
                                    d["to"], d["ws"], d["wsb"], None)

    assert call_ex(2) == -1                        # unknown flag bit
    assert call_ex(0xFFFFFFFF) == -1
    assert b"flag" in L.wsp_last_error()
    assert call_ex(W.IO_CANONICAL, D=96) == -1     # same validation as wsp_window_attn
    assert call_ex(W.IO_CANONICAL, wsb=16) == -4
    # bf16 windows address rows with 31-bit byte offsets: 32767 heads x 128 x
    # 2 B = 8 MiB rows, so a window of >= 256 rows (here 5*20*36 = 3600 in one
    # window) is rejected before anything is launched.
    big = W.Plan(5, 20, 36, 1, 1, 1, W.REGULAR)
    for flags in (W.IO_LAYOUT, W.IO_CANONICAL):
        assert L.wsp_window_attn_ex(big.handle, a, b, c, None, None, None, 32767, 128, 0, W.BF16,
                                    ctypes.c_float(0), flags, o, None, None, 0, None) == -2
        assert b"2 GiB" in L.wsp_last_error()
    need = W.window_attn_workspace(p, 4, 64, 16, W.F32)
    assert need == min(p.n_windows, 16) * 16 * 4 * 64 * 4      # one float32 partial per chunk
    big = W.Plan(21, 68, 120, 4, 3, 3, W.REGULAR)                 # 100 windows: 16 chunks
    # bf16: 256 more bytes for the kernel's work-queue counters
    assert W.window_attn_workspace(big, 20, 128, 256, W.BF16) == 16 * 256 * 20 * 128 * 4 + 256
    assert W.window_attn_workspace(big, 20, 128, 256, W.BF16, per_window=True) == 100 * 256 * 20 * 128 * 4 + 256
    assert W.window_attn_workspace(p, 4, 64, 0, W.BF16) == 256
    assert W.window_attn_workspace(p, 4, 64, 0, W.F32) == 0


def test_rope_argument_errors():
    p = W.Plan(5, 20, 36, 2, 3, 3, W.REGULAR)
    c = W.canonical(5, 20, 36)
    other = W.Plan(5, 20, 40, 2, 3, 3, W.REGULAR)
    L = raw()
    a, b = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000)
    f0 = ctypes.c_float(0)

    def call(x=a, y=b, H=4, D=128, dt=W.BF16, src=c, dst=p, pos=p, Lt=16):
        return L.wsp_rope_relayout(x, y, H, D, dt, src.handle, dst.handle, pos.handle, Lt, f0, None)

    assert call(D=64) == -1 and b"head_dim 128" in L.wsp_last_error()
    assert call(x=None) == -1
    assert call(y=a) == -1                      # aliasing
    assert call(x=ctypes.c_void_p(0x1008)) == -1
    assert call(dt=7) == -1
    assert call(H=0) == -1
    assert call(Lt=-1) == -1
    assert call(pos=other) == -1                # grids differ
    assert L.wsp_rope_relayout(a, b, 4, 128, W.BF16, c.handle, None, p.handle, 0, f0, None) == -1
    assert L.wsp_rope_text(a, b, 16, 4, 64, W.BF16, f0, None) == -1
    assert L.wsp_rope_text(a, a, 16, 4, 128, W.BF16, f0, None) == -1
    assert L.wsp_rope_text(a, b, 0, 4, 128, W.BF16, f0, None) == 0      # nothing to do


def test_linear_rope_argument_errors():
    """wsp_linear_rope validates everything before touching the device."""
    c = W.canonical(5, 20, 36)
    p = W.Plan(5, 20, 36, 2, 3, 3, W.REGULAR)
    other = W.Plan(5, 20, 40, 2, 3, 3, W.REGULAR)
    tall = W.Plan(2, 6000, 2, 1, 1, 1, W.REGULAR)          # windows 3286 rows high > 2048
    tall_c = W.canonical(2, 6000, 2)
    L = raw()
    x, w, y = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    f0 = ctypes.c_float(0)
    n = 5 * 20 * 36

    def call(x=x, w=w, y=y, M=n + 16, N=256, K=64, dt=W.BF16, rows=c, pos=p, Lt=16):
        return L.wsp_linear_rope(x, w, y, M, N, K, dt, rows.handle if rows else None,
                                 pos.handle if pos else None, Lt, f0, None)

    assert call(M=n) == -1 and b"token count" in L.wsp_last_error()
    assert call(rows=None) == -1 and call(pos=None) == -1
    assert call(pos=other) == -1 and b"grids" in L.wsp_last_error()
    assert call(Lt=-1, M=n - 1) == -1
    assert call(dt=W.F32) == -1
    assert call(N=128) == -1                                 # not a multiple of 256
    assert call(K=96) == -1
    assert call(x=None) == -1
    assert call(y=x) == -1                                   # y aliases x
    assert call(w=ctypes.c_void_p(0x2008)) == -1             # misaligned
    assert call(rows=tall_c, pos=tall, M=2 * 6000 * 2, Lt=0) == -2 and b"extents" in L.wsp_last_error()


def test_attn_schedule_option():
    L = raw()
    assert L.wsp_set_attn_schedule(6) == -1
    assert L.wsp_set_attn_schedule(-1) == -1
    assert L.wsp_set_attn_schedule(1) == -1      # the removed static persistent schedule
    for sc in (W.SCHED_PER_ITEM, W.SCHED_PER_ITEM_128, W.SCHED_QUEUE, W.SCHED_QUEUE_128, W.SCHED_AUTO):
        W.set_attn_schedule(sc)


def test_attn_order_option():
    L = raw()
    assert L.wsp_set_attn_order(7) == -1
    for o in (W.ORDER_ID, W.ORDER_LPT, W.ORDER_LPT_XCD):
        W.set_attn_order(o)


def test_device_info_argument_errors():
    L = raw()
    n = ctypes.c_int32()
    assert L.wsp_device_info(None, ctypes.byref(n)) == -1
    assert L.wsp_device_info(ctypes.byref(n), None) == -1


def test_rope_attention_argument_errors():
    """wsp_window_attn_rope / _workspace validate before any device work."""
    p = W.Plan(5, 20, 36, 2, 3, 3, W.REGULAR)
    tall = W.Plan(2, 6000, 2, 1, 1, 1, W.REGULAR)   # windows 3286 rows high > 2048
    L = raw()
    a, b, o = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    f0 = ctypes.c_float(0)
    need = ctypes.c_size_t()
    assert L.wsp_window_attn_rope_workspace(p.handle, 4, 128, 16, W.BF16, ctypes.byref(need)) == 0
    rot = 5 * 20 * 36 * 4 * 128 * 2 + 2 * 16 * 4 * 128 * 2            # rotated k, text q, text k
    assert need.value == W.window_attn_workspace(p, 4, 128, 16, W.BF16) + rot
    assert L.wsp_window_attn_rope_workspace(p.handle, 4, 64, 16, W.BF16, ctypes.byref(need)) == -1
    assert L.wsp_window_attn_rope_workspace(p.handle, 4, 128, 16, W.F32, ctypes.byref(need)) == -1
    # + 256 bytes of work-queue counters
    assert W.window_attn_rope_workspace(p, 4, 16, per_window=True) == rot + p.n_windows * 16 * 4 * 128 * 4 + 256

    def call(pl=p, D=128, dt=W.BF16, ws=None, wb=0):
        return L.wsp_window_attn_rope(pl.handle, a, b, a, a, b, a, 4, D, 16, dt, f0, f0, 1, o, o, ws, wb, None)

    assert call(D=64) == -1 and b"head_dim 128" in L.wsp_last_error()
    assert call(dt=W.F32) == -1
    assert call(ws=o, wb=16) == -4                          # workspace too small
    assert call(pl=tall) == -2 and b"extents" in L.wsp_last_error()
