"""ctypes binding of libwsp.so (argument marshalling only).

Every step of the layer runs inside libwsp's HIP kernels; this module only
converts Python/torch arguments to the C ABI declared in include/wsp.h and
allocates output tensors with torch (device memory plumbing).  There is no
CPU fallback: if the library is missing the import of an entry point fails.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwsp.so")

REGULAR, SHIFTED, CANONICAL = 0, 1, 2
IO_LAYOUT, IO_CANONICAL = 0, 1
F32, BF16 = 0, 1
ORDER_LPT_XCD, ORDER_LPT, ORDER_ID = 0, 1, 2
SCHED_AUTO, SCHED_PER_ITEM, SCHED_PER_ITEM_128, SCHED_QUEUE, SCHED_QUEUE_128 = 0, 2, 3, 4, 5
METHODS = {"regular": REGULAR, "shifted": SHIFTED, "canonical": CANONICAL}

_c_int, _c_i64, _c_sz, _c_vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
_i32p, _i64p, _szp = (ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64),
                      ctypes.POINTER(ctypes.c_size_t))

_SIGNATURES = {
    "wsp_plan": (_c_int, [_c_int] * 7 + [ctypes.POINTER(_c_vp)]),
    "wsp_plan_info": (_c_int, [_c_vp, _i64p, _i32p, _i32p]),
    "wsp_plan_tables": (_c_int, [_c_vp, _i32p, _i32p, _i32p, _i32p, _i32p]),
    "wsp_plan_free": (None, [_c_vp]),
    "wsp_relayout": (_c_int, [_c_vp, _c_vp, _c_i64, _c_vp, _c_vp, _c_vp]),
    "wsp_window_attn_workspace": (_c_int, [_c_vp, _c_int, _c_int, _c_int, _c_int, _szp]),
    "wsp_window_attn": (_c_int, [_c_vp] * 7 + [_c_int, _c_int, _c_int, _c_int, ctypes.c_float,
                                                _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "wsp_window_attn_ex": (_c_int, [_c_vp] * 7 + [_c_int, _c_int, _c_int, _c_int, ctypes.c_float,
                                                   ctypes.c_uint, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "wsp_window_attn_noalloc": (_c_int, [_c_vp] * 7 + [_c_int, _c_int, _c_int, _c_int, ctypes.c_float,
                                                        ctypes.c_uint, _c_vp, _c_vp, _c_vp]),
    "wsp_rope_relayout": (_c_int, [_c_vp, _c_vp, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_int,
                                   ctypes.c_float, _c_vp]),
    "wsp_rope_text": (_c_int, [_c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, ctypes.c_float, _c_vp]),
    "wsp_window_attn_rope": (_c_int, [_c_vp] * 7 + [_c_int, _c_int, _c_int, _c_int, ctypes.c_float,
                                                     ctypes.c_float, ctypes.c_uint, _c_vp, _c_vp, _c_vp, _c_sz,
                                                     _c_vp]),
    "wsp_window_attn_rope_workspace": (_c_int, [_c_vp, _c_int, _c_int, _c_int, _c_int, _szp]),
    "wsp_fp8_amax": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_int, _c_vp, _c_vp]),
    "wsp_fp8_quantize": (_c_int, [_c_vp, _c_vp, _c_i64, _c_int, _c_int, _c_int, _c_vp, _c_vp]),
    "wsp_window_attn_qk8": (_c_int, [_c_vp] * 9 + [_c_int, _c_int, _c_int, ctypes.c_float, ctypes.c_uint,
                                                    _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "wsp_linear": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_int, _c_int, _c_int, _c_vp]),
    "wsp_linear_rope": (_c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_int,
                                 ctypes.c_float, _c_vp]),
    "wsp_set_attn_order": (_c_int, [_c_int]),
    "wsp_device_info": (_c_int, [_i32p, _i32p]),
    "wsp_set_attn_schedule": (_c_int, [_c_int]),
    "wsp_last_error": (ctypes.c_char_p, []),
    "wsp_version": (_c_int, []),
}

_lib = None


class WspError(RuntimeError):
    """A libwsp call returned an error status."""

    def __init__(self, name, code, msg):
        super().__init__(f"{name} failed ({code}): {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded libwsp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m video_dit_window_amd.build` (no CPU fallback exists)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype, fn.argtypes = res, args
        _lib = l
    return _lib


def _check(name, rc):
    if rc != 0:
        raise WspError(name, rc, lib().wsp_last_error().decode())


def _i32(a):
    return a.ctypes.data_as(_i32p)


class Plan:
    """A window layout (owns a wsp_plan_t)."""

    def __init__(self, T, H, W, nt=1, nh=1, nw=1, method=REGULAR):
        if isinstance(method, str):
            method = METHODS[method]
        h = _c_vp()
        _check("wsp_plan", lib().wsp_plan(T, H, W, nt, nh, nw, method, ctypes.byref(h)))
        self._h = h
        self.T, self.H, self.W, self.nt, self.nh, self.nw, self.method = T, H, W, nt, nh, nw, method
        n, nwin, win = ctypes.c_int64(), ctypes.c_int32(), (ctypes.c_int32 * 3)()
        _check("wsp_plan_info", lib().wsp_plan_info(h, ctypes.byref(n), ctypes.byref(nwin), win))
        self.n_tokens, self.n_windows, self.win_size = n.value, nwin.value, tuple(win)

    @property
    def handle(self):
        return self._h

    def tables(self):
        """Host copies of offsets, ids, inv, boxes [nwin, 6], lpt (int32)."""
        n, nw = self.n_tokens, self.n_windows
        t = {"offsets": np.empty(nw + 1, np.int32), "ids": np.empty(n, np.int32),
             "inv": np.empty(n, np.int32), "boxes": np.empty((nw, 6), np.int32),
             "lpt": np.empty(nw, np.int32)}
        _check("wsp_plan_tables", lib().wsp_plan_tables(
            self._h, _i32(t["offsets"]), _i32(t["ids"]), _i32(t["inv"]), _i32(t["boxes"]),
            _i32(t["lpt"])))
        return t

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.wsp_plan_free(h)
            self._h = None


def plan(T, H, W, nt, nh, nw, method) -> Plan:
    return Plan(T, H, W, nt, nh, nw, method)


def canonical(T, H, W) -> Plan:
    return Plan(T, H, W, 1, 1, 1, CANONICAL)


# ---------------------------------------------------------------- device calls
def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return _c_vp(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _on(stream):
    """Context in which torch allocates for work enqueued on `stream`: the
    caching allocator then hands a freed block to another allocation only
    after the work queued on that stream (a workspace dropped on return may
    still be in use by the kernels just enqueued there)."""
    import contextlib
    torch = _torch()
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def _dev_ptr(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _c_vp(t.data_ptr())


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {dt}")


def relayout(x, src: Plan, dst: Plan, out=None, stream=None):
    """y[j] = x[rows of src holding dst's token j] (whole rows, bytes unchanged)."""
    torch = _torch()
    if out is None:
        with _on(stream):
            out = torch.empty_like(x)
    row_bytes = x[0].numel() * x.element_size() if x.shape[0] else 0
    if x.shape[0] != src.n_tokens or out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("x/out shape does not match the plans")
    _check("wsp_relayout", lib().wsp_relayout(_dev_ptr(x, "x"), _dev_ptr(out, "out"), row_bytes,
                                              src.handle, dst.handle, _stream(stream)))
    return out


def linear(x, w, residual=None, out=None, stream=None):
    """y = x w^T (+ residual): x [M, K], w [N, K], y [M, N], bfloat16.
    residual may be `out` itself (in-place residual update)."""
    torch = _torch()
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [M, K] and w [N, K]")
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        with _on(stream):
            out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if tuple(out.shape) != (M, N) or out.dtype != x.dtype or w.dtype != x.dtype:
        raise ValueError("out must be [M, N] with the dtype of x and w")
    if residual is not None and (tuple(residual.shape) != (M, N) or residual.dtype != x.dtype):
        raise ValueError("residual must be [M, N] with the dtype of x")
    rp = None if residual is None else _dev_ptr(residual, "residual")
    _check("wsp_linear", lib().wsp_linear(_dev_ptr(x, "x"), _dev_ptr(w, "w"), rp, _dev_ptr(out, "out"), M, N, K,
                                          _dtype_code(x.dtype), _stream(stream)))
    return out


def linear_rope(x, w, rows: Plan, pos: Plan, text_len, theta=None, out=None, stream=None):
    """q or k projection with the window-local rotary embedding applied as it
    is stored (wsp_linear_rope): x [n + text_len, K] holds the video rows in
    the row order of `rows` followed by the text rows, w [N, K] with N =
    heads * 128; each video row turns by its token's window-local position in
    layout `pos`, text row i by (i, i, i)."""
    torch = _torch()
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [M, K] and w [N, K]")
    M, K = x.shape
    N = w.shape[0]
    if M != rows.n_tokens + int(text_len):
        raise ValueError("x must hold the plan's tokens followed by text_len text rows")
    if out is None:
        with _on(stream):
            out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if tuple(out.shape) != (M, N) or out.dtype != x.dtype or w.dtype != x.dtype:
        raise ValueError("out must be [M, N] with the dtype of x and w")
    _check("wsp_linear_rope", lib().wsp_linear_rope(
        _dev_ptr(x, "x"), _dev_ptr(w, "w"), _dev_ptr(out, "out"), M, N, K, _dtype_code(x.dtype), rows.handle,
        pos.handle, int(text_len), ctypes.c_float(0.0 if theta is None else theta), _stream(stream)))
    return out


def window_attn_workspace(p: Plan, n_heads, head_dim, text_len, dtype, per_window=False) -> int:
    """Workspace bytes of window_attn: the minimum the call accepts (float32
    text sums of min(n_windows, 16) chunks), or with per_window=True the size
    that selects one text partial per window (n_windows chunks: each text
    item then shares its window's K/V in L2 with the video items; faster)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    b = ctypes.c_size_t()
    _check("wsp_window_attn_workspace",
           lib().wsp_window_attn_workspace(p.handle, n_heads, head_dim, text_len, code, ctypes.byref(b)))
    if per_window:
        # the partials of every window, plus what the minimum holds beside them
        # (the bf16 kernel's work-queue counters)
        return p.n_windows * text_len * n_heads * head_dim * 4 + \
            (b.value - min(p.n_windows, 16) * text_len * n_heads * head_dim * 4)
    return b.value


def window_attn(p: Plan, q, k, v, txt_q, txt_k, txt_v, scale=None, out=None, txt_out=None,
                workspace=None, stream=None, canonical=False, per_window=True):
    """Joint window attention; returns (out [N,H,D], txt_out [Lt,H,D]).

    canonical=True: q, k, v and out rows are in canonical token order (the
    layout permutation happens inside the kernel, wsp_window_attn_ex).
    Without a workspace, one is allocated: per_window=True sizes it for one
    text partial per window (the faster text reduction), False for the
    minimum (16 chunks of windows)."""
    torch = _torch()
    N, Hh, D = q.shape
    Lt = txt_q.shape[0]
    code = _dtype_code(q.dtype)
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    for name, t in (("txt_k", txt_k), ("txt_v", txt_v)):
        if t.shape != txt_q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match txt_q in shape and q in dtype")
    if txt_q.shape[1:] != (Hh, D) or N != p.n_tokens:
        raise ValueError("shapes do not match the plan / each other")
    need = window_attn_workspace(p, Hh, D, Lt, code, per_window=per_window)
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if txt_out is None:
            txt_out = torch.empty_like(txt_q)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    tp = [(_dev_ptr(t, n) if Lt else _c_vp(0)) for n, t in
          (("txt_q", txt_q), ("txt_k", txt_k), ("txt_v", txt_v), ("txt_out", txt_out))]
    _check("wsp_window_attn_ex", lib().wsp_window_attn_ex(
        p.handle, _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), tp[0], tp[1], tp[2],
        Hh, D, Lt, code, ctypes.c_float(0.0 if scale is None else float(scale)),
        IO_CANONICAL if canonical else IO_LAYOUT,
        _dev_ptr(out, "out"), tp[3], _dev_ptr(workspace, "workspace"), ws_bytes, _stream(stream)))
    return out, txt_out


def window_attn_noalloc(p: Plan, q, k, v, txt_q, txt_k, txt_v, out, txt_out, scale=None, stream=None,
                        canonical=False):
    """wsp_window_attn_noalloc: window_attn without a workspace (the library's
    fixed scratch array) and without uploading anything; the plan's tables
    must be resident from an earlier window_attn call with the same
    arguments and the same text reduction (one partial per window when
    those fit in the scratch array, else 16 chunks: window_attn with
    per_window=noalloc_per_window(...)).  out and txt_out are the caller's."""
    N, Hh, D = q.shape
    Lt = txt_q.shape[0]
    if out.shape != q.shape or out.dtype != q.dtype or txt_out.shape != txt_q.shape or txt_out.dtype != q.dtype:
        raise ValueError("out / txt_out must match q / txt_q")
    if N != p.n_tokens or txt_q.shape[1:] != (Hh, D):
        raise ValueError("shapes do not match the plan / each other")
    tp = [(_dev_ptr(t, n) if Lt else _c_vp(0)) for n, t in
          (("txt_q", txt_q), ("txt_k", txt_k), ("txt_v", txt_v), ("txt_out", txt_out))]
    _check("wsp_window_attn_noalloc", lib().wsp_window_attn_noalloc(
        p.handle, _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), tp[0], tp[1], tp[2],
        Hh, D, Lt, _dtype_code(q.dtype), ctypes.c_float(0.0 if scale is None else float(scale)),
        IO_CANONICAL if canonical else IO_LAYOUT, _dev_ptr(out, "out"), tp[3], _stream(stream)))
    return out, txt_out


def noalloc_per_window(p: Plan, n_heads, head_dim, text_len, dtype=BF16) -> bool:
    """Whether wsp_window_attn_noalloc reduces the text with one partial per
    window (they fit in its 96 MiB scratch, beside the 256 bytes of bf16
    work-queue counters) rather than in 16 chunks."""
    queue = 256 if (dtype if isinstance(dtype, int) else _dtype_code(dtype)) == BF16 else 0
    return p.n_windows * text_len * n_heads * head_dim * 4 <= (96 << 20) - queue


def rope_relayout(x, src: Plan, dst: Plan, pos: Plan, text_len, theta=None, out=None, stream=None):
    """Rows of x [N, H, 128] moved from layout src to dst and rotated by the
    window-local axial indices (text_len + dt, dh, dw) of each token in
    layout pos (wsp_rope_relayout)."""
    torch = _torch()
    if out is None:
        with _on(stream):
            out = torch.empty_like(x)
    if x.shape[0] != src.n_tokens or out.shape != x.shape or out.dtype != x.dtype or x.dim() != 3:
        raise ValueError("x/out shape does not match the plans")
    _check("wsp_rope_relayout", lib().wsp_rope_relayout(
        _dev_ptr(x, "x"), _dev_ptr(out, "out"), x.shape[1], x.shape[2], _dtype_code(x.dtype),
        src.handle, dst.handle, pos.handle, int(text_len), ctypes.c_float(0.0 if theta is None else theta),
        _stream(stream)))
    return out


def rope_text(x, theta=None, out=None, stream=None):
    """Text rows x [Lt, H, 128] rotated by the axial indices (i, i, i) (wsp_rope_text)."""
    torch = _torch()
    if out is None:
        with _on(stream):
            out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or x.dim() != 3:
        raise ValueError("x/out shapes differ")
    if x.shape[0] == 0:
        return out
    _check("wsp_rope_text", lib().wsp_rope_text(
        _dev_ptr(x, "x"), _dev_ptr(out, "out"), x.shape[0], x.shape[1], x.shape[2], _dtype_code(x.dtype),
        ctypes.c_float(0.0 if theta is None else theta), _stream(stream)))
    return out


def device_info():
    """wsp_device_info on the current device: {"n_xcds": XCD count,
    "xcd_round_robin": whether work group b runs on XCD b mod n_xcds}."""
    n, rr = ctypes.c_int32(), ctypes.c_int32()
    _check("wsp_device_info", lib().wsp_device_info(ctypes.byref(n), ctypes.byref(rr)))
    return {"n_xcds": n.value, "xcd_round_robin": bool(rr.value)}


def window_attn_rope_workspace(p: Plan, n_heads, text_len, per_window=True) -> int:
    """Workspace bytes of window_attn_rope (bf16, head dim 128): the rotated
    text q and k, then the text partials -- the minimum the call accepts, or
    with per_window=True one partial per window (the faster text reduction)."""
    b = ctypes.c_size_t()
    _check("wsp_window_attn_rope_workspace",
           lib().wsp_window_attn_rope_workspace(p.handle, n_heads, 128, text_len, BF16, ctypes.byref(b)))
    if per_window:
        return b.value - window_attn_workspace(p, n_heads, 128, text_len, BF16) + \
            window_attn_workspace(p, n_heads, 128, text_len, BF16, per_window=True)
    return b.value


def window_attn_rope(p: Plan, q, k, v, txt_q, txt_k, txt_v, scale=None, theta=None, out=None, txt_out=None,
                     workspace=None, stream=None, canonical=True, per_window=True):
    """Window attention of rotated q, k (wsp_window_attn_rope): the same bits
    as rope_relayout / rope_text followed by window_attn, with the video
    rotation inside the attention kernel; q and k are not modified.
    bf16, head dim 128.  Returns (out, txt_out)."""
    torch = _torch()
    N, Hh, D = q.shape
    Lt = txt_q.shape[0]
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    for name, t in (("txt_k", txt_k), ("txt_v", txt_v)):
        if t.shape != txt_q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match txt_q in shape and q in dtype")
    if txt_q.shape[1:] != (Hh, D) or N != p.n_tokens:
        raise ValueError("shapes do not match the plan / each other")
    need = window_attn_rope_workspace(p, Hh, Lt, per_window=per_window)
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if txt_out is None:
            txt_out = torch.empty_like(txt_q)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    tp = [(_dev_ptr(t, n) if Lt else _c_vp(0)) for n, t in
          (("txt_q", txt_q), ("txt_k", txt_k), ("txt_v", txt_v), ("txt_out", txt_out))]
    _check("wsp_window_attn_rope", lib().wsp_window_attn_rope(
        p.handle, _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), tp[0], tp[1], tp[2],
        Hh, D, Lt, _dtype_code(q.dtype), ctypes.c_float(0.0 if scale is None else float(scale)),
        ctypes.c_float(0.0 if theta is None else float(theta)), IO_CANONICAL if canonical else IO_LAYOUT,
        _dev_ptr(out, "out"), tp[3], _dev_ptr(workspace, "workspace"), ws_bytes, _stream(stream)))
    return out, txt_out


def fp8_amax(*tensors, amax=None, stream=None):
    """Per-head max |x| (float32 [heads]) over [rows, heads, dim] tensors (wsp_fp8_amax)."""
    torch = _torch()
    H = tensors[0].shape[1]
    if amax is None:
        with _on(stream):  # the zero fill runs on the stream the kernels use
            amax = torch.zeros(H, dtype=torch.float32, device=tensors[0].device)
    for t in tensors:
        if t.dim() != 3 or t.shape[1] != H:
            raise ValueError("tensors must be [rows, heads, dim] with one head count")
        if t.shape[0] == 0:
            continue
        _check("wsp_fp8_amax", lib().wsp_fp8_amax(_dev_ptr(t, "x"), t.shape[0], H, t.shape[2],
                                                  _dtype_code(t.dtype), _dev_ptr(amax, "amax"), _stream(stream)))
    return amax


def fp8_quantize(x, amax, out=None, stream=None):
    """E4M3 codes (torch.uint8, same shape) of x * 448/amax[head] (wsp_fp8_quantize)."""
    torch = _torch()
    if out is None:
        with _on(stream):
            out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if x.shape[0]:
        _check("wsp_fp8_quantize", lib().wsp_fp8_quantize(
            _dev_ptr(x, "x"), _dev_ptr(out, "out"), x.shape[0], x.shape[1], x.shape[2], _dtype_code(x.dtype),
            _dev_ptr(amax, "amax"), _stream(stream)))
    return out


def window_attn_qk8(p: Plan, q8, k8, v, txt_q8, txt_k8, txt_v, amax_q, amax_k, scale=None, out=None,
                    txt_out=None, workspace=None, stream=None, canonical=False, per_window=True):
    """Window attention with E4M3 q / k codes and bf16 v (wsp_window_attn_qk8)."""
    torch = _torch()
    N, Hh, D = v.shape
    Lt = txt_v.shape[0]
    if q8.shape != v.shape or k8.shape != v.shape or q8.dtype != torch.uint8 or k8.dtype != torch.uint8:
        raise ValueError("q8 / k8 must be uint8 codes shaped like v")
    if v.dtype != torch.bfloat16 or txt_v.dtype != torch.bfloat16:
        raise ValueError("v and txt_v must be bfloat16")
    need = window_attn_workspace(p, Hh, D, Lt, BF16, per_window=per_window)
    with _on(stream):
        if out is None:
            out = torch.empty_like(v)
        if txt_out is None:
            txt_out = torch.empty_like(txt_v)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=v.device)
    tp = [(_dev_ptr(t, n) if Lt else _c_vp(0)) for n, t in
          (("txt_q8", txt_q8), ("txt_k8", txt_k8), ("txt_v", txt_v), ("txt_out", txt_out))]
    _check("wsp_window_attn_qk8", lib().wsp_window_attn_qk8(
        p.handle, _dev_ptr(q8, "q8"), _dev_ptr(k8, "k8"), _dev_ptr(v, "v"), tp[0], tp[1], tp[2],
        _dev_ptr(amax_q, "amax_q"), _dev_ptr(amax_k, "amax_k"), Hh, D, Lt,
        ctypes.c_float(0.0 if scale is None else float(scale)), IO_CANONICAL if canonical else IO_LAYOUT,
        _dev_ptr(out, "out"), tp[3], _dev_ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, txt_out


def set_attn_order(order: int):
    _check("wsp_set_attn_order", lib().wsp_set_attn_order(order))


def set_attn_schedule(schedule: int):
    _check("wsp_set_attn_schedule", lib().wsp_set_attn_schedule(schedule))


def version() -> int:
    return lib().wsp_version()
