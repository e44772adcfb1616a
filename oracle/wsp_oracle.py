"""Plain CPU oracle of the SeedVR2/NaDiT 3D-windowed joint-attention layer.

TEST INFRASTRUCTURE ONLY.  This module is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``; the
product library never calls it.  It shares no code, table or constant with
the HIP path: everything below is written out from the pages' definitions,
in float64 unless a caller asks for another dtype.

Sources (page titles and sections):
  [WSP]  "Window-Aligned Sequence Parallelism (SeedVR2)" -- sections
         "Motivation", "Window layouts", "Planner", "Plan A redistribution",
         "Text stream", "SeedVR2 integration".
  [USP]  "Parallelize new models with USP (text replica)" -- section
         "3. Attention with USP" (joint text tensors, SDPA call with
         dropout 0 and no causal mask, default scale).

Readings where the pages leave a step open (each one is listed, with its
reason, in the design notes of the repository):
  * half-window shift for an odd window: integer shift s = floor(w / 2)
    subtracted from every cut (so the first clipped window is ceil(w/2) long);
  * windows that would be empty are not emitted;
  * rounding is Python's round() (half to even) on IEEE doubles;
  * softmax scale 1/sqrt(D), no mask inside a window, no dropout;
  * segment order [video window; text] (order does not change the result of
    unmasked attention);
  * the text mean divides by the number of windows of the current layout.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, brute force on tiny inputs, invariants the pages state
and the shapes the workload descriptions print.  The one reading that no pin
can settle is the odd-window shift rounding above; it is a single constant,
``SHIFT_FLOOR``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "REGULAR", "SHIFTED", "CANONICAL", "MAX_TEMPORAL_WINDOW", "SHIFT_FLOOR",
    "window_size", "axis_intervals", "Plan", "plan", "canonical_plan",
    "relayout", "relayout_perm", "layer_schedule", "transitions",
    "joint_attention", "window_attn", "text_mean", "attn_flops", "relayout_bytes",
]

REGULAR = 0
SHIFTED = 1
CANONICAL = 2

# [WSP] "Window layouts": the temporal extent fed to the window-size rule is
# capped at 30 frames.
MAX_TEMPORAL_WINDOW = 30

# [WSP] "Window layouts": the shifted tiling moves each cut by half a window.
# For an odd window w that is not an integer; this oracle reads it as
# floor(w / 2).  (Unpinned by the pages; see the module docstring.)
SHIFT_FLOOR = True


# ---------------------------------------------------------------------------
# window geometry
# ---------------------------------------------------------------------------
def window_size(T: int, H: int, W: int, nt: int, nh: int, nw: int):
    """Window extents (wt, wh, ww) for a post-patch grid.

    [WSP] "Window layouts": the spatial window is normalised to a 45x80
    (720p) reference area -- scale = sqrt(45*80/(H*W)); the rounded, rescaled
    grid is split into nh x nw parts with a ceiling; the temporal window is
    ceil(min(T, 30) / nt).  Written as the page states it: float scale,
    Python round(), ceiling of a true division.
    """
    for name, val in (("T", T), ("H", H), ("W", W), ("nt", nt), ("nh", nh), ("nw", nw)):
        if int(val) != val or val <= 0:
            raise ValueError(f"{name} must be a positive integer, got {val!r}")
    scale = math.sqrt(45 * 80 / (H * W))
    wh = math.ceil(round(H * scale) / nh)
    ww = math.ceil(round(W * scale) / nw)
    wt = math.ceil(min(T, MAX_TEMPORAL_WINDOW) / nt)
    if wh <= 0 or ww <= 0 or wt <= 0:
        raise ValueError(f"window size rounds to zero: (wt, wh, ww) = ({wt}, {wh}, {ww})")
    return wt, wh, ww


def axis_intervals(n: int, w: int, method: int):
    """Half-open intervals [a, b) that cut one axis of length n.

    [WSP] "Window layouts": regular cuts sit at the multiples of w, the last
    interval ending at n.  Shifted cuts sit half a window earlier, and each
    interval is clamped to [0, n], so the first and last ones are shorter;
    nothing wraps from one end of the axis to the other (unlike a cyclic
    roll).  Empty intervals are not produced.
    """
    if method == REGULAR:
        s = 0
    elif method == SHIFTED:
        s = w // 2 if SHIFT_FLOOR else int(math.ceil(w / 2))
    else:
        raise ValueError(f"unknown window method {method!r}")
    out = []
    i = 0
    while i * w - s < n:
        a = max(i * w - s, 0)
        b = min((i + 1) * w - s, n)
        if b > a:
            out.append((a, b))
        i += 1
    return out


@dataclass
class Plan:
    """A window layout of a (T, H, W) token grid.

    ids[j]  -- canonical token id held at layout position j
    inv[c]  -- layout position of canonical token id c (inverse of ids)
    offsets -- window w owns layout positions offsets[w] .. offsets[w+1]-1
    boxes   -- per window (t0, t1, h0, h1, w0, w1), half-open
    lpt     -- window ids sorted by (-video token count, window id)
    """
    T: int
    H: int
    W: int
    method: int
    win: tuple
    boxes: np.ndarray
    offsets: np.ndarray
    ids: np.ndarray
    inv: np.ndarray
    lpt: np.ndarray
    extents: dict = field(default_factory=dict)

    @property
    def n_tokens(self) -> int:
        return self.T * self.H * self.W

    @property
    def n_windows(self) -> int:
        return len(self.offsets) - 1

    def lengths(self) -> np.ndarray:
        return np.diff(self.offsets)


def plan(T: int, H: int, W: int, nt: int, nh: int, nw: int, method: int) -> Plan:
    """Window tables of one layout.

    [WSP] "Window layouts": window ids count the w intervals in the outer
    loop and the t intervals in the inner loop; a window lists its tokens
    with t varying slowest and w fastest; token (t, h, w) has canonical id
    (t*H + h)*W + w.
    [WSP] "Planner": the largest-first order sorts windows by
    (-video_token_count, original_window_id).
    """
    wt, wh, ww = window_size(T, H, W, nt, nh, nw)
    ti = axis_intervals(T, wt, method)
    hi = axis_intervals(H, wh, method)
    wi = axis_intervals(W, ww, method)
    boxes, offsets, ids = [], [0], []
    for (w0, w1) in wi:
        for (h0, h1) in hi:
            for (t0, t1) in ti:
                boxes.append((t0, t1, h0, h1, w0, w1))
                for t in range(t0, t1):
                    for h in range(h0, h1):
                        row = (t * H + h) * W  # canonical id of (t, h, 0)
                        ids.extend(range(row + w0, row + w1))
                offsets.append(len(ids))
    ids = np.asarray(ids, dtype=np.int64)
    inv = np.empty_like(ids)
    inv[ids] = np.arange(len(ids), dtype=np.int64)
    offsets = np.asarray(offsets, dtype=np.int64)
    lengths = np.diff(offsets)
    lpt = np.asarray(sorted(range(len(lengths)), key=lambda k: (-int(lengths[k]), k)),
                     dtype=np.int64)
    return Plan(T, H, W, method, (wt, wh, ww), np.asarray(boxes, dtype=np.int64),
                offsets, ids, inv, lpt,
                {"t": [b - a for a, b in ti], "h": [b - a for a, b in hi],
                 "w": [b - a for a, b in wi]})


def canonical_plan(T: int, H: int, W: int) -> Plan:
    """The canonical (identity) layout: one window, ids = arange(T*H*W)."""
    n = T * H * W
    ar = np.arange(n, dtype=np.int64)
    return Plan(T, H, W, CANONICAL, (T, H, W), np.asarray([(0, T, 0, H, 0, W)]),
                np.asarray([0, n], dtype=np.int64), ar, ar.copy(),
                np.asarray([0], dtype=np.int64), {"t": [T], "h": [H], "w": [W]})


# ---------------------------------------------------------------------------
# relayout
# ---------------------------------------------------------------------------
def relayout_perm(src: Plan, dst: Plan) -> np.ndarray:
    """perm[j] = source position of the token that destination position j holds.

    [WSP] "Plan A redistribution": when every token stays on its rank the
    transition is a local permutation.  Destination position j holds canonical
    token dst.ids[j], which sits at position src.inv[dst.ids[j]] in the source.
    """
    if (src.T, src.H, src.W) != (dst.T, dst.H, dst.W):
        raise ValueError("relayout between different token grids")
    return src.inv[dst.ids]


def relayout(x: np.ndarray, src: Plan, dst: Plan) -> np.ndarray:
    """Move whole rows of x (first axis = layout position) from src to dst."""
    x = np.asarray(x)
    if x.shape[0] != src.n_tokens:
        raise ValueError("row count does not match the grid")
    return x[relayout_perm(src, dst)]


# ---------------------------------------------------------------------------
# layer schedule
# ---------------------------------------------------------------------------
def layer_schedule(num_layers: int):
    """[WSP] "Motivation": consecutive layers switch between the regular and
    the shifted layout; layer 0 is regular."""
    return [REGULAR if l % 2 == 0 else SHIFTED for l in range(num_layers)]


def transitions(schedule) -> int:
    """[WSP] "Window layouts": layout transitions follow the schedule itself
    (one per pair of adjacent layers whose methods differ)."""
    return sum(1 for a, b in zip(schedule, schedule[1:]) if a != b)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def joint_attention(q_vid, k_vid, v_vid, txt_q, txt_k, txt_v, scale=None,
                    dtype=np.float64, text_only=False):
    """Attention of one window and one head over the joint segment.

    q_vid/k_vid/v_vid: [L, D] video rows of the window; txt_q/k/v: [Lt, D].
    Returns (video_out [L, D] or None when ``text_only``, text_out [Lt, D]).

    [WSP] "SeedVR2 integration": the window's packed segment is
    [video window; replicated text].  [USP] "3. Attention with USP": the
    attention is SDPA of that joint sequence with no mask and no dropout;
    scale defaults to 1/sqrt(D).
    """
    D = np.shape(txt_q)[-1] if np.size(txt_q) else np.shape(q_vid)[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    K = np.concatenate([k_vid, txt_k], axis=0).astype(dtype)
    V = np.concatenate([v_vid, txt_v], axis=0).astype(dtype)
    if text_only:
        Q = np.asarray(txt_q).astype(dtype)
    else:
        Q = np.concatenate([q_vid, txt_q], axis=0).astype(dtype)
    P = _softmax_rows((Q @ K.T) * dtype(scale))
    O = P @ V
    if text_only:
        return None, O
    L = len(q_vid)
    return O[:L], O[L:]


def window_attn(p: Plan, q, k, v, txt_q, txt_k, txt_v, scale=None,
                windows=None, heads=None, dtype=np.float64, keep_windows=False):
    """Joint attention inside every window, plus the window-averaged text output.

    q, k, v:          [N, H, D] rows in p's layout.
    txt_q/k/v:        [Lt, H, D], the same for every window.
    returns (out [N, H, D], txt_out [Lt, H, D]) in ``dtype``; rows of windows
    not in ``windows`` (or heads not in ``heads``) are left as NaN, and the
    text mean then only covers the listed heads (its divisor is always the
    layout's window count).

    Each (window, head) is ``joint_attention``.  [WSP] "Text stream": every
    window yields one text output T_w; the next text state is the sum of all
    T_w divided by the number of windows (not a token-weighted mean).
    """
    q, k, v = (np.asarray(a) for a in (q, k, v))
    txt_q, txt_k, txt_v = (np.asarray(a) for a in (txt_q, txt_k, txt_v))
    N, Hh, D = q.shape
    Lt = txt_q.shape[0]
    if N != p.n_tokens or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q/k/v shape does not match the plan")
    if txt_q.shape != (Lt, Hh, D) or txt_k.shape != txt_q.shape or txt_v.shape != txt_q.shape:
        raise ValueError("text tensors must be [Lt, H, D]")
    windows = range(p.n_windows) if windows is None else list(windows)
    heads = range(Hh) if heads is None else list(heads)
    out = np.full((N, Hh, D), np.nan, dtype=dtype)
    tsum = np.zeros((Lt, Hh, D), dtype=dtype)
    per_window = {}
    for w in windows:
        a, b = int(p.offsets[w]), int(p.offsets[w + 1])
        for h in heads:
            ov, ot = joint_attention(q[a:b, h], k[a:b, h], v[a:b, h], txt_q[:, h], txt_k[:, h],
                                     txt_v[:, h], scale=scale, dtype=dtype)
            out[a:b, h, :] = ov
            tsum[:, h, :] += ot
            if keep_windows:
                per_window[(w, h)] = ot.copy()
    txt_out = text_mean(tsum, p.n_windows)
    if keep_windows:
        return out, txt_out, per_window
    return out, txt_out


def text_mean(text_sum, n_windows: int):
    """[WSP] "Text stream": T_next = (sum over windows of T_w) / window count."""
    if n_windows <= 0:
        raise ValueError("text mean over zero windows")
    return text_sum / n_windows


# ---------------------------------------------------------------------------
# algorithmic work (for reporting)
# ---------------------------------------------------------------------------
def attn_flops(p: Plan, n_heads: int, head_dim: int, text_len: int) -> int:
    """QK^T and PV multiply-adds (2 FLOP each) of all video and text queries:
    4 * D * H * sum_w (L_w + Lt)^2."""
    L = p.lengths().astype(np.int64) + text_len
    return int(4 * head_dim * n_heads * int((L * L).sum()))


def relayout_bytes(n_rows: int, row_bytes: int) -> int:
    """Read and write every row once, plus one 4-byte index per row."""
    return 2 * n_rows * row_bytes + 4 * n_rows
