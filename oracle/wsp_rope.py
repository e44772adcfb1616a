"""Plain CPU oracle of the window-local 3D rotary position embedding (RoPE).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: imported by
``tests/`` and ``__graft_entry__.smoke()``; the product library never calls
it and shares no code or table with it.  float64 throughout.

Source: "Window-Aligned Sequence Parallelism (SeedVR2)", section "Reference
quirks reproduced on purpose":
  * positions count from each window's own corner: a video token whose
    offset from that corner is (dt, dh, dw) is rotated as if it sat at
    (text_len + dt, dh, dw), so two windows use the same indices;
  * only 3 * (head_dim // 3) channels are rotated (126 for a 128-wide head),
    and the channels beyond that width are copied unchanged.

Readings where the page is silent (listed in the design notes; parity
unpinned for these three, every other step is pinned by
``tests/test_rope_pins.py``):
  * R1 the rotated span is split into three contiguous axis blocks
    [t | h | w] of span/3 channels each, rotated in adjacent pairs
    (2k, 2k+1): (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a);
  * R2 pair i of an axis block turns by position * theta**(-2 i / (span/3)),
    theta = 10000 (the common rotary base);
  * R3 text token i uses the axial indices (i, i, i) (plain 1-D RoPE), which
    is why video temporal indices start at text_len.
Only head dims whose axis block has an even width are accepted (span/3 even:
head dim 128 gives 42); others raise ValueError.
"""
from __future__ import annotations

import numpy as np

from .wsp_oracle import Plan

ROPE_THETA = 10000.0


def rope_span(head_dim: int) -> int:
    """Rotated channels: 3 * (head_dim // 3)."""
    return 3 * (head_dim // 3)


def rope_axis_dim(head_dim: int) -> int:
    """Channels per axis block (reading R1); must be even."""
    a = rope_span(head_dim) // 3
    if a % 2 or a == 0:
        raise ValueError(f"head_dim {head_dim}: axis block of {a} channels cannot be rotated in pairs")
    return a


def window_positions(p: Plan, text_len: int) -> np.ndarray:
    """[N, 3] axial indices of every canonical token in layout p:
    (text_len + t - t0, h - h0, w - w0) for the window box containing it."""
    pos = np.empty((p.n_tokens, 3), dtype=np.int64)
    for (t0, t1, h0, h1, w0, w1) in p.boxes:
        t, h, w = np.meshgrid(np.arange(t0, t1), np.arange(h0, h1), np.arange(w0, w1), indexing="ij")
        cid = ((t * p.H + h) * p.W + w).ravel()
        pos[cid, 0] = text_len + (t - t0).ravel()
        pos[cid, 1] = (h - h0).ravel()
        pos[cid, 2] = (w - w0).ravel()
    return pos


def text_positions(text_len: int) -> np.ndarray:
    """[Lt, 3] axial indices of the text tokens (reading R3): (i, i, i)."""
    i = np.arange(text_len, dtype=np.int64)
    return np.stack([i, i, i], axis=1)


def rope_angles(pos3: np.ndarray, head_dim: int, theta: float = ROPE_THETA) -> np.ndarray:
    """[n, span/2] rotation angle of every channel pair (readings R1, R2)."""
    a = rope_axis_dim(head_dim)
    inv_freq = theta ** (-2.0 * np.arange(a // 2, dtype=np.float64) / a)
    pos3 = np.asarray(pos3, dtype=np.float64)
    return np.concatenate([pos3[:, ax:ax + 1] * inv_freq[None, :] for ax in range(3)], axis=1)


def rope(x: np.ndarray, pos3: np.ndarray, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotate x [n, heads, head_dim] (all heads alike) by the axial indices
    pos3 [n, 3]; channels past the span are copied."""
    x = np.asarray(x, dtype=np.float64)
    n, _, d = x.shape
    span = rope_span(d)
    ang = rope_angles(pos3, d, theta)                  # [n, span/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    y = x.copy()
    x0, x1 = x[:, :, 0:span:2], x[:, :, 1:span:2]
    y[:, :, 0:span:2] = x0 * c - x1 * s
    y[:, :, 1:span:2] = x0 * s + x1 * c
    return y


def rope_relayout(x: np.ndarray, src: Plan, dst: Plan, pos_layout: Plan, text_len: int,
                  theta: float = ROPE_THETA) -> np.ndarray:
    """Rows of x moved from layout src to dst, each rotated by the
    window-local axial indices its token has in layout pos_layout."""
    from .wsp_oracle import relayout
    y = relayout(x, src, dst)
    return rope(y, window_positions(pos_layout, text_len)[dst.ids], theta)
