"""Plain CPU oracle of the multi-layer stack workload (test infrastructure only).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and nothing in the product
path.  Shares no code with the HIP path.

The pages define one windowed joint-attention layer ("Window-Aligned Sequence
Parallelism (SeedVR2)", sections "Motivation" and "Window layouts": layers
alternate between the regular and the shifted layout and the hidden state is
permuted between layouts at every layer boundary; "Text stream": the text
tokens get the mean of the per-window text outputs).  The 32-layer stack that
the benchmark workloads name around it is a synthetic harness, read here as
follows (the pages fix none of it):

  * per layer one set of random projections shared by video and text rows:
    q = x Wq^T, k = x Wk^T, v = x Wv^T, each [E, E] with E = heads * head_dim,
    no bias, no normalisation, no MLP, no rotary embedding;
  * the attention output of the video rows and the text mean of the text rows
    go through the output projection Wo and are added to the residual stream:
    x <- x + attn Wo^T (video rows) and t <- t + mean Wo^T (text rows);
  * layer 0 uses the regular layout, then the layouts alternate; the video
    rows enter in canonical order, are permuted into layer 0's layout, move
    between layouts at every boundary and are permuted back at the end;
  * storage points are bfloat16, rounded to nearest even exactly where the
    GPU path stores them: q / k / v, the attention output and the text mean,
    and the residual stream after each update.  Everything in between is
    float64 here (the GPU path accumulates in float32);
  * optionally (rope_theta given) q and k turn by the window-local 3D rotary
    embedding of the layer's layout after their projection (oracle/wsp_rope.py,
    "Reference quirks reproduced on purpose"; text token i at (i, i, i)) and
    are rounded to bfloat16 again.

Parity pins (tests/test_stack_pins.py): Wo = 0 leaves the stream unchanged;
zero query/key projections with identity value and output projections give
window means computed from coordinates; the projection orientation is pinned
by selection matrices; the rounding by exactly representable cases and ties.
"""
from __future__ import annotations

import numpy as np

from .wsp_oracle import canonical_plan, layer_schedule, plan, relayout, window_attn
from .wsp_rope import rope, text_positions, window_positions

__all__ = ["bf16_round", "linear", "stack_forward"]


def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value (8 significant bits, ties to even) of float64 x,
    returned as float64.  Finite inputs of normal bfloat16 range only."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)   # np.round: half to even


def linear(x, w, r=None) -> np.ndarray:
    """bf16(x w^T + r): x [M, K], w [N, K] (one output feature per row)."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    if r is not None:
        y = y + np.asarray(r, dtype=np.float64)
    return bf16_round(y)


def stack_forward(x_vid, x_txt, geo, weights, heads: int, head_dim: int, scale=None, first_layer: int = 0,
                  rope_theta=None):
    """One pass of the stack.

    x_vid: [N, E] video hidden state in canonical token order, x_txt: [Lt, E]
    text hidden state (both bfloat16 values held in float64); geo = (T, H, W,
    nt, nh, nw); weights: one (Wq, Wk, Wv, Wo) tuple per layer, each [E, E].
    first_layer: schedule index of weights[0] (the layers run are
    first_layer .. first_layer + len(weights) - 1 of the alternating
    schedule, so a pass can be resumed from any layer's state).
    rope_theta: rotary base of the optional q / k rotation (None: none).
    Returns the video state back in canonical order and the text state."""
    T, H, W = geo[:3]
    n_layers = len(weights)
    layouts = [plan(*geo, m) for m in layer_schedule(first_layer + n_layers)[first_layer:]]
    canon = canonical_plan(T, H, W)
    N, E = x_vid.shape
    Lt = x_txt.shape[0]
    x = relayout(np.asarray(x_vid, dtype=np.float64), canon, layouts[0])
    t = np.asarray(x_txt, dtype=np.float64)
    for l, (wq, wk, wv, wo) in enumerate(weights):
        X = np.concatenate([x, t], axis=0)
        q, k, v = linear(X, wq), linear(X, wk), linear(X, wv)
        if rope_theta is not None:
            # rows of X are the video tokens in layout l's order, then the text
            pos3 = np.concatenate([window_positions(layouts[l], Lt)[layouts[l].ids], text_positions(Lt)], axis=0)
            q, k = (bf16_round(rope(a.reshape(N + Lt, heads, head_dim), pos3, rope_theta)).reshape(N + Lt, -1)
                    for a in (q, k))
        split = lambda a: (a[:N].reshape(N, heads, head_dim), a[N:].reshape(Lt, heads, head_dim))
        (qv, qt), (kv, kt), (vv, vt) = split(q), split(k), split(v)
        out, mean = window_attn(layouts[l], qv, kv, vv, qt, kt, vt, scale=scale)
        A = np.concatenate([bf16_round(out).reshape(N, E), bf16_round(mean).reshape(Lt, E)], axis=0)
        X = linear(A, wo, r=X)
        x, t = X[:N], X[N:]
        if l + 1 < n_layers:
            x = relayout(x, layouts[l], layouts[l + 1])
    x = relayout(x, layouts[-1], canon)
    return x, t
