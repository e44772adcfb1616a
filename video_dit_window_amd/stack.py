"""Multi-layer stack around the windowed joint-attention layer (synthetic
harness of the 32-layer workload).

Each layer: q / k / v projections of the hidden state (video rows followed by
the text rows, one [N + Lt, E] buffer), windowed joint attention in the
layer's layout (regular for even layers, shifted for odd), the output
projection added to the residual stream, and the layout permutation of the
video rows to the next layer's layout.  The video rows enter and leave in
canonical token order.  With ``canonical_io=True`` the stream stays in
canonical order throughout and the attention kernel reads and writes through
each layout's ids table instead (no standalone permutations).

With ``rope_theta`` set, the q and k projections apply the window-local 3D
rotary embedding of the layer's layout as they store (wsp_linear_rope; text
row i at (i, i, i)), the step right before attention in the real block.

Orchestration only: every step is a libwsp call (wsp_linear,
wsp_linear_rope, wsp_window_attn_ex, wsp_relayout); this module allocates
buffers with torch and passes pointers.
"""
from __future__ import annotations

from . import _lib as L


class Stack:
    """Plans and work buffers for one geometry; weights are passed per call.

    weights: one (Wq, Wk, Wv, Wo) tuple per layer, each a bf16 [E, E] device
    tensor (one output feature per row), E = heads * head_dim."""

    def __init__(self, T, H, W, nt, nh, nw, n_layers, heads, head_dim, text_len, device="cuda",
                 canonical_io=False, rope_theta=None):
        torch = L._torch()
        self.geo = (T, H, W, nt, nh, nw)
        self.rope_theta = rope_theta
        self.n_layers, self.heads, self.head_dim, self.text_len = n_layers, heads, head_dim, text_len
        self.E = heads * head_dim
        self.canonical_io = canonical_io
        self.canon = L.canonical(T, H, W)
        self.layouts = [L.Plan(T, H, W, nt, nh, nw, L.REGULAR if l % 2 == 0 else L.SHIFTED)
                        for l in range(min(n_layers, 2))]
        # text rows keep their order: an identity plan moves them between buffers
        self.text_plan = L.canonical(1, 1, text_len) if text_len else None
        self.N = T * H * W
        rows = self.N + text_len
        bf16 = torch.bfloat16
        self.X = [torch.empty((rows, self.E), dtype=bf16, device=device) for _ in range(1 if canonical_io else 2)]
        self.q, self.k, self.v, self.A = (torch.empty((rows, self.E), dtype=bf16, device=device)
                                          for _ in range(4))
        need = max(L.window_attn_workspace(p, heads, head_dim, text_len, L.BF16, per_window=True)
                   for p in self.layouts)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)

    def layout(self, l):
        return self.layouts[l % 2]

    def _heads(self, t, rows):
        return t.view(rows, self.heads, self.head_dim)

    def layer(self, X, l, weights, stream=None):
        """Projections, attention and residual update of layer l on buffer X
        (video rows in layer l's layout, or canonical with canonical_io)."""
        wq, wk, wv, wo = weights
        N, Lt = self.N, self.text_len
        if self.rope_theta is None:
            for w, dst in ((wq, self.q), (wk, self.k)):
                L.linear(X, w, out=dst, stream=stream)
        else:
            rows = self.canon if self.canonical_io else self.layout(l)
            for w, dst in ((wq, self.q), (wk, self.k)):
                L.linear_rope(X, w, rows, self.layout(l), Lt, theta=self.rope_theta, out=dst, stream=stream)
        L.linear(X, wv, out=self.v, stream=stream)
        hv = lambda t: self._heads(t[:N], N)
        ht = lambda t: self._heads(t[N:], Lt)
        L.window_attn(self.layout(l), hv(self.q), hv(self.k), hv(self.v), ht(self.q), ht(self.k), ht(self.v),
                      out=hv(self.A), txt_out=ht(self.A), workspace=self.ws, stream=stream,
                      canonical=self.canonical_io)
        L.linear(self.A, wo, residual=X, out=X, stream=stream)

    def _move(self, src, dst, p_src, p_dst, stream):
        N = self.N
        L.relayout(src[:N], p_src, p_dst, out=dst[:N], stream=stream)
        if self.text_len:
            L.relayout(src[N:], self.text_plan, self.text_plan, out=dst[N:], stream=stream)

    def forward(self, x_vid, x_txt, weights, out_vid=None, out_txt=None, stream=None):
        """One pass; x_vid [N, E] canonical order, x_txt [Lt, E]; returns the
        video state in canonical order and the text state (new tensors unless
        out_vid / out_txt are given)."""
        torch = L._torch()
        N = self.N
        if len(weights) != self.n_layers:
            raise ValueError("one (Wq, Wk, Wv, Wo) tuple per layer is required")
        if out_vid is None:
            out_vid = torch.empty_like(x_vid)
        if out_txt is None:
            out_txt = torch.empty_like(x_txt)
        if self.canonical_io:
            X = self.X[0]
            L.relayout(x_vid, self.canon, self.canon, out=X[:N], stream=stream)
            if self.text_len:
                L.relayout(x_txt, self.text_plan, self.text_plan, out=X[N:], stream=stream)
            for l in range(self.n_layers):
                self.layer(X, l, weights[l], stream)
            L.relayout(X[:N], self.canon, self.canon, out=out_vid, stream=stream)
        else:
            X, Y = self.X
            L.relayout(x_vid, self.canon, self.layout(0), out=X[:N], stream=stream)
            if self.text_len:
                L.relayout(x_txt, self.text_plan, self.text_plan, out=X[N:], stream=stream)
            for l in range(self.n_layers):
                self.layer(X, l, weights[l], stream)
                if l + 1 < self.n_layers:
                    self._move(X, Y, self.layout(l), self.layout(l + 1), stream)
                    X, Y = Y, X
            L.relayout(X[:N], self.layout(self.n_layers - 1), self.canon, out=out_vid, stream=stream)
        if self.text_len:
            L.relayout(X[N:], self.text_plan, self.text_plan, out=out_txt, stream=stream)
        return out_vid, out_txt
