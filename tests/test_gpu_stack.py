"""GPU parity of the multi-layer stack workload: wsp_linear (bf16 projection)
and the stack driver against the CPU oracle (oracle/wsp_stack.py).

wsp_linear is compared element by element with the float64 product rounded
once to bfloat16: at most one bfloat16 ulp apart plus the float32
accumulation error bound K * 2^-24 * sum|x w| (float32 accumulation can move
a result across a rounding tie, or matter near zero), on ragged row counts,
with and without a residual, in place.  The stack runs 1, 3 and all 32 alternating
layers (31 layout transitions, a text mean per layer) on the tiny grid and
32 layers on a mid grid in full against the oracle, with the explicit
permutations and canonical-order I/O agreeing bit for bit; at 32 layers
every layer is also checked from the GPU's own state before it (so rounding
differences of earlier layers do not compound into the comparison), and the
end state against the oracle run from the input.  At the full 1080p,
2560-wide configuration one layer is checked on the largest window's rows
and the second (shifted) layer on the largest shifted window's rows.
"""
import numpy as np
import pytest

import oracle as O
import video_dit_window_amd as W
import wsp_inputs as I
from helpers import check_bf16, dev_bits, from_dev, log
from video_dit_window_amd.stack import Stack

pytestmark = pytest.mark.gpu


def bf16_dev(a):
    """float64 array of bf16 values -> device bf16 tensor (exact)."""
    import torch
    bits = I.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def rnd_bf16(shape, seed, std=1.0):
    return O.bf16_round(np.random.default_rng(seed).standard_normal(shape) * std)


def ulp_bf16(x):
    """Spacing of bfloat16 values at |x| (8 significant bits)."""
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, e - 8)


def check_linear(M, N, K, residual, in_place, seed):
    import torch
    x, w = rnd_bf16((M, K), seed), rnd_bf16((N, K), seed + 1, std=0.05)
    r = rnd_bf16((M, N), seed + 2) if residual else None
    dx, dw = bf16_dev(x), bf16_dev(w)
    dr = bf16_dev(r) if residual else None
    if in_place:
        y = W.linear(dx, dw, residual=dr, out=dr)
    else:
        y = W.linear(dx, dw, residual=dr)
    torch.cuda.synchronize()
    got, ref = from_dev(y), O.linear(x, w, r)
    err = np.abs(got - ref)
    acc = 2.0 * K * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T + (np.abs(r) if residual else 0.0))
    bound = ulp_bf16(np.abs(ref) + acc) + acc
    log(f"  linear M={M} N={N} K={K} res={residual} in_place={in_place}: max|err| = {err.max():.3e}, "
        f"elements not correctly rounded: {int((err > 0).sum())} of {err.size}")
    assert np.all(err <= bound), "beyond one bf16 ulp plus the float32 accumulation bound"
    check_bf16(got, ref, "linear")


@pytest.mark.parametrize("M,N,K", [(1, 256, 64), (300, 256, 192), (1000, 512, 640), (4099, 768, 2560)])
def test_linear(gpu, M, N, K):
    check_linear(M, N, K, residual=False, in_place=False, seed=M + N)


@pytest.mark.parametrize("in_place", [False, True])
def test_linear_residual(gpu, in_place):
    check_linear(777, 512, 256, residual=True, in_place=in_place, seed=9)


def test_linear_rejects_bad_shapes(gpu):
    """N not a multiple of 256, K not a multiple of 64 and float32 operands
    are refused with an error (nothing is launched)."""
    import torch
    z = lambda *shape, dt=torch.bfloat16: torch.zeros(shape, dtype=dt, device="cuda")
    for (n, k) in ((128, 64), (256, 96)):
        with pytest.raises(W.WspError):
            W.linear(z(8, k), z(n, k))
    with pytest.raises(W.WspError):
        W.linear(z(8, 64, dt=torch.float32), z(256, 64, dt=torch.float32))
    y = W.linear(z(0, 64), z(256, 64))      # no rows: nothing to do
    assert tuple(y.shape) == (0, 256)


def check_update(got, ref, inp, what):
    """Relative L2 error of the layer updates (stream minus its input)."""
    du, ru = got - inp, ref - inp
    rel = float(np.linalg.norm(du - ru) / max(np.linalg.norm(ru), 1e-30))
    log(f"  {what}: rel-L2 = {rel:.3e} (bar 2e-2)")
    assert rel <= 2e-2, f"{what}: relative L2 error {rel}"


GEO = (5, 20, 36, 2, 3, 3)
HEADS, HD, LT = 4, 64, 16


def stack_inputs(n_layers, seed, wstd=0.06):
    E = HEADS * HD
    N = GEO[0] * GEO[1] * GEO[2]
    x, t = rnd_bf16((N, E), seed), rnd_bf16((LT, E), seed + 1)
    weights = [tuple(rnd_bf16((E, E), seed + 10 + 4 * l + i, std=wstd) for i in range(4)) for l in range(n_layers)]
    return x, t, weights


@pytest.mark.parametrize("n_layers", [1, 3])
def test_stack_tiny(gpu, n_layers):
    """A few alternating layers on the tiny grid (4 heads x 64, 16 text
    tokens): explicit permutations and canonical-order I/O agree bit for bit
    and match the oracle."""
    import torch
    x, t, weights = stack_inputs(n_layers, seed=40 + n_layers)
    dw = [tuple(bf16_dev(a) for a in wl) for wl in weights]
    res = {}
    for canon in (False, True):
        st = Stack(*GEO, n_layers, HEADS, HD, LT, canonical_io=canon)
        res[canon] = st.forward(bf16_dev(x), bf16_dev(t), dw)
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits(res[False][0]), dev_bits(res[True][0])), "video state: I/O orders differ"
    assert np.array_equal(dev_bits(res[False][1]), dev_bits(res[True][1])), "text state: I/O orders differ"
    ref_x, ref_t = O.stack_forward(x, t, GEO, weights, HEADS, HD)
    check_bf16(from_dev(res[False][0]), ref_x, f"stack {n_layers} layers video")
    check_bf16(from_dev(res[False][1]), ref_t, f"stack {n_layers} layers text")
    # The stream is dominated by its input (checked element-wise above); its
    # update must match too, in relative L2 within the bf16 bar.
    for got, ref, inp, what in ((res[False][0], ref_x, x, "video"), (res[False][1], ref_t, t, "text")):
        check_update(from_dev(got), ref, inp, f"stack {n_layers} layers {what} update")


STACK32 = [  # (name, geometry, heads, head_dim, text_len, weight std, seed)
    ("tiny", GEO, HEADS, HD, LT, 0.03, 60),
    ("mid", (6, 30, 52, 2, 3, 3), 2, 128, 40, 0.03, 70),
]


def oracle_layer_attention(xi, ti, geo, wl, heads, hd, layer):
    """Attention output of one stack layer computed by the oracle from the
    stream state (xi canonical order, ti text rows): q/k/v projections,
    window attention in the layer's layout and the text mean, returned with
    the video rows in canonical order."""
    N, E = xi.shape
    lt = ti.shape[0]
    lay = O.plan(*geo, O.REGULAR if layer % 2 == 0 else O.SHIFTED)
    can = O.canonical_plan(*geo[:3])
    X = np.concatenate([O.relayout(xi, can, lay), ti], axis=0)
    q, k, v = (O.linear(X, wm) for wm in wl[:3])
    split = lambda a: (a[:N].reshape(N, heads, hd), a[N:].reshape(lt, heads, hd))
    (qv, qt), (kv, kt), (vv, vt) = split(q), split(k), split(v)
    out, mean = O.window_attn(lay, qv, kv, vv, qt, kt, vt)
    return O.relayout(out.reshape(N, E), lay, can), mean.reshape(lt, E)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", STACK32, ids=[c[0] for c in STACK32])
def test_stack_32_layers(gpu, case):
    """The 32-layer alternating stack (layer 0 regular, 31 transitions).
    Weight std 0.03 at width 256 keeps the stream bounded over 32 layers (the
    tiny tests' 0.06 makes it grow ~200-fold, where float32 and float64
    arithmetic part ways whatever the implementation).  Every layer is
    checked from the GPU's own state before it: its attention output (video
    rows and text mean) at the attention bar, and the stream after its
    residual update.  A layer's update is then only a few bf16 steps of the
    stream, too fine to compare as a difference of two rounded streams, so the
    attention output stands in for it (the projection with its residual add
    is checked on its own by test_linear_residual)."""
    import torch
    name, geo, heads, hd, lt, wstd, seed = case
    E, N = heads * hd, geo[0] * geo[1] * geo[2]
    rng = np.random.default_rng(seed)
    x, t = O.bf16_round(rng.standard_normal((N, E))), O.bf16_round(rng.standard_normal((lt, E)))
    weights = [tuple(O.bf16_round(rng.standard_normal((E, E)) * wstd) for _ in range(4)) for _ in range(32)]
    dw = [tuple(bf16_dev(a) for a in wl) for wl in weights]
    dx, dt = bf16_dev(x), bf16_dev(t)
    # GPU state after every prefix of layers and the last layer's attention
    # output, canonical-order I/O
    states, attn = [(x, t)], []
    for n in range(1, 33):
        st = Stack(*geo, n, heads, hd, lt, canonical_io=True)
        xo, to = st.forward(dx, dt, dw[:n])
        torch.cuda.synchronize()
        states.append((from_dev(xo), from_dev(to)))
        attn.append(from_dev(st.A))
    # the whole pass with explicit permutations: same bits
    xe, te = Stack(*geo, 32, heads, hd, lt, canonical_io=False).forward(dx, dt, dw)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(xe), states[32][0]), "video state: I/O orders differ"
    assert np.array_equal(from_dev(te), states[32][1]), "text state: I/O orders differ"
    log(f"  {name}: every layer from the GPU's own state before it")
    for l in range(32):
        (xi, ti), (xg, tg) = states[l], states[l + 1]
        ra, rm = oracle_layer_attention(xi, ti, geo, weights[l], heads, hd, l)
        check_bf16(attn[l][:N], ra, f"{name} layer {l} attention, video rows")
        check_bf16(attn[l][N:], rm, f"{name} layer {l} text mean")
        rx, rt = O.stack_forward(xi, ti, geo, weights[l:l + 1], heads, hd, first_layer=l)
        check_bf16(xg, rx, f"{name} layer {l} video state")
        check_bf16(tg, rt, f"{name} layer {l} text state")
    # End to end, 32 roundings of the stream apart: the relative L2 part of
    # the bf16 bar (the element bar is applied per layer above, where one
    # layer's arithmetic is compared; over 32 layers single elements drift by
    # rounding-boundary crossings that compound).
    rx, rt = O.stack_forward(x, t, geo, weights, heads, hd)
    for got, ref, what in ((states[32][0], rx, "video"), (states[32][1], rt, "text")):
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        ratio = float(np.max(np.abs(got - ref) / (3e-2 + 2e-2 * np.abs(ref))))
        log(f"  {name} 32 layers {what} from the input: rel-L2 {rel:.3e} (bar 2e-2), element ratio {ratio:.3f}")
        assert np.isfinite(got).all() and rel <= 2e-2, f"{name} 32 layers {what}: relative L2 error {rel}"


def test_stack_1080p_one_layer_sampled(gpu):
    """One layer of the 1080p, 20 x 128, 256-text-token configuration: the
    video rows of the largest window (all heads, all 2560 features) against
    the oracle's projections and window attention of that window."""
    import torch
    w = I.WORKLOADS["1080p_bf16"]
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    E, Lt, N = w.heads * w.head_dim, w.text_len, w.n_tokens
    rng = np.random.default_rng(77)
    log("  generating 1080p stack inputs")
    x = O.bf16_round(rng.standard_normal((N, E), dtype=np.float32))
    t = O.bf16_round(rng.standard_normal((Lt, E), dtype=np.float32))
    wts = [O.bf16_round(rng.standard_normal((E, E), dtype=np.float32) * 0.02) for _ in range(4)]
    st = Stack(*geo, 1, w.heads, w.head_dim, Lt)
    xo, to = st.forward(bf16_dev(x), bf16_dev(t), [tuple(bf16_dev(a) for a in wts)])
    torch.cuda.synchronize()
    op = O.plan(*geo, O.REGULAR)
    win = int(op.lpt[0])
    ids = op.ids[op.offsets[win]:op.offsets[win + 1]]
    log(f"  oracle for window {win} ({len(ids)} rows)")
    X = np.concatenate([x[ids], t], axis=0)
    q, k, v = (O.linear(X, wm).reshape(-1, w.heads, w.head_dim) for wm in wts[:3])
    L = len(ids)
    out = np.empty((L, w.heads, w.head_dim))
    for h in range(w.heads):
        out[:, h], _ = O.joint_attention(q[:L, h], k[:L, h], v[:L, h], q[L:, h], k[L:, h], v[L:, h])
    ref = O.linear(O.bf16_round(out).reshape(L, E), wts[3], r=x[ids])
    got = from_dev(xo[torch.from_numpy(ids.astype(np.int64)).cuda()])
    check_bf16(got, ref, f"1080p stack layer, window {win}")
    check_update(got, ref, x[ids], f"1080p stack layer update, window {win}")


def test_stack_1080p_two_layers_sampled(gpu):
    """Two layers of the 1080p, 20 x 128, 256-text-token configuration with
    canonical-order I/O (the benchmark's stack): the second, shifted layer on
    the rows of the largest shifted window, computed by the oracle from the
    GPU's state after the first layer (video rows of that window and the text
    rows), and the first layer on the largest regular window's rows."""
    import torch
    w = I.WORKLOADS["1080p_bf16"]
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    E, Lt, N = w.heads * w.head_dim, w.text_len, w.n_tokens
    rng = np.random.default_rng(78)
    log("  generating 1080p stack inputs")
    x = O.bf16_round(rng.standard_normal((N, E), dtype=np.float32))
    t = O.bf16_round(rng.standard_normal((Lt, E), dtype=np.float32))
    wts = [[O.bf16_round(rng.standard_normal((E, E), dtype=np.float32) * 0.02) for _ in range(4)] for _ in range(2)]
    dw = [tuple(bf16_dev(a) for a in wl) for wl in wts]
    dx, dt = bf16_dev(x), bf16_dev(t)
    x1, t1 = Stack(*geo, 1, w.heads, w.head_dim, Lt, canonical_io=True).forward(dx, dt, dw[:1])
    x2, _ = Stack(*geo, 2, w.heads, w.head_dim, Lt, canonical_io=True).forward(dx, dt, dw)
    torch.cuda.synchronize()
    host_t1 = from_dev(t1)

    def oracle_window(xin, tin, ws, method):
        op = O.plan(*geo, method)
        win = int(op.lpt[0])
        ids = op.ids[op.offsets[win]:op.offsets[win + 1]]
        X = np.concatenate([xin(ids), tin], axis=0)
        q, k, v = (O.linear(X, wm).reshape(-1, w.heads, w.head_dim) for wm in ws[:3])
        L = len(ids)
        out = np.empty((L, w.heads, w.head_dim))
        for h in range(w.heads):
            out[:, h], _ = O.joint_attention(q[:L, h], k[:L, h], v[:L, h], q[L:, h], k[L:, h], v[L:, h])
        return win, ids, O.linear(O.bf16_round(out).reshape(L, E), ws[3], r=xin(ids))

    rows = lambda dev: (lambda ids: from_dev(dev[torch.from_numpy(ids.astype(np.int64)).cuda()]))
    win, ids, ref = oracle_window(lambda i: x[i], t, wts[0], O.REGULAR)
    got = rows(x1)(ids)
    check_bf16(got, ref, f"1080p stack layer 0, regular window {win}")
    check_update(got, ref, x[ids], f"1080p stack layer 0 update, regular window {win}")
    win, ids, ref = oracle_window(rows(x1), host_t1, wts[1], O.SHIFTED)
    got = rows(x2)(ids)
    check_bf16(got, ref, f"1080p stack layer 1, shifted window {win}")
    check_update(got, ref, rows(x1)(ids), f"1080p stack layer 1 update, shifted window {win}")


# ---- q / k projections with the window-local rotary embedding (wsp_linear_rope)

ROPE_GEO = (6, 30, 52, 2, 3, 3)     # 9360 video rows: the last 256-row tile is ragged
ROPE_CASES = [("canonical", "regular"), ("canonical", "shifted"), ("regular", "regular"),
              ("shifted", "shifted"), ("canonical", "canonical")]


def rope_plans(geo):
    return {"canonical": W.canonical(*geo[:3]), "regular": W.Plan(*geo, W.REGULAR),
            "shifted": W.Plan(*geo, W.SHIFTED)}


def linear_rope_chain(dx, dw, g, rows, pos, text_len, theta):
    """wsp_linear, then wsp_rope_relayout (src = dst = rows) over the video
    rows and wsp_rope_text over the text rows."""
    import torch
    plain = W.linear(dx, dw)
    n, heads = g[rows].n_tokens, dw.shape[0] // 128
    ref = torch.empty_like(plain)
    W.rope_relayout(plain[:n].view(n, heads, 128), g[rows], g[rows], g[pos], text_len, theta=theta,
                    out=ref[:n].view(n, heads, 128))
    if text_len:
        W.rope_text(plain[n:].view(text_len, heads, 128), theta=theta, out=ref[n:].view(text_len, heads, 128))
    return ref


@pytest.mark.parametrize("text_len", [0, 19])
@pytest.mark.parametrize("case", ROPE_CASES, ids=["-".join(c) for c in ROPE_CASES])
def test_linear_rope_bit_identical_to_chain(gpu, case, text_len):
    """The rotation in the projection's epilogue leaves exactly what the
    projection followed by the stand-alone rotation kernels leaves (4 heads,
    K = 192, rows in canonical or layout order; theta 500 with text)."""
    import torch
    rows, pos = case
    g = rope_plans(ROPE_GEO)
    M = g[rows].n_tokens + text_len
    seed = 300 + 7 * ROPE_CASES.index(case) + text_len
    dx, dw = bf16_dev(rnd_bf16((M, 192), seed)), bf16_dev(rnd_bf16((512, 192), seed + 1, std=0.08))
    theta = 500.0 if text_len else None
    y = W.linear_rope(dx, dw, g[rows], g[pos], text_len, theta=theta)
    ref = linear_rope_chain(dx, dw, g, rows, pos, text_len, theta)
    torch.cuda.synchronize()
    same = torch.equal(y.view(torch.int16), ref.view(torch.int16))
    log(f"  linear_rope rows {rows}, positions of {pos}, text_len {text_len}: bit-identical = {same}")
    assert same


def oracle_linear_rope(x, w, ids_rows, pos_plan, text_len, theta=O.ROPE_THETA):
    """Oracle of the rotated projection for rows x (video rows first, tokens
    ids_rows, then text rows): bf16(rope(bf16(x w^T))) and the per-element
    error allowance of the GPU's float32 arithmetic."""
    n = len(ids_rows)
    p = O.linear(x, w)
    heads = w.shape[0] // 128
    pos3 = np.concatenate([O.window_positions(pos_plan, text_len)[ids_rows], O.text_positions(text_len)], axis=0)
    ref = O.bf16_round(O.rope(p.reshape(-1, heads, 128), pos3, theta).reshape(p.shape))
    # the product may round to the neighbouring bf16 value (float32
    # accumulation, as test_linear's bound); a rotated pair mixes both of its
    # channels' errors; the result rounds once more (2^-8 relative)
    acc = 2.0 * x.shape[1] * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T)
    d = (ulp_bf16(np.abs(p) + acc) + acc).reshape(-1, heads, 64, 2)
    pair = np.repeat(d.sum(axis=3, keepdims=True), 2, axis=3)
    pair[:, :, 63, :] = d[:, :, 63, :]                 # channels 126, 127 pass through
    return ref, 2.0 ** -8 * np.abs(ref) + 1e-6 + pair.reshape(p.shape)


@pytest.mark.parametrize("method", ["regular", "shifted"])
@pytest.mark.parametrize("rows", ["canonical", "layout"])
def test_linear_rope_oracle(gpu, method, rows):
    """Against the float64 oracle: the projection rounded to bf16, rotated by
    the oracle's window-local positions (text rows at (i, i, i)), rounded
    again -- element by element within the float32 allowance, and at the bf16
    bar."""
    import torch
    T, H, Wd, nt, nh, nw = ROPE_GEO
    om = O.REGULAR if method == "regular" else O.SHIFTED
    op = O.plan(*ROPE_GEO, om)
    g = rope_plans(ROPE_GEO)
    ids = np.arange(T * H * Wd) if rows == "canonical" else op.ids
    rp = g["canonical"] if rows == "canonical" else g[method]
    Lt = 40
    x = rnd_bf16((len(ids) + Lt, 256), 330 + len(method) + len(rows))
    w = rnd_bf16((512, 256), 331, std=0.08)
    y = W.linear_rope(bf16_dev(x), bf16_dev(w), rp, g[method], Lt)
    torch.cuda.synchronize()
    ref, bound = oracle_linear_rope(x, w, ids, op, Lt)
    got = from_dev(y)
    err = np.abs(got - ref)
    log(f"  linear_rope {rows} rows, {method} positions: max|err| {err.max():.3e}, "
        f"{int((err > bound).sum())} beyond the allowance")
    assert np.all(err <= bound)
    check_bf16(got, ref, f"linear_rope {rows} rows, {method} positions")


def test_linear_rope_1080p(gpu):
    """The 1080p q / k projection (171360 video rows in canonical order + 256
    text rows, 2560 -> 2560, 20 heads of 128), rotated for the shifted layout:
    bit-identical to the two-pass chain over the whole output, and sampled
    rows (video rows of several windows and text rows) against the oracle."""
    import torch
    w = I.WORKLOADS["1080p_bf16"]
    geo = (w.T, w.H, w.W, w.nt, w.nh, w.nw)
    E, Lt, N = w.heads * w.head_dim, w.text_len, w.n_tokens
    g = rope_plans(geo)
    rng = np.random.default_rng(91)
    log("  generating 1080p projection inputs")
    xb = I.f32_to_bf16_bits(rng.standard_normal((N + Lt, E), dtype=np.float32))
    wb = I.f32_to_bf16_bits(rng.standard_normal((E, E), dtype=np.float32) * np.float32(0.02))
    dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    dx, dw = dev(xb), dev(wb)
    y = W.linear_rope(dx, dw, g["canonical"], g["shifted"], Lt)
    ref = linear_rope_chain(dx, dw, g, "canonical", "shifted", Lt, None)
    torch.cuda.synchronize()
    same = torch.equal(y.view(torch.int16), ref.view(torch.int16))
    log(f"  1080p linear_rope vs chain: bit-identical = {same}")
    assert same
    del ref
    sample = np.concatenate([rng.choice(N, 96, replace=False), [0, N - 1], N + np.arange(0, Lt, 37), [N + Lt - 1]])
    x = I.bf16_bits_to_f32(xb[sample]).astype(np.float64)
    wv = I.bf16_bits_to_f32(wb).astype(np.float64)
    op = O.plan(*geo, O.SHIFTED)
    vid = sample < N
    pos = np.concatenate([O.window_positions(op, Lt)[sample[vid]], O.text_positions(Lt)[sample[~vid] - N]], axis=0)
    p = O.linear(x, wv)
    want = O.bf16_round(O.rope(p.reshape(-1, w.heads, 128), pos).reshape(p.shape))
    got = from_dev(y[torch.from_numpy(sample.astype(np.int64)).cuda()])
    check_bf16(got, want, "1080p linear_rope, sampled rows")


def test_linear_rope_rejects_bad_arguments(gpu):
    """Row count not the plan's tokens + text, float32 operands, N not a
    multiple of 256: refused before any launch."""
    import torch
    g = rope_plans(ROPE_GEO)
    n = g["canonical"].n_tokens
    z = lambda *shape, dt=torch.bfloat16: torch.zeros(shape, dtype=dt, device="cuda")
    with pytest.raises(ValueError):
        W.linear_rope(z(n + 3, 64), z(256, 64), g["canonical"], g["regular"], 2)
    with pytest.raises(W.WspError):
        W.linear_rope(z(n, 64, dt=torch.float32), z(256, 64, dt=torch.float32), g["canonical"], g["regular"], 0)
    with pytest.raises(W.WspError):
        W.linear_rope(z(n, 64), z(128, 64), g["canonical"], g["regular"], 0)


@pytest.mark.parametrize("n_layers", [1, 3])
def test_stack_rope_tiny(gpu, n_layers):
    """Layers with rotated q / k (2 heads of 128, 16 text tokens) on the tiny
    grid: explicit permutations and canonical-order I/O agree bit for bit and
    match the oracle's stack with the rotation."""
    import torch
    heads, hd, lt = 2, 128, 16
    E, N = heads * hd, GEO[0] * GEO[1] * GEO[2]
    rng = np.random.default_rng(500 + n_layers)
    x, t = O.bf16_round(rng.standard_normal((N, E))), O.bf16_round(rng.standard_normal((lt, E)))
    weights = [tuple(O.bf16_round(rng.standard_normal((E, E)) * 0.05) for _ in range(4)) for _ in range(n_layers)]
    dw = [tuple(bf16_dev(a) for a in wl) for wl in weights]
    res = {}
    for canon in (False, True):
        st = Stack(*GEO, n_layers, heads, hd, lt, canonical_io=canon, rope_theta=10000.0)
        res[canon] = st.forward(bf16_dev(x), bf16_dev(t), dw)
    plain = Stack(*GEO, n_layers, heads, hd, lt, canonical_io=True).forward(bf16_dev(x), bf16_dev(t), dw)
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits(res[False][0]), dev_bits(res[True][0])), "video state: I/O orders differ"
    assert np.array_equal(dev_bits(res[False][1]), dev_bits(res[True][1])), "text state: I/O orders differ"
    assert not np.array_equal(dev_bits(res[True][0]), dev_bits(plain[0])), "the rotation changed nothing"
    ref_x, ref_t = O.stack_forward(x, t, GEO, weights, heads, hd, rope_theta=10000.0)
    check_bf16(from_dev(res[True][0]), ref_x, f"rope stack {n_layers} layers video")
    check_bf16(from_dev(res[True][1]), ref_t, f"rope stack {n_layers} layers text")
    for got, ref, inp, what in ((res[True][0], ref_x, x, "video"), (res[True][1], ref_t, t, "text")):
        check_update(from_dev(got), ref, inp, f"rope stack {n_layers} layers {what} update")
