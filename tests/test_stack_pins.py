"""Pins of the stack-workload oracle (oracle/wsp_stack.py) against closed forms.

The multi-layer stack is a synthetic harness around the pages' layer (random
projections, residual stream, alternating layouts); these tests tie its
oracle to results that follow from the definitions without running its code
path: bfloat16 rounding on exactly representable values and ties, the
orientation of the projection by selection matrices, a zero output
projection that must leave the stream unchanged, and zero query/key
projections whose uniform attention gives window means computed from
coordinates.  With the optional q / k rotation: zero q / k projections are
unaffected by it (it touches q and k only), and windows of one shape and the
same content give equal outputs (positions restart in every window).
"""
import numpy as np
import pytest

import oracle as O
import wsp_inputs as I
from test_oracle_pins import membership


def test_bf16_round_exact_cases():
    u = 2.0 ** -7                                      # bfloat16 spacing in [1, 2)
    cases = [(1.0, 1.0), (1 + u, 1 + u), (1 + u / 2, 1.0),          # tie -> even (1.0)
             (1 + 3 * u / 2, 1 + 2 * u),                              # tie -> even (1 + 2u)
             (1 + u / 2 + 2.0 ** -30, 1 + u), (-(1 + 3 * u / 2), -(1 + 2 * u)),
             (3.0, 3.0), (0.0, 0.0), (2.0 ** 100 * (1 + u / 2), 2.0 ** 100),
             (0.1, 0.10009765625)]                                    # 0x3dcd
    for x, want in cases:
        assert O.bf16_round(x) == want, (x, O.bf16_round(x), want)


def test_bf16_round_matches_float32_rounding():
    """On float32 inputs a single rounding to bfloat16 is what the input
    generator's float32 -> bfloat16 conversion computes."""
    x = np.random.default_rng(5).standard_normal(20000).astype(np.float32) * 7
    via_bits = I.bf16_bits_to_f32(I.f32_to_bf16_bits(x)).astype(np.float64)
    assert np.array_equal(O.bf16_round(x.astype(np.float64)), via_bits)


def test_linear_orientation_by_selection_matrix():
    rng = np.random.default_rng(1)
    x = O.bf16_round(rng.standard_normal((7, 12)))
    perm = np.array([3, 0, 11, 5, 5, 7])
    w = np.zeros((6, 12))
    w[np.arange(6), perm] = 1.0                        # row n of w picks column perm[n] of x
    assert np.array_equal(O.linear(x, w), x[:, perm])
    r = O.bf16_round(rng.standard_normal((7, 6)))
    assert np.array_equal(O.linear(x, w, r), O.bf16_round(x[:, perm] + r))
    assert np.array_equal(O.linear(x, 2 * w), 2 * x[:, perm])


GEO = (5, 20, 36, 2, 3, 3)
HEADS, HD, LT = 2, 16, 5
E = HEADS * HD


def inputs(seed):
    rng = np.random.default_rng(seed)
    N = GEO[0] * GEO[1] * GEO[2]
    return O.bf16_round(rng.standard_normal((N, E))), O.bf16_round(rng.standard_normal((LT, E)))


def test_zero_output_projection_is_identity():
    x, t = inputs(2)
    rng = np.random.default_rng(3)
    w = [tuple(O.bf16_round(rng.standard_normal((E, E)) * 0.1) for _ in range(3)) + (np.zeros((E, E)),)
         for _ in range(3)]
    xo, to = O.stack_forward(x, t, GEO, w, HEADS, HD)
    assert np.array_equal(xo, x) and np.array_equal(to, t)


@pytest.mark.parametrize("n_layers", [1, 2])
def test_uniform_attention_gives_window_means(n_layers):
    """Wq = Wk = 0 makes every score 0, so each query's output is the mean of
    the value rows of its window and the text rows; with Wv = Wo = I a layer
    adds bf16(that mean) to the stream.  Windows come from the closed-form
    membership (regular layout for layer 0, shifted for layer 1), the text
    update from the mean over windows of the per-window means."""
    x, t = inputs(4)
    z, eye = np.zeros((E, E)), np.eye(E)
    w = [(z, z, eye, eye)] * n_layers
    xo, to = O.stack_forward(x, t, GEO, w, HEADS, HD)
    xe, te = x.copy(), t.copy()
    for l in range(n_layers):
        method = O.REGULAR if l % 2 == 0 else O.SHIFTED
        _, win, nwin = membership(*GEO, method)
        means = np.zeros((nwin, E))
        for wi in range(nwin):
            rows = np.concatenate([xe[win == wi], te], axis=0)
            means[wi] = rows.mean(axis=0)
        xe = O.bf16_round(xe + O.bf16_round(means[win]))
        te = O.bf16_round(te + O.bf16_round(np.broadcast_to(means.mean(axis=0), te.shape)))
    np.testing.assert_allclose(xo, xe, rtol=0, atol=1e-12)
    np.testing.assert_allclose(to, te, rtol=0, atol=1e-12)


@pytest.mark.parametrize("first_layer", [1, 2, 5])
def test_resumed_layer_uses_its_schedule_layout(first_layer):
    """first_layer resumes the schedule: one layer at index l runs in the
    regular layout for even l and the shifted one for odd l (window means of
    the closed-form membership, as above), and layers 0..2 in one pass equal
    layer 0 followed by a pass resumed at layer 1."""
    x, t = inputs(6)
    z, eye = np.zeros((E, E)), np.eye(E)
    xo, to = O.stack_forward(x, t, GEO, [(z, z, eye, eye)], HEADS, HD, first_layer=first_layer)
    method = O.REGULAR if first_layer % 2 == 0 else O.SHIFTED
    _, win, nwin = membership(*GEO, method)
    means = np.stack([np.concatenate([x[win == wi], t], axis=0).mean(axis=0) for wi in range(nwin)])
    np.testing.assert_allclose(xo, O.bf16_round(x + O.bf16_round(means[win])), rtol=0, atol=1e-12)
    np.testing.assert_allclose(to, O.bf16_round(t + O.bf16_round(np.broadcast_to(means.mean(axis=0), t.shape))),
                               rtol=0, atol=1e-12)
    rng = np.random.default_rng(8)
    w = [tuple(O.bf16_round(rng.standard_normal((E, E)) * 0.05) for _ in range(4)) for _ in range(3)]
    full = O.stack_forward(x, t, GEO, w, HEADS, HD)
    x1, t1 = O.stack_forward(x, t, GEO, w[:1], HEADS, HD)
    rest = O.stack_forward(x1, t1, GEO, w[1:], HEADS, HD, first_layer=1)
    assert np.array_equal(full[0], rest[0]) and np.array_equal(full[1], rest[1])


def test_rope_stack_with_zero_qk_is_plain():
    """The rotation acts on q and k only: with Wq = Wk = 0 every score is 0
    with or without it, so the two stacks agree exactly."""
    rng = np.random.default_rng(12)
    heads, hd, lt = 1, 128, 3
    e = heads * hd
    N = GEO[0] * GEO[1] * GEO[2]
    x, t = O.bf16_round(rng.standard_normal((N, e))), O.bf16_round(rng.standard_normal((lt, e)))
    z = np.zeros((e, e))
    w = [(z, z) + tuple(O.bf16_round(rng.standard_normal((e, e)) * 0.1) for _ in range(2)) for _ in range(2)]
    plain = O.stack_forward(x, t, GEO, w, heads, hd)
    rot = O.stack_forward(x, t, GEO, w, heads, hd, rope_theta=10000.0)
    assert np.array_equal(plain[0], rot[0]) and np.array_equal(plain[1], rot[1])


def test_rope_stack_positions_restart_per_window():
    """The shifted layout of a 2 x 4 x 6 grid (nt = 1, nh = nw = 2) has two
    windows, the frames t = 0 and t = 1 (4 x 6 tokens each).  Video rows that
    depend on (h, w) only give both windows the same content at the same
    window-local positions, so one shifted layer with the rotation leaves
    both frames' rows equal; in the regular layout (one 2 x 4 x 6 window) the
    frames sit at temporal positions text_len + 0 and + 1 and come out
    different, so the rotation does see the temporal position."""
    geo = (2, 4, 6, 1, 2, 2)
    heads, hd, lt = 1, 128, 3
    e = heads * hd
    for method, boxes in ((O.SHIFTED, [(0, 1, 0, 4, 0, 6), (1, 2, 0, 4, 0, 6)]), (O.REGULAR, [(0, 2, 0, 4, 0, 6)])):
        assert [tuple(int(v) for v in b) for b in O.plan(*geo, method).boxes] == boxes
    rng = np.random.default_rng(13)
    frame = O.bf16_round(rng.standard_normal((24, e)))
    x = np.concatenate([frame, frame], axis=0)         # canonical order: t = 0 rows, then t = 1 rows
    t = O.bf16_round(rng.standard_normal((lt, e)))
    w = [tuple(O.bf16_round(rng.standard_normal((e, e)) * 0.1) for _ in range(4))]
    xs, _ = O.stack_forward(x, t, geo, w, heads, hd, first_layer=1, rope_theta=10000.0)
    assert np.array_equal(xs[:24], xs[24:])
    xr, _ = O.stack_forward(x, t, geo, w, heads, hd, first_layer=0, rope_theta=10000.0)
    assert not np.array_equal(xr[:24], xr[24:])
    xn, _ = O.stack_forward(x, t, geo, w, heads, hd, first_layer=0)
    assert np.array_equal(xn[:24], xn[24:])             # without the rotation the frames stay equal
