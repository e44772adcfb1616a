"""Pins of the RoPE oracle (oracle/wsp_rope.py) against what the page fixes
and what rotations must satisfy, independent of the oracle's own formulas.

Fixed by the page ("Window-Aligned Sequence Parallelism (SeedVR2)", section
"Reference quirks reproduced on purpose"): a video token's rotary indices
are its offsets from its own window's corner, with the temporal one moved up
by the text length; the rotated width is the largest multiple of three not
above the head dimension, and the leftover channels are copied.  Mathematical invariants of any
axial rotary embedding: identity at position 0, norm preservation,
composition of rotations, dependence of q.k on the position difference only,
axis separation.  The readings on the frequency base, the adjacent-pair
layout and the text positions (R1-R3 of the oracle) are pinned to their
stated form by hand-derived angles in tests/golden/rope_angles.json; the page
itself does not fix them.
"""
import json
import os

import numpy as np
import pytest

import oracle as O

D = 128


def rng(seed):
    return np.random.default_rng([77, seed])


def test_span_and_axis_block():
    assert O.rope_span(128) == 126          # 3 * (128 // 3): two channels are left unrotated
    assert O.rope_axis_dim(128) == 42
    with pytest.raises(ValueError):
        O.rope_axis_dim(64)                 # 3 * 21 = 63: axis blocks of 21 cannot pair


@pytest.mark.parametrize("method", [O.REGULAR, O.SHIFTED])
def test_window_positions_are_window_local(method):
    """Brute force on the tiny grid: find each token's window by scanning the
    boxes, subtract the box corner, add text_len on the temporal axis."""
    T, H, W, Lt = 5, 20, 36, 16
    p = O.plan(T, H, W, 2, 3, 3, method)
    pos = O.window_positions(p, Lt)
    for cid in rng(1).integers(0, T * H * W, size=300):
        t, h, w = cid // (H * W), (cid // W) % H, cid % W
        hits = [b for b in p.boxes if b[0] <= t < b[1] and b[2] <= h < b[3] and b[4] <= w < b[5]]
        assert len(hits) == 1
        t0, _, h0, _, w0, _ = hits[0]
        assert tuple(pos[cid]) == (Lt + t - t0, h - h0, w - w0)
    # positions count from each window's own corner, which sits at (Lt, 0, 0)
    for (t0, t1, h0, h1, w0, w1) in p.boxes:
        assert tuple(pos[(t0 * H + h0) * W + w0]) == (Lt, 0, 0)


def test_canonical_layout_positions_are_global():
    T, H, W = 3, 4, 5
    pos = O.window_positions(O.canonical_plan(T, H, W), 7)
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    assert np.array_equal(pos, np.stack([7 + t.ravel(), h.ravel(), w.ravel()], 1))


def test_identity_at_zero_and_pass_through():
    x = rng(2).standard_normal((9, 3, D))
    assert np.array_equal(O.rope(x, np.zeros((9, 3), np.int64)), x)
    pos = rng(3).integers(1, 50, size=(9, 3))
    y = O.rope(x, pos)
    assert np.array_equal(y[..., 126:], x[..., 126:])          # the two pass-through channels
    assert np.all(np.abs(y[..., :126] - x[..., :126]).max(axis=(0, 1)) > 0)  # every rotated channel moves


def test_norm_preserved_per_pair():
    x = rng(4).standard_normal((20, 2, D))
    y = O.rope(x, rng(5).integers(0, 300, size=(20, 3)))
    nx = x[..., 0:126:2] ** 2 + x[..., 1:126:2] ** 2
    ny = y[..., 0:126:2] ** 2 + y[..., 1:126:2] ** 2
    assert np.allclose(nx, ny, rtol=1e-12, atol=1e-12)


def test_rotations_compose_and_invert():
    x = rng(6).standard_normal((11, 2, D))
    a, b = rng(7).integers(-40, 40, size=(11, 3)), rng(8).integers(-40, 40, size=(11, 3))
    assert np.allclose(O.rope(O.rope(x, a), b), O.rope(x, a + b), atol=1e-12)
    assert np.allclose(O.rope(O.rope(x, a), -a), x, atol=1e-12)


def test_scores_depend_on_position_difference_only():
    q, k = rng(9).standard_normal((1, 1, D)), rng(10).standard_normal((1, 1, D))
    p, r = np.array([[12, 3, 7]]), np.array([[5, 9, 1]])
    s0 = float((O.rope(q, p) * O.rope(k, r)).sum())
    for shift in ([1, 0, 0], [0, 4, 0], [0, 0, 9], [30, 2, 11]):
        d = np.array([shift])
        assert abs(float((O.rope(q, p + d) * O.rope(k, r + d)).sum()) - s0) < 1e-10


def test_axes_rotate_their_own_blocks():
    x = rng(11).standard_normal((4, 1, D))
    base = np.array([[3, 4, 5]] * 4)
    for axis, (lo, hi) in enumerate([(0, 42), (42, 84), (84, 126)]):
        moved = base.copy()
        moved[:, axis] += 6
        diff = np.abs(O.rope(x, moved) - O.rope(x, base)).max(axis=(0, 1))
        assert np.all(diff[lo:hi] > 0) and np.all(diff[:lo] == 0) and np.all(diff[hi:] == 0)


def test_rope_relayout_matches_rotation_after_move():
    T, H, W, Lt = 5, 20, 36, 16
    c, r, s = O.canonical_plan(T, H, W), O.plan(T, H, W, 2, 3, 3, O.REGULAR), O.plan(T, H, W, 2, 3, 3, O.SHIFTED)
    x = rng(12).standard_normal((T * H * W, 2, D))
    y = O.rope_relayout(x, c, r, r, Lt)
    # row j of y is canonical token r.ids[j], rotated by its regular-layout window position
    j = 123
    cid = r.ids[j]
    assert np.allclose(y[j], O.rope(x[cid:cid + 1], O.window_positions(r, Lt)[cid:cid + 1])[0])
    # moving between layouts does not change a token's rotation, only its row
    y2 = O.rope_relayout(x, c, s, r, Lt)
    assert np.allclose(O.relayout(y2, s, r), y)


# ---------------------------------------------------------------- hand-derived goldens
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rope_angles.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def check_pairs(axial, pairs):
    """Rotate unit vectors through O.rope at the given axial indices and
    compare every listed pair with the hand-derived (cos, sin); every other
    channel of a one-hot input must stay where it is."""
    pos = np.asarray([axial], dtype=np.int64)
    ang = O.rope_angles(pos, D)[0]
    for p in pairs:
        c0, c1 = p["channels"]
        assert abs(ang[c0 // 2] - p["angle"]) <= 1e-12 * max(1.0, abs(p["angle"])), p
        for src, want in ((c0, (p["cos"], p["sin"])), (c1, (-p["sin"], p["cos"]))):
            x = np.zeros((1, 1, D))
            x[0, 0, src] = 1.0
            y = O.rope(x, pos)[0, 0]
            assert abs(y[c0] - want[0]) <= 1e-12 and abs(y[c1] - want[1]) <= 1e-12, (p, src, y[c0], y[c1])
            others = np.delete(y, [c0, c1])
            assert np.all(others == 0.0)


@pytest.mark.parametrize("case", golden()["cases"], ids=lambda c: c["name"])
def test_rope_angles_match_hand_derivation(case):
    """Pins the readings on the frequency base and exponent (10000^(-2i/42)),
    the block order [t | h | w] with adjacent pairs, and the rotation
    direction: a wrong exponent, interleaved axes, half-split pairs or the
    opposite sign each move at least one listed value."""
    check_pairs(case["axial"], case["pairs"])


def test_rope_text_positions_match_hand_derivation():
    """Text token i sits at (i, i, i) (reading on text positions)."""
    case = [c for c in golden()["cases"] if c["name"] == "text token 5"][0]
    assert tuple(O.text_positions(6)[5]) == tuple(case["axial"])
    check_pairs(O.text_positions(6)[5], case["pairs"])


@pytest.mark.parametrize("entry", golden()["window_positions"], ids=lambda e: e["method"])
def test_window_positions_and_angles_match_hand_derivation(entry):
    T, H, W = entry["grid"]
    p = O.plan(T, H, W, *entry["n"], O.SHIFTED if entry["method"] == "shifted" else O.REGULAR)
    t, h, w = entry["token"]
    cid = (t * H + h) * W + w
    assert cid == entry["canonical_id"]
    assert tuple(O.window_positions(p, entry["text_len"])[cid]) == tuple(entry["axial"])
    check_pairs(entry["axial"], entry["pairs"])
