"""Pins of the CPU oracle against things other than itself.

Each test ties an oracle function to a fact the pages or mathematics fix:
shapes printed in the workload descriptions, hand derivations of the
window rule (tests/golden/window_tables.json), a closed-form window
membership written independently of the oracle's loops, brute force over
all small geometries, SDPA (the library routine the text-replica page calls)
on single-window and masked formulations, and closed forms of attention.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "window_tables.json")))
METHOD = {"regular": O.REGULAR, "shifted": O.SHIFTED}


# ---------------------------------------------------------------- helpers
def membership(T, H, W, nt, nh, nw, method):
    """Window id and in-window order of every canonical token, in closed form.

    Independent of the oracle's nested loops: along an axis with window w
    and shift s a coordinate c falls in interval (c + s) // w; windows are
    numbered with the w axis outermost and t innermost.  Returns the layout
    order of canonical ids obtained by sorting tokens by (window, t, h, w).
    """
    wt, wh, ww = O.window_size(T, H, W, nt, nh, nw)

    def axis(n, w):
        s = (w // 2) if method == O.SHIFTED else 0
        c = np.arange(n)
        idx = (c + s) // w
        return idx, int(idx.max()) + 1

    it, ct = axis(T, wt)
    ih, ch = axis(H, wh)
    iw, cw = axis(W, ww)
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    win = (iw[w] * ch + ih[h]) * ct + it[t]
    cid = (t * H + h) * W + w
    order = np.lexsort((w.ravel(), h.ravel(), t.ravel(), win.ravel()))
    return cid.ravel()[order], win.ravel(), ct * ch * cw


def sdpa(q, k, v, mask=None):
    """torch's scaled_dot_product_attention in float64 on the CPU, [S, D] per head."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=None if mask is None else torch.from_numpy(mask)[None],
        dropout_p=0.0, is_causal=False)
    return out[0].numpy()


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- window size
@pytest.mark.parametrize("case", GOLD["printed"], ids=lambda c: c["claim"][:30])
def test_printed_workload_shapes(case):
    T, H, W = case["grid"]
    p = O.plan(T, H, W, *case["n"], METHOD[case["method"]])
    if "wh_ww" in case:
        assert list(p.win[1:]) == case["wh_ww"]
    if "windows_per_axis" in case:
        assert [len(p.extents[a]) for a in "thw"] == case["windows_per_axis"]
    if "n_windows" in case:
        assert p.n_windows == case["n_windows"]
    if "max_box" in case:
        assert [max(p.extents[a]) for a in "thw"] == case["max_box"]
        assert list(p.win) == case["max_box"]
    if "spatial_windows" in case:
        assert [len(p.extents["h"]), len(p.extents["w"])] == case["spatial_windows"]
    if "wt" in case:
        assert p.win[0] == case["wt"]


@pytest.mark.parametrize("case", GOLD["derived"], ids=lambda c: f"{c['grid']}-{c['method']}")
def test_hand_derived_tables(case):
    T, H, W = case["grid"]
    p = O.plan(T, H, W, *case["n"], METHOD[case["method"]])
    assert list(p.win) == case["win"]
    assert p.extents == case["extents"]
    if "offsets" in case:
        assert p.offsets.tolist() == case["offsets"]
    if "n_windows" in case:
        assert p.n_windows == case["n_windows"]
    if "full_windows_2430" in case:
        assert int((p.lengths() == 2430).sum()) == case["full_windows_2430"]


def test_resolution_invariance():
    """Window size does not depend on resolution at the 16:9 latent grids
    ("Motivation": the count of windows grows, never their size)."""
    sizes = {O.window_size(21, H, W, 4, 3, 3)[1:] for H, W in [(45, 80), (68, 120), (90, 160), (135, 240)]}
    assert sizes == {(15, 27)}
    p720 = O.plan(21, 45, 80, 4, 3, 3, O.REGULAR)
    p4k = O.plan(21, 135, 240, 4, 3, 3, O.REGULAR)
    assert p4k.n_windows > p720.n_windows


@pytest.mark.parametrize("case", GOLD["half_even"], ids=lambda c: f"{c['H']}x{c['W']}")
def test_round_half_to_even(case):
    H, W = case["H"], case["W"]
    assert H * math.sqrt(3600 / (H * W)) == case["H_scaled"]  # an exact tie
    assert O.window_size(1, H, W, *case["n"])[1:] == (case["wh"], case["ww"])


@pytest.mark.parametrize("case", GOLD["temporal_cap"], ids=lambda c: f"T{c['T']}nt{c['nt']}")
def test_temporal_cap(case):
    p = O.plan(case["T"], 45, 80, case["nt"], 3, 3, O.REGULAR)
    assert p.win[0] == case["wt"]
    assert p.extents["t"] == case["t_extents"]


@pytest.mark.parametrize("bad", [(0, 4, 4, 1, 1, 1), (2, -1, 4, 1, 1, 1), (2, 4, 4, 0, 1, 1),
                                 (1, 1, 20000, 1, 1, 1), (2, 4, 4, 1, 1, 2.5)])
def test_invalid_geometry_raises(bad):
    with pytest.raises(ValueError):
        O.window_size(*bad)


# ---------------------------------------------------------------- tables
# The spatial window is about 45/nh x 80/nw tokens whatever the grid, so
# small grids need large nh, nw to hold more than one window per axis.
SMALL = [(T, H, W, nt, nh, nw)
         for T, H, W in [(1, 1, 1), (3, 5, 7), (4, 6, 9), (7, 12, 11), (12, 8, 12), (2, 12, 5)]
         for nt, nh, nw in [(1, 1, 1), (2, 3, 3), (3, 25, 40), (2, 11, 17), (4, 60, 60)]]


@pytest.mark.parametrize("geo", SMALL)
@pytest.mark.parametrize("method", [O.REGULAR, O.SHIFTED])
def test_tables_match_closed_form_membership(geo, method):
    p = O.plan(*geo, method)
    ids, _, nwin = membership(*geo, method)
    assert np.array_equal(p.ids, ids)
    assert p.n_windows == nwin


def test_tables_brute_force_small_grids():
    """Exact partition, disjoint axis-aligned boxes without wraparound, offsets
    = prefix sum of box volumes, ids row-major inside each box -- over every
    grid with T, H, W <= 6 over a spread of window counts."""
    for T, H, W in itertools.product(range(1, 7), repeat=3):
        for n in itertools.product((1, 2, 3), (1, 13, 29, 60), (1, 17, 40, 80)):
            for method in (O.REGULAR, O.SHIFTED):
                p = O.plan(T, H, W, *n, method)
                N = T * H * W
                assert np.array_equal(np.sort(p.ids), np.arange(N))
                assert np.array_equal(p.inv[p.ids], np.arange(N))
                paint = np.zeros((T, H, W), dtype=np.int64)
                for wid, (t0, t1, h0, h1, w0, w1) in enumerate(p.boxes):
                    assert 0 <= t0 < t1 <= T and 0 <= h0 < h1 <= H and 0 <= w0 < w1 <= W
                    paint[t0:t1, h0:h1, w0:w1] += 1
                    vol = (t1 - t0) * (h1 - h0) * (w1 - w0)
                    assert p.offsets[wid + 1] - p.offsets[wid] == vol
                    seg = p.ids[p.offsets[wid]:p.offsets[wid + 1]]
                    tt, hh, ww = np.meshgrid(np.arange(t0, t1), np.arange(h0, h1),
                                             np.arange(w0, w1), indexing="ij")
                    assert np.array_equal(seg, ((tt * H + hh) * W + ww).ravel())
                assert (paint == 1).all()


def test_interval_cuts_closed_form():
    """Interior cuts of the regular tiling are the multiples of w; those of the
    shifted tiling are the c with (c + floor(w/2)) % w == 0."""
    for n in range(1, 41):
        for w in range(1, 13):
            for method, s in ((O.REGULAR, 0), (O.SHIFTED, w // 2)):
                iv = O.axis_intervals(n, w, method)
                assert iv[0][0] == 0 and iv[-1][1] == n
                assert all(a < b for a, b in iv)
                assert all(iv[i][1] == iv[i + 1][0] for i in range(len(iv) - 1))
                cuts = [b for _, b in iv[:-1]]
                assert cuts == [c for c in range(1, n) if (c + s) % w == 0]
                assert all(b - a <= w for a, b in iv)


def test_canonical_ids_are_windowed_arange():
    """'Window layouts': the canonical id is what windowing arange yields."""
    for method in (O.REGULAR, O.SHIFTED):
        p = O.plan(5, 20, 36, 2, 3, 3, method)
        c = O.canonical_plan(5, 20, 36)
        arange = np.arange(p.n_tokens)
        assert np.array_equal(O.relayout(arange, c, p), p.ids)
        assert np.array_equal(O.relayout(p.ids, p, c), arange)


def roll_partition(T, H, W, win):
    """Tiling after a cyclic roll by half a window on every axis: windows wrap."""
    labels = np.zeros((T, H, W), dtype=np.int64)
    wt, wh, ww = win
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    key = (((t + wt // 2) % T) // wt, ((h + wh // 2) % H) // wh, ((w + ww // 2) % W) // ww)
    _, labels = np.unique(np.stack([k.ravel() for k in key], 1), axis=0, return_inverse=True)
    return labels.reshape(-1)


def same_partition(a, b):
    """Whether two labelings of the same tokens define the same set of blocks."""
    pairs = set(zip(a.tolist(), b.tolist()))
    return len(pairs) == len(set(a.tolist())) == len(set(b.tolist()))


@pytest.mark.parametrize("geo", [(5, 20, 36, 2, 3, 3), (21, 68, 120, 4, 3, 3), (7, 12, 11, 2, 30, 20)])
def test_shifted_differs_from_regular_and_from_roll(geo):
    reg = O.plan(*geo, O.REGULAR)
    shf = O.plan(*geo, O.SHIFTED)
    _, lab_reg, _ = membership(*geo, O.REGULAR)
    _, lab_shf, _ = membership(*geo, O.SHIFTED)
    assert not same_partition(lab_reg, lab_shf)
    assert not np.array_equal(reg.ids, shf.ids)
    assert not same_partition(lab_shf, roll_partition(*geo[:3], shf.win))


def test_ragged_edges():
    """'Window layouts' consequences: edge windows are clipped, so counts are ragged."""
    for method in (O.REGULAR, O.SHIFTED):
        L = O.plan(21, 68, 120, 4, 3, 3, method).lengths()
        assert L.min() < L.max() == 6 * 15 * 27


def test_lpt_order_brute_force():
    for geo in [(21, 68, 120, 4, 3, 3), (5, 20, 36, 2, 3, 3), (7, 12, 11, 2, 30, 20)]:
        for method in (O.REGULAR, O.SHIFTED):
            p = O.plan(*geo, method)
            L = p.lengths()
            want = sorted(range(p.n_windows), key=lambda w: (-L[w], w))
            assert p.lpt.tolist() == want
            # ties keep ascending window id
            for a, b in zip(p.lpt[:-1], p.lpt[1:]):
                assert L[a] > L[b] or (L[a] == L[b] and a < b)


# ---------------------------------------------------------------- schedule
def test_31_transitions_for_32_alternating_layers():
    s = O.layer_schedule(32)
    assert O.transitions(s) == 31
    assert s[0] == O.REGULAR and s[1] == O.SHIFTED
    assert O.transitions([O.REGULAR] * 4) == 0


# ---------------------------------------------------------------- relayout
def test_relayout_round_trips():
    c = O.canonical_plan(5, 20, 36)
    r = O.plan(5, 20, 36, 2, 3, 3, O.REGULAR)
    s = O.plan(5, 20, 36, 2, 3, 3, O.SHIFTED)
    x = rand((c.n_tokens, 3), 1)
    for a, b in itertools.permutations([c, r, s], 2):
        assert np.array_equal(O.relayout(O.relayout(x, a, b), b, a), x)
    for a in (c, r, s):
        assert np.array_equal(O.relayout(x, a, a), x)
    assert np.array_equal(O.relayout(O.relayout(O.relayout(x, c, r), r, s), s, c), x)
    # a row in the destination is the token the destination's ids name
    y = O.relayout(O.relayout(x, c, r), r, s)
    assert np.array_equal(y, x[s.ids])


def test_relayout_rejects_other_grid():
    with pytest.raises(ValueError):
        O.relayout_perm(O.plan(5, 20, 36, 2, 3, 3, 0), O.plan(5, 20, 35, 2, 3, 3, 0))


# ---------------------------------------------------------------- attention
def test_single_window_equals_global_sdpa():
    """One window covering the grid: joint attention = SDPA over [video; text]."""
    T, H, W = 2, 6, 10
    p = O.plan(T, H, W, 1, 1, 1, O.REGULAR)
    assert p.n_windows == 1
    N, Hh, D, Lt = p.n_tokens, 2, 8, 3
    q, k, v = (rand((N, Hh, D), s) for s in (1, 2, 3))
    tq, tk, tv = (rand((Lt, Hh, D), s) for s in (4, 5, 6))
    out, txt = O.window_attn(p, q, k, v, tq, tk, tv)
    for h in range(Hh):
        ref = sdpa(np.concatenate([q[:, h], tq[:, h]]), np.concatenate([k[:, h], tk[:, h]]),
                   np.concatenate([v[:, h], tv[:, h]]))
        np.testing.assert_allclose(out[:, h], ref[:N], rtol=0, atol=1e-12)
        np.testing.assert_allclose(txt[:, h], ref[N:], rtol=0, atol=1e-12)


@pytest.mark.parametrize("method", [O.REGULAR, O.SHIFTED])
def test_masked_global_formulation(method):
    """Video outputs equal global SDPA in canonical order under the mask
    'same window' built from coordinates; the text output equals the mean,
    over windows, of SDPA of the text queries masked to one window."""
    geo = (3, 9, 16, 2, 9, 16)
    p = O.plan(*geo, method)
    assert p.n_windows >= 16
    c = O.canonical_plan(*geo[:3])
    _, win, nwin = membership(*geo, method)
    N, Hh, D, Lt = p.n_tokens, 2, 8, 4
    qc, kc, vc = (rand((N, Hh, D), s) for s in (7, 8, 9))
    tq, tk, tv = (rand((Lt, Hh, D), s) for s in (10, 11, 12))
    out, txt = O.window_attn(p, O.relayout(qc, c, p), O.relayout(kc, c, p),
                             O.relayout(vc, c, p), tq, tk, tv)
    out_c = O.relayout(out, p, c)
    vid_mask = np.concatenate([win[:, None] == win[None, :], np.ones((N, Lt), bool)], axis=1)
    for h in range(Hh):
        K = np.concatenate([kc[:, h], tk[:, h]])
        V = np.concatenate([vc[:, h], tv[:, h]])
        ref = sdpa(qc[:, h], K, V, vid_mask)
        np.testing.assert_allclose(out_c[:, h], ref, rtol=0, atol=1e-12)
        acc = np.zeros((Lt, D))
        for w in range(nwin):
            m = np.concatenate([np.broadcast_to(win == w, (Lt, N)), np.ones((Lt, Lt), bool)], 1)
            acc += sdpa(tq[:, h], K, V, m)
        np.testing.assert_allclose(txt[:, h], acc / nwin, rtol=0, atol=1e-12)


def test_two_token_closed_form_pins_scale_and_text_keys():
    """A 1x1x1 grid has one video token; with one text token the video query's
    weight on itself is sigmoid((q.k_v - q.k_t)/sqrt(D))."""
    p = O.plan(1, 1, 1, 1, 1, 1, O.REGULAR)
    D = 16
    q, k, v = (rand((1, 1, D), s) for s in (20, 21, 22))
    tq, tk, tv = (rand((1, 1, D), s) for s in (23, 24, 25))
    out, txt = O.window_attn(p, q, k, v, tq, tk, tv)
    for Q, o in ((q[0, 0], out[0, 0]), (tq[0, 0], txt[0, 0])):
        a = 1.0 / (1.0 + math.exp(-(Q @ k[0, 0] - Q @ tk[0, 0]) / math.sqrt(D)))
        np.testing.assert_allclose(o, a * v[0, 0] + (1 - a) * tv[0, 0], rtol=1e-13, atol=1e-13)
    # an explicit scale replaces 1/sqrt(D)
    out2, _ = O.window_attn(p, q, k, v, tq, tk, tv, scale=0.25)
    a = 1.0 / (1.0 + math.exp(-(q[0, 0] @ (k[0, 0] - tk[0, 0])) * 0.25))
    np.testing.assert_allclose(out2[0, 0], a * v[0, 0] + (1 - a) * tv[0, 0], rtol=1e-13)


@pytest.mark.parametrize("method", [O.REGULAR, O.SHIFTED])
def test_zero_keys_closed_form_window_count_mean(method):
    """K = 0 makes every weight uniform.  With text values 0 and video values
    c_w on window w: video outputs are c_w*L_w/(L_w+Lt) and the text output
    is the mean over windows of that value -- a window-count mean, which
    differs from the token-weighted mean ('Text stream')."""
    geo = (5, 20, 36, 2, 3, 3)
    p = O.plan(*geo, method)
    N, Hh, D, Lt = p.n_tokens, 2, 4, 16
    L = p.lengths()
    c = np.arange(1, p.n_windows + 1, dtype=np.float64)
    v = np.repeat(c, L)[:, None, None] * np.ones((N, Hh, D))
    q = rand((N, Hh, D), 30)
    tq = rand((Lt, Hh, D), 31)
    zeros = np.zeros((N, Hh, D))
    out, txt = O.window_attn(p, q, zeros, v, tq, np.zeros((Lt, Hh, D)), np.zeros((Lt, Hh, D)))
    per_w = c * L / (L + Lt)
    np.testing.assert_allclose(out[:, 0, 0], np.repeat(per_w, L), rtol=1e-13)
    np.testing.assert_allclose(txt, np.full((Lt, Hh, D), per_w.mean()), rtol=1e-13)
    token_weighted = (per_w * L).sum() / L.sum()
    assert abs(per_w.mean() - token_weighted) > 1e-3


def test_text_mean_divides_by_window_count():
    s = rand((3, 2, 4), 40)
    np.testing.assert_allclose(O.text_mean(s, 8), s / 8)
    with pytest.raises(ValueError):
        O.text_mean(s, 0)


def test_window_and_head_subsets_match_full():
    geo = (3, 9, 16, 2, 9, 16)
    p = O.plan(*geo, O.SHIFTED)
    N, Hh, D, Lt = p.n_tokens, 3, 8, 5
    q, k, v = (rand((N, Hh, D), s) for s in (50, 51, 52))
    tq, tk, tv = (rand((Lt, Hh, D), s) for s in (53, 54, 55))
    out, txt = O.window_attn(p, q, k, v, tq, tk, tv)
    sub, txt1 = O.window_attn(p, q, k, v, tq, tk, tv, windows=[2, 5], heads=[1])
    for w in (2, 5):
        a, b = p.offsets[w], p.offsets[w + 1]
        np.testing.assert_array_equal(sub[a:b, 1], out[a:b, 1])
    sub_all, txt_all = O.window_attn(p, q, k, v, tq, tk, tv, heads=[1])
    np.testing.assert_allclose(txt_all[:, 1], txt[:, 1], rtol=1e-14)


def test_flop_and_byte_counts():
    p = O.plan(21, 68, 120, 4, 3, 3, O.REGULAR)
    L = p.lengths()
    assert O.attn_flops(p, 20, 128, 256) == 4 * 128 * 20 * int(((L + 256) ** 2).sum())
    assert abs(O.attn_flops(p, 20, 128, 256) - 4.4997e12) / 4.4997e12 < 1e-4
    assert O.relayout_bytes(171360, 5120) == 2 * 171360 * 5120 + 4 * 171360
