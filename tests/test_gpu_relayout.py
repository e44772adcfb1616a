"""GPU parity of wsp_relayout: bit-exact against the oracle's row gather."""
import numpy as np
import pytest

import oracle as O
import video_dit_window_amd as W
from helpers import dev_bits, log

pytestmark = pytest.mark.gpu


def _plans(geo):
    T, H, Wd, nt, nh, nw = geo
    return ({"canonical": O.canonical_plan(T, H, Wd), "regular": O.plan(*geo, O.REGULAR),
             "shifted": O.plan(*geo, O.SHIFTED)},
            {"canonical": W.canonical(T, H, Wd), "regular": W.Plan(*geo, W.REGULAR),
             "shifted": W.Plan(*geo, W.SHIFTED)})


@pytest.mark.parametrize("row_elems", [8, 24, 2560, 2568])
def test_relayout_bit_exact_all_pairs(gpu, row_elems):
    import torch
    geo = (6, 30, 52, 2, 3, 3)
    op, wp = _plans(geo)
    n = op["canonical"].n_tokens
    rng = np.random.default_rng(row_elems)
    x = rng.integers(-32768, 32767, size=(n, row_elems), dtype=np.int16)
    xd = torch.from_numpy(x).cuda()
    for a in op:
        for b in op:
            y = W.relayout(xd, wp[a], wp[b])
            torch.cuda.synchronize()
            ref = O.relayout(x, op[a], op[b])
            assert np.array_equal(y.cpu().numpy(), ref), (a, b)
    log(f"  relayout rows of {row_elems * 2} B: all 9 layout pairs bit-exact")


def test_relayout_round_trip_and_identity(gpu):
    import torch
    geo = (7, 12, 11, 2, 30, 20)
    op, wp = _plans(geo)
    n = op["canonical"].n_tokens
    x = torch.randint(-2**31, 2**31 - 1, (n, 12), dtype=torch.int32, device="cuda")
    r = W.relayout(x, wp["canonical"], wp["regular"])
    s = W.relayout(r, wp["regular"], wp["shifted"])
    back = W.relayout(s, wp["shifted"], wp["canonical"])
    same = W.relayout(x, wp["canonical"], wp["canonical"])
    torch.cuda.synchronize()
    assert torch.equal(back, x) and torch.equal(same, x)
    ar = torch.arange(n, dtype=torch.int32, device="cuda").repeat_interleave(4).view(n, 4)
    ids = W.relayout(ar, wp["canonical"], wp["shifted"])[:, 0].cpu().numpy()
    assert np.array_equal(ids, op["shifted"].ids)


def test_relayout_full_1080p_qkv_rows(gpu):
    """[171360, 20*128] bf16 rows (5120 B), canonical -> regular -> shifted ->
    canonical, bit-exact against the oracle at every step."""
    import torch
    geo = (21, 68, 120, 4, 3, 3)
    op, wp = _plans(geo)
    n = op["canonical"].n_tokens
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randint(-32768, 32767, (n, 20, 128), dtype=torch.int16, device="cuda", generator=g)
    xh = x.cpu().numpy()
    cur, cur_h, name = x, xh, "canonical"
    for nxt in ("regular", "shifted", "canonical"):
        y = W.relayout(cur.view(torch.bfloat16), wp[name], wp[nxt]).view(torch.int16)
        torch.cuda.synchronize()
        ref = O.relayout(cur_h, op[name], op[nxt])
        assert np.array_equal(y.cpu().numpy(), ref), (name, nxt)
        cur, cur_h, name = y, ref, nxt
    assert torch.equal(cur, x)
    log("  1080p relayout chain bit-exact")
