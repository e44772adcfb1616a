// Host planner: window geometry, layout tables, relayout permutations and the
// ordered work list of the attention kernels.
//
// Window rule and layouts: "Window-Aligned Sequence Parallelism (SeedVR2)",
// section "Window layouts".  Largest-first order: same page, section "Planner".

#include <algorithm>
#include <cmath>
#include <numeric>

#include "wsp_internal.h"

namespace wsp {

namespace {

// The temporal extent entering the size rule is capped at 30 frames.
constexpr int kMaxTemporalWindow = 30;

struct Interval {
    int a, b;
};

// Cuts of one axis of length n with window w.  Regular: [i*w, min((i+1)*w, n)).
// Shifted: every cut moves back by floor(w/2) and is clipped to [0, n]; the
// first interval is therefore ceil(w/2) long and no interval wraps.
void axis_cuts(int n, int w, int method, std::vector<Interval> &out) {
    out.clear();
    const int64_t s = (method == WSP_SHIFTED) ? w / 2 : 0;
    for (int64_t i = 0; i * w - s < n; ++i) {
        const int64_t a = std::max<int64_t>(i * w - s, 0);
        const int64_t b = std::min<int64_t>((i + 1) * w - s, n);
        if (b > a) out.push_back({int(a), int(b)});
    }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int build_plan(int T, int H, int W, int nt, int nh, int nw, int method, wsp_plan_t &p) {
    if (T <= 0 || H <= 0 || W <= 0)
        return fail(WSP_EINVAL, "grid extents must be positive (T=" + std::to_string(T) +
                                    ", H=" + std::to_string(H) + ", W=" + std::to_string(W) + ")");
    if (method != WSP_REGULAR && method != WSP_SHIFTED && method != WSP_CANONICAL)
        return fail(WSP_EINVAL, "unknown window method " + std::to_string(method));
    const int64_t n = int64_t(T) * H * W;
    if (n >= (int64_t(1) << 31))
        return fail(WSP_ERANGE, "T*H*W = " + std::to_string(n) + " does not fit int32 token ids");
    p.T = T; p.H = H; p.W = W; p.nt = nt; p.nh = nh; p.nw = nw; p.method = method;
    p.n = n;

    std::vector<Interval> ti, hi, wi;
    if (method == WSP_CANONICAL) {
        p.wt = T; p.wh = H; p.ww = W;
        ti = {{0, T}}; hi = {{0, H}}; wi = {{0, W}};
    } else {
        if (nt <= 0 || nh <= 0 || nw <= 0)
            return fail(WSP_EINVAL, "window counts nt, nh, nw must be positive");
        // Size rule, evaluated in IEEE double like the page's Python:
        // scale = sqrt(45*80 / (H*W)); round() ties to even (nearbyint under
        // the default rounding mode).
        const double scale = std::sqrt(3600.0 / (double(H) * double(W)));
        const double rh = std::nearbyint(double(H) * scale);
        const double rw = std::nearbyint(double(W) * scale);
        if (!(rh >= 1.0) || !(rw >= 1.0))
            return fail(WSP_EINVAL, "window size rounds to zero for H=" + std::to_string(H) +
                                        ", W=" + std::to_string(W));
        if (rh > 2e9 || rw > 2e9) return fail(WSP_ERANGE, "rescaled grid too large");
        p.wh = int(ceil_div(int64_t(rh), nh));
        p.ww = int(ceil_div(int64_t(rw), nw));
        p.wt = int(ceil_div(std::min(T, kMaxTemporalWindow), nt));
        axis_cuts(T, p.wt, method, ti);
        axis_cuts(H, p.wh, method, hi);
        axis_cuts(W, p.ww, method, wi);
    }

    const size_t nwin = ti.size() * hi.size() * wi.size();
    try {
        p.offsets.assign(1, 0);
        p.offsets.reserve(nwin + 1);
        p.boxes.clear();
        p.boxes.reserve(6 * nwin);
        p.ids.resize(size_t(n));
        p.inv.resize(size_t(n));
        p.lpt.resize(nwin);
    } catch (const std::bad_alloc &) {
        return fail(WSP_ENOMEM, "host allocation of plan tables failed");
    }
    // w outermost, t innermost; row-major (t, h, w) inside each box.
    int64_t pos = 0;
    for (const Interval &iw : wi)
        for (const Interval &ih : hi)
            for (const Interval &it : ti) {
                p.boxes.insert(p.boxes.end(), {it.a, it.b, ih.a, ih.b, iw.a, iw.b});
                for (int t = it.a; t < it.b; ++t)
                    for (int h = ih.a; h < ih.b; ++h) {
                        const int64_t row = (int64_t(t) * H + h) * W;
                        for (int w = iw.a; w < iw.b; ++w) {
                            p.ids[size_t(pos)] = int32_t(row + w);
                            p.inv[size_t(row + w)] = int32_t(pos);
                            ++pos;
                        }
                    }
                p.offsets.push_back(int32_t(pos));
            }
    p.nwin = int32_t(nwin);
    p.max_rows = p.max_span = 0;
    p.max_ext[0] = p.max_ext[1] = p.max_ext[2] = 0;
    for (size_t w = 0; w < nwin; ++w)
        for (int a = 0; a < 3; ++a)
            p.max_ext[a] = std::max(p.max_ext[a], p.boxes[6 * w + 2 * a + 1] - p.boxes[6 * w + 2 * a]);
    for (size_t w = 0; w < nwin; ++w) {
        const int32_t a = p.offsets[w], b = p.offsets[w + 1];
        p.max_rows = std::max<int64_t>(p.max_rows, b - a);
        // Rows are in row-major (t, h, w) order: the first has the smallest
        // canonical id and the last the largest.
        if (b > a) p.max_span = std::max<int64_t>(p.max_span, int64_t(p.ids[b - 1]) - p.ids[a] + 1);
    }
    // Largest first, ties by window id.
    std::iota(p.lpt.begin(), p.lpt.end(), 0);
    std::stable_sort(p.lpt.begin(), p.lpt.end(), [&](int32_t a, int32_t b) {
        const int32_t la = p.offsets[a + 1] - p.offsets[a], lb = p.offsets[b + 1] - p.offsets[b];
        return la > lb;
    });
    return WSP_OK;
}

void window_positions(const wsp_plan_t &p, std::vector<int32_t> &pos) {
    // "Window-Aligned Sequence Parallelism (SeedVR2)", section "Reference
    // quirks reproduced on purpose": RoPE positions are offsets from each
    // window's own corner.
    pos.assign(size_t(p.n), 0);
    for (int32_t w = 0; w < p.nwin; ++w) {
        const int32_t *b = &p.boxes[6 * size_t(w)];
        for (int t = b[0]; t < b[1]; ++t)
            for (int h = b[2]; h < b[3]; ++h)
                for (int x = b[4]; x < b[5]; ++x)
                    pos[size_t((int64_t(t) * p.H + h) * p.W + x)] =
                        (t - b[0]) | ((h - b[2]) << 10) | ((x - b[4]) << 21);
    }
}

void relayout_perm(const wsp_plan_t &src, const wsp_plan_t &dst, std::vector<int32_t> &perm) {
    // Destination row j holds canonical token dst.ids[j], found at src.inv[...].
    perm.resize(size_t(dst.n));
    for (int64_t j = 0; j < dst.n; ++j) perm[size_t(j)] = src.inv[size_t(dst.ids[size_t(j)])];
}

void window_descs(const wsp_plan_t &p, bool gather, std::vector<WinDesc> &wins) {
    wins.resize(size_t(p.nwin));
    for (int32_t w = 0; w < p.nwin; ++w) {
        WinDesc &d = wins[size_t(w)];
        d.off = p.offsets[w];
        d.lw = p.offsets[w + 1] - d.off;
        // a window's rows in canonical order ascend (row-major in t, h, w):
        // its first id is the smallest and its last the largest
        d.vrow0 = gather ? p.ids[d.off] : d.off;
        d.vrows = gather ? p.ids[d.off + d.lw - 1] - p.ids[d.off] + 1 : d.lw;
    }
}

int build_items(const wsp_plan_t &p, int n_heads, int text_len, int bm, int order, bool gather,
                int n_chunks, std::vector<ItemDesc> &items) {
    constexpr int kXcds = 8;
    constexpr int kKeyTile = 64;
    std::vector<WinDesc> wins;
    window_descs(p, gather, wins);
    std::vector<int32_t> worder(size_t(p.nwin));
    if (order == WSP_ORDER_ID)
        std::iota(worder.begin(), worder.end(), 0);
    else
        worder = p.lpt;
    // Cost of a query tile over one window: its 64-key tiles.
    auto key_tiles = [&](int32_t w) { return ceil_div(int64_t(wins[size_t(w)].lw) + text_len, kKeyTile); };
    const int64_t text_tiles = ceil_div(text_len, bm);
    const int G = text_len > 0 ? n_chunks : 0;
    const bool per_window = G == p.nwin;
    // With one partial per window, a window whose text rows fit in the empty
    // part of its last video query tile takes tiles of the joint sequence
    // [video rows; text rows] (item chunk = w); the others keep a video
    // sequence and text items of their own (which then run full tiles).  The
    // test uses 256-row tiles whatever bm is, so that every tile height puts
    // the same rows in each 32-row wave (a wave's rows share its rescaling
    // steps): the schedules stay bit-identical.  Joint tiles never take more
    // tiles than separate ones.
    constexpr int64_t kJointTile = 256;
    auto joint = [&](int32_t w) {
        const int64_t lw = wins[size_t(w)].lw;
        return per_window &&
               ceil_div(lw + text_len, kJointTile) < ceil_div(lw, kJointTile) + ceil_div(text_len, kJointTile);
    };
    auto query_rows = [&](int32_t w) { return int64_t(wins[size_t(w)].lw) + (joint(w) ? text_len : 0); };
    if (text_tiles > 0xFFFF) return fail(WSP_ERANGE, "text_len needs more than 65535 query tiles");
    for (int32_t w = 0; w < p.nwin; ++w)
        if (ceil_div(query_rows(w), bm) > 0xFFFF)
            return fail(WSP_ERANGE, "window " + std::to_string(w) + " needs more than 65535 query tiles");

    // Groups of items that read the same K/V: all query tiles of a (window,
    // head); in chunk mode all text query tiles of a (chunk, head) form a
    // group of their own.  Each group has a cost in key tiles.
    struct Group {
        int64_t cost;
        std::vector<ItemDesc> items;
    };
    auto text_items = [&](int c, int h, std::vector<ItemDesc> &out) {
        const int w0 = chunk_begin(c, p.nwin, G), w1 = chunk_begin(c + 1, p.nwin, G);
        for (int64_t t = 0; t < text_tiles; ++t) {
            ItemDesc d{};
            d.w = w0;
            d.hq = (h << 16) | int(t);
            d.nwin = w1 - w0;
            d.chunk = c;
            out.push_back(d);
        }
    };
    std::vector<Group> groups;
    if (G > 0 && !per_window) {
        for (int c = 0; c < G; ++c) {
            int64_t cost = 0;
            for (int w = chunk_begin(c, p.nwin, G); w < chunk_begin(c + 1, p.nwin, G); ++w) cost += key_tiles(w);
            for (int h = 0; h < n_heads; ++h) {
                Group g{cost * text_tiles, {}};
                text_items(c, h, g.items);
                groups.push_back(std::move(g));
            }
        }
        // a text item covers a whole chunk of windows (several times a video
        // item): those groups go first, largest first
        std::stable_sort(groups.begin(), groups.end(),
                         [](const Group &a, const Group &b) { return a.cost > b.cost; });
    }
    for (int32_t w : worder) {
        const int64_t tiles = ceil_div(query_rows(w), bm);
        const bool own_text = per_window && !joint(w);
        for (int h = 0; h < n_heads; ++h) {
            Group g{(tiles + (own_text ? text_tiles : 0)) * key_tiles(w), {}};
            for (int64_t t = 0; t < tiles; ++t) {
                ItemDesc d{};
                d.w = w;
                d.hq = (h << 16) | int(t);
                d.chunk = joint(w) ? w : -1;
                d.win = wins[size_t(w)];
                const int32_t *bx = &p.boxes[6 * size_t(w)];
                d.eh = bx[3] - bx[2];
                d.ew = bx[5] - bx[4];
                g.items.push_back(d);
            }
            if (own_text) text_items(w, h, g.items);
            groups.push_back(std::move(g));
        }
    }
    items.clear();
    if (order != WSP_ORDER_LPT_XCD) {
        for (const Group &g : groups) items.insert(items.end(), g.items.begin(), g.items.end());
        return int(items.size());
    }
    // Work groups are handed to the XCDs round-robin by block index, so block
    // b runs on XCD b % 8.  Each group -- whose items all read the same K/V --
    // goes whole to the least-loaded XCD, in list order, and each XCD's list
    // keeps that order.
    std::vector<std::vector<ItemDesc>> lists(kXcds);
    std::vector<int64_t> load(kXcds, 0);
    for (const Group &g : groups) {
        const int x = int(std::min_element(load.begin(), load.end()) - load.begin());
        lists[size_t(x)].insert(lists[size_t(x)].end(), g.items.begin(), g.items.end());
        load[size_t(x)] += g.cost;
    }
    size_t longest = 0;
    for (auto &l : lists) longest = std::max(longest, l.size());
    ItemDesc idle{};
    idle.w = -1;
    items.assign(longest * kXcds, idle);
    for (int x = 0; x < kXcds; ++x)
        for (size_t s = 0; s < lists[x].size(); ++s) items[s * kXcds + x] = lists[x][s];
    return int(items.size());
}

}  // namespace wsp
