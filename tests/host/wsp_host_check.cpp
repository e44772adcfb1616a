// Host-side check of libwsp's planner and C-ABI argument handling, built
// with g++ and -fsanitize=address,undefined (test infrastructure: compiled
// and run by tests/test_host_sanitized.py on the CPU, no GPU needed).
//
// It links the library's host sources (plan.cpp, abi.cpp) against stub
// kernel launchers that abort if reached, and exercises:
//   * wsp_plan / wsp_plan_info / wsp_plan_tables / wsp_plan_free over the
//     five workload grids and a sweep of small geometries (tables must be
//     permutations, offsets box volumes, boxes inside the grid);
//   * the relayout permutations and window-position tables of every pair;
//   * the attention work lists for every order, both I/O orders and both
//     tile heights: every (window, head, query tile) exactly once -- tiles of
//     the joint rows [video; text] where a window has its own partial and
//     that saves a tile -- and every other (chunk, head, text query tile)
//     exactly once, chunks partitioning the windows in id order, window rows
//     matching the window table;
//   * argument validation of every entry point that takes device pointers
//     (NULL, misaligned, aliasing, bad sizes) -- these return before any
//     device call.
// Any failed check prints its location and makes the exit status nonzero.

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <set>
#include <tuple>
#include <vector>

#include "wsp_internal.h"

namespace wsp {
// ---- stub launchers: the host check never reaches a kernel ----------------
// The tile sizes mirror the kernels' (256 / 128 query rows per bf16 item, 64
// per float32 item, 256 x 64 projection tiles, 32 KiB amax rows); they only
// feed argument validation here.
[[noreturn]] static void reached(const char *what) {
    std::fprintf(stderr, "host check: kernel launcher %s reached\n", what);
    std::abort();
}
int attn_bf16_tile_m(bool small) { return small ? 128 : 256; }
int attn_f32_tile_m(int) { return 64; }
int gemm_bf16_tile_n() { return 256; }
int gemm_bf16_tile_k() { return 64; }
int fp8_max_row_chunks() { return 2048; }
hipError_t launch_relayout(const void *, void *, const int32_t *, int64_t, int64_t, hipStream_t) { reached("relayout"); }
hipError_t launch_attn_bf16(int, bool, bool, const void *, const void *, const void *, const void *, const void *,
                            const void *, void *, float *, const int32_t *, const ItemDesc *, const WinDesc *, int,
                            const float *, const float *, const RopeTables *, int, int, float, uint32_t *, int, int,
                            int, hipStream_t) {
    reached("attn_bf16");
}
hipError_t launch_attn_f32(int, const float *, const float *, const float *, const float *, const float *,
                           const float *, float *, float *, const int32_t *, const ItemDesc *, const WinDesc *, int,
                           int, int, float, hipStream_t) {
    reached("attn_f32");
}
hipError_t launch_rope(const void *, void *, const int32_t *, const int32_t *, const int32_t *, const float2 *,
                       int64_t, int, int, int, hipStream_t) {
    reached("rope");
}
hipError_t launch_fp8_amax(const void *, float *, int64_t, int, int, int, hipStream_t) { reached("fp8_amax"); }
hipError_t launch_fp8_quantize(const void *, void *, const float *, int64_t, int, int, int, hipStream_t) {
    reached("fp8_quantize");
}
hipError_t launch_gemm_bf16(const void *, const void *, void *, const void *, int64_t, int, int, const GemmRope *,
                            hipStream_t) {
    reached("gemm");
}
hipError_t launch_text_mean(const float *, void *, int64_t, int, int, int, hipStream_t) { reached("text_mean"); }
hipError_t launch_xcd_probe(int32_t *, int, hipStream_t) { reached("xcd_probe"); }
}  // namespace wsp

using namespace wsp;

static int g_fail = 0;
#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            if (g_fail < 20) std::fprintf(stderr, "%s:%d: CHECK(%s)\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                                \
        }                                                                            \
    } while (0)

static void check_plan(int T, int H, int W, int nt, int nh, int nw, int method) {
    wsp_plan_t *p = nullptr;
    const int rc = wsp_plan(T, H, W, nt, nh, nw, method, &p);
    if (rc != WSP_OK) {  // only degenerate sizes may fail
        CHECK(p == nullptr);
        return;
    }
    int64_t n = 0;
    int32_t nwin = 0, win[3];
    CHECK(wsp_plan_info(p, &n, &nwin, win) == WSP_OK);
    CHECK(n == int64_t(T) * H * W && nwin >= 1);
    std::vector<int32_t> off(static_cast<size_t>(nwin) + 1), ids(static_cast<size_t>(n)),
        inv(static_cast<size_t>(n)), boxes(6 * static_cast<size_t>(nwin)), lpt(static_cast<size_t>(nwin));
    CHECK(wsp_plan_tables(p, off.data(), ids.data(), inv.data(), boxes.data(), lpt.data()) == WSP_OK);
    CHECK(off[0] == 0 && off[size_t(nwin)] == n);
    std::vector<char> seen(size_t(n), 0);
    for (int64_t j = 0; j < n; ++j) {
        const int32_t c = ids[size_t(j)];
        CHECK(c >= 0 && c < n);
        if (c < 0 || c >= n) continue;
        CHECK(!seen[size_t(c)]);
        seen[size_t(c)] = 1;
        CHECK(inv[size_t(c)] == j);
    }
    for (int32_t w = 0; w < nwin; ++w) {
        const int32_t *b = &boxes[6 * size_t(w)];
        CHECK(0 <= b[0] && b[0] < b[1] && b[1] <= T && 0 <= b[2] && b[2] < b[3] && b[3] <= H && 0 <= b[4] &&
              b[4] < b[5] && b[5] <= W);
        CHECK(off[size_t(w) + 1] - off[size_t(w)] == (b[1] - b[0]) * (b[3] - b[2]) * (b[5] - b[4]));
    }
    std::set<int32_t> ls(lpt.begin(), lpt.end());
    CHECK(int(ls.size()) == nwin);

    // relayout permutations to and from the canonical layout, and positions
    wsp_plan_t *c = nullptr;
    CHECK(wsp_plan(T, H, W, 1, 1, 1, WSP_CANONICAL, &c) == WSP_OK);
    std::vector<int32_t> perm;
    relayout_perm(*c, *p, perm);
    for (int64_t j = 0; j < n; ++j) CHECK(perm[size_t(j)] == ids[size_t(j)]);
    relayout_perm(*p, *c, perm);
    for (int64_t j = 0; j < n; ++j) CHECK(perm[size_t(j)] == inv[size_t(j)]);
    if (p->max_ext[0] <= 1024 && p->max_ext[1] <= 2048 && p->max_ext[2] <= 2048) {
        std::vector<int32_t> pos;
        window_positions(*p, pos);
        CHECK(int64_t(pos.size()) == n);
    }

    // work lists
    for (int gather = 0; gather < 2; ++gather) {
        std::vector<WinDesc> wins;
        window_descs(*p, gather != 0, wins);
        for (int32_t w = 0; w < nwin; ++w) {
            const WinDesc &d = wins[size_t(w)];
            CHECK(d.off == off[size_t(w)] && d.lw == off[size_t(w) + 1] - off[size_t(w)]);
            if (gather) {
                CHECK(d.vrow0 == ids[size_t(d.off)]);
                for (int32_t r = 0; r < d.lw; ++r) {
                    const int64_t rel = int64_t(ids[size_t(d.off + r)]) - d.vrow0;
                    CHECK(rel >= 0 && rel < d.vrows);
                }
            } else {
                CHECK(d.vrow0 == d.off && d.vrows == d.lw);
            }
        }
        for (int order : {WSP_ORDER_LPT_XCD, WSP_ORDER_LPT, WSP_ORDER_ID})
            for (int bm : {64, 128, 256})
                for (int Lt : {0, 1, 40, 300})
                    for (int heads : {1, 3}) {
                      for (int G : {text_chunks(nwin), int(nwin)}) {
                        std::vector<ItemDesc> items;
                        const int cnt = build_items(*p, heads, Lt, bm, order, gather != 0, G, items);
                        CHECK(cnt == int(items.size()));
                        std::set<std::tuple<int, int, int>> vid, txt;
                        int64_t real = 0;
                        // one partial per window: joint tiles [video; text] for the
                        // windows where they save a tile, text items for the others
                        const bool per_window = Lt > 0 && G == int(nwin);
                        auto joint = [&](int32_t w) {
                            const int64_t lw = off[size_t(w) + 1] - off[size_t(w)];
                            return per_window && (lw + Lt + 255) / 256 < (lw + 255) / 256 + (Lt + 255) / 256;
                        };
                        for (const ItemDesc &it : items) {
                            if (it.w < 0) continue;
                            ++real;
                            const int h = it.hq >> 16, t = it.hq & 0xFFFF;
                            CHECK(h >= 0 && h < heads);
                            if (it.nwin == 0) {
                                CHECK(it.w < nwin);
                                if (it.w >= nwin) continue;
                                const WinDesc &d = wins[size_t(it.w)];
                                CHECK(it.win.off == d.off && it.win.lw == d.lw && it.win.vrow0 == d.vrow0 &&
                                      it.win.vrows == d.vrows);
                                CHECK(it.chunk == (joint(it.w) ? it.w : -1));
                                CHECK(int64_t(t) * bm < d.lw + (joint(it.w) ? Lt : 0));
                                CHECK(vid.insert({it.w, h, t}).second);
                                // the box extents give every row's canonical offset in the window
                                CHECK(it.eh > 0 && it.ew > 0);
                                if (gather && h == 0 && t == 0) {
                                    const uint32_t eh = uint32_t(it.eh), ew = uint32_t(it.ew);
                                    for (int32_t r = 0; r < d.lw; ++r) {
                                        const uint32_t q1 = uint32_t(r) / ew, dt = q1 / eh;
                                        const int64_t rel = int64_t(dt) * p->H * p->W + int64_t(q1 - dt * eh) * p->W +
                                                            int64_t(uint32_t(r) - q1 * ew);
                                        CHECK(rel == int64_t(ids[size_t(d.off + r)]) - d.vrow0);
                                    }
                                }
                            } else {
                                CHECK(Lt > 0);
                                CHECK(it.chunk >= 0 && it.chunk < G);
                                CHECK(!per_window || (it.nwin == 1 && !joint(it.w)));
                                CHECK(it.w == chunk_begin(it.chunk, nwin, G));
                                CHECK(it.w + it.nwin == chunk_begin(it.chunk + 1, nwin, G));
                                CHECK(int64_t(t) * bm < Lt);
                                CHECK(txt.insert({it.chunk, h, t}).second);
                            }
                        }
                        int64_t want_vid = 0;
                        int64_t want_txt = 0;
                        for (int32_t w = 0; w < nwin; ++w) {
                            want_vid += heads * ((int64_t(off[size_t(w) + 1] - off[size_t(w)]) + (joint(w) ? Lt : 0) +
                                                  bm - 1) / bm);
                            if (per_window && !joint(w)) want_txt += heads * ((Lt + bm - 1) / bm);
                        }
                        if (Lt > 0 && !per_window) want_txt = int64_t(G) * heads * ((Lt + bm - 1) / bm);
                        CHECK(int64_t(vid.size()) == want_vid);
                        CHECK(int64_t(txt.size()) == want_txt);
                        CHECK(real == want_vid + want_txt);
                      }
                    }
    }
    // chunks cover the windows once, in id order
    {
        const int G = text_chunks(nwin);
        CHECK(G >= 1 && G <= kTextChunks && G <= nwin);
        CHECK(chunk_begin(0, nwin, G) == 0 && chunk_begin(G, nwin, G) == nwin);
        for (int cc = 0; cc < G; ++cc) CHECK(chunk_begin(cc + 1, nwin, G) > chunk_begin(cc, nwin, G));
    }
    wsp_plan_free(c);
    wsp_plan_free(p);
}

static void check_arguments() {
    wsp_plan_t *p = nullptr, *other = nullptr;
    CHECK(wsp_plan(5, 20, 36, 2, 3, 3, WSP_SHIFTED, &p) == WSP_OK);
    CHECK(wsp_plan(5, 20, 37, 2, 3, 3, WSP_SHIFTED, &other) == WSP_OK);
    alignas(16) static uint8_t buf[4][64];
    void *a = buf[0], *b = buf[1], *c = buf[2], *o = buf[3];
    void *mis = buf[0] + 8;
    // planner errors
    wsp_plan_t *bad = reinterpret_cast<wsp_plan_t *>(0x1);
    CHECK(wsp_plan(0, 20, 36, 2, 3, 3, WSP_REGULAR, &bad) == WSP_EINVAL && bad == nullptr);
    CHECK(wsp_plan(5, 20, 36, 0, 3, 3, WSP_REGULAR, &bad) == WSP_EINVAL);
    CHECK(wsp_plan(5, 20, 36, 2, 3, 3, 9, &bad) == WSP_EINVAL);
    CHECK(wsp_plan(2048, 2048, 2048, 2, 3, 3, WSP_REGULAR, &bad) == WSP_ERANGE);
    CHECK(wsp_plan(5, 20, 36, 2, 3, 3, WSP_REGULAR, nullptr) == WSP_EINVAL);
    CHECK(wsp_plan_info(nullptr, nullptr, nullptr, nullptr) == WSP_EINVAL);
    CHECK(wsp_plan_tables(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == WSP_EINVAL);
    wsp_plan_free(nullptr);
    // relayout
    CHECK(wsp_relayout(a, b, 16, p, other, nullptr) == WSP_EINVAL);
    CHECK(wsp_relayout(a, b, 24, p, p, nullptr) == WSP_EINVAL);
    CHECK(wsp_relayout(a, a, 16, p, p, nullptr) == WSP_EINVAL);
    CHECK(wsp_relayout(mis, b, 16, p, p, nullptr) == WSP_EINVAL);
    CHECK(wsp_relayout(nullptr, b, 16, p, p, nullptr) == WSP_EINVAL);
    // workspace and attention
    size_t ws = 0;
    CHECK(wsp_window_attn_workspace(p, 4, 64, 16, WSP_F32, &ws) == WSP_OK);
    CHECK(ws == size_t(text_chunks(p->nwin)) * 16 * 4 * 64 * 4);
    CHECK(wsp_window_attn_workspace(p, 4, 96, 16, WSP_F32, &ws) == WSP_EINVAL);
    CHECK(wsp_window_attn_workspace(p, 0, 64, 16, WSP_F32, &ws) == WSP_EINVAL);
    auto attn = [&](const void *q, const void *k, void *out, void *w, size_t wb, int H, int D, int Lt, int dt,
                    unsigned flags) {
        return wsp_window_attn_ex(p, q, k, c, a, b, c, H, D, Lt, dt, 0.f, flags, out, o, w, wb, nullptr);
    };
    CHECK(attn(a, b, o, buf[3], 0, 4, 96, 16, WSP_BF16, 0) == WSP_EINVAL);
    CHECK(attn(nullptr, b, o, buf[3], 0, 4, 64, 16, WSP_BF16, 0) == WSP_EINVAL);
    CHECK(attn(mis, b, o, buf[3], 0, 4, 64, 16, WSP_BF16, 0) == WSP_EINVAL);
    CHECK(attn(a, b, a, buf[3], 0, 4, 64, 16, WSP_BF16, 0) == WSP_EINVAL);
    CHECK(attn(a, b, o, buf[3], 16, 4, 64, 16, WSP_BF16, 0) == WSP_EWORKSPACE);
    CHECK(attn(a, b, o, nullptr, 1 << 30, 4, 64, 16, WSP_BF16, 0) == WSP_EWORKSPACE);
    CHECK(attn(a, b, o, buf[3], 0, 4, 64, 16, WSP_BF16, 2) == WSP_EINVAL);
    CHECK(attn(a, b, o, buf[3], 0, 4, 64, 16, 7, 0) == WSP_EINVAL);
    // fp8 q/k attention
    const float *am = reinterpret_cast<const float *>(buf[0]);
    CHECK(wsp_window_attn_qk8(p, a, b, c, a, b, c, am, am, 4, 64, 16, 0.f, 0, o, o, nullptr, 0, nullptr) ==
          WSP_EINVAL);
    CHECK(wsp_window_attn_qk8(p, a, b, c, a, b, c, nullptr, am, 4, 128, 16, 0.f, 0, o, o, nullptr, 0,
                              nullptr) == WSP_EINVAL);
    // attention with in-kernel rotary embedding
    size_t wr = 0;
    CHECK(wsp_window_attn_rope_workspace(p, 4, 128, 16, WSP_BF16, &wr) == WSP_OK);
    CHECK(wsp_window_attn_workspace(p, 4, 128, 16, WSP_BF16, &ws) == WSP_OK);
    CHECK(wr == ws + 3600 * 4 * 128 * 2 + 2 * 16 * 4 * 128 * 2);  // rotated k, text q, text k (bf16)
    CHECK(wsp_window_attn_rope_workspace(p, 4, 64, 16, WSP_BF16, &wr) == WSP_EINVAL);
    CHECK(wsp_window_attn_rope_workspace(p, 4, 128, 16, WSP_F32, &wr) == WSP_EINVAL);
    auto rattn = [&](wsp_plan_t *pl, void *w, size_t wb, int D, int dt) {
        return wsp_window_attn_rope(pl, a, b, c, a, b, c, 4, D, 16, dt, 0.f, 0.f, 1, o, o, w, wb, nullptr);
    };
    CHECK(rattn(p, buf[3], 0, 64, WSP_BF16) == WSP_EINVAL);
    CHECK(rattn(p, buf[3], 0, 128, WSP_F32) == WSP_EINVAL);
    CHECK(rattn(p, buf[3], 16, 128, WSP_BF16) == WSP_EWORKSPACE);
    CHECK(rattn(p, buf[3], ws, 128, WSP_BF16) == WSP_EWORKSPACE);  // partials only, no room for the rotated rows
    wsp_plan_t *tall = nullptr;                                     // windows 3286 rows high: beyond 2048
    CHECK(wsp_plan(2, 6000, 2, 1, 1, 1, WSP_REGULAR, &tall) == WSP_OK);
    CHECK(rattn(tall, buf[3], 0, 128, WSP_BF16) == WSP_ERANGE);
    wsp_plan_free(tall);
    // rope, fp8, linear, options
    CHECK(wsp_rope_relayout(a, b, 4, 64, WSP_BF16, p, p, p, 0, 0.f, nullptr) == WSP_EINVAL);
    CHECK(wsp_rope_relayout(a, b, 4, 128, WSP_BF16, p, p, other, 0, 0.f, nullptr) == WSP_EINVAL);
    CHECK(wsp_rope_text(a, a, 16, 4, 128, WSP_BF16, 0.f, nullptr) == WSP_EINVAL);
    CHECK(wsp_rope_text(a, b, 0, 4, 128, WSP_BF16, 0.f, nullptr) == WSP_OK);
    CHECK(wsp_fp8_amax(a, 1, 4, 64, WSP_BF16, nullptr, nullptr) == WSP_EINVAL);
    CHECK(wsp_fp8_amax(a, 1, 4, 96, WSP_BF16, reinterpret_cast<float *>(b), nullptr) == WSP_EINVAL);
    CHECK(wsp_fp8_quantize(a, b, -1, 4, 64, WSP_BF16, am, nullptr) == WSP_EINVAL);
    CHECK(wsp_linear(a, b, nullptr, o, 8, 100, 64, WSP_BF16, nullptr) == WSP_EINVAL);
    CHECK(wsp_linear(a, b, nullptr, o, 8, 256, 60, WSP_BF16, nullptr) == WSP_EINVAL);
    CHECK(wsp_linear(a, b, nullptr, a, 8, 256, 64, WSP_BF16, nullptr) == WSP_EINVAL);
    CHECK(wsp_linear(a, b, nullptr, o, 0, 256, 64, WSP_BF16, nullptr) == WSP_OK);
    // wsp_linear_rope: M must be the plan's tokens + text rows; plans of one grid
    const int64_t n_p = 5 * 20 * 36;
    CHECK(wsp_linear_rope(a, b, o, n_p, 256, 64, WSP_BF16, p, p, 16, 0.f, nullptr) == WSP_EINVAL);
    CHECK(wsp_linear_rope(a, b, o, n_p + 16, 256, 64, WSP_BF16, nullptr, p, 16, 0.f, nullptr) == WSP_EINVAL);
    CHECK(wsp_linear_rope(a, b, o, n_p + 16, 256, 64, WSP_BF16, p, other, 16, 0.f, nullptr) == WSP_EINVAL);
    CHECK(wsp_linear_rope(a, b, o, n_p + 16, 128, 64, WSP_BF16, p, p, 16, 0.f, nullptr) == WSP_EINVAL);
    CHECK(wsp_linear_rope(a, b, a, n_p + 16, 256, 64, WSP_BF16, p, p, 16, 0.f, nullptr) == WSP_EINVAL);
    CHECK(wsp_linear_rope(a, b, o, n_p - 1, 256, 64, WSP_BF16, p, p, -1, 0.f, nullptr) == WSP_EINVAL);
    wsp_plan_t *tall2 = nullptr;
    CHECK(wsp_plan(2, 6000, 2, 1, 1, 1, WSP_REGULAR, &tall2) == WSP_OK);
    CHECK(wsp_linear_rope(a, b, o, 2 * 6000 * 2, 256, 64, WSP_BF16, tall2, tall2, 0, 0.f, nullptr) == WSP_ERANGE);
    wsp_plan_free(tall2);
    CHECK(wsp_set_attn_order(7) == WSP_EINVAL);
    int nx = 0, rr = 0;
    CHECK(wsp_device_info(nullptr, &rr) == WSP_EINVAL);
    CHECK(wsp_device_info(&nx, nullptr) == WSP_EINVAL);
    CHECK(wsp_set_attn_schedule(1) == WSP_EINVAL);
    CHECK(wsp_last_error()[0] != '\0');
    wsp_plan_free(other);
    wsp_plan_free(p);
}

int main() {
    // the five workload grids
    const int grids[][6] = {{5, 20, 36, 2, 3, 3},     {21, 45, 80, 4, 3, 3}, {21, 68, 120, 4, 3, 3},
                            {31, 135, 240, 4, 3, 3},  {3, 12, 20, 1, 1, 1}, {4, 20, 36, 4, 9, 9}};
    for (const auto &g : grids)
        for (int m : {WSP_REGULAR, WSP_SHIFTED}) check_plan(g[0], g[1], g[2], g[3], g[4], g[5], m);
    check_plan(5, 20, 36, 1, 1, 1, WSP_CANONICAL);
    // small geometries, including degenerate and tie-rounding ones
    for (int T = 1; T <= 7; T += 3)
        for (int H = 1; H <= 13; H += 4)
            for (int W = 1; W <= 17; W += 5)
                for (int n = 1; n <= 4; ++n)
                    for (int m : {WSP_REGULAR, WSP_SHIFTED}) check_plan(T, H, W, n, n, 5 - n, m);
    check_plan(2, 75, 192, 2, 3, 3, WSP_SHIFTED);
    check_plan(2, 25, 576, 2, 3, 3, WSP_SHIFTED);
    check_plan(40, 8, 8, 1, 2, 2, WSP_SHIFTED);
    check_arguments();
    if (g_fail) {
        std::fprintf(stderr, "host check: %d failures\n", g_fail);
        return 1;
    }
    std::printf("host check: ok\n");
    return 0;
}
