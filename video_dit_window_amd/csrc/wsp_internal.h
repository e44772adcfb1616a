// Internal declarations of libwsp: the plan object, host table builders and
// the kernel launchers.  Not part of the public ABI (include/wsp.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "wsp.h"

namespace wsp {

// Work item of the attention kernels: x = window id (-1: nothing to do),
// y = (head << 16) | query tile.
using Item = int2;

// Work item of the per-item bf16 kernel with its window resolved on the host,
// so that a work group starts with one scalar load instead of a chain of
// dependent table loads.
struct alignas(32) ItemDesc {
    int32_t w;      // window id (-1: nothing to do)
    int32_t hq;     // (head << 16) | query tile
    int32_t off;    // first layout row of the window
    int32_t lw;     // video rows of the window
    int32_t vrow0;  // tensor row the window's video rows are addressed from
                    // (layout order: off; canonical order: its smallest id)
    int32_t vrows;  // tensor rows from vrow0 that the window's rows span
    int32_t pad[2];
};

struct DeviceTables {
    int32_t *offsets = nullptr;                                 // [n_windows + 1]
    int32_t *ids = nullptr;                                     // [n_tokens]
    int32_t *rel = nullptr;                                     // [n_tokens] ids - first id of the window
    int32_t *pos = nullptr;                                     // [n_tokens] window positions
    std::map<std::tuple<int, int, int, int>, int32_t *> perm;   // src layout -> perm
    // (H, Lt, BM, order, persistent work groups) -> work list
    std::map<std::tuple<int, int, int, int, int>, std::pair<Item *, int>> items;
    // (H, Lt, BM, order, canonical-order I/O) -> resolved work list
    std::map<std::tuple<int, int, int, int, int>, std::pair<ItemDesc *, int>> descs;
};

}  // namespace wsp

struct wsp_plan_t {
    int T = 0, H = 0, W = 0, nt = 0, nh = 0, nw = 0, method = 0;
    int wt = 0, wh = 0, ww = 0;
    int64_t n = 0;
    int32_t nwin = 0;
    int64_t max_rows = 0;   // largest window (rows)
    int64_t max_span = 0;   // largest canonical-id span of a window (last id - first id + 1)
    int32_t max_ext[3] = {0, 0, 0};  // largest window extent along t, h, w
    std::vector<int32_t> offsets, ids, inv, boxes, lpt;
    std::mutex mu;                               // guards dev
    std::map<int, wsp::DeviceTables> dev;        // per device ordinal
};

namespace wsp {

// ---- errors --------------------------------------------------------------
int fail(int code, const std::string &msg);
int hip_fail(hipError_t e, const char *what);
#define WSP_HIP(call)                                   \
    do {                                                \
        hipError_t e_ = (call);                         \
        if (e_ != hipSuccess) return hip_fail(e_, #call); \
    } while (0)

// ---- host planner (plan.cpp) ---------------------------------------------
int build_plan(int T, int H, int W, int nt, int nh, int nw, int method, wsp_plan_t &p);
void relayout_perm(const wsp_plan_t &src, const wsp_plan_t &dst, std::vector<int32_t> &perm);
// Window-local offset (dt, dh, dw) of every canonical token, packed as
// dt | dh << 10 | dw << 21 (extents checked against 1024 / 2048 by the caller).
void window_positions(const wsp_plan_t &p, std::vector<int32_t> &pos);
// Attention work list; returns items.size().  n_groups == 0: one item per
// work group (grid = items.size()); n_groups > 0: persistent lists for that
// many work groups, items[r * n_groups + g] (padded with x = -1).
int build_items(const wsp_plan_t &p, int n_heads, int text_len, int bm, int order, int n_groups,
                std::vector<Item> &items);

// ---- device tables (abi.cpp) ----------------------------------------------
int device_offsets(wsp_plan_t &p, int dev, int32_t **out);
int device_ids(wsp_plan_t &p, int dev, int32_t **out);
int device_perm(const wsp_plan_t &src, wsp_plan_t &dst, int dev, int32_t **out);
int device_positions(wsp_plan_t &p, int dev, int32_t **out);
int device_items(wsp_plan_t &p, int dev, int n_heads, int text_len, int bm, int order,
                 int n_groups, Item **out, int *count);
int device_rel_ids(wsp_plan_t &p, int dev, int32_t **out);
int device_item_descs(wsp_plan_t &p, int dev, int n_heads, int text_len, int bm, int order,
                      bool gather, ItemDesc **out, int *count);

// ---- kernel launchers -------------------------------------------------------
// relayout.hip
hipError_t launch_relayout(const void *x, void *y, const int32_t *perm, int64_t n_rows,
                           int64_t row_bytes, hipStream_t s);
// attn_bf16.hip: the per-item bf16 kernel (one work group per item) and its
// query-tile height: 256 rows, or 128 with `small` (4-wave work groups, two
// per CU).  rel != NULL selects canonical-order q/k/v/out: video
// row r of window w is tensor row vrow0(w) + rel[offsets[w] + r] (the plan's
// ids relative to the window's smallest id; items resolved to match).
int attn_bf16_tile_m(bool small);
hipError_t launch_attn_bf16(int head_dim, bool small, const void *q, const void *k, const void *v,
                            const void *tq, const void *tk, const void *tv, void *out,
                            float *ws, const int32_t *rel, const ItemDesc *items, int n_items,
                            int n_heads, int text_len, float scale, hipStream_t s);
// attn_bf16_persist.hip: the persistent bf16 kernel (short windows): n_groups
// resident work groups walk items[r * n_groups + g], r < rounds.
int attn_bf16_persist_tile_m();
hipError_t launch_attn_bf16_persist(int head_dim, const void *q, const void *k, const void *v,
                                    const void *tq, const void *tk, const void *tv, void *out,
                                    float *ws, const int32_t *offsets, const int32_t *ids,
                                    const int32_t *rel, const Item *items, int n_groups, int rounds,
                                    int n_heads, int text_len, float scale, hipStream_t s);
// attn_f32.hip
int attn_f32_tile_m(int head_dim);
hipError_t launch_attn_f32(int head_dim, const float *q, const float *k, const float *v,
                           const float *tq, const float *tk, const float *tv, float *out,
                           float *ws, const int32_t *offsets, const int32_t *ids,
                           const Item *items, int n_items, int n_heads, int text_len, float scale,
                           hipStream_t s);
// rope.hip: rows of x (perm[j], or j) rotated into y[j]; positions from the
// packed table pos[cid[j]] (+ text_len on t) or, with pos == NULL, (j, j, j);
// cs = [P][21] (cos, sin) pairs.  Head dim 128 only.
hipError_t launch_rope(const void *x, void *y, const int32_t *perm, const int32_t *cid,
                       const int32_t *pos, const float2 *cs, int64_t n_rows, int n_heads, int dtype,
                       int text_len, hipStream_t s);
// fp8.hip: per-head amax (max-accumulated as float bits) and E4M3 codes.
int fp8_max_row_chunks();
hipError_t launch_fp8_amax(const void *x, float *amax, int64_t n_rows, int n_heads, int head_dim,
                           int dtype, hipStream_t s);
hipError_t launch_fp8_quantize(const void *x, void *y, const float *amax, int64_t n_rows,
                               int n_heads, int head_dim, int dtype, hipStream_t s);
// attn_qk8.hip: attention with E4M3 q / k codes (head dim 128, bf16 v / out).
int attn_qk8_tile_m();
hipError_t launch_attn_qk8(const void *q, const void *k, const void *v, const void *tq,
                           const void *tk, const void *tv, void *out, float *ws,
                           const int32_t *offsets, const int32_t *ids, const Item *items,
                           int n_items, const float *amax_q, const float *amax_k, int n_heads,
                           int text_len, float scale, hipStream_t s);
// gemm_bf16.hip: y[M,N] = x[M,K] w[N,K]^T (+ r), bf16; N % tile_n == 0,
// K % tile_k == 0 (checked by the caller).
int gemm_bf16_tile_n();
int gemm_bf16_tile_k();
hipError_t launch_gemm_bf16(const void *x, const void *w, void *y, const void *r, int64_t M, int N,
                            int K, hipStream_t s);
// text_mean.hip
hipError_t launch_text_mean(const float *ws, void *txt_out, int64_t per_window, int n_windows,
                            int dtype, hipStream_t s);

}  // namespace wsp
