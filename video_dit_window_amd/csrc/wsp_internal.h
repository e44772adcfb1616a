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

// Text outputs are reduced over windows in fixed chunks: the windows of a
// plan split into G runs of consecutive ids, each summed (float32, id order)
// into one partial of the workspace, and the partials are added in chunk
// order by the text-mean kernel.  G is min(n_windows, kTextChunks) (the
// workspace every call accepts): text work items then loop over a chunk's
// windows.  Or G = n_windows -- one partial per window -- when the caller's
// workspace holds that many: a window's text rows are then queried beside its
// video rows, from the same K/V stream on the same XCD -- in the same query
// tiles (the joint sequence [video; text] cut into tiles) where that saves a
// tile, else by text items of that one window.
constexpr int kTextChunks = 16;
inline int text_chunks(int n_windows) { return n_windows < kTextChunks ? n_windows : kTextChunks; }
// First window of chunk c (chunk c covers windows chunk_begin(c) ..
// chunk_begin(c + 1) - 1).
inline int chunk_begin(int c, int n_windows, int n_chunks) {
    return int(int64_t(c) * n_windows / n_chunks);
}

// Rows of one window as the attention kernels address them.
struct alignas(16) WinDesc {
    int32_t off;    // first layout row of the window
    int32_t lw;     // video rows of the window
    int32_t vrow0;  // tensor row the window's video rows are addressed from
                    // (layout order: off; canonical order: its smallest id)
    int32_t vrows;  // tensor rows from vrow0 that the window's rows span
};

// Work item of the attention kernels, resolved on the host so that a work
// group starts with one scalar load.
//  video item (nwin == 0): query tile `hq & 0xFFFF` of window w, head
//    hq >> 16; the window's rows in `win`.  chunk < 0: tiles of the video
//    rows; chunk >= 0: tiles of the joint query rows [video rows; text rows],
//    the normalised outputs of the text rows stored to partial `chunk`;
//  text item (nwin > 0): query tile `hq & 0xFFFF` of the text rows, head
//    hq >> 16, attended in turn over windows w .. w + nwin - 1 (rows from the
//    per-plan WinDesc table); the normalised outputs are summed into the
//    float32 partial `chunk` of the workspace.
//  w < 0: nothing to do.
//  eh, ew (video items): the window's box extents along h and w: row r of
//    the window, (dt, dh, dw) with r = (dt * eh + dh) * ew + dw, lies
//    dt*H*W + dh*W + dw canonical rows past its first row, so canonical-order
//    kernels form the row ids of a video item without reading the ids table.
struct alignas(16) ItemDesc {
    int32_t w;
    int32_t hq;
    int32_t nwin;
    int32_t chunk;
    WinDesc win;
    int32_t eh, ew;
    int32_t pad[2];
};
static_assert(sizeof(ItemDesc) == 48, "one 48-byte scalar load per work item");

struct DeviceTables {
    int32_t *offsets = nullptr;                                 // [n_windows + 1]
    int32_t *ids = nullptr;                                     // [n_tokens]
    int32_t *rel = nullptr;                                     // [n_tokens] ids - first id of the window
    int32_t *pos = nullptr;                                     // [n_tokens] window positions
    int32_t *lpos = nullptr;                                    // [n_tokens] window positions, layout order
    WinDesc *wins[2] = {nullptr, nullptr};                      // [n_windows] layout / canonical order
    std::map<std::tuple<int, int, int, int>, int32_t *> perm;   // src layout -> perm
    // (H, Lt, BM, order, canonical-order I/O, text chunks) -> work list
    std::map<std::tuple<int, int, int, int, int, int>, std::pair<ItemDesc *, int>> items;
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
// Window rows as the attention kernels address them (gather: canonical-order
// tensors, vrow0 = the window's smallest canonical id).
void window_descs(const wsp_plan_t &p, bool gather, std::vector<WinDesc> &wins);
// Attention work list, ordered for dispatch: the query tiles of every
// (window, head) -- of its video rows, or (one chunk per window, where that
// saves a tile) of [video rows; text rows] -- and text items of every other
// (chunk, head, text tile); returns its length or a negative status.
int build_items(const wsp_plan_t &p, int n_heads, int text_len, int bm, int order, bool gather,
                int n_chunks, std::vector<ItemDesc> &items);

// ---- device tables (abi.cpp) ----------------------------------------------
int device_offsets(wsp_plan_t &p, int dev, int32_t **out);
int device_ids(wsp_plan_t &p, int dev, int32_t **out);
int device_perm(const wsp_plan_t &src, wsp_plan_t &dst, int dev, int32_t **out);
int device_positions(wsp_plan_t &p, int dev, int32_t **out);
int device_rel_ids(wsp_plan_t &p, int dev, int32_t **out);
// Window positions in layout order (pos[ids[j]]), for the in-kernel RoPE.
int device_layout_positions(wsp_plan_t &p, int dev, int32_t **out);
int device_windows(wsp_plan_t &p, int dev, bool gather, WinDesc **out);
int device_items(wsp_plan_t &p, int dev, int n_heads, int text_len, int bm, int order, bool gather,
                 int n_chunks, ItemDesc **out, int *count);

// ---- kernel launchers -------------------------------------------------------
// relayout.hip
hipError_t launch_relayout(const void *x, void *y, const int32_t *perm, int64_t n_rows,
                           int64_t row_bytes, hipStream_t s);
// Ticket counters of the bf16 kernel's work queue, at the start of the
// caller's workspace (256 bytes, cleared by the launch itself).
constexpr int kQueueWords = 64;
constexpr size_t kQueueBytes = sizeof(uint32_t) * kQueueWords;
// attn_bf16.hip: the matrix-core kernel, one work group per item: 256 query
// rows, or 128 with `small` (4-wave work groups, two per CU).  queue != NULL
// launches resident work groups instead (as many as fit on the device) that
// take the items from n_lists lists in turn (n_lists 8: list x = items
// 8t + x, taken by the work groups running on XCD x; 1: the whole list) --
// the queue's counters are cleared by a kernel launched just before.
// grid_hw = H*W and grid_w = W of the plan's grid (canonical-order row ids of
// video items from their window boxes).  rel != NULL
// selects canonical-order q/k/v/out: video row r of window w is tensor row
// vrow0(w) + rel[offsets[w] + r] (the plan's ids relative to the window's
// smallest id; items and windows resolved to match).  q8: q, k (and the text
// ones) are E4M3 codes with per-head scales amax/448 (head dim 128 only).
// ws receives the float32 text partials of the items' chunks.
int attn_bf16_tile_m(bool small);
// In-kernel rotary embedding of the video queries (bf16, head dim 128):
// cs = (cos, sin) of 21 pairs per position (positions 0 .. text_len +
// largest temporal extent - 1 at least); pos[layout row] = the row's window
// offset dt | dh << 10 | dw << 21 (axial positions text_len + dt, dh, dw).
struct RopeTables {
    const float2 *cs = nullptr;
    const int32_t *pos = nullptr;
};
hipError_t launch_attn_bf16(int head_dim, bool small, bool q8, const void *q, const void *k, const void *v,
                            const void *tq, const void *tk, const void *tv, void *out, float *ws,
                            const int32_t *rel, const ItemDesc *items, const WinDesc *wins, int n_items,
                            const float *amax_q, const float *amax_k, const RopeTables *rope, int n_heads,
                            int text_len, float scale, uint32_t *queue, int n_lists, int grid_hw, int grid_w,
                            hipStream_t s);
// attn_f32.hip: the float32 kernel (same items; ids != NULL: canonical-order
// tensors, video row r of window w is tensor row ids[offsets[w] + r]).
int attn_f32_tile_m(int head_dim);
hipError_t launch_attn_f32(int head_dim, const float *q, const float *k, const float *v,
                           const float *tq, const float *tk, const float *tv, float *out,
                           float *ws, const int32_t *ids, const ItemDesc *items, const WinDesc *wins,
                           int n_items, int n_heads, int text_len, float scale, hipStream_t s);
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
// gemm_bf16.hip: y[M,N] = x[M,K] w[N,K]^T (+ r), bf16; N % tile_n == 0,
// K % tile_k == 0 (checked by the caller).  rope != NULL (r must be NULL):
// every 128-feature head of row m is rotated after the bf16 rounding, by the
// axial position of pos[cid[m]] (+ text_len on t) for m < n_video, else
// (m - n_video) on all three axes; cs = [P][21] (cos, sin) pairs.
struct GemmRope {
    const int32_t *cid = nullptr;
    const int32_t *pos = nullptr;
    const float2 *cs = nullptr;
    int n_video = 0;
    int text_len = 0;
};
int gemm_bf16_tile_n();
int gemm_bf16_tile_k();
hipError_t launch_gemm_bf16(const void *x, const void *w, void *y, const void *r, int64_t M, int N,
                            int K, const GemmRope *rope, hipStream_t s);
// xcd_probe.hip: xcc[b] = the XCD that work group b of an n_blocks launch ran on.
hipError_t launch_xcd_probe(int32_t *xcc, int n_blocks, hipStream_t s);
// abi.cpp: the XCD count of device dev and whether work group b of a launch
// runs on XCD b mod that count (probed once per device; without probe, a
// device not probed yet reports 8 and round-robin).
int device_xcds(int dev, int *n_xcds, bool *round_robin, bool probe);
// text_mean.hip: txt_out = (sum of the n_parts float32 partials, in order) /
// n_windows, rounded once to dtype.
hipError_t launch_text_mean(const float *ws, void *txt_out, int64_t per_part, int n_parts,
                            int n_windows, int dtype, hipStream_t s);

}  // namespace wsp
