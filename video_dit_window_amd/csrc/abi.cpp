// C entry points of libwsp: argument validation, per-device table caches and
// kernel dispatch.  See include/wsp.h for the contract of each call.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "wsp_internal.h"

namespace wsp {

namespace {
thread_local std::string g_last_error;
std::atomic<int> g_attn_order{WSP_ORDER_LPT_XCD};
std::atomic<int> g_attn_sched{WSP_SCHED_AUTO};

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

std::tuple<int, int, int, int> layout_key(const wsp_plan_t &p) {
    if (p.method == WSP_CANONICAL) return {WSP_CANONICAL, 0, 0, 0};
    return {p.method, p.nt, p.nh, p.nw};
}

template <typename T>
int upload(const T *host, size_t count, T **dev_out) {
    T *d = nullptr;
    const size_t bytes = std::max<size_t>(count, 1) * sizeof(T);
    hipError_t e = hipMalloc(reinterpret_cast<void **>(&d), bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(e == hipErrorOutOfMemory ? WSP_ENOMEM : WSP_EDEVICE,
                    std::string("hipMalloc of a plan table failed: ") + hipGetErrorString(e));
    }
    if (count) {
        e = hipMemcpy(d, host, count * sizeof(T), hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            (void)hipFree(d);
            return hip_fail(e, "hipMemcpy of a plan table");
        }
    }
    *dev_out = d;
    return WSP_OK;
}

}  // namespace

int fail(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(WSP_EDEVICE, std::string(what) + " failed: " + hipGetErrorString(e));
}

int device_offsets(wsp_plan_t &p, int dev, int32_t **out) {
    std::lock_guard<std::mutex> lk(p.mu);
    DeviceTables &t = p.dev[dev];
    if (!t.offsets) {
        int rc = upload(p.offsets.data(), p.offsets.size(), &t.offsets);
        if (rc) return rc;
    }
    *out = t.offsets;
    return WSP_OK;
}

int device_ids(wsp_plan_t &p, int dev, int32_t **out) {
    std::lock_guard<std::mutex> lk(p.mu);
    DeviceTables &t = p.dev[dev];
    if (!t.ids) {
        int rc = upload(p.ids.data(), p.ids.size(), &t.ids);
        if (rc) return rc;
    }
    *out = t.ids;
    return WSP_OK;
}

int device_positions(wsp_plan_t &p, int dev, int32_t **out) {
    std::lock_guard<std::mutex> lk(p.mu);
    DeviceTables &t = p.dev[dev];
    if (!t.pos) {
        std::vector<int32_t> pos;
        try {
            window_positions(p, pos);
        } catch (const std::bad_alloc &) {
            return fail(WSP_ENOMEM, "host allocation of a position table failed");
        }
        int rc = upload(pos.data(), pos.size(), &t.pos);
        if (rc) return rc;
    }
    *out = t.pos;
    return WSP_OK;
}

int device_perm(const wsp_plan_t &src, wsp_plan_t &dst, int dev, int32_t **out) {
    const auto key = layout_key(src);
    {
        std::lock_guard<std::mutex> lk(dst.mu);
        auto &m = dst.dev[dev].perm;
        auto it = m.find(key);
        if (it != m.end()) {
            *out = it->second;
            return WSP_OK;
        }
    }
    std::vector<int32_t> perm;
    try {
        relayout_perm(src, dst, perm);
    } catch (const std::bad_alloc &) {
        return fail(WSP_ENOMEM, "host allocation of a relayout permutation failed");
    }
    int32_t *d = nullptr;
    int rc = upload(perm.data(), perm.size(), &d);
    if (rc) return rc;
    std::lock_guard<std::mutex> lk(dst.mu);
    auto &m = dst.dev[dev].perm;
    auto ins = m.emplace(key, d);
    if (!ins.second) (void)hipFree(d);  // another thread uploaded it first
    *out = ins.first->second;
    return WSP_OK;
}

int device_rel_ids(wsp_plan_t &p, int dev, int32_t **out) {
    std::lock_guard<std::mutex> lk(p.mu);
    DeviceTables &t = p.dev[dev];
    if (!t.rel) {
        std::vector<int32_t> rel;
        try {
            rel.resize(p.ids.size());
        } catch (const std::bad_alloc &) {
            return fail(WSP_ENOMEM, "host allocation of the relative id table failed");
        }
        for (int32_t w = 0; w < p.nwin; ++w)
            for (int32_t j = p.offsets[w]; j < p.offsets[w + 1]; ++j) rel[j] = p.ids[j] - p.ids[p.offsets[w]];
        int rc = upload(rel.data(), rel.size(), &t.rel);
        if (rc) return rc;
    }
    *out = t.rel;
    return WSP_OK;
}

int device_layout_positions(wsp_plan_t &p, int dev, int32_t **out) {
    std::lock_guard<std::mutex> lk(p.mu);
    DeviceTables &t = p.dev[dev];
    if (!t.lpos) {
        std::vector<int32_t> pos, lpos;
        try {
            window_positions(p, pos);
            lpos.resize(p.ids.size());
        } catch (const std::bad_alloc &) {
            return fail(WSP_ENOMEM, "host allocation of a position table failed");
        }
        for (size_t j = 0; j < lpos.size(); ++j) lpos[j] = pos[size_t(p.ids[j])];
        int rc = upload(lpos.data(), lpos.size(), &t.lpos);
        if (rc) return rc;
    }
    *out = t.lpos;
    return WSP_OK;
}

namespace {
struct XcdInfo {
    int n = 0;
    bool round_robin = false;
};
std::mutex g_xcd_mu;
std::map<int, XcdInfo> g_xcd;  // device ordinal -> probed work-group placement
}  // namespace

int device_xcds(int dev, int *n_xcds, bool *round_robin, bool probe) {
    std::lock_guard<std::mutex> lk(g_xcd_mu);
    auto it = g_xcd.find(dev);
    if (it == g_xcd.end() && !probe) {  // not known yet: report the assumed placement
        *n_xcds = 8;
        *round_robin = true;
        return WSP_OK;
    }
    if (it == g_xcd.end()) {
        // One synchronous probe per device (like the first table upload):
        // 1024 one-wave work groups report the XCD they ran on.
        constexpr int kBlocks = 1024;
        int32_t *d = nullptr;
        hipError_t e = hipMalloc(reinterpret_cast<void **>(&d), kBlocks * sizeof(int32_t));
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(e == hipErrorOutOfMemory ? WSP_ENOMEM : WSP_EDEVICE,
                        std::string("hipMalloc of the XCD probe failed: ") + hipGetErrorString(e));
        }
        std::vector<int32_t> xcc(kBlocks, -1);
        e = launch_xcd_probe(d, kBlocks, nullptr);
        if (e == hipSuccess) e = hipMemcpy(xcc.data(), d, kBlocks * sizeof(int32_t), hipMemcpyDeviceToHost);
        (void)hipFree(d);
        if (e != hipSuccess) return hip_fail(e, "XCD probe");
        XcdInfo info;
        info.n = 1 + *std::max_element(xcc.begin(), xcc.end());
        info.round_robin = true;
        for (int b = 0; b < kBlocks; ++b) info.round_robin = info.round_robin && xcc[size_t(b)] == b % info.n;
        it = g_xcd.emplace(dev, info).first;
    }
    *n_xcds = it->second.n;
    *round_robin = it->second.round_robin;
    return WSP_OK;
}

int device_windows(wsp_plan_t &p, int dev, bool gather, WinDesc **out) {
    std::lock_guard<std::mutex> lk(p.mu);
    DeviceTables &t = p.dev[dev];
    WinDesc *&d = t.wins[gather ? 1 : 0];
    if (!d) {
        std::vector<WinDesc> wins;
        try {
            window_descs(p, gather, wins);
        } catch (const std::bad_alloc &) {
            return fail(WSP_ENOMEM, "host allocation of the window table failed");
        }
        int rc = upload(wins.data(), wins.size(), &d);
        if (rc) return rc;
    }
    *out = d;
    return WSP_OK;
}

int device_items(wsp_plan_t &p, int dev, int n_heads, int text_len, int bm, int order, bool gather,
                 int n_chunks, ItemDesc **out, int *count) {
    const auto key = std::make_tuple(n_heads, text_len, bm, order, int(gather), n_chunks);
    {
        std::lock_guard<std::mutex> lk(p.mu);
        auto &m = p.dev[dev].items;
        auto it = m.find(key);
        if (it != m.end()) {
            *out = it->second.first;
            *count = it->second.second;
            return WSP_OK;
        }
    }
    std::vector<ItemDesc> items;
    int rc;
    try {
        rc = build_items(p, n_heads, text_len, bm, order, gather, n_chunks, items);
    } catch (const std::bad_alloc &) {
        return fail(WSP_ENOMEM, "host allocation of the attention work list failed");
    }
    if (rc < 0) return rc;
    ItemDesc *d = nullptr;
    rc = upload(items.data(), items.size(), &d);
    if (rc) return rc;
    std::lock_guard<std::mutex> lk(p.mu);
    auto &m = p.dev[dev].items;
    auto ins = m.emplace(key, std::make_pair(d, int(items.size())));
    if (!ins.second) (void)hipFree(d);
    *out = ins.first->second.first;
    *count = ins.first->second.second;
    return WSP_OK;
}

}  // namespace wsp

using namespace wsp;

extern "C" {

const char *wsp_last_error(void) { return g_last_error.c_str(); }

int wsp_version(void) { return WSP_VERSION; }

int wsp_plan(int T, int H, int W, int nt, int nh, int nw, int method, wsp_plan_t **out) {
    g_last_error.clear();
    if (!out) return fail(WSP_EINVAL, "out is NULL");
    *out = nullptr;
    wsp_plan_t *p = new (std::nothrow) wsp_plan_t;
    if (!p) return fail(WSP_ENOMEM, "plan allocation failed");
    int rc = build_plan(T, H, W, nt, nh, nw, method, *p);
    if (rc) {
        delete p;
        return rc;
    }
    *out = p;
    return WSP_OK;
}

int wsp_plan_info(const wsp_plan_t *p, int64_t *n_tokens, int32_t *n_windows, int32_t *win_size) {
    g_last_error.clear();
    if (!p) return fail(WSP_EINVAL, "plan is NULL");
    if (n_tokens) *n_tokens = p->n;
    if (n_windows) *n_windows = p->nwin;
    if (win_size) {
        win_size[0] = p->wt;
        win_size[1] = p->wh;
        win_size[2] = p->ww;
    }
    return WSP_OK;
}

int wsp_plan_tables(const wsp_plan_t *p, int32_t *offsets, int32_t *ids, int32_t *inv,
                    int32_t *boxes, int32_t *lpt) {
    g_last_error.clear();
    if (!p) return fail(WSP_EINVAL, "plan is NULL");
    if (offsets) std::memcpy(offsets, p->offsets.data(), p->offsets.size() * 4);
    if (ids) std::memcpy(ids, p->ids.data(), p->ids.size() * 4);
    if (inv) std::memcpy(inv, p->inv.data(), p->inv.size() * 4);
    if (boxes) std::memcpy(boxes, p->boxes.data(), p->boxes.size() * 4);
    if (lpt) std::memcpy(lpt, p->lpt.data(), p->lpt.size() * 4);
    return WSP_OK;
}

void wsp_plan_free(wsp_plan_t *p) {
    if (!p) return;
    int cur = -1;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (auto &kv : p->dev) {
        if (hipSetDevice(kv.first) != hipSuccess) continue;
        DeviceTables &t = kv.second;
        if (t.offsets) (void)hipFree(t.offsets);
        if (t.ids) (void)hipFree(t.ids);
        if (t.rel) (void)hipFree(t.rel);
        if (t.pos) (void)hipFree(t.pos);
        for (WinDesc *w : t.wins)
            if (w) (void)hipFree(w);
        for (auto &pm : t.perm) (void)hipFree(pm.second);
        for (auto &it : t.items) (void)hipFree(it.second.first);
    }
    if (have_cur) (void)hipSetDevice(cur);
    delete p;
}

int wsp_relayout(const void *x, void *y, int64_t row_bytes, const wsp_plan_t *src,
                 const wsp_plan_t *dst, void *stream) {
    g_last_error.clear();
    if (!src || !dst) return fail(WSP_EINVAL, "plan is NULL");
    if (src->T != dst->T || src->H != dst->H || src->W != dst->W)
        return fail(WSP_EINVAL, "relayout between plans of different grids");
    if (row_bytes <= 0 || row_bytes % 16)
        return fail(WSP_EINVAL, "row_bytes must be a positive multiple of 16, got " +
                                    std::to_string(row_bytes));
    if (!x || !y) return fail(WSP_EINVAL, "x or y is NULL");
    if (!aligned16(x) || !aligned16(y)) return fail(WSP_EINVAL, "x and y must be 16-byte aligned");
    if (x == y) return fail(WSP_EINVAL, "x and y must not alias");
    if (row_bytes > (int64_t(1) << 40) / std::max<int64_t>(dst->n, 1))
        return fail(WSP_ERANGE, "n_tokens * row_bytes too large");
    int dev = 0;
    WSP_HIP(hipGetDevice(&dev));
    int32_t *perm = nullptr;
    int rc = device_perm(*src, *const_cast<wsp_plan_t *>(dst), dev, &perm);
    if (rc) return rc;
    hipError_t e = launch_relayout(x, y, perm, dst->n, row_bytes, hipStream_t(stream));
    if (e != hipSuccess) return hip_fail(e, "relayout kernel launch");
    return WSP_OK;
}

int wsp_window_attn_workspace(const wsp_plan_t *p, int n_heads, int head_dim, int text_len,
                              int dtype, size_t *bytes) {
    g_last_error.clear();
    if (!p || !bytes) return fail(WSP_EINVAL, "plan or bytes is NULL");
    if (n_heads < 1 || n_heads > 32767) return fail(WSP_EINVAL, "n_heads must be in 1..32767");
    if (head_dim != 64 && head_dim != 128) return fail(WSP_EINVAL, "head_dim must be 64 or 128");
    if (text_len < 0) return fail(WSP_EINVAL, "text_len must be >= 0");
    if (dtype != WSP_F32 && dtype != WSP_BF16) return fail(WSP_EINVAL, "unknown dtype");
    const int G = text_chunks(p->nwin);
    const double b = double(G) * text_len * n_heads * head_dim * 4.0;
    if (b > 9e18) return fail(WSP_ERANGE, "workspace size overflows");
    *bytes = size_t(G) * size_t(text_len) * size_t(n_heads) * size_t(head_dim) * 4u +
             (dtype == WSP_BF16 ? kQueueBytes : 0);
    return WSP_OK;
}

int wsp_window_attn(const wsp_plan_t *pc, const void *q, const void *k, const void *v,
                    const void *txt_q, const void *txt_k, const void *txt_v, int n_heads,
                    int head_dim, int text_len, int dtype, float scale, void *out,
                    void *txt_out, void *workspace, size_t workspace_bytes, void *stream) {
    return wsp_window_attn_ex(pc, q, k, v, txt_q, txt_k, txt_v, n_heads, head_dim, text_len, dtype,
                              scale, WSP_ATTN_IO_LAYOUT, out, txt_out, workspace, workspace_bytes,
                              stream);
}

namespace {

constexpr int kRopeHeadDim = 128;
constexpr int kRopeAxisPairs = 21;

// (cos, sin) of position p times theta^(-2i/42), i < 21, for p < P; one table
// per (device, theta, P), built in double and kept until the process ends.
std::mutex g_rope_mu;
std::map<std::tuple<int, uint32_t, int>, float2 *> g_rope_tables;

int rope_table(int dev, float theta, int P, const float2 **out) {
    uint32_t tb;
    std::memcpy(&tb, &theta, sizeof tb);
    const auto key = std::make_tuple(dev, tb, P);
    std::lock_guard<std::mutex> lk(g_rope_mu);
    auto it = g_rope_tables.find(key);
    if (it != g_rope_tables.end()) {
        *out = it->second;
        return WSP_OK;
    }
    std::vector<float2> host;
    try {
        host.resize(size_t(P) * kRopeAxisPairs);
    } catch (const std::bad_alloc &) {
        return fail(WSP_ENOMEM, "host allocation of a rotary table failed");
    }
    const int axis = 2 * kRopeAxisPairs;
    for (int p = 0; p < P; ++p)
        for (int i = 0; i < kRopeAxisPairs; ++i) {
            const double a = double(p) * std::pow(double(theta), -2.0 * i / axis);
            host[size_t(p) * kRopeAxisPairs + i] = float2{float(std::cos(a)), float(std::sin(a))};
        }
    float2 *d = nullptr;
    int rc = upload(host.data(), host.size(), &d);
    if (rc) return rc;
    g_rope_tables.emplace(key, d);
    *out = d;
    return WSP_OK;
}

int rope_args(const void *x, const void *y, int n_heads, int head_dim, int dtype, int text_len,
              float &theta) {
    if (!x || !y) return fail(WSP_EINVAL, "x or y is NULL");
    if (!aligned16(x) || !aligned16(y)) return fail(WSP_EINVAL, "x and y must be 16-byte aligned");
    if (x == y) return fail(WSP_EINVAL, "x and y must not alias");
    if (head_dim != kRopeHeadDim)
        return fail(WSP_EINVAL, "rotary embedding needs head_dim 128 (three 42-channel axis blocks), got " +
                                    std::to_string(head_dim));
    if (n_heads < 1 || n_heads > 32767) return fail(WSP_EINVAL, "n_heads must be in 1..32767");
    if (dtype != WSP_F32 && dtype != WSP_BF16) return fail(WSP_EINVAL, "unknown dtype");
    if (text_len < 0 || text_len > (1 << 20)) return fail(WSP_EINVAL, "text_len must be in 0..2^20");
    if (!(theta > 0.0f) || !std::isfinite(theta)) theta = 10000.0f;
    return WSP_OK;
}

}  // namespace

namespace {

// ---- the no-allocation entry point's scratch --------------------------------
// Float32 text partials for wsp_window_attn_noalloc: a file-scope device array
// (each GPU the library runs on holds its own copy until the process ends).
// Host code never passes the array's name to a kernel: its device address
// comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(96) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_ptr;  // device ordinal -> device address of `scratch`

int scratch_address(int dev, void **out) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it == g_scratch_ptr.end()) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress of the scratch array");
        }
        it = g_scratch_ptr.emplace(dev, ptr).first;
    }
    *out = it->second;
    return WSP_OK;
}

// Device tables of one attention call, looked up only (nothing is uploaded
// or allocated): the no-allocation entry point runs on tables that a call of
// wsp_window_attn_ex with the same plan and shape left on the device.
int resident_tables(wsp_plan_t &p, int dev, int n_heads, int text_len, int bm, int order, bool gather,
                    int n_chunks, bool bf16, ItemDesc **items, int *n_items, WinDesc **wins, int32_t **ids,
                    int32_t **rel) {
    std::lock_guard<std::mutex> lk(p.mu);
    auto d = p.dev.find(dev);
    if (d != p.dev.end()) {
        DeviceTables &t = d->second;
        auto it = t.items.find(std::make_tuple(n_heads, text_len, bm, order, int(gather), n_chunks));
        WinDesc *w = t.wins[gather ? 1 : 0];
        const bool have_ids = !gather || (bf16 ? t.rel != nullptr : t.ids != nullptr);
        if (it != t.items.end() && w && have_ids) {
            *items = it->second.first;
            *n_items = it->second.second;
            *wins = w;
            *ids = gather && !bf16 ? t.ids : nullptr;
            *rel = gather && bf16 ? t.rel : nullptr;
            return WSP_OK;
        }
    }
    return fail(WSP_EINVAL,
                "the plan's device tables for this head count, text length, dtype, I/O order, schedule and "
                "text reduction are not on this device: call wsp_window_attn_ex once with the same arguments "
                "first (it uploads them; wsp_window_attn_noalloc allocates nothing)");
}

// Bytes of the rotated k (n_tokens rows) and the rotated text q and k that
// lead wsp_window_attn_rope's workspace (bf16, head dim 128), each part
// rounded up to 256.
size_t rope_part_bytes(int64_t rows, int n_heads) {
    return (size_t(rows) * size_t(n_heads) * kRopeHeadDim * 2u + 255u) & ~size_t(255);
}
size_t rope_bytes(const wsp_plan_t &p, int text_len, int n_heads) {
    return rope_part_bytes(p.n, n_heads) + 2 * rope_part_bytes(text_len, n_heads);
}

// Shared body of wsp_window_attn_ex (q8 = false), wsp_window_attn_qk8,
// wsp_window_attn_noalloc (no_alloc: resident tables, the scratch array as
// workspace) and wsp_window_attn_rope (rope_theta != NULL: the workspace
// starts with the rotated k, text q and text k; the video queries turn
// inside the attention kernel).
int window_attn_impl(const wsp_plan_t *pc, const void *q, const void *k, const void *v,
                     const void *txt_q, const void *txt_k, const void *txt_v, int n_heads,
                     int head_dim, int text_len, int dtype, bool q8, const float *amax_q,
                     const float *amax_k, float scale, unsigned flags, void *out, void *txt_out,
                     void *workspace, size_t workspace_bytes, void *stream, bool no_alloc = false,
                     const float *rope_theta = nullptr) {
    if (flags & ~unsigned(WSP_ATTN_IO_CANONICAL)) return fail(WSP_EINVAL, "unknown attention flags");
    const bool gather = (flags & WSP_ATTN_IO_CANONICAL) != 0;
    size_t need = 0;
    int rc = wsp_window_attn_workspace(pc, n_heads, head_dim, text_len, dtype, &need);
    if (rc) return rc;
    wsp_plan_t *p = const_cast<wsp_plan_t *>(pc);
    const bool rope = rope_theta != nullptr;
    float theta = rope ? *rope_theta : 0.f;
    size_t rot_bytes = 0;
    if (rope) {
        if (dtype != WSP_BF16 || head_dim != kRopeHeadDim)
            return fail(WSP_EINVAL, "rotary attention needs bf16 and head_dim 128");
        if (text_len > (1 << 20)) return fail(WSP_EINVAL, "text_len must be in 0..2^20");
        if (!(theta > 0.0f) || !std::isfinite(theta)) theta = 10000.0f;
        if (p->max_ext[0] > 1024 || p->max_ext[1] > 2048 || p->max_ext[2] > 2048)
            return fail(WSP_ERANGE, "window extents beyond 1024 (t) / 2048 (h, w)");
        rot_bytes = rope_bytes(*p, text_len, n_heads);
        need += rot_bytes;
    }
    for (const void *ptr : {q, k, v, static_cast<const void *>(out)}) {
        if (!ptr) return fail(WSP_EINVAL, "q, k, v and out must be non-NULL");
        if (!aligned16(ptr)) return fail(WSP_EINVAL, "q, k, v and out must be 16-byte aligned");
    }
    if (out == q || out == k || out == v) return fail(WSP_EINVAL, "out must not alias q, k or v");
    // The matrix-core kernel addresses a window's video rows (canonical
    // order: the rows between its smallest and largest canonical id) and the
    // text rows with 31-bit byte offsets from per-window buffer bases.
    if (dtype == WSP_BF16) {
        const int64_t row_bytes = int64_t(n_heads) * head_dim * 2;
        const int64_t rows = std::max<int64_t>(gather ? p->max_span : p->max_rows, text_len);
        if (rows * row_bytes >= (int64_t(1) << 31))
            return fail(WSP_ERANGE, gather ? "a window's canonical rows span 2 GiB or more"
                                           : "a window's rows (or the text rows) take 2 GiB or more");
        // Canonical order: the kernel forms row offsets as 24-bit products
        // (relative id x row bytes).  Exact: row_bytes <= 32767 * 128 * 2 < 2^24
        // (n_heads and head_dim checked above), and relative id < span <
        // 2^31 / row_bytes <= 2^24 because row_bytes >= 128.
    }
    if ((rope || (dtype == WSP_BF16 && !no_alloc)) && (!workspace || workspace_bytes < need))
        return fail(WSP_EWORKSPACE, "workspace of " + std::to_string(need) + " bytes required, got " +
                                        std::to_string(workspace_bytes));
    if ((rope || (dtype == WSP_BF16 && !no_alloc)) && !aligned16(workspace))
        return fail(WSP_EINVAL, "workspace must be 16-byte aligned");
    if (no_alloc && (text_len > 0 || dtype == WSP_BF16)) {
        if (need > kScratchBytes)
            return fail(WSP_ERANGE, "wsp_window_attn_noalloc: the text mean needs " + std::to_string(need) +
                                        " bytes of scratch, more than its fixed " + std::to_string(kScratchBytes) +
                                        " (use wsp_window_attn_ex)");
        workspace_bytes = kScratchBytes;
    }
    if (text_len > 0) {
        for (const void *ptr : {txt_q, txt_k, txt_v, static_cast<const void *>(txt_out)}) {
            if (!ptr) return fail(WSP_EINVAL, "text tensors and txt_out must be non-NULL when text_len > 0");
            if (!aligned16(ptr)) return fail(WSP_EINVAL, "text tensors must be 16-byte aligned");
        }
        if (!no_alloc) {
            if (!workspace || workspace_bytes < need)
                return fail(WSP_EWORKSPACE, "workspace of " + std::to_string(need) +
                                                " bytes required, got " + std::to_string(workspace_bytes));
            if (!aligned16(workspace)) return fail(WSP_EINVAL, "workspace must be 16-byte aligned");
        }
    }
    // Workspace: rotated k, text q and text k (rotary attention), the work
    // queue's counters (bf16), then the text partials.
    void *rot_k = nullptr, *rot_tq = nullptr, *rot_tk = nullptr;
    if (rope) {
        uint8_t *w = static_cast<uint8_t *>(workspace);
        rot_k = w;
        rot_tq = w + rope_part_bytes(p->n, n_heads);
        rot_tk = static_cast<uint8_t *>(rot_tq) + rope_part_bytes(text_len, n_heads);
        workspace = w + rot_bytes;
        workspace_bytes -= rot_bytes;
    }
    if (!(scale > 0.0f) || !std::isfinite(scale)) scale = 1.0f / std::sqrt(float(head_dim));
    // One text partial per window when the workspace holds them (each text
    // item then shares its window's K/V with the video items in L2), else
    // min(n_windows, 16) chunks.
    const size_t per_part = size_t(text_len) * size_t(n_heads) * size_t(head_dim) * 4u;
    const size_t queue_bytes = dtype == WSP_BF16 ? kQueueBytes : 0;
    const int n_chunks =
        workspace_bytes - queue_bytes >= per_part * size_t(p->nwin) ? p->nwin : text_chunks(p->nwin);
    int order = g_attn_order.load();
    // Short windows (joint sequences averaging < 1024 rows) take 128-row
    // query tiles: a window's partly empty last tile then wastes less.
    const int sched = g_attn_sched.load();
    const bool short_items = (double(p->n) / double(p->nwin) + text_len) < 1024.0;
    const bool small = sched == WSP_SCHED_PER_ITEM_128 || sched == WSP_SCHED_QUEUE_128 ||
                       (sched == WSP_SCHED_AUTO && short_items);
    const bool use_queue = sched == WSP_SCHED_QUEUE || sched == WSP_SCHED_QUEUE_128 || sched == WSP_SCHED_AUTO;
    const int bm = dtype != WSP_BF16 ? attn_f32_tile_m(head_dim) : attn_bf16_tile_m(small);

    int dev = 0;
    WSP_HIP(hipGetDevice(&dev));
    if (order == WSP_ORDER_LPT_XCD) {
        // The XCD grouping of the work list holds only where work group b
        // runs on XCD b mod 8; elsewhere plain largest-first order.
        // (the no-allocation entry point never probes: its tables, built by
        // an earlier wsp_window_attn_ex call, already reflect the probe)
        int n_xcds = 0;
        bool rr = false;
        if ((rc = device_xcds(dev, &n_xcds, &rr, !no_alloc))) return rc;
        if (n_xcds != 8 || !rr) order = WSP_ORDER_LPT;
    }
    ItemDesc *items = nullptr;
    WinDesc *wins = nullptr;
    int n_items = 0;
    int32_t *d_ids = nullptr, *d_rel = nullptr;
    if (no_alloc) {
        if ((rc = resident_tables(*p, dev, n_heads, text_len, bm, order, gather, n_chunks, dtype == WSP_BF16,
                                  &items, &n_items, &wins, &d_ids, &d_rel)))
            return rc;
        if ((text_len > 0 || dtype == WSP_BF16) && (rc = scratch_address(dev, &workspace))) return rc;
    } else {
        if ((rc = device_items(*p, dev, n_heads, text_len, bm, order, gather, n_chunks, &items, &n_items)))
            return rc;
        if ((rc = device_windows(*p, dev, gather, &wins))) return rc;
        if (gather && dtype == WSP_BF16 && (rc = device_rel_ids(*p, dev, &d_rel))) return rc;
        if (gather && dtype != WSP_BF16 && (rc = device_ids(*p, dev, &d_ids))) return rc;
    }
    hipStream_t s = hipStream_t(stream);
    uint32_t *queue = nullptr;
    if (queue_bytes) {
        queue = static_cast<uint32_t *>(workspace);
        workspace = static_cast<uint8_t *>(workspace) + queue_bytes;
    }
    float *ws = static_cast<float *>(workspace);
    hipError_t e;
    RopeTables rt;
    if (rope) {
        // k rotated once for every query tile that reads it (the stand-alone
        // rotation kernel, in the I/O order: canonical rows take positions by
        // canonical id, layout rows through the plan's ids), the text rows
        // at (i, i, i); the queries turn as the attention kernel loads them.
        const float2 *cs = nullptr;
        int32_t *pos = nullptr, *lpos = nullptr, *cid = nullptr;
        const int P = std::max({text_len + p->max_ext[0], p->max_ext[1], p->max_ext[2], text_len, 1});
        if ((rc = rope_table(dev, theta, P, &cs))) return rc;
        if ((rc = device_positions(*p, dev, &pos))) return rc;
        if ((rc = device_layout_positions(*p, dev, &lpos))) return rc;
        if (!gather && (rc = device_ids(*p, dev, &cid))) return rc;
        rt = RopeTables{cs, lpos};
        e = launch_rope(k, rot_k, nullptr, cid, pos, cs, p->n, n_heads, dtype, text_len, s);
        if (e == hipSuccess && text_len > 0)
            e = launch_rope(txt_q, rot_tq, nullptr, nullptr, nullptr, cs, text_len, n_heads, dtype, 0, s);
        if (e == hipSuccess && text_len > 0)
            e = launch_rope(txt_k, rot_tk, nullptr, nullptr, nullptr, cs, text_len, n_heads, dtype, 0, s);
        if (e != hipSuccess) return hip_fail(e, "rope kernel launch");
        k = rot_k;
        if (text_len > 0) {
            txt_q = rot_tq;
            txt_k = rot_tk;
        }
    }
    if (dtype == WSP_BF16)
        e = launch_attn_bf16(head_dim, small, q8, q, k, v, txt_q, txt_k, txt_v, out, ws, d_rel, items, wins,
                             n_items, amax_q, amax_k, rope ? &rt : nullptr, n_heads, text_len, scale,
                             use_queue ? queue : nullptr, order == WSP_ORDER_LPT_XCD ? 8 : 1, p->H * p->W, p->W, s);
    else
        e = launch_attn_f32(head_dim, static_cast<const float *>(q), static_cast<const float *>(k),
                            static_cast<const float *>(v), static_cast<const float *>(txt_q),
                            static_cast<const float *>(txt_k), static_cast<const float *>(txt_v),
                            static_cast<float *>(out), ws, d_ids, items, wins, n_items, n_heads,
                            text_len, scale, s);
    if (e != hipSuccess) return hip_fail(e, "window attention kernel launch");
    if (text_len > 0) {
        e = launch_text_mean(ws, txt_out, int64_t(text_len) * n_heads * head_dim, n_chunks, p->nwin, dtype, s);
        if (e != hipSuccess) return hip_fail(e, "text mean kernel launch");
    }
    return WSP_OK;
}

}  // namespace

int wsp_window_attn_ex(const wsp_plan_t *pc, const void *q, const void *k, const void *v,
                       const void *txt_q, const void *txt_k, const void *txt_v, int n_heads,
                       int head_dim, int text_len, int dtype, float scale, unsigned flags,
                       void *out, void *txt_out, void *workspace, size_t workspace_bytes,
                       void *stream) {
    g_last_error.clear();
    return window_attn_impl(pc, q, k, v, txt_q, txt_k, txt_v, n_heads, head_dim, text_len, dtype, false,
                            nullptr, nullptr, scale, flags, out, txt_out, workspace, workspace_bytes, stream);
}


int wsp_rope_relayout(const void *x, void *y, int n_heads, int head_dim, int dtype,
                      const wsp_plan_t *src, const wsp_plan_t *dst, const wsp_plan_t *pos,
                      int text_len, float theta, void *stream) {
    g_last_error.clear();
    if (!src || !dst || !pos) return fail(WSP_EINVAL, "plan is NULL");
    if (src->T != dst->T || src->H != dst->H || src->W != dst->W || pos->T != dst->T ||
        pos->H != dst->H || pos->W != dst->W)
        return fail(WSP_EINVAL, "plans of different grids");
    int rc = rope_args(x, y, n_heads, head_dim, dtype, text_len, theta);
    if (rc) return rc;
    if (pos->max_ext[0] > 1024 || pos->max_ext[1] > 2048 || pos->max_ext[2] > 2048)
        return fail(WSP_ERANGE, "window extents beyond 1024 (t) / 2048 (h, w)");
    const int P = std::max({text_len + pos->max_ext[0], pos->max_ext[1], pos->max_ext[2]});
    int dev = 0;
    WSP_HIP(hipGetDevice(&dev));
    int32_t *perm = nullptr, *cid = nullptr, *ptab = nullptr;
    const float2 *cs = nullptr;
    if ((rc = device_perm(*src, *const_cast<wsp_plan_t *>(dst), dev, &perm))) return rc;
    if ((rc = device_ids(*const_cast<wsp_plan_t *>(dst), dev, &cid))) return rc;
    if ((rc = device_positions(*const_cast<wsp_plan_t *>(pos), dev, &ptab))) return rc;
    if ((rc = rope_table(dev, theta, P, &cs))) return rc;
    hipError_t e = launch_rope(x, y, perm, cid, ptab, cs, dst->n, n_heads, dtype, text_len,
                               hipStream_t(stream));
    if (e != hipSuccess) return hip_fail(e, "rope kernel launch");
    return WSP_OK;
}

int wsp_rope_text(const void *x, void *y, int text_len, int n_heads, int head_dim, int dtype,
                  float theta, void *stream) {
    g_last_error.clear();
    int rc = rope_args(x, y, n_heads, head_dim, dtype, text_len, theta);
    if (rc) return rc;
    if (text_len == 0) return WSP_OK;
    int dev = 0;
    WSP_HIP(hipGetDevice(&dev));
    const float2 *cs = nullptr;
    if ((rc = rope_table(dev, theta, text_len, &cs))) return rc;
    hipError_t e = launch_rope(x, y, nullptr, nullptr, nullptr, cs, text_len, n_heads, dtype, 0,
                               hipStream_t(stream));
    if (e != hipSuccess) return hip_fail(e, "rope kernel launch");
    return WSP_OK;
}

int wsp_fp8_amax(const void *x, int64_t n_rows, int n_heads, int head_dim, int dtype, float *amax,
                 void *stream) {
    g_last_error.clear();
    if (!amax) return fail(WSP_EINVAL, "amax is NULL");
    if (n_rows < 0) return fail(WSP_EINVAL, "n_rows must be >= 0");
    if (n_rows > 0 && !x) return fail(WSP_EINVAL, "x is NULL");
    if (x && !aligned16(x)) return fail(WSP_EINVAL, "x must be 16-byte aligned");
    if (!aligned16(amax) && (reinterpret_cast<uintptr_t>(amax) & 3u))
        return fail(WSP_EINVAL, "amax must be 4-byte aligned");
    if (head_dim != 64 && head_dim != 128) return fail(WSP_EINVAL, "head_dim must be 64 or 128");
    if (dtype != WSP_F32 && dtype != WSP_BF16) return fail(WSP_EINVAL, "unknown dtype");
    const int elem = dtype == WSP_BF16 ? 2 : 4;
    if (n_heads < 1 || int64_t(n_heads) * head_dim * elem / 16 > fp8_max_row_chunks())
        return fail(WSP_EINVAL, "n_heads out of range (a row may hold at most " +
                                    std::to_string(fp8_max_row_chunks() * 16) + " bytes)");
    hipError_t e = launch_fp8_amax(x, amax, n_rows, n_heads, head_dim, dtype, hipStream_t(stream));
    if (e != hipSuccess) return hip_fail(e, "fp8 amax kernel launch");
    return WSP_OK;
}

int wsp_fp8_quantize(const void *x, void *y, int64_t n_rows, int n_heads, int head_dim, int dtype,
                     const float *amax, void *stream) {
    g_last_error.clear();
    if (!amax) return fail(WSP_EINVAL, "amax is NULL");
    if (n_rows < 0) return fail(WSP_EINVAL, "n_rows must be >= 0");
    if (n_rows > 0 && (!x || !y)) return fail(WSP_EINVAL, "x or y is NULL");
    if ((x && !aligned16(x)) || (y && !aligned16(y)))
        return fail(WSP_EINVAL, "x and y must be 16-byte aligned");
    if (head_dim != 64 && head_dim != 128) return fail(WSP_EINVAL, "head_dim must be 64 or 128");
    if (dtype != WSP_F32 && dtype != WSP_BF16) return fail(WSP_EINVAL, "unknown dtype");
    if (n_heads < 1 || n_heads > 32767) return fail(WSP_EINVAL, "n_heads must be in 1..32767");
    hipError_t e = launch_fp8_quantize(x, y, amax, n_rows, n_heads, head_dim, dtype, hipStream_t(stream));
    if (e != hipSuccess) return hip_fail(e, "fp8 quantize kernel launch");
    return WSP_OK;
}

int wsp_window_attn_rope_workspace(const wsp_plan_t *p, int n_heads, int head_dim, int text_len, int dtype,
                                   size_t *bytes) {
    g_last_error.clear();
    int rc = wsp_window_attn_workspace(p, n_heads, head_dim, text_len, dtype, bytes);
    if (rc) return rc;
    if (dtype != WSP_BF16 || head_dim != kRopeHeadDim)
        return fail(WSP_EINVAL, "rotary attention needs bf16 and head_dim 128");
    *bytes += rope_bytes(*p, text_len, n_heads);
    return WSP_OK;
}

int wsp_window_attn_rope(const wsp_plan_t *pc, const void *q, const void *k, const void *v,
                         const void *txt_q, const void *txt_k, const void *txt_v, int n_heads,
                         int head_dim, int text_len, int dtype, float scale, float theta, unsigned flags,
                         void *out, void *txt_out, void *workspace, size_t workspace_bytes, void *stream) {
    g_last_error.clear();
    return window_attn_impl(pc, q, k, v, txt_q, txt_k, txt_v, n_heads, head_dim, text_len, dtype, false,
                            nullptr, nullptr, scale, flags, out, txt_out, workspace, workspace_bytes, stream,
                            false, &theta);
}

int wsp_window_attn_noalloc(const wsp_plan_t *pc, const void *q, const void *k, const void *v,
                            const void *txt_q, const void *txt_k, const void *txt_v, int n_heads,
                            int head_dim, int text_len, int dtype, float scale, unsigned flags,
                            void *out, void *txt_out, void *stream) {
    g_last_error.clear();
    return window_attn_impl(pc, q, k, v, txt_q, txt_k, txt_v, n_heads, head_dim, text_len, dtype, false,
                            nullptr, nullptr, scale, flags, out, txt_out, nullptr, 0, stream, true);
}

int wsp_window_attn_qk8(const wsp_plan_t *pc, const void *q8, const void *k8, const void *v,
                        const void *txt_q8, const void *txt_k8, const void *txt_v,
                        const float *amax_q, const float *amax_k, int n_heads, int head_dim,
                        int text_len, float scale, unsigned flags, void *out, void *txt_out,
                        void *workspace, size_t workspace_bytes, void *stream) {
    g_last_error.clear();
    if (head_dim != 128) return fail(WSP_EINVAL, "the fp8 q/k attention needs head_dim 128");
    if (!amax_q || !amax_k) return fail(WSP_EINVAL, "amax_q and amax_k must be non-NULL");
    if (!aligned16(amax_q) && (reinterpret_cast<uintptr_t>(amax_q) & 3u))
        return fail(WSP_EINVAL, "amax_q must be 4-byte aligned");
    if (!aligned16(amax_k) && (reinterpret_cast<uintptr_t>(amax_k) & 3u))
        return fail(WSP_EINVAL, "amax_k must be 4-byte aligned");
    return window_attn_impl(pc, q8, k8, v, txt_q8, txt_k8, txt_v, n_heads, head_dim, text_len, WSP_BF16, true,
                            amax_q, amax_k, scale, flags, out, txt_out, workspace, workspace_bytes, stream);
}

namespace {

// Checks shared by wsp_linear and wsp_linear_rope; WSP_OK with M == 0 means
// nothing to do.
int linear_args(const void *x, const void *w, const void *r, const void *y, int64_t M, int N, int K,
                int dtype, const char *name) {
    if (dtype != WSP_BF16) return fail(WSP_EINVAL, std::string(name) + " supports WSP_BF16 only");
    if (M < 0) return fail(WSP_EINVAL, "M must be >= 0");
    if (N <= 0 || N % gemm_bf16_tile_n() != 0)
        return fail(WSP_EINVAL, "N must be a positive multiple of " + std::to_string(gemm_bf16_tile_n()));
    if (K <= 0 || K % gemm_bf16_tile_k() != 0 || K >= (1 << 20))
        return fail(WSP_EINVAL, "K must be a positive multiple of " + std::to_string(gemm_bf16_tile_k()) +
                                    " below 2^20");
    if (M == 0) return WSP_OK;
    if (M > int64_t(0x7FFFFFFF) - 256) return fail(WSP_ERANGE, "M is too large");
    if (!x || !w || !y) return fail(WSP_EINVAL, "x, w and y must be non-NULL");
    for (const void *ptr : {x, w, r, y})
        if (ptr && !aligned16(ptr)) return fail(WSP_EINVAL, "x, w, r and y must be 16-byte aligned");
    if (y == x || y == w) return fail(WSP_EINVAL, "y must not alias x or w");
    return WSP_OK;
}

}  // namespace

int wsp_linear(const void *x, const void *w, const void *r, void *y, int64_t M, int N, int K,
               int dtype, void *stream) {
    g_last_error.clear();
    int rc = linear_args(x, w, r, y, M, N, K, dtype, "wsp_linear");
    if (rc || M == 0) return rc;
    hipError_t e = launch_gemm_bf16(x, w, y, r, M, N, K, nullptr, hipStream_t(stream));
    if (e != hipSuccess) return hip_fail(e, "linear kernel launch");
    return WSP_OK;
}

int wsp_linear_rope(const void *x, const void *w, void *y, int64_t M, int N, int K, int dtype,
                    const wsp_plan_t *rows, const wsp_plan_t *pos, int text_len, float theta,
                    void *stream) {
    g_last_error.clear();
    if (!rows || !pos) return fail(WSP_EINVAL, "plan is NULL");
    if (rows->T != pos->T || rows->H != pos->H || rows->W != pos->W)
        return fail(WSP_EINVAL, "plans of different grids");
    if (text_len < 0 || text_len > (1 << 20)) return fail(WSP_EINVAL, "text_len must be in 0..2^20");
    if (M != rows->n + int64_t(text_len))
        return fail(WSP_EINVAL, "M must be the plan's token count plus text_len (" +
                                    std::to_string(rows->n + int64_t(text_len)) + "), got " + std::to_string(M));
    int rc = linear_args(x, w, nullptr, y, M, N, K, dtype, "wsp_linear_rope");
    if (rc || M == 0) return rc;
    if (pos->max_ext[0] > 1024 || pos->max_ext[1] > 2048 || pos->max_ext[2] > 2048)
        return fail(WSP_ERANGE, "window extents beyond 1024 (t) / 2048 (h, w)");
    if (!(theta > 0.0f) || !std::isfinite(theta)) theta = 10000.0f;
    const int P = std::max({text_len + pos->max_ext[0], pos->max_ext[1], pos->max_ext[2], 1});
    int dev = 0;
    WSP_HIP(hipGetDevice(&dev));
    int32_t *cid = nullptr, *ptab = nullptr;
    const float2 *cs = nullptr;
    if ((rc = device_ids(*const_cast<wsp_plan_t *>(rows), dev, &cid))) return rc;
    if ((rc = device_positions(*const_cast<wsp_plan_t *>(pos), dev, &ptab))) return rc;
    if ((rc = rope_table(dev, theta, P, &cs))) return rc;
    const GemmRope rp{cid, ptab, cs, int(rows->n), text_len};
    hipError_t e = launch_gemm_bf16(x, w, y, nullptr, M, N, K, &rp, hipStream_t(stream));
    if (e != hipSuccess) return hip_fail(e, "linear kernel launch");
    return WSP_OK;
}

int wsp_device_info(int *n_xcds, int *xcd_round_robin) {
    g_last_error.clear();
    if (!n_xcds || !xcd_round_robin) return fail(WSP_EINVAL, "n_xcds and xcd_round_robin must be non-NULL");
    int dev = 0;
    WSP_HIP(hipGetDevice(&dev));
    bool rr = false;
    int rc = device_xcds(dev, n_xcds, &rr, true);
    if (rc) return rc;
    *xcd_round_robin = rr ? 1 : 0;
    return WSP_OK;
}

int wsp_set_attn_order(int order) {
    g_last_error.clear();
    if (order != WSP_ORDER_LPT_XCD && order != WSP_ORDER_LPT && order != WSP_ORDER_ID)
        return fail(WSP_EINVAL, "unknown attention order " + std::to_string(order));
    g_attn_order.store(order);
    return WSP_OK;
}

int wsp_set_attn_schedule(int schedule) {
    g_last_error.clear();
    if (schedule != WSP_SCHED_AUTO && schedule != WSP_SCHED_PER_ITEM && schedule != WSP_SCHED_PER_ITEM_128 &&
        schedule != WSP_SCHED_QUEUE && schedule != WSP_SCHED_QUEUE_128)
        return fail(WSP_EINVAL, "unknown attention schedule");
    g_attn_sched.store(schedule);
    return WSP_OK;
}

}  // extern "C"
