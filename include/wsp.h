/*
 * wsp.h -- C ABI of the MI355X (gfx950) 3D-windowed joint-attention layer.
 *
 * The layer is the one described on the page "Window-Aligned Sequence
 * Parallelism (SeedVR2)": a post-patch (T, H, W) video token grid is cut into
 * regular or half-window-shifted, boundary-clipped 3D windows ("Window
 * layouts"); inside each window the video tokens attend jointly with the
 * replicated text tokens ("SeedVR2 integration"); the per-window text outputs
 * are averaged over the window count ("Text stream"); and activations are
 * permuted between layouts at layer boundaries ("Plan A redistribution",
 * local-permutation case).  The joint call shape -- image Q/K/V plus separate
 * text Q/K/V -- follows "Parallelize new models with USP (text replica)",
 * section "3. Attention with USP".
 *
 * Conventions for every entry point:
 *   - Return value: WSP_OK (0) or a negative wsp_status.  On error nothing is
 *     launched and wsp_last_error() returns a message (thread-local, valid
 *     until the calling thread's next wsp_* call).
 *   - Device pointers are owned by the caller; the library never frees or
 *     keeps them.  Plans are owned by the library until wsp_plan_free().
 *   - `stream` is a hipStream_t (NULL = the null stream).  Device work is
 *     enqueued on it and the call returns without waiting for it.  The only
 *     synchronous step is the first device use of a plan (or of a plan pair
 *     in wsp_relayout, or of a new head/text-length shape in
 *     wsp_window_attn) on a device: its index tables are then copied to that
 *     device once and cached with the plan; and the first attention call on
 *     a device probes how work groups reach its dies (wsp_device_info).
 *   - Tensors are dense row-major.  A "row" is one token: [n_heads, head_dim]
 *     elements for attention tensors, `row_bytes` bytes for wsp_relayout.
 *   - Calls on different streams that share a plan are safe; output buffers
 *     must not overlap inputs.
 */
#ifndef WSP_H
#define WSP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Window layout of one token grid (opaque). */
typedef struct wsp_plan_t wsp_plan_t;

enum wsp_method {
    WSP_REGULAR = 0,   /* slice(i*w, min((i+1)*w, n)) on every axis           */
    WSP_SHIFTED = 1,   /* every cut moved back by floor(w/2), clipped to [0,n) */
    WSP_CANONICAL = 2  /* identity layout: one window, ids = 0..N-1           */
};

enum wsp_dtype { WSP_F32 = 0, WSP_BF16 = 1 };

enum wsp_status {
    WSP_OK = 0,
    WSP_EINVAL = -1,      /* bad argument: geometry, method, dtype, pointer, size */
    WSP_ERANGE = -2,      /* a size does not fit the library's index types        */
    WSP_ENOMEM = -3,      /* host or device allocation failed                     */
    WSP_EWORKSPACE = -4,  /* workspace missing or smaller than required           */
    WSP_EDEVICE = -5      /* a HIP runtime call failed (message holds HIP's text) */
};

/* Order in which wsp_window_attn hands work to the GPU (tuning/measurement). */
enum wsp_order {
    WSP_ORDER_LPT_XCD = 0, /* largest window first, (window, head) groups spread
                              over the 8 XCDs so each group's tiles share one L2
                              (where wsp_device_info finds work groups placed
                              round-robin over 8 XCDs; else as WSP_ORDER_LPT)  */
    WSP_ORDER_LPT = 1,     /* largest window first, plain block order            */
    WSP_ORDER_ID = 2       /* window id order                                    */
};

/* Schedule of the bf16 attention kernel (wsp_set_attn_schedule).  Value 1
 * (a persistent schedule of earlier versions) is no longer accepted. */
enum wsp_schedule {
    WSP_SCHED_AUTO = 0,         /* by mean window length (wsp_set_attn_schedule) */
    WSP_SCHED_PER_ITEM = 2,     /* one work group per 256-query-row item         */
    WSP_SCHED_PER_ITEM_128 = 3, /* one work group per 128-query-row item         */
    WSP_SCHED_QUEUE = 4,        /* resident work groups, 256-row items in turn   */
    WSP_SCHED_QUEUE_128 = 5     /* resident work groups, 128-row items in turn   */
};

/*
 * wsp_plan -- build the window tables of one layout.
 *
 * "Window-Aligned Sequence Parallelism (SeedVR2)", section "Window layouts":
 *   scale = sqrt(45*80 / (H*W)) (IEEE double, the 720p reference area);
 *   wh = ceil(round(H*scale) / nh), ww = ceil(round(W*scale) / nw) with
 *   round() ties-to-even; wt = ceil(min(T, 30) / nt).  Regular cuts at
 *   multiples of the window; shifted cuts at k*w - floor(w/2), clipped to the
 *   axis (empty windows are not produced).  Window ids run over the w
 *   intervals in the outer loop, then h, then t in the inner loop; a window's
 *   tokens are listed with t slowest and w fastest; token (t, h, w) has the
 *   canonical id (t*H + h)*W + w.
 *   Section "Planner": the largest-first order sorts windows by
 *   (-video token count, window id).
 *
 * T, H, W     grid extents (> 0, T*H*W < 2^31)
 * nt, nh, nw  window counts of the size rule (> 0); ignored for WSP_CANONICAL
 * method      enum wsp_method
 * out         receives the new plan (set to NULL on error)
 * Errors: WSP_EINVAL (non-positive size, unknown method, a window size that
 * rounds to zero), WSP_ERANGE (T*H*W >= 2^31), WSP_ENOMEM.
 */
int wsp_plan(int T, int H, int W, int nt, int nh, int nw, int method, wsp_plan_t **out);

/*
 * wsp_plan_info -- sizes of a plan.  Any output pointer may be NULL.
 * n_tokens  T*H*W;  n_windows  window count;  win_size  {wt, wh, ww}
 * Errors: WSP_EINVAL (p is NULL).
 */
int wsp_plan_info(const wsp_plan_t *p, int64_t *n_tokens, int32_t *n_windows, int32_t *win_size);

/*
 * wsp_plan_tables -- copy the host tables of a plan into caller buffers.
 * Any pointer may be NULL (that table is skipped).
 * offsets  [n_windows + 1]  window w owns layout rows offsets[w]..offsets[w+1]-1
 * ids      [n_tokens]       canonical id held at each layout row
 * inv      [n_tokens]       layout row of each canonical id (ids[inv[c]] == c)
 * boxes    [6 * n_windows]  t0,t1,h0,h1,w0,w1 (half-open) per window
 * lpt      [n_windows]      window ids, largest first, ties by id
 * Errors: WSP_EINVAL (p is NULL).
 */
int wsp_plan_tables(const wsp_plan_t *p, int32_t *offsets, int32_t *ids, int32_t *inv,
                    int32_t *boxes, int32_t *lpt);

/* wsp_plan_free -- release a plan and its cached device tables (NULL is a no-op).
 * The caller must make sure no enqueued work still reads them. */
void wsp_plan_free(wsp_plan_t *p);

/*
 * wsp_relayout -- local permutation between two layouts of the same grid.
 *
 * "Window-Aligned Sequence Parallelism (SeedVR2)", sections "Motivation" and
 * "Plan A redistribution": a layout transition in which no token changes
 * owner is a local permutation.  y[j] = x[inv_src[ids_dst[j]]]: row j of
 * the output is the row of x that holds canonical token ids_dst[j].  Bytes
 * are moved unchanged (any dtype).
 *
 * x, y       device pointers, [n_tokens, row_bytes] each, 16-byte aligned,
 *            non-overlapping
 * row_bytes  bytes per token row, a positive multiple of 16
 * src, dst   plans of the same (T, H, W) grid (either may be WSP_CANONICAL)
 * Errors: WSP_EINVAL (NULL or misaligned pointer, bad row_bytes, grids
 * differ, x == y), WSP_ERANGE (n_tokens*row_bytes overflows), WSP_ENOMEM,
 * WSP_EDEVICE.
 */
int wsp_relayout(const void *x, void *y, int64_t row_bytes, const wsp_plan_t *src,
                 const wsp_plan_t *dst, void *stream);

/*
 * wsp_window_attn_workspace -- the smallest device workspace (bytes)
 * wsp_window_attn accepts: Q + G * text_len * n_heads * head_dim * 4 with
 * G = min(n_windows, 16), one float32 partial text sum per chunk of
 * consecutive windows (the windows split into G runs of ids, run c starting
 * at floor(c * n_windows / G)), and Q = 256 bytes for WSP_BF16 (the work
 * queue's ticket counters, cleared by each call), 0 for WSP_F32.  1080p-
 * shaped layer (20 x 128, 256 text tokens): 42 MB; 4K-shaped (512 text
 * tokens): 84 MB.  A workspace of Q + n_windows * text_len * n_heads *
 * head_dim * 4 bytes or more (262 MB at 1080p, 2.6 GB at 4K) selects one
 * partial per window: a
 * window's text rows are then queried beside its video rows -- in the same
 * query tiles where that saves a tile -- sharing that window's K/V in L2
 * (about 2% faster at 1080p).  The video output of the two modes may differ
 * in the last bits (a wave's 32 query rows share their rescaling steps).
 * Errors: WSP_EINVAL (bad plan/shape/dtype), WSP_ERANGE.
 */
int wsp_window_attn_workspace(const wsp_plan_t *p, int n_heads, int head_dim, int text_len,
                              int dtype, size_t *bytes);

/*
 * wsp_window_attn -- joint attention inside every window of p, and the
 * window-averaged text output.
 *
 * "Window-Aligned Sequence Parallelism (SeedVR2)", section "SeedVR2
 * integration": each window attends over the packed segment
 * [video window; replicated text]; section "Text stream": each window yields
 * one text output T_w and the text result is (sum over windows of T_w) /
 * window count.  "Parallelize new models with USP (text replica)", section
 * "3. Attention with USP": the attention is SDPA without mask or dropout,
 * with image and text Q/K/V passed as separate tensors.
 *
 * For window w (layout rows a = offsets[w] .. b = offsets[w+1]-1) and head h:
 *   Q = [q[a:b, h]; txt_q[:, h]],  K = [k[a:b, h]; txt_k[:, h]],
 *   V = [v[a:b, h]; txt_v[:, h]],  O = softmax(Q K^T * scale) V;
 *   out[a:b, h] = the first b-a rows of O; T_w = the last text_len rows.
 *   txt_out[:, h] = (sum_w T_w) / n_windows, summed in float32 in a fixed
 *   order -- window order inside each of G chunks of consecutive windows,
 *   then the chunk sums in chunk order -- and rounded once to dtype.  G is
 *   n_windows when workspace_bytes >= n_windows * text_len * n_heads *
 *   head_dim * 4, else min(n_windows, 16) (wsp_window_attn_workspace); for a
 *   given G the result is bit-identical from run to run and across dispatch
 *   orders.
 *
 * p                 plan; q/k/v/out rows are in its layout
 * q, k, v           device, [n_tokens, n_heads, head_dim] of dtype
 * txt_q/k/v         device, [text_len, n_heads, head_dim] of dtype (may be
 *                   NULL when text_len == 0)
 * n_heads           1 .. 32767;  head_dim  64 or 128;  text_len  >= 0
 * dtype             WSP_BF16 (MFMA path, float32 accumulation and softmax)
 *                   or WSP_F32 (float32 throughout)
 * scale             softmax scale; <= 0 selects 1/sqrt(head_dim)
 * out               device, [n_tokens, n_heads, head_dim] of dtype
 * txt_out           device, [text_len, n_heads, head_dim] of dtype (NULL
 *                   allowed when text_len == 0)
 * workspace         device, >= wsp_window_attn_workspace() bytes, 16-byte
 *                   aligned (may be NULL only for WSP_F32 with text_len ==
 *                   0); contents on entry are ignored; it holds the work
 *                   queue's counters and the chunk sums until the kernels
 *                   of the same call have read them (calls sharing a
 *                   workspace must be ordered on one stream)
 * Errors: WSP_EINVAL (pointer NULL or not 16-byte aligned, unsupported
 * head_dim/dtype, n_heads out of range), WSP_ERANGE (a window longer than
 * the kernel's tile index range), WSP_EWORKSPACE, WSP_ENOMEM, WSP_EDEVICE.
 */
int wsp_window_attn(const wsp_plan_t *p, const void *q, const void *k, const void *v,
                    const void *txt_q, const void *txt_k, const void *txt_v, int n_heads,
                    int head_dim, int text_len, int dtype, float scale, void *out,
                    void *txt_out, void *workspace, size_t workspace_bytes, void *stream);

/* Flags of wsp_window_attn_ex. */
enum wsp_attn_flags {
    WSP_ATTN_IO_LAYOUT = 0,    /* q, k, v and out rows are in p's layout (as wsp_window_attn) */
    WSP_ATTN_IO_CANONICAL = 1  /* q, k, v and out rows are in canonical token order */
};

/*
 * wsp_window_attn_ex -- wsp_window_attn with the layout permutation fused in.
 *
 * "Window-Aligned Sequence Parallelism (SeedVR2)", sections "Motivation" and
 * "Plan A redistribution": a layout transition in which no token changes
 * owner is a local permutation.  With WSP_ATTN_IO_CANONICAL the tensors q, k,
 * v and out hold rows in canonical token order (row c = canonical id c, the
 * layout WSP_CANONICAL); video row r of window w is read from (and its output
 * written to) canonical row ids[offsets[w] + r] of p, so no separate
 * wsp_relayout is needed before or after the call.  The result equals
 * wsp_relayout(p -> canonical) applied to wsp_window_attn on inputs relayouted
 * canonical -> p, bit for bit.  txt_* and txt_out are unchanged.
 *
 * Arguments, layouts, ownership and errors as wsp_window_attn, plus
 * flags  WSP_ATTN_IO_LAYOUT or WSP_ATTN_IO_CANONICAL (other bits: WSP_EINVAL).
 * bf16 with WSP_ATTN_IO_CANONICAL also returns WSP_ERANGE when a window's
 * canonical rows (smallest to largest id) span 2 GiB or more of q/k/v.
 * The first canonical call for a plan on a device uploads its ids table (and,
 * for bf16, the same ids relative to each window's smallest id).
 */
int wsp_window_attn_ex(const wsp_plan_t *p, const void *q, const void *k, const void *v,
                       const void *txt_q, const void *txt_k, const void *txt_v, int n_heads,
                       int head_dim, int text_len, int dtype, float scale, unsigned flags,
                       void *out, void *txt_out, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * wsp_window_attn_noalloc -- wsp_window_attn_ex for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same kernels and results, bit for bit;
 * it calls no hipMalloc, hipFree or allocating routine:
 *   - the work queue's counters (256 bytes, bf16) and the text mean's
 *     float32 partials go to a fixed scratch array of 96 MiB that the
 *     library holds on each GPU it runs on until the process ends.  One
 *     partial per window when those fit (n_windows * text_len * n_heads *
 *     head_dim * 4 bytes <= 96 MiB - 256, e.g. the 720p-shaped layer), else
 *     min(n_windows, 16) chunk partials (42 MB for the 1080p-shaped layer,
 *     84 MB for the 4K-shaped one); a larger need returns WSP_ERANGE;
 *   - the plan's device tables must already be on the device: a call of
 *     wsp_window_attn_ex with the same plan, n_heads, head_dim, text_len,
 *     dtype and flags, the same wsp_set_attn_order / _schedule setting and a
 *     workspace selecting the same text reduction uploads them; without one
 *     this call returns WSP_EINVAL and launches nothing.  The first call on
 *     a device also looks up the scratch array's device address once
 *     (hipGetSymbolAddress).
 * Every call on one GPU shares that GPU's scratch array: calls that overlap
 * in time on one GPU (different streams, or host threads) race and must be
 * ordered by the caller.  The kernels write every scratch element they read
 * within the call, so nothing needs clearing between calls.
 * Arguments as wsp_window_attn_ex without the workspace; errors as
 * wsp_window_attn_ex plus the two above.
 */
int wsp_window_attn_noalloc(const wsp_plan_t *p, const void *q, const void *k, const void *v,
                            const void *txt_q, const void *txt_k, const void *txt_v, int n_heads,
                            int head_dim, int text_len, int dtype, float scale, unsigned flags,
                            void *out, void *txt_out, void *stream);

/*
 * wsp_rope_relayout -- window-local 3D rotary position embedding, fused with
 * the row move between two layouts (for q and k; v takes wsp_relayout).
 *
 * "Window-Aligned Sequence Parallelism (SeedVR2)", section "Reference quirks
 * reproduced on purpose": a video token is rotated by its offset (dt, dh, dw)
 * from the corner of its own window, the temporal index raised by text_len
 * (tokens of different windows may share indices); the rotated width is
 * 3 * (head_dim / 3) channels (126 for head_dim 128) and the rest are
 * copied unchanged.  Where the page is silent this library
 * takes: three contiguous 42-channel axis blocks [t | h | w], each rotated in
 * adjacent pairs (2k, 2k+1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a),
 * pair i of a block turning by position * theta^(-2i/42).
 *
 * y[j] = rotate(x[row of src holding dst's token j], axial indices of that
 * token in layout `pos`).  With pos == dst this is the rotation a window
 * layer applies; with src == dst == pos's grid in canonical order it rotates
 * canonical-order q / k for the layout `pos` (for wsp_window_attn_ex with
 * canonical I/O).
 *
 * x, y       device pointers, [n_tokens, n_heads, head_dim] of dtype,
 *            16-byte aligned, non-overlapping
 * head_dim   128 (the only size whose axis blocks pair up); n_heads 1..32767
 * src, dst, pos  plans of the same grid; pos's window extents <= 1024 (t),
 *            2048 (h, w)
 * text_len   text tokens ahead of the video in the temporal index (>= 0)
 * theta      rotary base (<= 0 or non-finite: 10000)
 * The first call for a (theta, position count) pair on a device builds a
 * small (cos, sin) table (double precision, rounded to float32) that lives
 * until the process ends; the first call for a plan uploads its tables.
 * Errors: WSP_EINVAL (NULL / misaligned / aliasing pointers, grids differ,
 * head_dim, dtype, n_heads, text_len), WSP_ERANGE (window extents),
 * WSP_ENOMEM, WSP_EDEVICE.
 */
int wsp_rope_relayout(const void *x, void *y, int n_heads, int head_dim, int dtype,
                      const wsp_plan_t *src, const wsp_plan_t *dst, const wsp_plan_t *pos,
                      int text_len, float theta, void *stream);

/*
 * wsp_rope_text -- rotary embedding of the text rows: text token i uses the
 * axial indices (i, i, i) (plain 1-D rotary positions; the page places video
 * temporal indices after text_len, the text takes 0 .. text_len-1).
 * x, y [text_len, n_heads, head_dim]; arguments and errors as
 * wsp_rope_relayout.  text_len == 0 is a no-op.
 */
int wsp_rope_text(const void *x, void *y, int text_len, int n_heads, int head_dim, int dtype,
                  float theta, void *stream);

/*
 * wsp_window_attn_rope -- window attention of rotated queries and keys:
 * wsp_window_attn_ex's result for q, k rotated as wsp_rope_relayout (src =
 * dst = pos = p, or canonical order with pos = p) and txt_q, txt_k rotated
 * as wsp_rope_text would rotate them -- bit for bit.  The video queries turn
 * inside the attention kernel as each work item loads them; k is rotated
 * once by the stand-alone rotation kernel into the workspace (every query
 * tile of a window reads each key row, so rotating keys on the kernel's
 * loads would repeat the work per query tile), the text rows likewise.
 * q, k, txt_q and txt_k are left untouched.
 *
 * "Window-Aligned Sequence Parallelism (SeedVR2)", section "Reference quirks
 * reproduced on purpose" (window-local axial indices, temporal index raised
 * by text_len); section "SeedVR2 integration" (attention over [video window;
 * text]); the readings of wsp_rope_relayout (axis blocks, pair layout, theta).
 *
 * Arguments as wsp_window_attn_ex, plus theta (rotary base; <= 0 or
 * non-finite: 10000).  dtype must be WSP_BF16 and head_dim 128.
 * workspace  device, >= wsp_window_attn_rope_workspace() bytes, 16-byte
 *            aligned, never NULL: the rotated k (n_tokens * n_heads * 128 *
 *            2 bytes), text q and text k (text_len * n_heads * 128 * 2 bytes
 *            each), each part rounded up to 256, then the float32 text
 *            partials as in wsp_window_attn_ex (one per window when the rest
 *            holds text_len * n_heads * 128 * 4 bytes per window, else
 *            min(n_windows, 16) chunks).
 * Errors: as wsp_window_attn_ex; WSP_EINVAL for another dtype or head_dim;
 * WSP_ERANGE for window extents beyond 1024 (t) / 2048 (h, w).
 */
int wsp_window_attn_rope(const wsp_plan_t *p, const void *q, const void *k, const void *v,
                         const void *txt_q, const void *txt_k, const void *txt_v, int n_heads,
                         int head_dim, int text_len, int dtype, float scale, float theta, unsigned flags,
                         void *out, void *txt_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * wsp_window_attn_rope_workspace -- the smallest workspace (bytes) of
 * wsp_window_attn_rope: wsp_window_attn_workspace's plus the rotated k,
 * text q and text k.  Errors: as wsp_window_attn_workspace; WSP_EINVAL
 * unless dtype is WSP_BF16 and head_dim 128.
 */
int wsp_window_attn_rope_workspace(const wsp_plan_t *p, int n_heads, int head_dim, int text_len, int dtype,
                                   size_t *bytes);

/*
 * wsp_fp8_amax -- per-head largest |x| of a [n_rows, n_heads, head_dim]
 * tensor, max-accumulated into amax[n_heads] (float32, device memory; the
 * caller zeroes it before the first call, then may accumulate several
 * tensors -- e.g. the video and the text keys -- into one scale).
 *
 * Low-precision attention variant: the page "Scaling Video Training with
 * Parallelism" reports that low precision pays off in a neighbouring system;
 * the quantisation recipe here (per-head scale 448 / amax, OCP E4M3 codes) is
 * this library's own.
 * x  device, 16-byte aligned; dtype WSP_BF16 or WSP_F32; head_dim 64 or
 *    128; a row may hold at most 32 KiB.
 * Errors: WSP_EINVAL, WSP_EDEVICE.
 */
int wsp_fp8_amax(const void *x, int64_t n_rows, int n_heads, int head_dim, int dtype, float *amax,
                 void *stream);

/*
 * wsp_fp8_quantize -- y = OCP E4M3 codes (1 byte each) of x * (448 /
 * amax[head]): the scale a correctly rounded float32 division, the product
 * one float32 multiply, then round to nearest even, saturated at +-448
 * (amax 0 gives scale 1).  x and y [n_rows, n_heads, head_dim]; y holds one
 * byte per element.  Arguments and errors as wsp_fp8_amax.
 */
int wsp_fp8_quantize(const void *x, void *y, int64_t n_rows, int n_heads, int head_dim, int dtype,
                     const float *amax, void *stream);

/*
 * wsp_window_attn_qk8 -- wsp_window_attn_ex with E4M3 queries and keys.
 *
 * The scores come from the codes q8, k8, txt_q8, txt_k8 (wsp_fp8_quantize
 * with the per-head amax_q of q and txt_q, amax_k of k and txt_k) on the
 * gfx950 FP8 matrix cores and are dequantised by (amax_q/448)(amax_k/448);
 * softmax, probabilities, v and the outputs are as in the bf16 path (v,
 * txt_v, out, txt_out bfloat16).  Windows, text mean, flags
 * (WSP_ATTN_IO_CANONICAL), workspace (as for WSP_BF16), stream and errors as
 * wsp_window_attn_ex; head_dim must be 128.
 */
int wsp_window_attn_qk8(const wsp_plan_t *p, const void *q8, const void *k8, const void *v,
                        const void *txt_q8, const void *txt_k8, const void *txt_v,
                        const float *amax_q, const float *amax_k, int n_heads, int head_dim,
                        int text_len, float scale, unsigned flags, void *out, void *txt_out,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * wsp_device_info -- how work groups reach the current device's dies: the
 * number of XCDs (accelerated compute dies) a launch spreads over, and
 * whether work group b runs on XCD b mod that count.  Probed once per
 * device by a one-wave kernel reading each work group's XCC_ID register
 * (synchronous, like the first upload of a plan's tables; the first
 * attention call on a device runs the same probe).  The XCD-grouped work
 * list (WSP_ORDER_LPT_XCD) is used only where the count is 8 and the
 * placement round-robin; otherwise the attention calls fall back to
 * WSP_ORDER_LPT.
 * Errors: WSP_EINVAL (NULL pointers), WSP_ENOMEM, WSP_EDEVICE.
 */
int wsp_device_info(int *n_xcds, int *xcd_round_robin);

/*
 * wsp_set_attn_order -- process-wide dispatch order of wsp_window_attn
 * (enum wsp_order; default WSP_ORDER_LPT_XCD).  "Window-Aligned Sequence
 * Parallelism (SeedVR2)", section "Planner": ragged windows are balanced by
 * token count, largest first; here that order sequences GPU work groups.
 * Results do not depend on the order.  Errors: WSP_EINVAL.
 */
int wsp_set_attn_order(int order);

/*
 * wsp_set_attn_schedule -- process-wide schedule of the bf16 attention
 * kernel (enum wsp_schedule; default WSP_SCHED_AUTO).
 * WSP_SCHED_PER_ITEM: one work group (8 wavefronts) per 256-query-row item.
 * WSP_SCHED_PER_ITEM_128: one work group (4 wavefronts, two per compute
 * unit) per 128-query-row item: less of a window's last query tile is
 * empty.  WSP_SCHED_QUEUE / WSP_SCHED_QUEUE_128: the same items taken in
 * turn by resident work groups (as many as fit on the device), each from
 * the list of its XCD first (with WSP_ORDER_LPT_XCD) and then from the
 * others until all are empty; the ticket counters sit in the workspace.  An
 * item's start-up then overlaps the previous item's output stores and no
 * work group waits for a dispatch.  WSP_SCHED_AUTO: WSP_SCHED_QUEUE_128 when
 * a window's joint sequence averages fewer than 1024 rows, else
 * WSP_SCHED_QUEUE.  All four run the same per-wavefront arithmetic in the
 * same order, so results are bit-identical; the order set by
 * wsp_set_attn_order applies to all.  Errors: WSP_EINVAL.
 */
int wsp_set_attn_schedule(int schedule);

/*
 * wsp_linear -- y = x w^T (+ r): the bfloat16 projection of the 32-layer
 * stack workload (q / k / v projections of the hidden state and the output
 * projection added to the residual stream).  The pages define the attention
 * layer only; this entry point serves the synthetic multi-layer harness
 * built around it, with random weights.
 *
 * x: [M, K], w: [N, K] (one output feature per row), y and r: [M, N]; all
 * row-major bfloat16 device arrays owned by the caller; float32 accumulation
 * and one rounding to bfloat16 after adding r.  r may be NULL (no residual)
 * or equal to y (in-place residual update); y must not alias x or w.
 * dtype must be WSP_BF16.  Requirements: M >= 0 (M = 0 does nothing),
 * N a positive multiple of 256, K a positive multiple of 64, K < 2^20,
 * 16-byte aligned pointers.  Asynchronous on `stream`; errors: WSP_EINVAL,
 * WSP_ERANGE (M beyond 2^31 - 257 rows), WSP_EDEVICE (launch failure);
 * nothing is launched on error.
 */
int wsp_linear(const void *x, const void *w, const void *r, void *y, int64_t M, int N, int K,
               int dtype, void *stream);

/*
 * wsp_linear_rope -- the q or k projection of a window layer with the
 * window-local 3D rotary embedding applied as the products are stored:
 * y = rotate(bf16(x w^T)), bit for bit what wsp_linear (r = NULL) followed by
 * wsp_rope_relayout (src = dst = rows, pos) on the video rows and
 * wsp_rope_text on the text rows would leave, without that second pass over
 * y.
 *
 * "Window-Aligned Sequence Parallelism (SeedVR2)", section "Reference quirks
 * reproduced on purpose" (a video token turns by its offset from its own
 * window's corner, the temporal index raised by text_len; a 128-wide head
 * turns its first 126 channels and copies the last two); the readings of
 * wsp_rope_relayout (axis blocks, pair layout, theta, text positions
 * (i, i, i)).
 *
 * x [M, K], w [N, K], y [M, N]: row-major bfloat16 device arrays owned by the
 * caller, 16-byte aligned, y aliasing neither x nor w.  M = rows' token count
 * + text_len: rows 0 .. n-1 are the video tokens in the row order of plan
 * `rows` (a canonical plan for canonical order, or a layout), rows n ..
 * n+text_len-1 the text tokens 0 .. text_len-1.  Every 128 output features
 * form one head (N a positive multiple of 256), rotated alike; each video row
 * turns by its token's window-local position in layout `pos` (same grid as
 * `rows`; window extents <= 1024 (t), 2048 (h, w)).  K as wsp_linear.
 * theta: rotary base (<= 0 or non-finite: 10000).  dtype must be WSP_BF16.
 * The first call for a plan uploads its id / position tables and the first
 * call for a (theta, position count) pair its (cos, sin) table, kept until the
 * process ends (as wsp_rope_relayout).  Asynchronous on `stream`; errors:
 * WSP_EINVAL (arguments as wsp_linear, NULL plans, grids differ, M, text_len
 * outside 0..2^20), WSP_ERANGE (M, window extents), WSP_ENOMEM, WSP_EDEVICE;
 * nothing is launched on error.
 */
int wsp_linear_rope(const void *x, const void *w, void *y, int64_t M, int N, int K, int dtype,
                    const wsp_plan_t *rows, const wsp_plan_t *pos, int text_len, float theta,
                    void *stream);

/* wsp_last_error -- message of the calling thread's last failed call ("" if none). */
const char *wsp_last_error(void);

/* wsp_version -- ABI version of this header (major*10000 + minor*100 + patch). */
int wsp_version(void);

#define WSP_VERSION 20400

#ifdef __cplusplus
}
#endif

#endif /* WSP_H */
