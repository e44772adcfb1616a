// Float32 window joint attention (vector ALU, float32 throughout).
//
// "Window-Aligned Sequence Parallelism (SeedVR2)", section "SeedVR2
// integration": each window attends over the packed segment
// [video window; replicated text].  "Parallelize new models with USP (text
// replica)", section "3. Attention with USP": plain SDPA, no mask, no dropout.
//
// Work items as in attn_bf16.hip: a video item is (window, head, 64 query
// rows) -- of the window's video rows, or of its joint rows [video; text]
// (the text rows' outputs stored to the window's float32 partial) -- and
// writes `out`; a text item is (chunk of consecutive windows, head, 64 text
// query rows): its queries attend over each window of the chunk in turn and
// the normalised outputs T_w are summed in window order into the chunk's
// float32 partial of the workspace.  Four lanes share a
// query, each holding a quarter of the head dimension (element d = 16*e +
// 4*sub + 0..3 for lane `sub`), so a K/V row read from LDS is one 64-byte
// broadcast per quarter.  Keys stream through LDS in tiles of 32 rows with an
// online (running max) softmax.

#include "wsp_internal.h"

namespace wsp {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;       // queries per work group
constexpr int kBN = 32;       // keys per LDS tile
constexpr int kThreads = 256; // 4 lanes per query

// ids != NULL: q, k, v and out rows are in canonical token order and video
// row r of window w is canonical row ids[offsets[w] + r].
template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ tq, const float *__restrict__ tk, const float *__restrict__ tv,
    float *__restrict__ out, float *__restrict__ ws, const int32_t *__restrict__ ids,
    const ItemDesc *__restrict__ items, const WinDesc *__restrict__ wins, int H, int Lt, float scale) {
    constexpr int E = D / 16;  // float4 groups per lane
    __shared__ f32x4 Ks[kBN][D / 4];
    __shared__ f32x4 Vs[kBN][D / 4];

    const ItemDesc it = items[blockIdx.x];
    if (it.w < 0) return;
    const bool text = it.nwin > 0;
    const int h = it.hq >> 16, qt = it.hq & 0xFFFF;
    const int64_t rs = int64_t(H) * D;  // row stride (elements)
    const int tid = threadIdx.x, sub = tid & 3, qi = tid >> 2;
    const int qrow = qt * kBM + qi;
    // nv video rows of the window, then (text and joint items) text rows
    const bool joint = !text && it.chunk >= 0;
    const int nv = text ? 0 : it.win.lw;
    const int nq = nv + (text || joint ? Lt : 0);

    // Query row (zeros past the end of the item's query rows).
    f32x4 qv[E];
    const float *qp = nullptr;
    if (qrow < nq) {
        const int64_t r = qrow >= nv ? int64_t(qrow - nv)
                                     : (ids ? int64_t(ids[it.win.off + qrow]) : int64_t(it.win.off) + qrow);
        qp = (qrow >= nv ? tq : q) + r * rs + int64_t(h) * D;
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        qv[e] = qp ? *reinterpret_cast<const f32x4 *>(qp + 16 * e + 4 * sub) : f32x4{0, 0, 0, 0};

    const int n_loop = text ? it.nwin : 1;
    for (int wi = 0; wi < n_loop; ++wi) {
        const WinDesc wd = text ? wins[it.w + wi] : it.win;
        const int64_t off = wd.off;
        const int Lw = wd.lw;
        const int M = Lw + Lt;
        auto vrow = [&](int r) -> int64_t { return ids ? int64_t(ids[off + r]) : off + r; };
        f32x4 o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = f32x4{0, 0, 0, 0};
        float m_run = -INFINITY, l_run = 0.f;

        const int ntiles = (M + kBN - 1) / kBN;
        for (int j = 0; j < ntiles; ++j) {
            __syncthreads();
            // Stage K and V rows j*32 .. j*32+31 (video rows, then text rows).
            for (int c = tid; c < kBN * (D / 4); c += kThreads) {
                const int r = c / (D / 4), col = c % (D / 4);
                const int kr = j * kBN + r;
                f32x4 kk = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
                if (kr < Lw) {
                    const int64_t o_ = vrow(kr) * rs + int64_t(h) * D + 4 * col;
                    kk = *reinterpret_cast<const f32x4 *>(k + o_);
                    vv = *reinterpret_cast<const f32x4 *>(v + o_);
                } else if (kr < M) {
                    const int64_t o_ = int64_t(kr - Lw) * rs + int64_t(h) * D + 4 * col;
                    kk = *reinterpret_cast<const f32x4 *>(tk + o_);
                    vv = *reinterpret_cast<const f32x4 *>(tv + o_);
                }
                Ks[r][col] = kk;
                Vs[r][col] = vv;
            }
            __syncthreads();

            float s[kBN];
            float mx = -INFINITY;
#pragma unroll
            for (int kk = 0; kk < kBN; ++kk) {
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const f32x4 kv = Ks[kk][4 * e + sub];
                    acc = fmaf(qv[e].x, kv.x, acc);
                    acc = fmaf(qv[e].y, kv.y, acc);
                    acc = fmaf(qv[e].z, kv.z, acc);
                    acc = fmaf(qv[e].w, kv.w, acc);
                }
                acc += __shfl_xor(acc, 1);
                acc += __shfl_xor(acc, 2);
                s[kk] = (j * kBN + kk < M) ? acc * scale : -INFINITY;
                mx = fmaxf(mx, s[kk]);
            }
            const float m_new = fmaxf(m_run, mx);
            const float alpha = expf(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] *= alpha;
#pragma unroll
            for (int kk = 0; kk < kBN; ++kk) {
                const float p = expf(s[kk] - m_new);
                l_run += p;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const f32x4 vv = Vs[kk][4 * e + sub];
                    o[e].x = fmaf(p, vv.x, o[e].x);
                    o[e].y = fmaf(p, vv.y, o[e].y);
                    o[e].z = fmaf(p, vv.z, o[e].z);
                    o[e].w = fmaf(p, vv.w, o[e].w);
                }
            }
            m_run = m_new;
        }

        if (qrow >= nq) continue;
        const float inv = 1.0f / l_run;
        if (qrow >= nv) {
            // the partial `chunk`: a text item writes it on its chunk's first
            // window and adds the later ones in window order (same thread,
            // same addresses); a joint item is its window's only writer
            float *dst = ws + ((int64_t(it.chunk) * Lt + (qrow - nv)) * H + h) * D;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                f32x4 *p = reinterpret_cast<f32x4 *>(dst + 16 * e + 4 * sub);
                const f32x4 val = o[e] * inv;
                *p = wi > 0 ? *p + val : val;
            }
        } else {
            float *dst = out + vrow(qrow) * rs + int64_t(h) * D;
#pragma unroll
            for (int e = 0; e < E; ++e) *reinterpret_cast<f32x4 *>(dst + 16 * e + 4 * sub) = o[e] * inv;
        }
    }
}

}  // namespace

int attn_f32_tile_m(int) { return kBM; }

hipError_t launch_attn_f32(int head_dim, const float *q, const float *k, const float *v,
                           const float *tq, const float *tk, const float *tv, float *out,
                           float *ws, const int32_t *ids, const ItemDesc *items, const WinDesc *wins,
                           int n_items, int n_heads, int text_len, float scale, hipStream_t s) {
    if (n_items <= 0) return hipSuccess;
    if (head_dim == 128)
        attn_f32_kernel<128><<<dim3(n_items), dim3(kThreads), 0, s>>>(
            q, k, v, tq, tk, tv, out, ws, ids, items, wins, n_heads, text_len, scale);
    else if (head_dim == 64)
        attn_f32_kernel<64><<<dim3(n_items), dim3(kThreads), 0, s>>>(
            q, k, v, tq, tk, tv, out, ws, ids, items, wins, n_heads, text_len, scale);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace wsp
