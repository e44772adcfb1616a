// bfloat16 window joint attention on gfx950 matrix cores (MFMA).
//
// "Window-Aligned Sequence Parallelism (SeedVR2)", section "SeedVR2
// integration": each window attends over the packed segment
// [video window; replicated text]; section "Text stream": each window yields
// one text output, averaged over windows afterwards.  "Parallelize new
// models with USP (text replica)", section "3. Attention with USP": plain
// SDPA (no mask, no dropout, scale 1/sqrt(D) unless given).
//
// Work item = (window w, head h, query tile of BM rows) of the joint query
// sequence [q rows of w; txt_q]; the key/value sequence is [k/v rows of w;
// txt_k/v].  A work group has 4 wavefronts; each owns QB blocks of 32 query
// rows.  Per 64-key tile:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, K from LDS (A), Q in VGPRs (B);
//                 the transposed product leaves each lane with ONE query
//                 (column) and 16 keys per 32x32 block, so the softmax row
//                 statistics need only in-lane reductions plus one swap
//                 between the two 32-lane halves.
//   online softmax in float32 (exp2 with the scale folded into one FMA);
//   O^T += V^T P^T  the probabilities stay in VGPRs as the B operand
//                 (bf16); V^T comes from LDS, where V is stored as blocks of
//                 4 keys x 1 dim (8 bytes) so one lane reads 4 keys of one
//                 head dimension with a single 8-byte LDS load.
// K/V tiles are double-buffered in LDS; the next tile's global loads are in
// flight while the current tile is multiplied.  Video query rows write bf16
// `out`; text query rows write their normalised float32 output to the
// workspace (reduced over windows in id order by the text-mean kernel).

#include <cstdlib>

#include "wsp_internal.h"

namespace wsp {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 wavefronts
constexpr float kLog2e = 1.4426950408889634f;

template <int D, int QB>
struct Shape {
    static constexpr int BM = 4 * 32 * QB;            // query rows per work group
    static constexpr int KSTEPS = D / 16;             // k-steps of S^T over the head dim
    static constexpr int DT = D / 32;                 // 32-row blocks of O^T
    static constexpr int CH = D / 8;                  // 16-byte chunks per row
    static constexpr int K_ROW = 2 * D + 16;          // LDS bytes per K row (padded)
    static constexpr int K_BYTES = kBN * K_ROW;
    static constexpr int VB_BYTES = 8 * D;            // one block of 4 keys x D dims
    static constexpr int V_BYTES = (kBN / 4) * VB_BYTES;
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int K_LOADS = kBN * CH / kThreads;
    static constexpr int V_PAIRS = (kBN / 4) * CH;    // (key block, chunk) pairs
    static_assert(kBN * CH % kThreads == 0, "K tile must split evenly over threads");
    static_assert(V_PAIRS <= kThreads, "V tile must fit one pass");
};

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum of a lane's value and the value of the lane 32 apart (the other
// half of the same query's keys).  A cross-half exchange through the LDS
// crossbar (ds_bpermute); one call per tile.
__device__ inline float halves_max(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ inline float halves_sum(float x) { return x + __shfl_xor(x, 32, 64); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to a packed bf16 pair (round to nearest even), one v_cvt_pk.
__device__ inline bf16x2 to_bf16x2(float lo, float hi) {
    return __builtin_convertvector(f32x2{lo, hi}, bf16x2);
}
__device__ inline uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, to_bf16x2(lo, hi));
}

// Row r of the joint sequence [video rows of the window; text rows], with r
// clamped to the last row M-1: rows past the end read real data, which the
// score mask (keys) or the store guard (queries) then discards.  Branch-free:
// two selects.
__device__ inline const uint16_t *joint_row(const uint16_t *vid, const uint16_t *txt, int r,
                                            int Lw, int M, int64_t off, int64_t rs, int64_t hd) {
    r = min(r, M - 1);
    const bool is_vid = r < Lw;
    const int64_t row = is_vid ? off + r : int64_t(r - Lw);
    return (is_vid ? vid : txt) + row * rs + hd;
}

// Rescale threshold of the running softmax maximum, in log2 units: the
// accumulators are rescaled only when a tile's maximum exceeds the running
// maximum by more than this, so probabilities stay below 2^8.
constexpr float kRescaleLog2 = 8.0f;

template <int D, int QB>
__global__ __launch_bounds__(kThreads, 3 - QB) void attn_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ tq,
    const uint16_t *__restrict__ tk, const uint16_t *__restrict__ tv,
    uint16_t *__restrict__ out, float *__restrict__ ws, const int32_t *__restrict__ offsets,
    const Item *__restrict__ items, int H, int Lt, float c2) {
    using S_ = Shape<D, QB>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * S_::STAGE];

    const Item it = items[blockIdx.x];
    if (it.x < 0) return;
    const int w = it.x, h = it.y >> 16, qt = it.y & 0xFFFF;
    const int64_t off = offsets[w];
    const int Lw = offsets[w + 1] - int(off);
    const int M = Lw + Lt;
    const int64_t rs = int64_t(H) * D, hd = int64_t(h) * D;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;

    // Query rows of this lane (B operand of S^T = K Q^T): 8 dims per k-step.
    bf16x8 Qr[QB][S_::KSTEPS];
    int qrow[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        qrow[b] = qt * S_::BM + (wave * QB + b) * 32 + l32;
        const uint16_t *p = joint_row(q, tq, qrow[b], Lw, M, off, rs, hd);
#pragma unroll
        for (int s = 0; s < S_::KSTEPS; ++s)
            Qr[b][s] = *reinterpret_cast<const bf16x8 *>(p + 16 * s + 8 * hh);
    }

    // Global -> register staging of one K/V tile.  Each thread loads fixed
    // rows of every tile: K rows rk + 256/CH*i (16-byte column kcol), V rows
    // 4*vkb + r (column vdc).  Tiles made only of video rows advance
    // per-thread row pointers by a whole tile; tiles that reach the text rows
    // or the padded end pick each row through joint_row().
    u32x4 kreg[S_::K_LOADS], vreg[4];
    const int kcol = tid % S_::CH, krow = tid / S_::CH;
    const int vdc = tid % S_::CH, vkb = tid / S_::CH;  // V: 16-byte chunk, block of 4 keys
    const bool v_loader = tid < S_::V_PAIRS;
    const int64_t tile_step = int64_t(kBN) * rs;
    const uint16_t *kp0 = k + (off + krow) * rs + hd + 8 * kcol;
    const uint16_t *vp0 = v + (off + 4 * vkb) * rs + hd + 8 * vdc;
    constexpr int KSTRIDE = kThreads / S_::CH;  // rows between a thread's K loads
    auto gload = [&](int j) {
        if ((j + 1) * kBN <= Lw) {
            const int64_t o = int64_t(j) * tile_step;
#pragma unroll
            for (int i = 0; i < S_::K_LOADS; ++i)
                kreg[i] = *reinterpret_cast<const u32x4 *>(kp0 + o + int64_t(KSTRIDE * i) * rs);
            if (v_loader) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vreg[r] = *reinterpret_cast<const u32x4 *>(vp0 + o + int64_t(r) * rs);
            }
        } else {
#pragma unroll
            for (int i = 0; i < S_::K_LOADS; ++i) {
                const uint16_t *p = joint_row(k, tk, j * kBN + krow + KSTRIDE * i, Lw, M, off, rs, hd);
                kreg[i] = *reinterpret_cast<const u32x4 *>(p + 8 * kcol);
            }
            if (v_loader) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint16_t *p = joint_row(v, tv, j * kBN + 4 * vkb + r, Lw, M, off, rs, hd);
                    vreg[r] = *reinterpret_cast<const u32x4 *>(p + 8 * vdc);
                }
            }
        }
    };
    // Register -> LDS.  K rows are stored padded; V is transposed into
    // 16-byte groups [dim 2x: keys 0..3][dim 2x+1: keys 0..3] of one key
    // block, the group index XOR-swizzled so a quarter-wave of writes and a
    // half-wave of 8-byte reads each touch distinct banks.
    auto lstore = [&](int buf) {
        uint8_t *Kb = smem + buf * S_::STAGE;
        uint8_t *Vb = Kb + S_::K_BYTES;
#pragma unroll
        for (int i = 0; i < S_::K_LOADS; ++i)
            *reinterpret_cast<u32x4 *>(Kb + (krow + KSTRIDE * i) * S_::K_ROW + kcol * 16) = kreg[i];
        if (v_loader) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t a0 = vreg[0][x], a1 = vreg[1][x], a2 = vreg[2][x], a3 = vreg[3][x];
                u32x4 g;
                g[0] = (a0 & 0xFFFFu) | (a1 << 16);
                g[1] = (a2 & 0xFFFFu) | (a3 << 16);
                g[2] = (a0 >> 16) | (a1 & 0xFFFF0000u);
                g[3] = (a2 >> 16) | (a3 & 0xFFFF0000u);
                const int G = 4 * vdc + x, P = G ^ ((G >> 4) & 3);
                *reinterpret_cast<u32x4 *>(Vb + vkb * S_::VB_BYTES + P * 16) = g;
            }
        }
    };

    f32x16 O[QB][S_::DT];
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        m_run[b] = -INFINITY;
        l_run[b] = 0.f;
#pragma unroll
        for (int t = 0; t < S_::DT; ++t) O[b][t] = f32x16{};
    }

    // LDS byte offset of this lane's V^T operand inside a key block.
    int voff[S_::DT];
#pragma unroll
    for (int t = 0; t < S_::DT; ++t) {
        const int d = 32 * t + l32, G = d >> 1, P = G ^ ((G >> 4) & 3);
        voff[t] = P * 16 + (d & 1) * 8;
    }

    const int ntiles = (M + kBN - 1) / kBN;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int j = 0; j < ntiles; ++j) {
        const int buf = j & 1;
        if (j + 1 < ntiles) gload(j + 1);
        const uint8_t *Kb = smem + buf * S_::STAGE;
        const uint8_t *Vb = Kb + S_::K_BYTES;

        // S^T for 64 keys (two 32-key blocks) x 32 queries per block b.
        f32x16 S[QB][2];
#pragma unroll
        for (int b = 0; b < QB; ++b) S[b][0] = S[b][1] = f32x16{};
#pragma unroll
        for (int s = 0; s < S_::KSTEPS; ++s) {
#pragma unroll
            for (int mk = 0; mk < 2; ++mk) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                    Kb + (32 * mk + l32) * S_::K_ROW + (16 * s + 8 * hh) * 2);
#pragma unroll
                for (int b = 0; b < QB; ++b) S[b][mk] = mfma(a, Qr[b][s], S[b][mk]);
            }
        }
        // Keys past the end of the joint sequence (last tile only).
        if ((j + 1) * kBN > M) {
#pragma unroll
            for (int mk = 0; mk < 2; ++mk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j * kBN + 32 * mk + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key >= M) {
#pragma unroll
                        for (int b = 0; b < QB; ++b) S[b][mk][r] = -INFINITY;
                    }
                }
        }
        // Online softmax.  The running maximum m_run moves (and O, l are
        // rescaled) only when some lane of the wave sees a tile maximum more
        // than 2^kRescaleLog2 above it -- a wave-uniform branch taken on the
        // first tile and rarely after.  P^T leaves as bf16 B operands, one
        // per 16-key k-step.
        float mx[QB];
        bool grow = false;
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            float m = S[b][0][0];
#pragma unroll
            for (int mk = 0; mk < 2; ++mk)
#pragma unroll
                for (int r = 0; r < 16; ++r) m = fmaxf(m, S[b][mk][r]);
            mx[b] = halves_max(m);
            grow |= (mx[b] - m_run[b]) * c2 > kRescaleLog2;
        }
        if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                const float m_new = fmaxf(m_run[b], mx[b]);
                const float alpha = __builtin_amdgcn_exp2f((m_run[b] - m_new) * c2);
                m_run[b] = m_new;
                l_run[b] *= alpha;
#pragma unroll
                for (int t = 0; t < S_::DT; ++t) O[b][t] *= alpha;
            }
        }
        // p = 2^(s*c2 - m*c2), packed to bf16 pairs; the row sum adds the
        // same rounded values the PV product uses (one dot2 per pair).
        bf16x8 P[QB][4];
        const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            const float mc = m_run[b] * c2;
            float sum = l_run[b];
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
                const int mk = cs >> 1, r0 = 8 * (cs & 1);
                u32x4 pk;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(S[b][mk][r0 + 2 * i], c2, -mc));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(S[b][mk][r0 + 2 * i + 1], c2, -mc));
                    const bf16x2 pp = to_bf16x2(p0, p1);
                    sum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, sum, false);
                    pk[i] = __builtin_bit_cast(uint32_t, pp);
                }
                P[b][cs] = __builtin_bit_cast(bf16x8, pk);
            }
            l_run[b] = sum;
        }
        // O^T += V^T P^T over the tile's four 16-key k-steps.
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) {
            const uint8_t *v0 = Vb + (4 * cs + hh) * S_::VB_BYTES;      // keys 16cs+4hh+0..3
            const uint8_t *v1 = Vb + (4 * cs + 2 + hh) * S_::VB_BYTES;  // keys 16cs+8+4hh+0..3
#pragma unroll
            for (int t = 0; t < S_::DT; ++t) {
                const u32x2 lo = *reinterpret_cast<const u32x2 *>(v0 + voff[t]);
                const u32x2 hi = *reinterpret_cast<const u32x2 *>(v1 + voff[t]);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
                for (int b = 0; b < QB; ++b) O[b][t] = mfma(a, P[b][cs], O[b][t]);
            }
        }
        if (j + 1 < ntiles) lstore(buf ^ 1);
        __syncthreads();
    }

    // Normalise and store: lane holds query qrow[b], dims 32t + 8g + 4hh + 0..3.
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const float l = halves_sum(l_run[b]);
        if (qrow[b] >= M) continue;
        const float inv = 1.0f / l;
        if (qrow[b] < Lw) {
            uint16_t *dst = out + (off + qrow[b]) * rs + hd;
#pragma unroll
            for (int t = 0; t < S_::DT; ++t)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x16 &o = O[b][t];
                    u32x2 st;
                    st[0] = pack_bf16(o[4 * g] * inv, o[4 * g + 1] * inv);
                    st[1] = pack_bf16(o[4 * g + 2] * inv, o[4 * g + 3] * inv);
                    *reinterpret_cast<u32x2 *>(dst + 32 * t + 8 * g + 4 * hh) = st;
                }
        } else {
            float *dst = ws + ((int64_t(w) * Lt + (qrow[b] - Lw)) * H + h) * D;
#pragma unroll
            for (int t = 0; t < S_::DT; ++t)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x16 &o = O[b][t];
                    *reinterpret_cast<f32x4 *>(dst + 32 * t + 8 * g + 4 * hh) =
                        f32x4{o[4 * g] * inv, o[4 * g + 1] * inv, o[4 * g + 2] * inv, o[4 * g + 3] * inv};
                }
        }
    }
}

// Query blocks of 32 rows per wavefront (1 or 2).  One block keeps a wave
// within 256 registers, so two waves share each SIMD (the default); two
// blocks halve the LDS reads per MFMA but run one wave per SIMD.  The
// WSP_ATTN_QB environment variable selects 2 for measurements.
int query_blocks() {
    static const int qb = [] {
        const char *e = std::getenv("WSP_ATTN_QB");
        return (e && std::atoi(e) == 2) ? 2 : 1;
    }();
    return qb;
}

template <int D, int QB>
void launch(const void *q, const void *k, const void *v, const void *tq, const void *tk,
            const void *tv, void *out, float *ws, const int32_t *offsets, const Item *items,
            int n_items, int n_heads, int text_len, float c2, hipStream_t s) {
    auto U = [](const void *p) { return static_cast<const uint16_t *>(p); };
    attn_bf16_kernel<D, QB><<<dim3(n_items), dim3(kThreads), 0, s>>>(
        U(q), U(k), U(v), U(tq), U(tk), U(tv), static_cast<uint16_t *>(out), ws, offsets, items,
        n_heads, text_len, c2);
}

}  // namespace

int attn_bf16_tile_m(int) { return 4 * 32 * query_blocks(); }

hipError_t launch_attn_bf16(int head_dim, const void *q, const void *k, const void *v,
                            const void *tq, const void *tk, const void *tv, void *out,
                            float *ws, const int32_t *offsets, const Item *items, int n_items,
                            int n_heads, int text_len, float scale, hipStream_t s) {
    if (n_items <= 0) return hipSuccess;
    const float c2 = scale * kLog2e;
    const int qb = query_blocks();
    if (head_dim == 128 && qb == 2)
        launch<128, 2>(q, k, v, tq, tk, tv, out, ws, offsets, items, n_items, n_heads, text_len, c2, s);
    else if (head_dim == 128)
        launch<128, 1>(q, k, v, tq, tk, tv, out, ws, offsets, items, n_items, n_heads, text_len, c2, s);
    else if (head_dim == 64 && qb == 2)
        launch<64, 2>(q, k, v, tq, tk, tv, out, ws, offsets, items, n_items, n_heads, text_len, c2, s);
    else if (head_dim == 64)
        launch<64, 1>(q, k, v, tq, tk, tv, out, ws, offsets, items, n_items, n_heads, text_len, c2, s);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace wsp
