// Window-local 3D rotary position embedding, fused with the row move between
// layouts (one read and one write of each q / k row).
//
// "Window-Aligned Sequence Parallelism (SeedVR2)", section "Reference quirks
// reproduced on purpose": a video token turns by its offset (dt, dh, dw) from
// its own window's corner, the temporal component raised by text_len, so
// tokens of different windows share positions; the rotated width is three
// times head_dim / 3 (126 for a 128-wide head) and the remaining two channels
// are copied.  The rotated span is three contiguous axis blocks
// [t | h | w] of 42 channels, each rotated in adjacent pairs (2k, 2k+1), pair
// i of a block by position * theta^(-2i/42); text token i uses (i, i, i).
// The (cos, sin) of every (position, pair) comes from a host-built table
// (double precision, rounded to float32); rotation in float32, one rounding
// to the tensor's dtype.
//
// One wavefront per destination row, 16 bytes per lane per step (8 bf16 or
// 4 float32 channels = 4 or 2 pairs, never straddling a head), four steps'
// non-temporal loads issued before their stores as in the plain relayout.

#include "wsp_internal.h"

namespace wsp {

namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;      // 16-byte chunks per lane loaded before their stores
constexpr int kHeadDim = 128;
constexpr int kSpan = 126;      // 3 * (128 / 3)
constexpr int kAxisPairs = 21;  // 42 channels per axis block

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
__global__ __launch_bounds__(64 * kWaves) void rope_kernel(
    const u32x4 *__restrict__ x, u32x4 *__restrict__ y, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ cid, const int32_t *__restrict__ pos, const float2 *__restrict__ cs,
    int64_t n_rows, int chunks_per_row, int text_len) {
    const int64_t row = int64_t(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int lane = threadIdx.x & 63;
    const int64_t srow = perm ? int64_t(perm[row]) : row;
    int p[3];
    if (pos) {
        const uint32_t v = uint32_t(pos[cid ? int64_t(cid[row]) : row]);
        p[0] = text_len + int(v & 1023u);
        p[1] = int((v >> 10) & 2047u);
        p[2] = int(v >> 21);
    } else {
        p[0] = p[1] = p[2] = int(row);
    }
    constexpr int EL = BF16 ? 8 : 4;         // channels per 16-byte chunk
    constexpr int CPH = kHeadDim / EL;       // chunks per head
    static_assert(64 % CPH == 0, "a lane must see the same channels in every head");
    // The lane's chunks all start at channel d0 of their head, so its pairs
    // and their (cos, sin) are the same for every chunk of the row.
    const int d0 = (lane % CPH) * EL;
    float2 t[EL / 2];
#pragma unroll
    for (int e = 0; e < EL / 2; ++e) {
        const int k = d0 / 2 + e;
        t[e] = float2{1.f, 0.f};             // pass-through pairs (not applied)
        if (2 * k < kSpan) {
            const int axis = k / kAxisPairs;
            t[e] = cs[p[axis] * kAxisPairs + (k - axis * kAxisPairs)];
        }
    }
    const u32x4 *src = x + srow * chunks_per_row;
    u32x4 *dst = y + row * chunks_per_row;
    for (int base = 0; base < chunks_per_row; base += 64 * kUnroll) {
        u32x4 raw[kUnroll];
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int ch = base + lane + 64 * i;
            if (ch < chunks_per_row) raw[i] = __builtin_nontemporal_load(src + ch);
        }
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int ch = base + lane + 64 * i;
            if (ch >= chunks_per_row) continue;
            uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < EL / 2; ++e) {   // pair index k = d0/2 + e
                f32x2 v;
                if constexpr (BF16) {
                    v = __builtin_convertvector(__builtin_bit_cast(bf16x2, w[e]), f32x2);
                } else {
                    v = f32x2{__uint_as_float(w[2 * e]), __uint_as_float(w[2 * e + 1])};
                }
                if (2 * (d0 / 2 + e) < kSpan)
                    v = f32x2{fmaf(v.x, t[e].x, -v.y * t[e].y), fmaf(v.x, t[e].y, v.y * t[e].x)};
                if constexpr (BF16) {
                    o[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
                } else {
                    o[2 * e] = __float_as_uint(v.x);
                    o[2 * e + 1] = __float_as_uint(v.y);
                }
            }
            __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, dst + ch);
        }
    }
}

}  // namespace

hipError_t launch_rope(const void *x, void *y, const int32_t *perm, const int32_t *cid,
                       const int32_t *pos, const float2 *cs, int64_t n_rows, int n_heads, int dtype,
                       int text_len, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    const int64_t row_bytes = int64_t(n_heads) * kHeadDim * (dtype == WSP_BF16 ? 2 : 4);
    const int chunks = int(row_bytes / 16);
    const dim3 grid(unsigned((n_rows + kWaves - 1) / kWaves)), block(64 * kWaves);
    const u32x4 *xs = static_cast<const u32x4 *>(x);
    u32x4 *ys = static_cast<u32x4 *>(y);
    if (dtype == WSP_BF16)
        rope_kernel<true><<<grid, block, 0, s>>>(xs, ys, perm, cid, pos, cs, n_rows, chunks, text_len);
    else
        rope_kernel<false><<<grid, block, 0, s>>>(xs, ys, perm, cid, pos, cs, n_rows, chunks, text_len);
    return hipGetLastError();
}

}  // namespace wsp
