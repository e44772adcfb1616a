// FP8 (OCP E4M3) quantisation of query / key rows for the low-precision
// attention variant: per-head absolute maximum, then codes of x * 448/amax.
//
// Format: 1 sign, 4 exponent (bias 7), 3 mantissa bits, largest finite 448
// (gfx950's v_cvt_pk_fp8_f32, round to nearest even).  The scale 448/amax is a
// correctly rounded float32 division and the product x*scale one float32
// multiply, so the codes are reproducible bit for bit on the host.

#include "wsp_internal.h"

namespace wsp {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAmaxThreads = 256;
constexpr int kAmaxSlots = 8;  // 16-byte chunks per thread and row: rows up to 32 KiB

// amax[h] = max(amax[h], |x[r, h, :]|) over all rows, as float bits (the bit
// patterns of non-negative floats order like unsigned integers).  Each thread
// keeps the running maximum of fixed chunk columns over a strided set of rows
// (four rows in flight); the lanes sharing a head then reduce by shuffles and
// one lane per head and wave issues the atomic.
template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const u32x4 *__restrict__ x,
                                                            unsigned int *__restrict__ amax,
                                                            int64_t n_rows, int chunks,
                                                            int chunks_per_head) {
    uint32_t m[kAmaxSlots];
#pragma unroll
    for (int s = 0; s < kAmaxSlots; ++s) m[s] = 0;
    auto absmax = [](uint32_t acc, const u32x4 &v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (BF16) {
                acc = max(acc, max((v[e] & 0x7FFFu) << 16, (v[e] >> 16 & 0x7FFFu) << 16));
            } else {
                acc = max(acc, v[e] & 0x7FFFFFFFu);
            }
        }
        return acc;
    };
    constexpr int kRowsInFlight = 4;
    const int64_t stride = int64_t(gridDim.x) * kRowsInFlight;
    for (int64_t r0 = int64_t(blockIdx.x) * kRowsInFlight; r0 < n_rows; r0 += stride) {
#pragma unroll
        for (int s = 0; s < kAmaxSlots; ++s) {
            const int c = threadIdx.x + s * kAmaxThreads;
            if (c < chunks) {
                u32x4 v[kRowsInFlight];
#pragma unroll
                for (int i = 0; i < kRowsInFlight; ++i)
                    v[i] = r0 + i < n_rows ? x[(r0 + i) * chunks + c] : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int i = 0; i < kRowsInFlight; ++i) m[s] = absmax(m[s], v[i]);
            }
        }
    }
    // Lanes c .. c+cph-1 (consecutive in the wave; cph is 8, 16 or 32) share a head.
#pragma unroll
    for (int s = 0; s < kAmaxSlots; ++s) {
        const int c = threadIdx.x + s * kAmaxThreads;
        uint32_t v = c < chunks ? m[s] : 0u;
        for (int d = 1; d < chunks_per_head; d <<= 1) v = max(v, uint32_t(__shfl_xor(int(v), d, 64)));
        if (c < chunks && c % chunks_per_head == 0) atomicMax(amax + c / chunks_per_head, v);
    }
}

constexpr int kQWaves = 4;

// y[r] = E4M3 codes of x[r] * (448 / amax[head]); one wavefront per row.
template <bool BF16>
__global__ __launch_bounds__(64 * kQWaves) void quantize_kernel(const u32x4 *__restrict__ x,
                                                               uint8_t *__restrict__ y,
                                                               const float *__restrict__ amax,
                                                               int64_t n_rows, int chunks,
                                                               int chunks_per_head) {
    const int64_t row = int64_t(blockIdx.x) * kQWaves + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int lane = threadIdx.x & 63;
    constexpr int EL = BF16 ? 8 : 4;  // elements per 16-byte input chunk
    const u32x4 *src = x + row * chunks;
    uint8_t *dst = y + row * int64_t(chunks) * EL;
    for (int c = lane; c < chunks; c += 64) {
        const float a = amax[c / chunks_per_head];
        const float scale = a > 0.0f ? __fdiv_rn(448.0f, a) : 1.0f;
        const u32x4 v = __builtin_nontemporal_load(src + c);
        float f[EL];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (BF16) {
                f[2 * e] = __uint_as_float(v[e] << 16);
                f[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
            } else {
                f[e] = __uint_as_float(v[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < EL; ++e) f[e] = fminf(fmaxf(__fmul_rn(f[e], scale), -448.0f), 448.0f);
        uint32_t w[EL / 4];
#pragma unroll
        for (int g = 0; g < EL / 4; ++g) {
            uint32_t t = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * g], f[4 * g + 1], 0, false);
            w[g] = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * g + 2], f[4 * g + 3], t, true);
        }
        if constexpr (BF16)
            *reinterpret_cast<uint2 *>(dst + int64_t(c) * EL) = uint2{w[0], w[1]};
        else
            *reinterpret_cast<uint32_t *>(dst + int64_t(c) * EL) = w[0];
    }
}

}  // namespace

int fp8_max_row_chunks() { return kAmaxThreads * kAmaxSlots; }

hipError_t launch_fp8_amax(const void *x, float *amax, int64_t n_rows, int n_heads, int head_dim,
                           int dtype, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    const int elem = dtype == WSP_BF16 ? 2 : 4;
    const int cph = head_dim * elem / 16, chunks = n_heads * cph;
    const unsigned grid = unsigned(std::min<int64_t>((n_rows + 3) / 4, 1024));
    const u32x4 *xs = static_cast<const u32x4 *>(x);
    unsigned int *bits = reinterpret_cast<unsigned int *>(amax);
    if (dtype == WSP_BF16)
        amax_kernel<true><<<grid, kAmaxThreads, 0, s>>>(xs, bits, n_rows, chunks, cph);
    else
        amax_kernel<false><<<grid, kAmaxThreads, 0, s>>>(xs, bits, n_rows, chunks, cph);
    return hipGetLastError();
}

hipError_t launch_fp8_quantize(const void *x, void *y, const float *amax, int64_t n_rows,
                               int n_heads, int head_dim, int dtype, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    const int elem = dtype == WSP_BF16 ? 2 : 4;
    const int cph = head_dim * elem / 16, chunks = n_heads * cph;
    const dim3 grid(unsigned((n_rows + kQWaves - 1) / kQWaves)), block(64 * kQWaves);
    const u32x4 *xs = static_cast<const u32x4 *>(x);
    uint8_t *ys = static_cast<uint8_t *>(y);
    if (dtype == WSP_BF16)
        quantize_kernel<true><<<grid, block, 0, s>>>(xs, ys, amax, n_rows, chunks, cph);
    else
        quantize_kernel<false><<<grid, block, 0, s>>>(xs, ys, amax, n_rows, chunks, cph);
    return hipGetLastError();
}

}  // namespace wsp
