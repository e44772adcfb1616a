// Layout permutation: y[j] = x[perm[j]] for whole rows.
//
// "Window-Aligned Sequence Parallelism (SeedVR2)", sections "Motivation" and
// "Plan A redistribution": a layout transition whose tokens all stay put is a
// local permutation of rows.  The kernel is a pure HBM copy: one wavefront per
// destination row, each lane moving 16-byte chunks, all loads of a lane
// issued before its stores so a row's bytes are in flight together.

#include "wsp_internal.h"

namespace wsp {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;       // rows per work group
constexpr int kUnroll = 4;      // 16-byte chunks per lane per pass (4 KB per wave)

__global__ __launch_bounds__(kWaves * 64) void relayout_kernel(
    const u32x4 *__restrict__ x, u32x4 *__restrict__ y, const int32_t *__restrict__ perm,
    int64_t n_rows, int64_t chunks_per_row) {
    const int64_t row = int64_t(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int lane = threadIdx.x & 63;
    const int64_t src = perm[row];
    const u32x4 *s = x + src * chunks_per_row;
    u32x4 *d = y + row * chunks_per_row;
    for (int64_t base = 0; base < chunks_per_row; base += 64 * kUnroll) {
        u32x4 r[kUnroll];
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int64_t c = base + lane + 64 * i;
            if (c < chunks_per_row) r[i] = __builtin_nontemporal_load(s + c);
        }
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int64_t c = base + lane + 64 * i;
            if (c < chunks_per_row) __builtin_nontemporal_store(r[i], d + c);
        }
    }
}

}  // namespace

hipError_t launch_relayout(const void *x, void *y, const int32_t *perm, int64_t n_rows,
                           int64_t row_bytes, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    const int64_t blocks = (n_rows + kWaves - 1) / kWaves;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    relayout_kernel<<<dim3(unsigned(blocks)), dim3(kWaves * 64), 0, s>>>(
        static_cast<const u32x4 *>(x), static_cast<u32x4 *>(y), perm, n_rows, row_bytes / 16);
    return hipGetLastError();
}

}  // namespace wsp
