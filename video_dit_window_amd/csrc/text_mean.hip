// Window-averaged text output.
//
// "Window-Aligned Sequence Parallelism (SeedVR2)", section "Text stream":
// every window yields one text output T_w and the next text state is the sum
// over windows divided by the window count (not a token-weighted mean).  The
// attention kernels leave one float32 partial per chunk of consecutive
// windows, [n_parts][Lt*H*D] (each the sum of its windows' T_w in id order);
// each thread adds four consecutive elements of the partials in chunk order
// (a fixed order: bit-identical results run to run, whatever order the work
// groups ran in), divides once by the window count and rounds once.

#include "wsp_internal.h"

namespace wsp {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint16_t to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__global__ __launch_bounds__(256) void text_mean_kernel(const float *__restrict__ ws,
                                                        void *__restrict__ out,
                                                        int64_t per_part, int n_parts, int n_windows,
                                                        int out_bf16) {
    const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (i >= per_part) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const float *p = ws + i;
#pragma unroll 4
    for (int c = 0; c < n_parts; ++c) acc += *reinterpret_cast<const f32x4 *>(p + int64_t(c) * per_part);
    const float n = float(n_windows);
    acc = acc / n;
    if (out_bf16) {
        uint16_t *o = static_cast<uint16_t *>(out) + i;
        const uint32_t lo = uint32_t(to_bf16_bits(acc.x)) | (uint32_t(to_bf16_bits(acc.y)) << 16);
        const uint32_t hi = uint32_t(to_bf16_bits(acc.z)) | (uint32_t(to_bf16_bits(acc.w)) << 16);
        *reinterpret_cast<uint2 *>(o) = make_uint2(lo, hi);
    } else {
        *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + i) = acc;
    }
}

}  // namespace

hipError_t launch_text_mean(const float *ws, void *txt_out, int64_t per_part, int n_parts,
                            int n_windows, int dtype, hipStream_t s) {
    if (per_part <= 0) return hipSuccess;
    const int64_t blocks = (per_part / 4 + 255) / 256;
    text_mean_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(ws, txt_out, per_part, n_parts,
                                                                   n_windows, dtype == WSP_BF16);
    return hipGetLastError();
}

}  // namespace wsp
