// Shared device helpers of the bf16 window-attention kernels (types, tile
// shape, LDS swizzle, MFMA wrapper, bf16 packing, joint-sequence row
// offsets).  Internal to libwsp.
#pragma once

#include "wsp_internal.h"

namespace wsp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kBN = 64;        // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format,
// no swizzle, no index stride).
constexpr int kBufferFlags = 0x00020000;

// Largest per-lane tile sum of probabilities accepted without moving the
// running maximum: every probability then stays below 2^20, far inside the
// range of float32 accumulation and of bf16 operands.
constexpr float kMaxTileSum = 1048576.0f;

template <int D, int kWaves = 4>
struct Shape {
    static constexpr int KSTEPS = D / 16;        // k-steps of S^T over the head dim
    static constexpr int DT = D / 32;            // 32-row blocks of O^T
    static constexpr int CH = D / 8;             // 16-byte chunks per row
    static constexpr int ROW = 2 * D;            // bytes per K/V row in LDS
    static constexpr int TILE = kBN * ROW;       // one K (or V) tile
    static constexpr int ROWS_PER_LOAD = 1024 / ROW;            // rows per wave DMA
    static constexpr int LOADS = kBN / ROWS_PER_LOAD / kWaves;  // DMAs per wave per tile
    static_assert(LOADS * ROWS_PER_LOAD * kWaves == kBN, "tile must split over the waves");
};

// XOR swizzle of the 16-byte chunk index within row r (see the file comment).
template <int D>
__device__ __host__ constexpr int swz(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum of a lane's value and the value of the lane 32 apart (the other
// half of the same query's keys), through ds_bpermute.
__device__ inline float halves_max(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ inline float halves_sum(float x) { return x + __shfl_xor(x, 32, 64); }

// Two floats to a packed bf16 pair (round to nearest even), one v_cvt_pk.
__device__ inline bf16x2 to_bf16x2(float lo, float hi) {
    return __builtin_convertvector(f32x2{lo, hi}, bf16x2);
}
__device__ inline uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, to_bf16x2(lo, hi));
}

}  // namespace
}  // namespace wsp
