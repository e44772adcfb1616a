// bfloat16 linear layer on gfx950 matrix cores: y = x w^T (+ r).
//
// The projections around the windowed attention of a transformer layer: the
// q / k / v projections of the hidden state and the output projection added
// to the residual stream.  The pages describe the attention layer only; the
// 32-layer stack that uses these projections is a synthetic harness with
// random weights, so this kernel is plumbing for it, not part of the method.
//
// x: [M, K] row-major, w: [N, K] row-major (one output feature per row, the
// nn.Linear layout), y and r: [M, N] row-major, all bfloat16; float32
// accumulation, one rounding at the end (after adding r).
//
// A work group computes a 256 x 256 tile of y with 8 wavefronts (4 along M x
// 2 along N, 64 x 128 each, 2 per SIMD).  The product is formed transposed,
// y^T = w x^T, on v_mfma_f32_32x32x16_bf16 with w rows as the A operand and x
// rows as B, so that each lane ends up holding four consecutive output
// features of one row per 32 x 32 block (8-byte stores).  K advances in
// 64-element slabs: both 256-row slabs move global -> LDS by direct
// buffer-load DMA (16 bytes per lane, rows of 128 bytes, the 16-byte chunks
// XOR-swizzled by (row / 2) % 8 so that the 32-row operand reads spread over
// the banks), double-buffered against the products of the previous slab.
// Tiles are mapped so that the 256-row slabs of x go round-robin to the 8
// XCDs (work group b runs on XCD b % 8); on an XCD, groups of slabs that
// fill its 32 CUs once run w tile by w tile, so that work groups running
// side by side share their x slabs and w tiles through the XCD's L2.
//
// ROPE: the q / k projections of a window layer, with the window-local 3D
// rotary embedding applied where the products are stored ("Window-Aligned
// Sequence Parallelism (SeedVR2)", section "Reference quirks reproduced on
// purpose": a video token turns by its offset from its own window's corner,
// the temporal index raised by the text length; a 128-wide head turns its
// first 126 channels, in three 42-channel axis blocks of adjacent pairs, and
// copies the last two; text token i uses (i, i, i)).
// Every 128 output features form one head.  The epilogue holds four
// consecutive features of a row per lane, i.e. two whole pairs, so each pair
// turns in registers: the product is rounded to bfloat16 first and the
// rotation runs in float32 from that value, then rounds again -- the same
// steps as the stand-alone rotation kernel applied to the stored projection,
// so the result is bit-identical to that two-pass chain without its extra
// read and write of q and k.

#include "wsp_internal.h"

namespace wsp {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kGBM = 256, kGBN = 256, kGBK = 64;
constexpr int kGWaves = 8;
constexpr int kGRow = kGBK * 2;              // bytes per slab row in LDS
constexpr int kGTile = kGBM * kGRow;         // one 256-row slab: 32 KB
constexpr int kGLoads = kGBM / 8 / kGWaves;  // DMA instructions per wave per slab (8 rows each)
constexpr int kBufferFlags = 0x00020000;     // raw buffer resource word 3 on gfx9-family parts
constexpr int kCusPerXcd = 32;               // MI355X: 256 CUs in 8 XCDs

__device__ __host__ constexpr int gswz(int r) { return (r >> 1) & 7; }

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int kRopeSpanPairs = 63;  // pairs 0..62 turn, pair 63 (channels 126, 127) passes
constexpr int kRopeAxisPairs = 21;  // 42 channels per axis block

// Pair k (two bf16 channels packed in w) of a head rotated by the row's
// (cos, sin) entry cs[pb[axis of k] + k]: float32 arithmetic, one rounding;
// pair 63 passes through.
__device__ inline uint32_t rope_pair(uint32_t w, int k, const int (&pb)[3], const float2 *__restrict__ cs) {
    if (k >= kRopeSpanPairs) return w;
    const int ax = k >= 2 * kRopeAxisPairs ? 2 : (k >= kRopeAxisPairs ? 1 : 0);
    const float2 t = cs[pb[ax] + k];
    const f32x2 f = __builtin_convertvector(__builtin_bit_cast(bf16x2, w), f32x2);
    const f32x2 o = {fmaf(f.x, t.x, -f.y * t.y), fmaf(f.x, t.y, f.y * t.x)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(o, bf16x2));
}

template <bool RES, bool ROPE>
__global__ __launch_bounds__(64 * kGWaves, 2) void gemm_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, uint16_t *y,
    const uint16_t *r, int M, int N, int K, int m_tiles, int n_tiles, int group, GemmRope rp) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer resources exist only in the device pass
    __shared__ __attribute__((aligned(1024))) uint8_t sx0[kGTile];
    __shared__ __attribute__((aligned(1024))) uint8_t sw0[kGTile];
    __shared__ __attribute__((aligned(1024))) uint8_t sx1[kGTile];
    __shared__ __attribute__((aligned(1024))) uint8_t sw1[kGTile];

    // Tile of this work group: x slab m_t goes to XCD m_t % 8.  On that XCD
    // the slots run through groups of `group` x slabs (the last group: the
    // slabs left over), and within a group through the w tiles, each w tile
    // for the group's slabs side by side.  The host sizes a group so that it
    // fills the XCD's CUs once (group x n_tiles ~ 32): the work groups that
    // run at a time on an XCD then share their x slabs and w tiles through
    // the XCD's L2.
    const int b = int(blockIdx.x), xcd = b & 7, slot = b >> 3;
    const int m8 = (m_tiles + 7) / 8, full = (m8 / group) * group * n_tiles;
    const int gs = slot < full ? group : m8 - (m8 / group) * group;  // > 0 wherever used
    const int g0 = slot < full ? (slot / (group * n_tiles)) * group : (m8 / group) * group;
    const int in = slot < full ? slot % (group * n_tiles) : slot - full;
    const int m_t = (g0 + in % gs) * 8 + xcd, n_t = in / gs;
    if (m_t >= m_tiles) return;
    const int m0 = m_t * kGBM, n0 = n_t * kGBN;
    const int rows_x = min(kGBM, M - m0);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;
    const int wm = wave & 3, wn = wave >> 2;  // wave tile: x rows wm*64.., w rows wn*128..

    // DMA: instruction i of wave `wave` moves slab rows wave*32 + 8i + lane/8,
    // lane's 16 bytes landing at LDS chunk lane%8 and coming from the row's
    // chunk (lane%8) ^ gswz(row).  x rows past M repeat row M-1 (their
    // outputs are not stored).
    const uint32_t kbytes = uint32_t(K) * 2u;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x + int64_t(m0) * K), 0, int(uint32_t(rows_x) * kbytes), kBufferFlags);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(w + int64_t(n0) * K), 0, int(uint32_t(kGBN) * kbytes), kBufferFlags);
    int xoff[kGLoads], woff[kGLoads];
#pragma unroll
    for (int i = 0; i < kGLoads; ++i) {
        const int row = wave * 32 + 8 * i + lane / 8;
        const int chunk = 16 * ((lane & 7) ^ gswz(row));
        xoff[i] = min(row, rows_x - 1) * int(kbytes) + chunk;
        woff[i] = row * int(kbytes) + chunk;
    }
    auto dma = [&](uint8_t LDS_AS *dx, uint8_t LDS_AS *dw, int slab) {
        const int soff = slab * kGRow;
#pragma unroll
        for (int i = 0; i < kGLoads; ++i) {
            const int lo = (wave * 32 + 8 * i) * kGRow;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (void LDS_AS *)(dx + lo), 16, xoff[i], soff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (void LDS_AS *)(dw + lo), 16, woff[i], soff, 0, 0);
        }
    };

    // Operand addresses: w block nb (A): row wn*128 + 32nb + l32; x block mb
    // (B): row wm*64 + 32mb + l32; k-step s reads logical chunk 2s + hh.
    int waddr[4], xaddr[2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) waddr[nb] = (wn * 128 + 32 * nb + l32) * kGRow;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) xaddr[mb] = (wm * 64 + 32 * mb + l32) * kGRow;
    const int sw = gswz(l32);  // rows differ by multiples of 32 from l32: same swizzle

    f32x16 acc[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x16{};

    auto slab = [&](const uint8_t LDS_AS *cx, const uint8_t LDS_AS *cw, uint8_t LDS_AS *nx, uint8_t LDS_AS *nw,
                    int s, int n_slabs) {
        if (s + 1 < n_slabs) dma(nx, nw, s + 1);
        bf16x8 wa[2][4], xb[2][2];
        auto rd = [&](int ks, int buf) {
            const int c = 16 * ((2 * ks + hh) ^ sw);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) wa[buf][nb] = *reinterpret_cast<const bf16x8 LDS_AS *>(cw + waddr[nb] + c);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) xb[buf][mb] = *reinterpret_cast<const bf16x8 LDS_AS *>(cx + xaddr[mb] + c);
        };
        rd(0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int ks = 0; ks < kGBK / 16; ++ks) {
            // The operands of k-step ks+1 are read between the products of
            // step ks (one read after each of the first six products).
            if (ks + 1 < kGBK / 16) rd(ks + 1, (ks + 1) & 1);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma(wa[ks & 1][nb], xb[ks & 1][mb], acc[mb][nb]);
            if (ks + 1 < kGBK / 16) {
#pragma unroll
                for (int i = 0; i < 6; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's DMA of slab s+1 has landed
        __syncthreads();                     // ... every wave's, and all are done with slab s
    };

    const int n_slabs = K / kGBK;
    uint8_t LDS_AS *const x0 = (uint8_t LDS_AS *)sx0;
    uint8_t LDS_AS *const w0 = (uint8_t LDS_AS *)sw0;
    uint8_t LDS_AS *const x1 = (uint8_t LDS_AS *)sx1;
    uint8_t LDS_AS *const w1 = (uint8_t LDS_AS *)sw1;
    dma(x0, w0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int s = 0; s < n_slabs; s += 2) {
        slab(x0, w0, x1, w1, s, n_slabs);
        if (s + 1 < n_slabs) slab(x1, w1, x0, w0, s + 1, n_slabs);
    }

    // Epilogue: acc[mb][nb] register 4g + e holds y[m][n] with m = m0 +
    // wm*64 + 32mb + l32 and n = n0 + wn*128 + 32nb + 8g + 4hh + e.  The
    // wave's 128 features are one head (n0 + wn*128 is a multiple of 128):
    // feature pair 16nb + 4g + 2hh + h of it sits in register pair (4g + 2h,
    // 4g + 2h + 1).
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int m = m0 + wm * 64 + 32 * mb + l32;
        if (m >= M) continue;
        uint16_t *yrow = y + int64_t(m) * N + n0 + wn * 128 + 4 * hh;
        const uint16_t *rrow = RES ? r + int64_t(m) * N + n0 + wn * 128 + 4 * hh : nullptr;
        // ROPE: cs index of pair k of the row is pb[axis of k] + k (the
        // row's axial position times 21, less the axis block's first pair).
        int pb[3] = {0, 0, 0};
        if constexpr (ROPE) {
            int p0, p1, p2;
            if (m < rp.n_video) {
                const uint32_t v = uint32_t(rp.pos[rp.cid[m]]);
                p0 = rp.text_len + int(v & 1023u);
                p1 = int((v >> 10) & 2047u);
                p2 = int(v >> 21);
            } else {
                p0 = p1 = p2 = m - rp.n_video;
            }
            pb[0] = p0 * kRopeAxisPairs;
            pb[1] = (p1 - 1) * kRopeAxisPairs;
            pb[2] = (p2 - 2) * kRopeAxisPairs;
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[mb][nb][4 * g + e];
                if constexpr (RES) {
                    const u32x2 rv = *reinterpret_cast<const u32x2 *>(rrow + 32 * nb + 8 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t bits = (rv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                        v[e] += __builtin_bit_cast(float, bits << 16);
                    }
                }
                uint32_t s0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v[0], v[1]}, bf16x2));
                uint32_t s1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v[2], v[3]}, bf16x2));
                if constexpr (ROPE) {
                    const int k0 = 16 * nb + 4 * g + 2 * hh;  // pair of s0; s1 holds pair k0 + 1
                    s0 = rope_pair(s0, k0, pb, rp.cs);
                    s1 = rope_pair(s1, k0 + 1, pb, rp.cs);
                }
                *reinterpret_cast<u32x2 *>(yrow + 32 * nb + 8 * g) = u32x2{s0, s1};
            }
    }
#endif
}

}  // namespace

int gemm_bf16_tile_n() { return kGBN; }
int gemm_bf16_tile_k() { return kGBK; }

hipError_t launch_gemm_bf16(const void *x, const void *w, void *y, const void *r, int64_t M, int N,
                            int K, const GemmRope *rope, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (rope && (r || N % 128 != 0 || !rope->cid || !rope->pos || !rope->cs)) return hipErrorInvalidValue;
    const int m_tiles = int((M + kGBM - 1) / kGBM), n_tiles = N / kGBN;
    const int group = std::max(1, (kCusPerXcd + n_tiles / 2) / n_tiles);
    const int64_t blocks = int64_t((m_tiles + 7) / 8) * 8 * n_tiles;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    auto U = [](const void *p) { return static_cast<const uint16_t *>(p); };
    const dim3 grid{unsigned(blocks)}, block{64 * kGWaves};
    uint16_t *Y = static_cast<uint16_t *>(y);
    if (rope)
        gemm_bf16_kernel<false, true><<<grid, block, 0, s>>>(U(x), U(w), Y, nullptr, int(M), N, K, m_tiles,
                                                             n_tiles, group, *rope);
    else if (r)
        gemm_bf16_kernel<true, false><<<grid, block, 0, s>>>(U(x), U(w), Y, U(r), int(M), N, K, m_tiles,
                                                             n_tiles, group, GemmRope{});
    else
        gemm_bf16_kernel<false, false><<<grid, block, 0, s>>>(U(x), U(w), Y, nullptr, int(M), N, K, m_tiles,
                                                              n_tiles, group, GemmRope{});
    return hipGetLastError();
}

}  // namespace wsp
