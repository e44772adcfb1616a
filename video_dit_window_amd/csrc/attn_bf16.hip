// Window joint attention on gfx950 matrix cores (MFMA): bfloat16 q/k/v, or
// OCP E4M3 q/k codes with bfloat16 v.
//
// "Window-Aligned Sequence Parallelism (SeedVR2)", section "SeedVR2
// integration": each window attends over the packed segment
// [video window; replicated text]; section "Text stream": each window yields
// one text output, averaged over windows afterwards.  "Parallelize new
// models with USP (text replica)", section "3. Attention with USP": plain
// SDPA (no mask, no dropout, scale 1/sqrt(D) unless given).  The E4M3 variant
// follows the low-precision result of "Scaling Video Training with
// Parallelism" (a neighbouring system); its recipe is this library's own.
//
// Work items (host-built list, one work group each):
//   video item  (window w, head h, tile of 256 video query rows of w): the
//               queries attend over [k/v rows of w; txt_k/v] and write `out`;
//   text item   (chunk c of consecutive windows, head h, tile of 256 text
//               query rows): the same queries attend over each window of the
//               chunk in turn (an independent softmax per window) and the
//               normalised outputs T_w are summed, in window order, into the
//               float32 partial c of the workspace (the text-mean kernel then
//               adds the partials in chunk order and divides by the window
//               count).  The query rows are loaded once per item.
// A work group is 8 wavefronts of 32 query rows (one work group per CU), 2
// waves per SIMD, < 256 registers each (or, for short windows, 4 wavefronts
// and 128 rows, two work groups per CU).
//
// Per 64-key tile and wavefront, in two 32-key halves (block 1's score
// products run between the pieces of block 0's softmax, and the products of
// block 0's probabilities between the pieces of block 1's, so that a wave
// keeps its own matrix and vector work overlapped):
//   S^T = K Q^T     K from LDS as the A operand, Q in registers as B:
//                   v_mfma_f32_32x32x16_bf16 (bf16), or
//                   v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 codes (unit E8M0
//                   scales; the dequantisation rides in the exponent scale).
//                   The transposed product leaves each lane with ONE query
//                   column and 32 of its keys.
//   softmax         float32, exp2 with the scale folded into one FMA; the
//                   running maximum is set on a window's first half tile and
//                   moves only when a half's probabilities would exceed 2^20
//                   (detected from the row sum).
//   O^T += V^T P^T  the probabilities stay in registers as bf16 B operands;
//                   V^T comes from the row-major V tile through the gfx950
//                   LDS transpose read (ds_read_b64_tr_b16).
// K and V tiles travel global -> LDS by direct DMA loads (buffer loads to
// LDS, 16 bytes per lane, no staging registers), double-buffered: the DMA of tile
// j+1 runs while tile j is multiplied.  Rows are stored unpadded, their
// 16-byte chunks XOR-swizzled by row so that the K operand reads and the
// transpose reads hit distinct banks.

#include "attn_bf16_common.h"

namespace wsp {

namespace {

// Waves per work group: 8 x 32 query rows, one work group per CU (2 waves
// per SIMD); or 4 x 32 rows, two work groups per CU (short windows: less of
// a window's last query tile is empty).  Same per-wave arithmetic.
constexpr int kItemWaves = 8, kSmallItemWaves = 4;
// s_getreg operand: hwreg XCC_ID (20), offset 0, 4 bits.
constexpr int kHwRegXccId = ((4 - 1) << 11) | (0 << 6) | 20;

typedef int v8i __attribute__((ext_vector_type(8)));
constexpr int kE8M0One = 127;  // E8M0 exponent of 1.0

__device__ inline f32x16 mfma8(v8i a, v8i b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kE8M0One, 0, kE8M0One);
}

// K tiles: rows of 2D bytes (bf16) or D bytes (E4M3 codes).
template <int D, int kWaves, bool Q8>
struct KShape {
    static constexpr int ROW = Q8 ? D : 2 * D;                 // bytes per K row in LDS
    static constexpr int CH = ROW / 16;                        // 16-byte chunks per row
    static constexpr int TILE = kBN * ROW;
    static constexpr int ROWS_PER_LOAD = 1024 / ROW;           // rows per wave DMA
    static constexpr int LOADS = kBN / ROWS_PER_LOAD / kWaves; // DMAs per wave per tile
    static_assert(LOADS * ROWS_PER_LOAD * kWaves == kBN, "tile must split over the waves");
};

// XOR swizzle of the 16-byte chunks of an E4M3 K row (8 chunks): the 32-row
// operand reads (2 chunks per lane) hit distinct banks.
__device__ __host__ constexpr int swz8(int r) { return (r >> 1) & 7; }
template <int D, bool Q8>
__device__ __host__ constexpr int kswz(int r) {
    return Q8 ? swz8(r) : swz<D>(r);
}

// Window-local rotary embedding of the queries inside the kernel (ROPE).
constexpr int kRopePairs = 21;  // pairs per axis block (42 of 128 channels)

// Rotation of query chunk c = 2S + hh of a row: bf16 channels 8c .. 8c+7,
// i.e. pairs 8S + 4hh + e (e < 4; pair k of axis block k / 21), with the
// row's table offsets p21[a] = position_a * 21 (positions Lt + dt, dh, dw);
// cs = (cos, sin) of 21 pairs per position.  Pairs 0..62 turn, pair 63
// (channels 126, 127) passes through.  The axis and in-block index of each
// pair are compile-time up to the lane's hh.  Same float32 steps and one
// rounding to bf16 as the stand-alone rotation kernel.
template <int S>
__device__ inline u32x4 rope_q_chunk(u32x4 w, int hh, const int (&p21)[3], const float2 *__restrict__ cs) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int k0 = 8 * S + e, k1 = k0 + 4;
        const int ax0 = k0 / kRopePairs, ax1 = k1 / kRopePairs;
        const int i0 = k0 - kRopePairs * ax0, i1 = k1 - kRopePairs * ax1;
        int idx;
        if (ax0 == ax1) idx = p21[ax0] + i0 + 4 * hh;
        else idx = hh ? (ax1 < 3 ? p21[ax1] + i1 : 0) : p21[ax0] + i0;
        const float2 t = cs[idx];
        const float x0 = __uint_as_float(w[e] << 16), x1 = __uint_as_float(w[e] & 0xFFFF0000u);
        const uint32_t r = pack_bf16(fmaf(x0, t.x, -x1 * t.y), fmaf(x0, t.y, x1 * t.x));
        o[e] = (ax1 >= 3 && hh) ? w[e] : r;  // pair 63 (channels 126, 127) passes through
    }
    return o;
}
template <int S, int N>
__device__ inline void rope_q_row(bf16x8 (&Qr)[N], int hh, const int (&p21)[3], const float2 *__restrict__ cs) {
    if constexpr (S < N) {
        Qr[S] = __builtin_bit_cast(bf16x8, rope_q_chunk<S>(__builtin_bit_cast(u32x4, Qr[S]), hh, p21, cs));
        rope_q_row<S + 1, N>(Qr, hh, p21, cs);
    }
}

// GATHER: q, k, v and out hold rows in canonical token order; video row r
// of window w is canonical row vrow0 + rel[off + r] (the plan's ids relative
// to the window's smallest id), so the layout permutation happens inside the
// loads and the output stores.  Q8: q, k, tq, tk are E4M3 codes (D = 128).
// ROPE (bf16, D = 128): the video query rows are rotated by their
// window-local positions as an item loads them; k, tq and tk arrive rotated.
template <int D, int kWaves, bool GATHER, bool Q8, bool ROPE>
__global__ __launch_bounds__(64 * kWaves, 2) void attn_bf16_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint8_t *__restrict__ tq, const uint8_t *__restrict__ tk, const uint16_t *__restrict__ tv,
    uint16_t *__restrict__ out, float *__restrict__ ws, const int32_t *__restrict__ rel,
    const ItemDesc *__restrict__ items, const WinDesc *__restrict__ wins,
    const float *__restrict__ amax_q, const float *__restrict__ amax_k, const float2 *__restrict__ rope_cs,
    const int32_t *__restrict__ rope_pos, int H, int Lt, float c2_unit, uint32_t *__restrict__ queue,
    int n_items, int n_lists, int grid_hw, int grid_w) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer resources exist only in the device pass
    using VS = Shape<D, kWaves>;       // V tiles (bf16 rows)
    using KS = KShape<D, kWaves, Q8>;  // K tiles
    static_assert(!Q8 || D == 128, "E4M3 scores need head_dim 128");
    static_assert(!ROPE || (D == 128 && !Q8), "in-kernel RoPE: bf16 rows of head_dim 128");
    constexpr int kBM = 32 * kWaves;   // query rows per work group
    constexpr int QE = Q8 ? 1 : 2;     // bytes per q / k element
    // Two stages, each a K tile followed by a V tile.
    constexpr int kStage = KS::TILE + VS::TILE;
    // The stages; after an item's last tile also the staging area of its
    // video outputs (32 rows of 2D bytes per wave, rows kOutRow apart: the
    // 16-byte pad spreads a column over the banks, and the lane's addresses
    // stay one base plus constants).
    constexpr int kOutRow = VS::ROW + 16;
    constexpr int kOut = kWaves * 32 * kOutRow;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStage > kOut ? 2 * kStage : kOut];

    const int64_t rs = int64_t(H) * D;  // elements per tensor row
    const uint32_t krow_bytes = uint32_t(rs) * QE, vrow_bytes = uint32_t(rs) * 2u;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;

    // DMA of one K/V tile.  For V, wave `wave` moves rows wave*(64/kWaves)
    // + ROWS_PER_LOAD*i + lane/CH (i < LOADS); the lane's 16 bytes land at
    // LDS chunk lane%CH of its row and come from the row's chunk
    // (lane%CH) ^ swz(row).  K likewise with its own row size.
    const int vdrow0 = wave * (kBN / kWaves) + lane / VS::CH;
    const int kdrow0 = wave * (kBN / kWaves) + lane / KS::CH;
    int vdchunk[VS::LOADS], kdchunk[KS::LOADS];  // bytes into the row
#pragma unroll
    for (int i = 0; i < VS::LOADS; ++i)
        vdchunk[i] = 16 * ((lane % VS::CH) ^ swz<D>(vdrow0 + VS::ROWS_PER_LOAD * i));
#pragma unroll
    for (int i = 0; i < KS::LOADS; ++i)
        kdchunk[i] = 16 * ((lane % KS::CH) ^ kswz<D, Q8>(kdrow0 + KS::ROWS_PER_LOAD * i));
    auto klo = [&](int i) { return (wave * (kBN / kWaves) + KS::ROWS_PER_LOAD * i) * KS::ROW; };
    auto vlo = [&](int i) { return KS::TILE + (wave * (kBN / kWaves) + VS::ROWS_PER_LOAD * i) * VS::ROW; };
    // Every DMA is a buffer load (MUBUF): the global/flat DMA forms would
    // make the compiler wait for all outstanding LDS reads (lgkmcnt(0)) while
    // a DMA is in flight.  Video rows come through resources based at the
    // window's first row (gather mode: its smallest canonical row, the first
    // in row-major order), text rows through resources based at the text
    // tensors; the host checks that every offset fits 31 bits.  A resource's
    // byte range also bounds every access.  (The window's row range is held
    // in scalar registers: a resource in vector registers would turn every
    // DMA into a loop over lanes.)
    auto rsrc = [&](const void *base, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), kBufferFlags);
    };

    // LDS byte offsets of this lane's operands inside a stage.
    //  K (A of S^T), bf16: row 32*mk + l32, logical chunk 2s + hh.
    //  K, E4M3: row 32*mk + l32, logical chunks 4s + 2hh + e (e < 2).
    int kaddr[Q8 ? 1 : VS::KSTEPS];
    int kaddr8[2][2];
    if constexpr (Q8) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 2; ++e) kaddr8[s][e] = l32 * KS::ROW + 16 * ((4 * s + 2 * hh + e) ^ swz8(l32));
    } else {
#pragma unroll
        for (int s = 0; s < VS::KSTEPS; ++s) kaddr[s] = l32 * KS::ROW + 16 * ((2 * s + hh) ^ swz<D>(l32));
    }
    //  V^T (A of O^T) by transpose reads: for O^T block t and half B of a
    //  16-key k-step, lane i = lane%16 of 16-lane group g reads 8 bytes of
    //  row 16*cs + 8*B + 4*hh + i/4, dims 32t + 16*(g%2) + 4*(i%4) .. +3;
    //  the transpose hands lane l dim 32t + l%32 of those four rows.
    const int gi = lane & 15, ghalf = (lane >> 4) & 1;
    int vaddr[VS::DT][2];
#pragma unroll
    for (int t = 0; t < VS::DT; ++t)
#pragma unroll
        for (int B = 0; B < 2; ++B) {
            const int row = 8 * B + 4 * hh + (gi >> 2);
            const int dim = 32 * t + 16 * ghalf + 4 * (gi & 3);
            vaddr[t][B] = KS::TILE + row * VS::ROW + 16 * ((dim >> 3) ^ swz<D>(row)) + 2 * (dim & 7);
        }

    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    uint8_t LDS_AS *const st0 = (uint8_t LDS_AS *)lds;
    uint8_t LDS_AS *const st1 = st0 + kStage;

    // Gather mode: relative ids of the rows of a tile, one set per DMA (V
    // rows; E4M3 K rows have their own map).
    struct Ids {
        int v[VS::LOADS];
        int k[Q8 ? KS::LOADS : 1];
    };
    // Ids of tile j of a window whose relative ids are addressed by `irs`.
    auto load_ids = [&](__amdgpu_buffer_rsrc_t irs, Ids &d, int j) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < VS::LOADS; ++i)
            d.v[i] = __builtin_amdgcn_raw_buffer_load_b32(irs, 4 * (j * kBN + vdrow0 + VS::ROWS_PER_LOAD * i), 0, 0);
        if constexpr (Q8) {
#pragma unroll
            for (int i = 0; i < KS::LOADS; ++i)
                d.k[i] = __builtin_amdgcn_raw_buffer_load_b32(irs, 4 * (j * kBN + kdrow0 + KS::ROWS_PER_LOAD * i), 0, 0);
        }
    };
    // Gather mode: the window's relative ids, read by buffer loads whose
    // per-lane offset holds the row (the range check covers it: rows past
    // the window read 0, and such rows only reach the DMA as masked keys).
    auto ids_rsrc = [&](const WinDesc &wd) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(GATHER ? rel + wd.off : rel), 0,
                                                 GATHER ? 4 * wd.lw : 0, kBufferFlags);
    };

    // The work: the item at blockIdx.x; or, with a queue, resident work
    // groups that take items in turn from a list (list x holds items
    // n_lists * t + x, then idle padding; queue[x], zero at launch, hands out
    // its tickets t), so an item's start-up overlaps the previous item's
    // stores and no work group waits for a dispatch.  A work group starts on
    // the list of the XCD it runs on (every item of a (window, head) group
    // then reads the group's K/V from one L2) and, once that list is empty,
    // moves on to the next ones, so every list drains wherever the work
    // groups run.  Thread 0 takes the next ticket as an item starts and
    // publishes it at the item's first barrier; every wave then requests the
    // next item's descriptor (lanes 0..11 hold its words).  s_next has two
    // slots used in turn: a slot is rewritten only after every wave has
    // passed the barrier that follows its reads.
    __shared__ int s_next[2];
    int xq = 0, b = blockIdx.x, par = 0, empty_lists = 0;
    auto take = [&]() __attribute__((always_inline)) {
        if (tid == 0)
            s_next[par] = n_lists * int(__hip_atomic_fetch_add(queue + xq, 1u, __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT)) + xq;
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(s_next[par]);
        par ^= 1;
    };
    if (queue) {
        if (n_lists > 1) xq = int(__builtin_amdgcn_s_getreg(kHwRegXccId) & 7u);
        take();
    }
    ItemDesc it{};
    it.w = -1;
    if (b < n_items) it = items[b];
    for (;;) {
    if (it.w < 0) {  // list xq is empty
        if (!queue || ++empty_lists >= n_lists) break;
        xq = xq + 1 == n_lists ? 0 : xq + 1;
        take();
        it.w = -1;
        if (b < n_items) it = items[b];
        continue;
    }
    uint32_t ticket = 0;
    if (queue && tid == 0)
        ticket = __hip_atomic_fetch_add(queue + xq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t next_desc = 0;
    const bool text = it.nwin > 0;
    const int h = it.hq >> 16, qt = it.hq & 0xFFFF;
    const int64_t hd = int64_t(h) * D;  // elements
    // Scores in log2 units: S * c2; E4M3 scores carry both dequantisation factors.
    float c2 = c2_unit;
    if constexpr (Q8) c2 = c2_unit * (amax_q[h] * (1.0f / 448.0f)) * (amax_k[h] * (1.0f / 448.0f));

    // Query row of this lane (B operand of S^T = K Q^T): the item's query
    // rows are nv video rows of its window (through the ids table in gather
    // mode), then -- joint items, or text items (nv = 0) -- text rows.  Its
    // tensor row also addresses the output store.
    const bool joint = !text && it.chunk >= 0;
    const int nv = text ? 0 : it.win.lw;
    const int nq = nv + (text || joint ? Lt : 0);
    const int qrow = qt * kBM + wave * 32 + l32;
    // ROPE: the query row's window offset, requested first: its (cos, sin)
    // loads depend on it and then run beside the query row's own load.
    uint32_t qpk = 0;
    if constexpr (ROPE) {
        if (qrow < nv) qpk = uint32_t(rope_pos[it.win.off + qrow]);
    }
    // Gather mode: the first tile's row ids are requested with the query
    // row's id, so that the query load and the first DMA start together.
    // Gather mode: video rows take their ids from the window's box (row r =
    // (dt*eh + dh)*ew + dw lies dt*H*W + dh*W + dw canonical rows past the
    // first), so the query and first-tile loads wait for no table read.
    auto box_rel = [&](int r) {
        const uint32_t eh = uint32_t(it.eh), ew = uint32_t(it.ew);
        const uint32_t q1 = uint32_t(r) / ew, dt = q1 / eh;
        return int(dt * uint32_t(grid_hw) + (q1 - dt * eh) * uint32_t(grid_w) + (uint32_t(r) - q1 * ew));
    };
    // (rows past the window get id 0, as from the table's range check)
    auto box_ids0 = [&](Ids &d) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < VS::LOADS; ++i) {
            const int r = vdrow0 + VS::ROWS_PER_LOAD * i;
            d.v[i] = r < nv ? box_rel(r) : 0;
        }
        if constexpr (Q8) {
#pragma unroll
            for (int i = 0; i < KS::LOADS; ++i) {
                const int r = kdrow0 + KS::ROWS_PER_LOAD * i;
                d.k[i] = r < nv ? box_rel(r) : 0;
            }
        }
    };
    int64_t qtrow;
    {
        const int r = min(qrow, nq - 1);
        if (r >= nv) qtrow = r - nv;
        else if (GATHER) qtrow = int64_t(it.win.vrow0) + box_rel(r);
        else qtrow = int64_t(it.win.off) + r;
    }
    // bf16: lane half hh holds dims 16s + 8hh .. +7 of k-step s.  E4M3:
    // bytes [64s + 32hh, +32) of the row (the K operands use the same map).
    bf16x8 Qr[Q8 ? 1 : VS::KSTEPS];
    v8i Qr8[2];
    {
        const uint8_t *p = (min(qrow, nq - 1) >= nv ? tq : q) + (qtrow * rs + hd) * QE;
        if constexpr (Q8) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(p + 64 * s + 32 * hh);
                const u32x4 b = *reinterpret_cast<const u32x4 *>(p + 64 * s + 32 * hh + 16);
                Qr8[s] = v8i{int(a[0]), int(a[1]), int(a[2]), int(a[3]), int(b[0]), int(b[1]), int(b[2]), int(b[3])};
            }
        } else {
#pragma unroll
            for (int s = 0; s < VS::KSTEPS; ++s)
                Qr[s] = *reinterpret_cast<const bf16x8 *>(p + 2 * (16 * s + 8 * hh));
        }
    }
    const __amdgpu_buffer_rsrc_t tkrs = rsrc(tk + hd * QE, uint32_t(Lt) * krow_bytes);
    const __amdgpu_buffer_rsrc_t tvrs = rsrc(tv + hd, uint32_t(Lt) * vrow_bytes);

    // A wave whose 32 query rows all lie past the item's query rows (the
    // last query tile of a sequence) only moves its share of the K/V tiles
    // and meets the barriers: the SIMD it shares then runs the other wave
    // alone.
    const bool active = qt * kBM + wave * 32 < nq;

    // A video item runs one window; a text item each window of its chunk.
    const int n_loop = text ? it.nwin : 1;
    for (int wi = 0; wi < n_loop; ++wi) {
        const WinDesc wd = text ? wins[it.w + wi] : it.win;
        const int Lw = wd.lw;
        const int M = Lw + Lt;  // joint key/value sequence [video rows; text rows]
        const int64_t vrow0 = wd.vrow0;
        const uint32_t vrows = uint32_t(wd.vrows);
        const __amdgpu_buffer_rsrc_t krs = rsrc(k + (vrow0 * rs + hd) * QE, vrows * krow_bytes);
        const __amdgpu_buffer_rsrc_t vrs = rsrc(v + vrow0 * rs + hd, vrows * vrow_bytes);
        // Layout order: the lane's first row as a per-lane offset (its chunk
        // added at the load), the tile and row steps in the scalar offset.
        const int kdbase = kdrow0 * int(krow_bytes), vdbase = vdrow0 * int(vrow_bytes);
        // Gather mode: the ids of the next tile's rows are loaded one tile
        // ahead of their DMA.  Two register sets alternate: the next tile's
        // ids are requested before the current tile's DMA, so the tile's
        // closing vmcnt wait does not end on them.  The DMA offset is one
        // 24-bit multiply-add, exact because the host's limits keep the row
        // bytes and the relative ids below 2^24 and every offset below 2^31.
        const __amdgpu_buffer_rsrc_t irs = ids_rsrc(wd);
        auto kid = [&](const Ids &d, int i) { return Q8 ? d.k[i] : d.v[i]; };
        // The window's video rows travel with cache policy CP: 0 where other
        // items of the same XCD read the same K/V from L2 (video items, and a
        // text item of a single window, which runs beside that window's video
        // items); non-temporal (2) for a text item over a chunk of several
        // windows, the only reader of that K/V on its XCD, so that streaming
        // it does not evict the video groups' K/V.  Text rows (shared by
        // every item) keep the default.
        // (The tile-step lambdas are forced inline: left to the inliner, the
        // 4-wave layout-order kernel called one and kept its closure in
        // scratch memory.)
        auto dma_cp = [&](auto cp_c, uint8_t LDS_AS *dst, int j, Ids &idp,
                          Ids &idn) __attribute__((always_inline)) {
            constexpr int CP = decltype(cp_c)::value;
            if constexpr (GATHER) load_ids(irs, idn, j + 1);
            if (!GATHER && (j + 1) * kBN <= Lw) {
                const int ks = j * kBN * int(krow_bytes), vs = j * kBN * int(vrow_bytes);
#pragma unroll
                for (int i = 0; i < KS::LOADS; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + klo(i)), 16, kdbase + kdchunk[i],
                                                             ks + KS::ROWS_PER_LOAD * i * int(krow_bytes), 0, CP);
#pragma unroll
                for (int i = 0; i < VS::LOADS; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + vlo(i)), 16, vdbase + vdchunk[i],
                                                             vs + VS::ROWS_PER_LOAD * i * int(vrow_bytes), 0, CP);
            } else if (GATHER && (j + 1) * kBN <= Lw) {
#pragma unroll
                for (int i = 0; i < KS::LOADS; ++i) {
                    const int o = int(__umul24(uint32_t(kid(idp, i)), krow_bytes)) + kdchunk[i];
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + klo(i)), 16, o, 0, 0, CP);
                }
#pragma unroll
                for (int i = 0; i < VS::LOADS; ++i) {
                    const int o = int(__umul24(uint32_t(idp.v[i]), vrow_bytes)) + vdchunk[i];
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + vlo(i)), 16, o, 0, 0, CP);
                }
            } else {
                // Row by row: video rows, then text rows; rows past the joint
                // sequence clamped to its last row.
#pragma unroll
                for (int i = 0; i < KS::LOADS; ++i) {
                    const int r = min(j * kBN + kdrow0 + KS::ROWS_PER_LOAD * i, M - 1);
                    if (r < Lw) {
                        const int o = (GATHER ? int(__umul24(uint32_t(kid(idp, i)), krow_bytes))
                                              : r * int(krow_bytes)) + kdchunk[i];
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + klo(i)), 16, o, 0, 0, CP);
                    } else {
                        const int o = (r - Lw) * int(krow_bytes) + kdchunk[i];
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(tkrs, (void LDS_AS *)(dst + klo(i)), 16, o, 0, 0, 0);
                        // Keeps the compiler from merging the two arms into one
                        // load with a per-lane resource (issued as a loop over
                        // lanes).
                        asm volatile("");
                    }
                }
#pragma unroll
                for (int i = 0; i < VS::LOADS; ++i) {
                    const int r = min(j * kBN + vdrow0 + VS::ROWS_PER_LOAD * i, M - 1);
                    if (r < Lw) {
                        const int o = (GATHER ? int(__umul24(uint32_t(idp.v[i]), vrow_bytes))
                                              : r * int(vrow_bytes)) + vdchunk[i];
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + vlo(i)), 16, o, 0, 0, CP);
                    } else {
                        const int o = (r - Lw) * int(vrow_bytes) + vdchunk[i];
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(tvrs, (void LDS_AS *)(dst + vlo(i)), 16, o, 0, 0, 0);
                        asm volatile("");
                    }
                }
            }
        };
        auto dma = [&](uint8_t LDS_AS *dst, int j, Ids &idp, Ids &idn) __attribute__((always_inline)) {
            if (it.nwin > 1) dma_cp(std::integral_constant<int, 2>{}, dst, j, idp, idn);
            else dma_cp(std::integral_constant<int, 0>{}, dst, j, idp, idn);
        };

        f32x16 O[VS::DT];
#pragma unroll
        for (int t = 0; t < VS::DT; ++t) O[t] = f32x16{};
        float m_run = -INFINITY, l_run = 0.f;
        const int ntiles = (M + kBN - 1) / kBN;
        // A tile's last PV k-step (V^T operands va[1], probabilities P[3])
        // is multiplied at the start of the next tile, after that tile's
        // first K operand reads are issued (their latency hides under it),
        // and after the window's last tile.  Zero operands make the first
        // tile's deferred step a no-op.
        bf16x8 P[4];
        bf16x8 va[2][VS::DT];
        P[3] = bf16x8{};
#pragma unroll
        for (int t = 0; t < VS::DT; ++t) va[1][t] = bf16x8{};
        auto deferred = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int t = 0; t < VS::DT; ++t) O[t] = mfma(va[1][t], P[3], O[t]);
        };

        // One tile: cur holds tile j; the DMA of tile j+1 goes to nxt.
        auto tile = [&](const uint8_t LDS_AS *cur, uint8_t LDS_AS *nxt, int j, Ids &idu,
                        Ids &idn) __attribute__((always_inline)) {
            if (j + 1 < ntiles) dma(nxt, j + 1, idu, idn);
            if (active) {
            // Wave priority 1 until block 0's softmax is settled, then 0:
            // of the two waves of a SIMD, the one behind in its tile wins
            // issue, so the pair reaches the closing barrier together.
            __builtin_amdgcn_s_setprio(1);

            // S^T for 64 keys (two 32-key blocks) x this wave's 32 queries.
            // Block 0's products first; block 1's run while block 0's softmax
            // goes, and the products of block 0's probabilities while block
            // 1's softmax goes (the online softmax takes the tile in two
            // 32-key halves).
            f32x16 S[2] = {f32x16{}, f32x16{}};
            const bool last = (j + 1) * kBN > M;  // keys past the end of the joint sequence
            // element r of S[mk] is key 32mk + 8(r/4) + (r%4) of the tile
            // counted from this lane's first, j*kBN + 4hh
            auto mask = [&](int mk) __attribute__((always_inline)) {
                const int lim = M - j * kBN - 4 * hh;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * mk + 8 * (r >> 2) + (r & 3) >= lim) S[mk][r] = -INFINITY;
            };
            // p = 2^(s*c2 - m_run*c2) of half h packed to bf16 pairs (P^T B
            // operands, one per 16-key k-step); the row sum adds the same
            // rounded values.
            // Piece q (0..7) of half h: the probabilities of S[h] registers
            // 8(q/4) + 2(q%4) and + 1, into word q%4 of pk[q/4].
            auto piece = [&](int h, int q, float mc, float &sum, u32x4 (&pk)[2]) __attribute__((always_inline)) {
                const int r = 8 * (q >> 2) + 2 * (q & 3);
                const float p0 = __builtin_amdgcn_exp2f(fmaf(S[h][r], c2, -mc));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(S[h][r + 1], c2, -mc));
                const bf16x2 pp = to_bf16x2(p0, p1);
                sum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, sum, false);
                pk[q >> 2][q & 3] = __builtin_bit_cast(uint32_t, pp);
            };
            auto probs = [&](int h) __attribute__((always_inline)) {
                const float mc = m_run * c2;
                float sum = 0.f;
                u32x4 pk[2];
#pragma unroll
                for (int q = 0; q < 8; ++q) piece(h, q, mc, sum, pk);
                P[2 * h] = __builtin_bit_cast(bf16x8, pk[0]);
                P[2 * h + 1] = __builtin_bit_cast(bf16x8, pk[1]);
                return sum;
            };
            // Only on a window's first half tile (m_run = -inf) and when some
            // probability of a half would exceed 2^20 does the wave take the
            // exact path: the half's maximum, rescale of O and l by
            // 2^((m_old - m_new)*c2), recompute.
            auto settle = [&](int h, float hsum, bool first) __attribute__((always_inline)) {
                if (first || __builtin_amdgcn_ballot_w64(!(hsum <= kMaxTileSum))) {
                    float m = S[h][0];
#pragma unroll
                    for (int r = 1; r < 16; ++r) m = fmaxf(m, S[h][r]);
                    const float m_new = fmaxf(m_run, halves_max(m));
                    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
                    m_run = m_new;
                    if (!first) {  // on the first half O and l are still zero
                        l_run *= alpha;
#pragma unroll
                        for (int t = 0; t < VS::DT; ++t) O[t] *= alpha;
                    }
                    hsum = probs(h);
                }
                l_run += hsum;
            };
            // V^T operands (transpose reads) of one 16-key step.
            auto vread = [&](int cs, bf16x8 (&dst)[VS::DT]) __attribute__((always_inline)) {
#pragma unroll
                for (int t = 0; t < VS::DT; ++t) {
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (s16x4 LDS_AS *)(cur + vaddr[t][0] + cs * 16 * VS::ROW));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (s16x4 LDS_AS *)(cur + vaddr[t][1] + cs * 16 * VS::ROW));
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                    dst[t] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
                }
            };
            float hs0 = 0.f, hs1 = 0.f;
            if constexpr (Q8) {
                // two 64-dim k-steps of E4M3 codes per key block
                v8i ka[2][2];
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int mk = 0; mk < 2; ++mk) {
                        const uint8_t LDS_AS *base = cur + mk * 32 * KS::ROW;
                        const u32x4 a = *reinterpret_cast<const u32x4 LDS_AS *>(base + kaddr8[s][0]);
                        const u32x4 b = *reinterpret_cast<const u32x4 LDS_AS *>(base + kaddr8[s][1]);
                        ka[s][mk] = v8i{int(a[0]), int(a[1]), int(a[2]), int(a[3]),
                                        int(b[0]), int(b[1]), int(b[2]), int(b[3])};
                    }
                deferred();
#pragma unroll
                for (int s = 0; s < 2; ++s) S[0] = mfma8(ka[s][0], Qr8[s], S[0]);
                if (last) mask(0);
#pragma unroll
                for (int s = 0; s < 2; ++s) S[1] = mfma8(ka[s][1], Qr8[s], S[1]);
                vread(0, va[0]);
                hs0 = probs(0);
            } else {
                // The K operands run two k-steps ahead of the products, over
                // block 0's eight k-steps and then block 1's.
                constexpr int KS2 = 2 * VS::KSTEPS;
                bf16x8 ka[KS2];
                auto kread = [&](int f) __attribute__((always_inline)) {
                    const int mk = f / VS::KSTEPS, st = f % VS::KSTEPS;
                    ka[f] = *reinterpret_cast<const bf16x8 LDS_AS *>(cur + kaddr[st] + mk * 32 * KS::ROW);
                };
                kread(0);
                kread(1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                deferred();
                __builtin_amdgcn_sched_group_barrier(0x008, VS::DT, 0);
#pragma unroll
                for (int f = 0; f < VS::KSTEPS; ++f) {
                    S[0] = mfma(ka[f], Qr[f], S[0]);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    kread(f + 2);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                if (last) mask(0);
                // block 1's products, each followed by its operand reads and
                // a piece of block 0's softmax (six vector instructions,
                // transcendental ones included).  Also on a window's first
                // tile, where m_run = -inf makes the softmax non-finite and
                // the exact path recomputes it: no branch splits this block.
                const float mc = m_run * c2;
                u32x4 pk[2];
                constexpr int PP = 8 / VS::KSTEPS;  // softmax pieces per product
#pragma unroll
                for (int f = 0; f < VS::KSTEPS; ++f) {
                    S[1] = mfma(ka[VS::KSTEPS + f], Qr[f], S[1]);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (f + 2 < VS::KSTEPS) {
                        kread(VS::KSTEPS + f + 2);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    if (f == 0) {
                        vread(0, va[0]);
                        __builtin_amdgcn_sched_group_barrier(0x100, 2 * VS::DT, 0);
                    }
#pragma unroll
                    for (int q = PP * f; q < PP * f + PP; ++q) piece(0, q, mc, hs0, pk);
                    __builtin_amdgcn_sched_group_barrier(0x402, 6 * PP, 0);
                }
                P[0] = __builtin_bit_cast(bf16x8, pk[0]);
                P[1] = __builtin_bit_cast(bf16x8, pk[1]);
                // (kept here on every tile: on a window's first tile these
                // values are recomputed, and the compiler would otherwise
                // move the softmax under that branch, after the products)
                asm volatile("" : "+v"(hs0), "+v"(P[0]), "+v"(P[1]));
            }
            __builtin_amdgcn_s_setprio(0);
            settle(0, hs0, j == 0);
            if (last) mask(1);

            // O^T += V^T P^T over the tile's four 16-key k-steps, the operands
            // of step cs+1 read while step cs multiplies; a piece of block
            // 1's softmax follows each product of steps 0 and 1.
            {
                const float mc = m_run * c2;
                u32x4 pk[2];
                constexpr int PP = 4 / VS::DT;  // softmax pieces per product
#pragma unroll
                for (int cs = 0; cs < 2; ++cs)
#pragma unroll
                    for (int t = 0; t < VS::DT; ++t) {
                        O[t] = mfma(va[cs & 1][t], P[cs], O[t]);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (t == 0) {
                            vread(cs + 1, va[(cs + 1) & 1]);
                            __builtin_amdgcn_sched_group_barrier(0x100, 2 * VS::DT, 0);
                        }
#pragma unroll
                        for (int q = PP * (VS::DT * cs + t); q < PP * (VS::DT * cs + t) + PP; ++q)
                            piece(1, q, mc, hs1, pk);
                        __builtin_amdgcn_sched_group_barrier(0x402, 6 * PP, 0);
                    }
                P[2] = __builtin_bit_cast(bf16x8, pk[0]);
                P[3] = __builtin_bit_cast(bf16x8, pk[1]);
            }
            settle(1, hs1, false);
            vread(3, va[1]);
#pragma unroll
            for (int t = 0; t < VS::DT; ++t) O[t] = mfma(va[0][t], P[2], O[t]);
            // (k-step 3 is multiplied at the start of the next tile)
            }
            // The DMA of tile j+1 has landed (vmcnt) and every wave is done with
            // `cur` before it is overwritten two tiles later.
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
        };

        // Both stages are free here: the previous window or item (if any)
        // ended on a tile's closing barrier.
        Ids idA, idB;
        if (queue && wi == 0) {
            // every wave has read back the previous item's staged outputs
            // (LDS only: that item's global stores may still be in flight)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        // (one DMA call per branch, so that the wait for a table read stays
        // in its own branch)
        if (!GATHER || !text) {
            if constexpr (GATHER) box_ids0(idA);
            dma(st0, 0, idA, idB);
        } else {
            load_ids(irs, idA, 0);
            dma(st0, 0, idA, idB);
        }
        if constexpr (ROPE) {
            // video queries rotated in registers (chunk 2s + hh of the row),
            // once the first tile's DMA is on its way
            if (wi == 0 && qrow < nv) {
                const int p21[3] = {(Lt + int(qpk & 1023u)) * kRopePairs, int((qpk >> 10) & 2047u) * kRopePairs,
                                    int(qpk >> 21) * kRopePairs};
                rope_q_row<0, VS::KSTEPS>(Qr, hh, p21, rope_cs);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
        // (the raw ticket: nothing reads the atomic's result before this
        // wait, which the first DMA needs anyway)
        asm volatile("" ::: "memory");
        if (queue && wi == 0 && tid == 0) s_next[par] = int(ticket);
        __syncthreads();
        if (queue && wi == 0) {
            const int nb = n_lists * __builtin_amdgcn_readfirstlane(s_next[par]) + xq;
            if (lane < 12)
                next_desc = nb < n_items ? reinterpret_cast<const uint32_t *>(items)[12 * nb + lane]
                                         : (lane == 0 ? ~0u : 0u);
        }
        for (int j = 0; j < ntiles; j += 2) {
            tile(st0, st1, j, idB, idA);
            if (j + 1 < ntiles) tile(st1, st0, j + 1, idA, idB);
        }
        if (active) deferred();
        // Nothing is in flight here (the last tile waited); saying so lets
        // the next item's descriptor be read after the outputs below without
        // waiting for their stores.
        __builtin_amdgcn_s_waitcnt(0x0F70);

        // Normalise.  The lane holds query qrow, dims 32t + 8g + 4hh + 0..3.
        const float l = halves_sum(l_run);
        const float inv = 1.0f / l;
        if (qrow >= nv && qrow < nq) {
            // A text row: T_w into the float32 partial `chunk`.  A text item
            // writes it on its chunk's first window and adds the later ones
            // in window order (the same lane reads back what it wrote); a
            // joint item is the only writer of its window's text rows.
            float *dst = ws + ((int64_t(it.chunk) * Lt + (qrow - nv)) * H + h) * D;
#pragma unroll
            for (int t = 0; t < VS::DT; ++t)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 *p = reinterpret_cast<f32x4 *>(dst + 32 * t + 8 * g + 4 * hh);
                    f32x4 val = f32x4{O[t][4 * g] * inv, O[t][4 * g + 1] * inv, O[t][4 * g + 2] * inv,
                                      O[t][4 * g + 3] * inv};
                    if (wi > 0) val = *p + val;
                    *p = val;
                }
        }
        // Video rows go out through LDS: each wave stages its rows in its own
        // part of the idle stage buffers, then stores whole 16-byte chunks,
        // CH consecutive lanes per row (full cache lines, instead of 8-byte
        // pieces of 32 rows per store).
        const int r0 = qt * kBM + wave * 32;  // the wave's first query row
        if (r0 < nv) {
            uint8_t LDS_AS *const ob = st0 + wave * 32 * kOutRow;
            if (qrow < nv) {
#pragma unroll
                for (int t = 0; t < VS::DT; ++t)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        u32x2 st;
                        st[0] = pack_bf16(O[t][4 * g] * inv, O[t][4 * g + 1] * inv);
                        st[1] = pack_bf16(O[t][4 * g + 2] * inv, O[t][4 * g + 3] * inv);
                        *reinterpret_cast<u32x2 LDS_AS *>(ob + l32 * kOutRow + 2 * (32 * t + 8 * g + 4 * hh)) = st;
                    }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the staged rows are in LDS
            constexpr int RPI = 64 / VS::CH;      // rows per store
            constexpr int NS = 32 / RPI;          // stores per wave
            const int nrows = min(32, nv - r0), rl = lane / VS::CH, c = lane % VS::CH;
            const uint8_t LDS_AS *const ib = ob + rl * kOutRow + 16 * c;
            // All row ids and staged chunks are requested before the first
            // store (rows past nrows read stale staging bytes that are never
            // stored), so the LDS round trips overlap.
            int trow[NS];
            u32x4 val[NS];
#pragma unroll
            for (int i = 0; i < NS; ++i)  // tensor row of the wave's row RPI*i + rl (held by that lane)
                trow[i] = __builtin_amdgcn_ds_bpermute(4 * rl + 4 * RPI * i, int(qtrow));
#pragma unroll
            for (int i = 0; i < NS; ++i) val[i] = *reinterpret_cast<const u32x4 LDS_AS *>(ib + RPI * i * kOutRow);
#pragma unroll
            for (int i = 0; i < NS; ++i)
                if (rl < nrows - RPI * i)
                    *reinterpret_cast<u32x4 *>(out + int64_t(trow[i]) * rs + hd + 8 * c) = val[i];
        }
    }
    if (!queue) break;
    // The next item: its descriptor words from lanes 0..11 (w < 0 ends the list).
    it.w = __builtin_amdgcn_readlane(int(next_desc), 0);
    it.hq = __builtin_amdgcn_readlane(int(next_desc), 1);
    it.nwin = __builtin_amdgcn_readlane(int(next_desc), 2);
    it.chunk = __builtin_amdgcn_readlane(int(next_desc), 3);
    it.win.off = __builtin_amdgcn_readlane(int(next_desc), 4);
    it.win.lw = __builtin_amdgcn_readlane(int(next_desc), 5);
    it.win.vrow0 = __builtin_amdgcn_readlane(int(next_desc), 6);
    it.win.vrows = __builtin_amdgcn_readlane(int(next_desc), 7);
    it.eh = __builtin_amdgcn_readlane(int(next_desc), 8);
    it.ew = __builtin_amdgcn_readlane(int(next_desc), 9);
    par ^= 1;
    }
#endif
}

}  // namespace

int attn_bf16_tile_m(bool small) { return 32 * (small ? kSmallItemWaves : kItemWaves); }

namespace {
// Clears the work queue's ticket counters ahead of a resident-work-group launch.
__global__ void clear_queue_kernel(uint32_t *queue) {
    if (threadIdx.x < kQueueWords) queue[threadIdx.x] = 0u;
}
}  // namespace

hipError_t launch_attn_bf16(int head_dim, bool small, bool q8, const void *q, const void *k, const void *v,
                            const void *tq, const void *tk, const void *tv, void *out, float *ws,
                            const int32_t *rel, const ItemDesc *items, const WinDesc *wins, int n_items,
                            const float *amax_q, const float *amax_k, const RopeTables *rope, int n_heads,
                            int text_len, float scale, uint32_t *queue, int n_lists, int grid_hw, int grid_w,
                            hipStream_t s) {
    if (n_items <= 0) return hipSuccess;
    if (queue && n_lists != 1 && n_lists != 8) return hipErrorInvalidValue;
    if (q8 && head_dim != 128) return hipErrorInvalidValue;
    if (rope && (q8 || head_dim != 128)) return hipErrorInvalidValue;
    const float c2 = scale * kLog2e;
    const RopeTables none{};
    const RopeTables &rt = rope ? *rope : none;
    auto B = [](const void *p) { return static_cast<const uint8_t *>(p); };
    auto U = [](const void *p) { return static_cast<const uint16_t *>(p); };
    hipError_t err = hipSuccess;
    auto launch = [&](auto kern, int waves) {
        int grid = n_items;
        if (queue) {
            // one resident work group per free slot of every compute unit
            int dev = 0, cus = 0, per_cu = 0;
            if ((err = hipGetDevice(&dev)) != hipSuccess) return;
            if ((err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return;
            if ((err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * waves, 0)) != hipSuccess)
                return;
            grid = std::min(n_items, std::max(1, cus * per_cu));
            clear_queue_kernel<<<1, 64, 0, s>>>(queue);
        }
        kern<<<dim3(grid), dim3(64 * waves), 0, s>>>(B(q), B(k), U(v), B(tq), B(tk), U(tv),
                                                      static_cast<uint16_t *>(out), ws, rel, items, wins, amax_q,
                                                      amax_k, rt.cs, rt.pos, n_heads, text_len, c2, queue, n_items,
                                                      n_lists, grid_hw, grid_w);
    };
    auto dispatch = [&](auto waves_c) {
        constexpr int NW = decltype(waves_c)::value;
        const bool g = rel != nullptr;
        if (rope) {
            g ? launch(attn_bf16_kernel<128, NW, true, false, true>, NW)
              : launch(attn_bf16_kernel<128, NW, false, false, true>, NW);
        } else if (q8) {
            g ? launch(attn_bf16_kernel<128, NW, true, true, false>, NW)
              : launch(attn_bf16_kernel<128, NW, false, true, false>, NW);
        } else if (head_dim == 128) {
            g ? launch(attn_bf16_kernel<128, NW, true, false, false>, NW)
              : launch(attn_bf16_kernel<128, NW, false, false, false>, NW);
        } else if (head_dim == 64) {
            g ? launch(attn_bf16_kernel<64, NW, true, false, false>, NW)
              : launch(attn_bf16_kernel<64, NW, false, false, false>, NW);
        } else {
            return hipErrorInvalidValue;
        }
        return hipSuccess;
    };
    const hipError_t e = small ? dispatch(std::integral_constant<int, kSmallItemWaves>{})
                               : dispatch(std::integral_constant<int, kItemWaves>{});
    if (e != hipSuccess) return e;
    if (err != hipSuccess) return err;
    return hipGetLastError();
}

}  // namespace wsp
