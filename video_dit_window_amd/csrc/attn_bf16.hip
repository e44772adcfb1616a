// bfloat16 window joint attention on gfx950 matrix cores (MFMA).
//
// "Window-Aligned Sequence Parallelism (SeedVR2)", section "SeedVR2
// integration": each window attends over the packed segment
// [video window; replicated text]; section "Text stream": each window yields
// one text output, averaged over windows afterwards.  "Parallelize new
// models with USP (text replica)", section "3. Attention with USP": plain
// SDPA (no mask, no dropout, scale 1/sqrt(D) unless given).
//
// Work item = (window w, head h, tile of 256 query rows) of the joint query
// sequence [q rows of w; txt_q]; the key/value sequence is [k/v rows of w;
// txt_k/v].  A work group is 8 wavefronts of 32 query rows (one work group
// per CU), 2 waves per SIMD, < 256 registers each (or, for short windows, 4
// wavefronts and 128 rows, two work groups per CU).
//
// Per 64-key tile and wavefront:
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16 with K from LDS as the A operand
//                   and Q in registers as B.  The transposed product leaves
//                   each lane with ONE query column and 32 of its keys.
//   softmax         float32, exp2 with the scale folded into one FMA; the
//                   running maximum is set on a work item's first tile and
//                   moves only when a tile's probabilities would exceed 2^20
//                   (detected from the row sum).
//   O^T += V^T P^T  the probabilities stay in registers as bf16 B operands;
//                   V^T comes from the row-major V tile through the gfx950
//                   LDS transpose read (ds_read_b64_tr_b16).
// K and V tiles travel global -> LDS by direct DMA loads (buffer loads to
// LDS, 16 bytes per lane, no staging registers), double-buffered: the DMA of tile
// j+1 runs while tile j is multiplied.  Rows are stored unpadded, their
// 16-byte chunks XOR-swizzled by row so that the K operand reads (16 rows,
// one chunk) and the transpose reads (4 rows x 4 chunks) hit distinct banks.
// Video query rows write bf16 `out`; text query rows write their normalised
// float32 output to the workspace, reduced over windows in id order by the
// text-mean kernel.

#include "attn_bf16_common.h"

namespace wsp {

namespace {

// Waves per work group: 8 x 32 query rows, one work group per CU (2 waves
// per SIMD); or 4 x 32 rows, two work groups per CU (short windows: less of
// a window's last query tile is empty).  Same per-wave arithmetic.
constexpr int kItemWaves = 8, kSmallItemWaves = 4;

// GATHER: q, k, v and out hold rows in canonical token order; the video row
// r of window w is canonical row vrow0 + rel[offsets[w] + r] (the plan's ids
// relative to the window's smallest id), so the layout permutation happens
// inside the loads and the output stores.
template <int D, int kWaves, bool GATHER>
__global__ __launch_bounds__(64 * kWaves, 2) void attn_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ tq,
    const uint16_t *__restrict__ tk, const uint16_t *__restrict__ tv,
    uint16_t *__restrict__ out, float *__restrict__ ws, const int32_t *__restrict__ rel,
    const ItemDesc *__restrict__ items, int H, int Lt, float c2) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer resources exist only in the device pass
    using S_ = Shape<D, kWaves>;
    constexpr int kBM = 32 * kWaves;  // query rows per work group
    // Two stages, each a K tile followed by a V tile.
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[2 * S_::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[2 * S_::TILE];

    // One scalar load: window, head, query tile and the window's rows.
    const ItemDesc it = items[blockIdx.x];
    if (it.w < 0) return;
    const int w = it.w, h = it.hq >> 16, qt = it.hq & 0xFFFF;
    const int64_t off = it.off;
    const int Lw = it.lw;
    const int M = Lw + Lt;
    const int64_t rs = int64_t(H) * D, hd = int64_t(h) * D;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;

    // Tensor row of video row r (< Lw) of this window.
    const int64_t vrow0 = it.vrow0;
    const int32_t *const wrel = GATHER ? rel + off : nullptr;
    auto vrow = [&](int r) -> int64_t { return GATHER ? vrow0 + wrel[r] : off + r; };

    // Query row of this lane (B operand of S^T = K Q^T): 8 dims per k-step.
    // Its tensor row (video rows: through the ids table) also addresses the
    // output store.
    bf16x8 Qr[S_::KSTEPS];
    const int qrow = qt * kBM + wave * 32 + l32;
    int64_t qtrow;
    {
        const int r = min(qrow, M - 1);
        const bool vid = r < Lw;
        qtrow = vid ? vrow(min(r, Lw - 1)) : int64_t(r - Lw);
        const uint16_t *p = (vid ? q : tq) + qtrow * rs + hd;
#pragma unroll
        for (int s = 0; s < S_::KSTEPS; ++s)
            Qr[s] = *reinterpret_cast<const bf16x8 *>(p + 16 * s + 8 * hh);
    }

    // DMA of one K/V tile.  Wave `wave` moves rows wave*16 + ROWS_PER_LOAD*i
    // + lane/CH (i < LOADS); lane's 16 bytes land at LDS chunk lane%CH of its
    // row and come from the row's chunk (lane%CH) ^ swz(row).
    const int drow0 = wave * (kBN / kWaves) + lane / S_::CH;
    const int dpc = lane % S_::CH;
    int dchunk[S_::LOADS];
#pragma unroll
    for (int i = 0; i < S_::LOADS; ++i) dchunk[i] = 8 * (dpc ^ swz<D>(drow0 + S_::ROWS_PER_LOAD * i));
    // Every DMA is a buffer load (MUBUF): the global/flat DMA forms would
    // make the compiler wait for all outstanding LDS reads (lgkmcnt(0)) while
    // a DMA is in flight.  Video rows come through resources based at the
    // window's first row (gather mode: its smallest canonical row, the first
    // in row-major order), text rows through resources based at the text
    // tensors; the host checks that every offset fits 31 bits.  Tiles made
    // only of video rows (layout order) keep a loop-invariant per-lane offset
    // and put the tile step in the scalar offset; other tiles load row by row
    // with rows past the joint sequence clamped to its last row.  A
    // resource's byte range also bounds every access.
    const uint32_t row_bytes = uint32_t(rs) * 2u;
    // (The window's row range comes with the work item, in scalar
    // registers: a resource held in vector registers would turn every DMA
    // into a loop over lanes.)
    const uint32_t vrows = uint32_t(it.vrows);
    auto rsrc = [&](const uint16_t *base, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0, int(bytes), kBufferFlags);
    };
    const __amdgpu_buffer_rsrc_t krs = rsrc(k + vrow0 * rs + hd, vrows * row_bytes);
    const __amdgpu_buffer_rsrc_t vrs = rsrc(v + vrow0 * rs + hd, vrows * row_bytes);
    const __amdgpu_buffer_rsrc_t tkrs = rsrc(tk + hd, uint32_t(Lt) * row_bytes);
    const __amdgpu_buffer_rsrc_t tvrs = rsrc(tv + hd, uint32_t(Lt) * row_bytes);
    int dvoff[S_::LOADS];
#pragma unroll
    for (int i = 0; i < S_::LOADS; ++i)
        dvoff[i] = (drow0 + S_::ROWS_PER_LOAD * i) * int(row_bytes) + 2 * dchunk[i];
    // Gather mode: relative ids of the rows of the next tile to move, loaded
    // one tile ahead of their DMA by buffer loads whose per-lane offset holds
    // the row (the range check covers it: rows past the window read 0, and
    // such rows only reach the DMA as masked keys).  Two register sets
    // alternate: the next tile's ids are requested before the current tile's
    // DMA, so the tile's closing vmcnt wait does not end on them.  The DMA
    // offset is one 24-bit multiply-add, exact because the host's limits keep
    // row_bytes and the relative ids below 2^24 and every offset below 2^31.
    const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t *>(GATHER ? wrel : rel), 0, GATHER ? 4 * Lw : 0, kBufferFlags);
    int idA[S_::LOADS], idB[S_::LOADS];
    auto load_ids = [&](int (&idp)[S_::LOADS], int j) {
#pragma unroll
        for (int i = 0; i < S_::LOADS; ++i)
            idp[i] = __builtin_amdgcn_raw_buffer_load_b32(irs, 4 * (j * kBN + drow0 + S_::ROWS_PER_LOAD * i),
                                                          0, 0);
    };
    auto dma = [&](uint8_t LDS_AS *dst, int j, int (&idp)[S_::LOADS], int (&idn)[S_::LOADS]) {
        if constexpr (GATHER) load_ids(idn, j + 1);
        if (!GATHER && (j + 1) * kBN <= Lw) {
            const int soff = j * kBN * int(row_bytes);
#pragma unroll
            for (int i = 0; i < S_::LOADS; ++i) {
                const int lo = (wave * (kBN / kWaves) + S_::ROWS_PER_LOAD * i) * S_::ROW;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + lo), 16, dvoff[i], soff, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + S_::TILE + lo), 16, dvoff[i],
                                                         soff, 0, 0);
            }
        } else if (GATHER && (j + 1) * kBN <= Lw) {
#pragma unroll
            for (int i = 0; i < S_::LOADS; ++i) {
                const int lo = (wave * (kBN / kWaves) + S_::ROWS_PER_LOAD * i) * S_::ROW;
                const int o = int(__umul24(uint32_t(idp[i]), row_bytes)) + 2 * dchunk[i];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + lo), 16, o, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + S_::TILE + lo), 16, o, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < S_::LOADS; ++i) {
                const int r = min(j * kBN + drow0 + S_::ROWS_PER_LOAD * i, M - 1);
                const int lo = (wave * (kBN / kWaves) + S_::ROWS_PER_LOAD * i) * S_::ROW;
                if (r < Lw) {
                    const int o = (GATHER ? int(__umul24(uint32_t(idp[i]), row_bytes)) : r * int(row_bytes)) +
                                  2 * dchunk[i];
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + lo), 16, o, 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + S_::TILE + lo), 16, o, 0,
                                                             0, 0);
                } else {
                    const int o = (r - Lw) * int(row_bytes) + 2 * dchunk[i];
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(tkrs, (void LDS_AS *)(dst + lo), 16, o, 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(tvrs, (void LDS_AS *)(dst + S_::TILE + lo), 16, o, 0,
                                                             0, 0);
                    // Keeps the compiler from merging the two arms into one
                    // load with a per-lane resource (issued as a loop over
                    // lanes).
                    asm volatile("");
                }
            }
        }
    };

    // LDS byte offsets of this lane's operands inside a stage.
    //  K (A of S^T): row 32*mk + l32, logical chunk 2s + hh.
    int kaddr[S_::KSTEPS];
#pragma unroll
    for (int s = 0; s < S_::KSTEPS; ++s)
        kaddr[s] = l32 * S_::ROW + 16 * ((2 * s + hh) ^ swz<D>(l32));
    //  V^T (A of O^T) by transpose reads: for O^T block t and half B of a
    //  16-key k-step, lane i = lane%16 of 16-lane group g reads 8 bytes of
    //  row 16*cs + 8*B + 4*hh + i/4, dims 32t + 16*(g%2) + 4*(i%4) .. +3;
    //  the transpose hands lane l dim 32t + l%32 of those four rows.
    const int gi = lane & 15, ghalf = (lane >> 4) & 1;
    int vaddr[S_::DT][2];
#pragma unroll
    for (int t = 0; t < S_::DT; ++t)
#pragma unroll
        for (int B = 0; B < 2; ++B) {
            const int row = 8 * B + 4 * hh + (gi >> 2);
            const int dim = 32 * t + 16 * ghalf + 4 * (gi & 3);
            vaddr[t][B] = S_::TILE + row * S_::ROW + 16 * ((dim >> 3) ^ swz<D>(row)) + 2 * (dim & 7);
        }

    f32x16 O[S_::DT];
#pragma unroll
    for (int t = 0; t < S_::DT; ++t) O[t] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    const int ntiles = (M + kBN - 1) / kBN;

    // One tile: cur holds tile j; the DMA of tile j+1 goes to nxt.
    // A wave whose 32 query rows all lie past the joint sequence (the last
    // query tile of a window) only moves its share of the K/V tiles and
    // meets the barriers: the SIMD it shares then runs the other wave alone.
    const bool active = qt * kBM + wave * 32 < M;
    auto tile = [&](const uint8_t LDS_AS *cur, uint8_t LDS_AS *nxt, int j, int (&idu)[S_::LOADS],
                    int (&idn)[S_::LOADS]) {
        if (j + 1 < ntiles) dma(nxt, j + 1, idu, idn);
        if (active) {

        // S^T for 64 keys (two 32-key blocks) x this wave's 32 queries.  The
        // K operands of k-step s+2 are read while step s multiplies.
        f32x16 S[2] = {f32x16{}, f32x16{}};
        bf16x8 ka[S_::KSTEPS][2];
        auto kread = [&](int s) {
#pragma unroll
            for (int mk = 0; mk < 2; ++mk)
                ka[s][mk] = *reinterpret_cast<const bf16x8 LDS_AS *>(cur + kaddr[s] + mk * 32 * S_::ROW);
        };
        kread(0);
        kread(1);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int s = 0; s < S_::KSTEPS; ++s) {
#pragma unroll
            for (int mk = 0; mk < 2; ++mk) S[mk] = mfma(ka[s][mk], Qr[s], S[mk]);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (s + 2 < S_::KSTEPS) {
                kread(s + 2);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
        }
        if ((j + 1) * kBN > M) {  // keys past the end of the joint sequence
            // element r of S[mk] is key 32mk + 8(r/4) + (r%4) of the tile
            // counted from this lane's first, j*kBN + 4hh
            const int lim = M - j * kBN - 4 * hh;
#pragma unroll
            for (int mk = 0; mk < 2; ++mk)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * mk + 8 * (r >> 2) + (r & 3) >= lim) S[mk][r] = -INFINITY;
        }

        // p = 2^(s*c2 - m_run*c2) packed to bf16 pairs (P^T B operands, one
        // per 16-key k-step); the row sum adds the same rounded values.
        bf16x8 P[4];
        auto probs = [&]() {
            const float mc = m_run * c2;
            float sum = 0.f;
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
                const int mk = cs >> 1, r0 = 8 * (cs & 1);
                u32x4 pk;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(S[mk][r0 + 2 * i], c2, -mc));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(S[mk][r0 + 2 * i + 1], c2, -mc));
                    const bf16x2 pp = to_bf16x2(p0, p1);
                    sum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, sum, false);
                    pk[i] = __builtin_bit_cast(uint32_t, pp);
                }
                P[cs] = __builtin_bit_cast(bf16x8, pk);
            }
            return sum;
        };
        // Only on the first tile (m_run = -inf) and when some probability
        // would exceed 2^20 does the wave take the exact path: tile maximum,
        // rescale of O and l by 2^((m_old - m_new)*c2), recompute.  The first
        // tile goes there directly.
        // V^T operands (transpose reads) of one 16-key step; those of the
        // first step are read while the softmax runs.
        auto vread = [&](int cs, bf16x8 (&dst)[S_::DT]) {
#pragma unroll
            for (int t = 0; t < S_::DT; ++t) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 LDS_AS *)(cur + vaddr[t][0] + cs * 16 * S_::ROW));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 LDS_AS *)(cur + vaddr[t][1] + cs * 16 * S_::ROW));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                dst[t] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
            }
        };
        bf16x8 va[2][S_::DT];
        vread(0, va[0]);
        float tsum = j == 0 ? 0.f : probs();
        if (j == 0 || __builtin_amdgcn_ballot_w64(!(tsum <= kMaxTileSum))) {
            float m = S[0][0];
#pragma unroll
            for (int mk = 0; mk < 2; ++mk)
#pragma unroll
                for (int r = 0; r < 16; ++r) m = fmaxf(m, S[mk][r]);
            const float m_new = fmaxf(m_run, halves_max(m));
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
            m_run = m_new;
            if (j != 0) {  // on the first tile O and l are still zero
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < S_::DT; ++t) O[t] *= alpha;
            }
            tsum = probs();
        }
        l_run += tsum;

        // O^T += V^T P^T over the tile's four 16-key k-steps, the operands
        // of step cs+1 read while step cs multiplies.
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) {
            if (cs + 1 < 4) vread(cs + 1, va[(cs + 1) & 1]);
#pragma unroll
            for (int t = 0; t < S_::DT; ++t) O[t] = mfma(va[cs & 1][t], P[cs], O[t]);
        }
        }
        // The DMA of tile j+1 has landed (vmcnt) and every wave is done with
        // `cur` before it is overwritten two tiles later.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    };

    uint8_t LDS_AS *const st0 = (uint8_t LDS_AS *)stage0;
    uint8_t LDS_AS *const st1 = (uint8_t LDS_AS *)stage1;
    if constexpr (GATHER) load_ids(idA, 0);
    dma(st0, 0, idA, idB);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int j = 0; j < ntiles; j += 2) {
        tile(st0, st1, j, idB, idA);
        if (j + 1 < ntiles) tile(st1, st0, j + 1, idA, idB);
    }

    // Normalise and store: lane holds query qrow, dims 32t + 8g + 4hh + 0..3.
    const float l = halves_sum(l_run);
    if (qrow >= M) return;
    const float inv = 1.0f / l;
    if (qrow < Lw) {
        uint16_t *dst = out + qtrow * rs + hd;
#pragma unroll
        for (int t = 0; t < S_::DT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 st;
                st[0] = pack_bf16(O[t][4 * g] * inv, O[t][4 * g + 1] * inv);
                st[1] = pack_bf16(O[t][4 * g + 2] * inv, O[t][4 * g + 3] * inv);
                *reinterpret_cast<u32x2 *>(dst + 32 * t + 8 * g + 4 * hh) = st;
            }
    } else {
        float *dst = ws + ((int64_t(w) * Lt + (qrow - Lw)) * H + h) * D;
#pragma unroll
        for (int t = 0; t < S_::DT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<f32x4 *>(dst + 32 * t + 8 * g + 4 * hh) =
                    f32x4{O[t][4 * g] * inv, O[t][4 * g + 1] * inv, O[t][4 * g + 2] * inv,
                          O[t][4 * g + 3] * inv};
    }
#endif
}

}  // namespace

int attn_bf16_tile_m(bool small) { return 32 * (small ? kSmallItemWaves : kItemWaves); }

hipError_t launch_attn_bf16(int head_dim, bool small, const void *q, const void *k, const void *v,
                            const void *tq, const void *tk, const void *tv, void *out,
                            float *ws, const int32_t *rel, const ItemDesc *items, int n_items,
                            int n_heads, int text_len, float scale, hipStream_t s) {
    if (n_items <= 0) return hipSuccess;
    const float c2 = scale * kLog2e;
    auto U = [](const void *p) { return static_cast<const uint16_t *>(p); };
    auto launch = [&](auto kern, int waves) {
        kern<<<dim3(n_items), dim3(64 * waves), 0, s>>>(U(q), U(k), U(v), U(tq), U(tk), U(tv),
                                                         static_cast<uint16_t *>(out), ws, rel, items, n_heads,
                                                         text_len, c2);
    };
    auto dispatch = [&](auto waves_c) {
        constexpr int NW = decltype(waves_c)::value;
        const bool g = rel != nullptr;
        if (head_dim == 128)
            g ? launch(attn_bf16_kernel<128, NW, true>, NW) : launch(attn_bf16_kernel<128, NW, false>, NW);
        else if (head_dim == 64)
            g ? launch(attn_bf16_kernel<64, NW, true>, NW) : launch(attn_bf16_kernel<64, NW, false>, NW);
        else
            return hipErrorInvalidValue;
        return hipSuccess;
    };
    const hipError_t e = small ? dispatch(std::integral_constant<int, kSmallItemWaves>{})
                               : dispatch(std::integral_constant<int, kItemWaves>{});
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace wsp
