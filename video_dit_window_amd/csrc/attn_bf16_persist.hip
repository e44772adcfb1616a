// bfloat16 window joint attention on gfx950 matrix cores, persistent form.
//
// Computes exactly what attn_bf16.hip computes ("Window-Aligned Sequence
// Parallelism (SeedVR2)", sections "SeedVR2 integration" and "Text stream";
// "Parallelize new models with USP (text replica)", section "3. Attention
// with USP": plain SDPA over [video window; text], scale 1/sqrt(D) unless
// given), with the same per-tile arithmetic and order, so results are
// bit-identical to it.  What differs is the schedule around the tiles:
//
// * One work group per compute unit stays resident for the whole launch and
//   walks its own host-built list of work items (window, head, 256 query
//   rows).  The lists come from the largest-first order: every (window,
//   head) group goes whole to one XCD (work group b runs on XCD b % 8) and
//   each of its query tiles to the least-loaded work group of that XCD, so
//   the tiles that stream the same K/V run side by side behind one L2.
// * The K/V tile stream never drains between items: the DMA issued during
//   an item's last key tile already fetches the first tile of the next item,
//   and the next item's query rows (and, with canonical-order I/O, the row
//   ids the next DMAs need) are loaded during that last tile too.  A fresh
//   work group per item instead waits for its queries and its first K/V tile
//   with the compute unit idle.
// * The masked tile (keys past the end of the joint sequence) is always an
//   item's last tile, so the steady loop carries no masking code.
//
// Per 64-key tile and wavefront (32 query rows), as in attn_bf16.hip:
// S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS, Q in registers), an
// online softmax in float32 whose running maximum moves only when a tile's
// probabilities would exceed 2^20, and O^T += V^T P^T with P kept as bf16
// operands and V^T read through the LDS transpose read.  K/V tiles move by
// direct buffer-load DMA into two LDS stages with XOR-swizzled 16-byte
// chunks.

#include <type_traits>

#include "attn_bf16_common.h"

namespace wsp {

namespace {

constexpr int kPkWaves = 8;
constexpr int kMid = 0, kPen = 1, kFin = 2;  // tile kinds, see `tile`
template <int K>
using KindC = std::integral_constant<int, K>;
constexpr int kPkBM = 32 * kPkWaves;  // query rows per work item

// One work item, wave-uniform.  np: its 64-key tiles rounded up to an even
// count (an extra tile is wholly past the end: no arithmetic, only the DMA
// slot), so that every item starts in the same LDS stage.  vrow0 / vrows:
// first tensor row and row count
// of the buffer resource the item's video K/V rows are read through (layout
// order: the window's rows; canonical order: the span from the window's
// smallest to its largest canonical id).
struct PkItem {
    int w, h, qt, Lw, M, np;
    int64_t off, hd, vrow0;
    uint32_t vrows;
    bool valid;
};

template <int D, bool GATHER>
__global__ __launch_bounds__(64 * kPkWaves, 2) void attn_bf16_persist_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ tq,
    const uint16_t *__restrict__ tk, const uint16_t *__restrict__ tv,
    uint16_t *__restrict__ out, float *__restrict__ ws, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ ids, const int32_t *__restrict__ rel, const Item *__restrict__ items,
    int rounds, int H, int Lt,
    float c2) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer resources exist only in the device pass
    using S_ = Shape<D, kPkWaves>;
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[2 * S_::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[2 * S_::TILE];
    // Query rows of the next item, moved in by DMA during the current item's
    // last tile; wave w's 32 rows at rows 32w.., chunks swizzled like K rows.
    __shared__ __attribute__((aligned(1024))) uint8_t qbuf[kPkBM * S_::ROW];

    const int G = int(gridDim.x), b = int(blockIdx.x);
    const int64_t rs = int64_t(H) * D;
    const uint32_t row_bytes = uint32_t(rs) * 2u;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;

    // Item r of this work group's list; lists end with x < 0 or at `rounds`.
    auto load_item = [&](int r) {
        PkItem t{};
        t.valid = false;
        if (r >= rounds) return t;
        const Item e = items[int64_t(r) * G + b];
        if (e.x < 0) return t;
        t.valid = true;
        t.w = e.x;
        t.h = e.y >> 16;
        t.qt = e.y & 0xFFFF;
        t.off = offsets[t.w];
        t.Lw = offsets[t.w + 1] - int(t.off);
        t.M = t.Lw + Lt;
        t.np = 2 * ((t.M + 2 * kBN - 1) / (2 * kBN));
        t.hd = int64_t(t.h) * D;
        if constexpr (GATHER) {
            const int32_t first = ids[t.off], last = ids[t.off + t.Lw - 1];
            t.vrow0 = first;
            t.vrows = uint32_t(last - first + 1);
        } else {
            t.vrow0 = t.off;
            t.vrows = uint32_t(t.Lw);
        }
        return t;
    };

    // DMA lane geometry: wave `wave` moves rows wave*8 + ROWS_PER_LOAD*i +
    // lane/CH (i < LOADS) of a tile; lane's 16 bytes land at LDS chunk
    // lane%CH of its row and come from the row's chunk (lane%CH) ^ swz(row).
    const int drow0 = wave * (kBN / kPkWaves) + lane / S_::CH;
    const int dpc = lane % S_::CH;
    int dchunk[S_::LOADS], dvoff[S_::LOADS];
#pragma unroll
    for (int i = 0; i < S_::LOADS; ++i) {
        dchunk[i] = 8 * (dpc ^ swz<D>(drow0 + S_::ROWS_PER_LOAD * i));
        dvoff[i] = (drow0 + S_::ROWS_PER_LOAD * i) * int(row_bytes) + 2 * dchunk[i];
    }
    auto rsrc = [&](const uint16_t *base, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0, int(bytes), kBufferFlags);
    };
    // Canonical-order I/O: ids, relative to the item's smallest id, of the
    // rows the next DMA moves, loaded one DMA ahead (idp_ok false: not
    // loaded, fetch at the DMA) by buffer loads over the window's entries
    // (rows past the window read 0 and reach the DMA only as masked keys).
    // A row's DMA offset is then one 24-bit multiply-add, exact because the
    // host's limits keep row_bytes and the relative ids below 2^24.
    int idp[S_::LOADS];
    bool idp_ok = false;
    auto rel_rsrc = [&](const PkItem &t) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(rel + t.off), 0, 4 * t.Lw, kBufferFlags);
    };
    auto load_ids = [&](const PkItem &t, int j) {
        const __amdgpu_buffer_rsrc_t irs = rel_rsrc(t);
#pragma unroll
        for (int i = 0; i < S_::LOADS; ++i)
            idp[i] = __builtin_amdgcn_raw_buffer_load_b32(irs, 4 * (j * kBN + drow0 + S_::ROWS_PER_LOAD * i), 0, 0);
        idp_ok = true;
    };
    // Tile j of item t into dst (K tile, then V tile).  Every DMA is a buffer
    // load: video rows through resources based at the item's first video row,
    // text rows through resources based at the text tensors; the host checks
    // that every offset fits 31 bits.  Tiles of video rows only (layout order)
    // keep the loop-invariant lane offsets and put the tile step in the scalar
    // offset; other tiles go row by row, rows past the joint sequence clamped
    // to its last row.
    auto dma = [&](uint8_t LDS_AS *dst, const PkItem &t, int j) {
        const __amdgpu_buffer_rsrc_t krs = rsrc(k + t.vrow0 * rs + t.hd, t.vrows * row_bytes);
        const __amdgpu_buffer_rsrc_t vrs = rsrc(v + t.vrow0 * rs + t.hd, t.vrows * row_bytes);
        if constexpr (GATHER) {
            if (!idp_ok) load_ids(t, j);
        }
        if (!GATHER && (j + 1) * kBN <= t.Lw) {
            const int soff = j * kBN * int(row_bytes);
#pragma unroll
            for (int i = 0; i < S_::LOADS; ++i) {
                const int lo = (wave * (kBN / kPkWaves) + S_::ROWS_PER_LOAD * i) * S_::ROW;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + lo), 16, dvoff[i], soff, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + S_::TILE + lo), 16, dvoff[i],
                                                         soff, 0, 0);
            }
        } else if (GATHER && (j + 1) * kBN <= t.Lw) {
#pragma unroll
            for (int i = 0; i < S_::LOADS; ++i) {
                const int lo = (wave * (kBN / kPkWaves) + S_::ROWS_PER_LOAD * i) * S_::ROW;
                const int o = int(__umul24(uint32_t(idp[i]), row_bytes)) + 2 * dchunk[i];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + lo), 16, o, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + S_::TILE + lo), 16, o, 0, 0, 0);
            }
        } else {
            const __amdgpu_buffer_rsrc_t tkrs = rsrc(tk + t.hd, uint32_t(Lt) * row_bytes);
            const __amdgpu_buffer_rsrc_t tvrs = rsrc(tv + t.hd, uint32_t(Lt) * row_bytes);
#pragma unroll
            for (int i = 0; i < S_::LOADS; ++i) {
                const int r = min(j * kBN + drow0 + S_::ROWS_PER_LOAD * i, t.M - 1);
                const int lo = (wave * (kBN / kPkWaves) + S_::ROWS_PER_LOAD * i) * S_::ROW;
                if (r < t.Lw) {
                    const int o = (GATHER ? int(__umul24(uint32_t(idp[i]), row_bytes)) : r * int(row_bytes)) +
                                  2 * dchunk[i];
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + lo), 16, o, 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + S_::TILE + lo), 16, o, 0,
                                                             0, 0);
                } else {
                    const int o = (r - t.Lw) * int(row_bytes) + 2 * dchunk[i];
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(tkrs, (void LDS_AS *)(dst + lo), 16, o, 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(tvrs, (void LDS_AS *)(dst + S_::TILE + lo), 16, o, 0,
                                                             0, 0);
                    // Keeps the two arms as two loads (a merged load with a
                    // per-lane resource would be issued lane by lane).
                    asm volatile("");
                }
            }
        }
        idp_ok = false;
    };

    // Query rows.  Lane (l32, hh) of wave `wave` owns joint row q_row(t) of
    // item t (B operand of S^T = K Q^T).  The DMA moves the wave's 32 rows:
    // instruction i, lane l -> row ROWS_PER_LOAD*i + l/CH of the wave's block,
    // LDS chunk l%CH holding the row's chunk (l%CH) ^ swz(row); video rows
    // come from q (canonical order: through the ids, fetched ahead into
    // qid[]), text rows from tq, rows past the joint sequence repeat its last.
    constexpr int QLOADS = 32 / S_::ROWS_PER_LOAD;
    auto q_row = [&](const PkItem &t) { return t.qt * kPkBM + wave * 32 + l32; };
    int qid[QLOADS];
    auto load_qids = [&](const PkItem &t) {
        const __amdgpu_buffer_rsrc_t irs = rel_rsrc(t);
#pragma unroll
        for (int i = 0; i < QLOADS; ++i)
            qid[i] = __builtin_amdgcn_raw_buffer_load_b32(
                irs, 4 * (t.qt * kPkBM + wave * 32 + S_::ROWS_PER_LOAD * i + lane / S_::CH), 0, 0);
    };
    auto q_dma = [&](const PkItem &t) {
        const __amdgpu_buffer_rsrc_t qrs = rsrc(q + t.vrow0 * rs + t.hd, t.vrows * row_bytes);
        const __amdgpu_buffer_rsrc_t tqrs = rsrc(tq + t.hd, uint32_t(Lt) * row_bytes);
#pragma unroll
        for (int i = 0; i < QLOADS; ++i) {
            const int rr = S_::ROWS_PER_LOAD * i + lane / S_::CH;  // row within the wave's block
            const int r = min(t.qt * kPkBM + wave * 32 + rr, t.M - 1);
            const int chunk = 16 * (dpc ^ swz<D>(rr));
            uint8_t LDS_AS *dst = (uint8_t LDS_AS *)qbuf + (wave * 32 + S_::ROWS_PER_LOAD * i) * S_::ROW;
            if (r < t.Lw) {
                const int o = (GATHER ? int(__umul24(uint32_t(qid[i]), row_bytes)) : r * int(row_bytes)) + chunk;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (void LDS_AS *)dst, 16, o, 0, 0, 0);
            } else {
                const int o = (r - t.Lw) * int(row_bytes) + chunk;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(tqrs, (void LDS_AS *)dst, 16, o, 0, 0, 0);
                asm volatile("");
            }
        }
    };
    // Reads this lane's query operands from qbuf (after the DMA has landed)
    // and waits for them, so that qbuf may be refilled afterwards.
    bf16x8 Qr[S_::KSTEPS];
    auto read_q = [&]() {
        const uint8_t LDS_AS *qb = (const uint8_t LDS_AS *)qbuf + (wave * 32 + l32) * S_::ROW;
#pragma unroll
        for (int s2 = 0; s2 < S_::KSTEPS; ++s2)
            Qr[s2] = *reinterpret_cast<const bf16x8 LDS_AS *>(qb + 16 * ((2 * s2 + hh) ^ swz<D>(l32)));
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    };
    // Tensor row of this lane's query (video rows; -1 for text rows).
    auto q_tensor_row = [&](const PkItem &t) -> int64_t {
        const int r = min(q_row(t), t.M - 1);
        if (r >= t.Lw) return -1;
        return GATHER ? int64_t(ids[t.off + r]) : t.off + r;
    };

    // LDS byte offsets of this lane's operands inside a stage.
    //  K (A of S^T): row 32*mk + l32, logical chunk 2s + hh.
    int kaddr[S_::KSTEPS];
#pragma unroll
    for (int s = 0; s < S_::KSTEPS; ++s) kaddr[s] = l32 * S_::ROW + 16 * ((2 * s + hh) ^ swz<D>(l32));
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

    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    f32x16 O[S_::DT];
    float m_run, l_run;

    PkItem cur = load_item(0);
    if (!cur.valid) return;
    PkItem nxt = load_item(1);
    int64_t qtrow = q_tensor_row(cur);
    int64_t qtrow_n = nxt.valid ? q_tensor_row(nxt) : -1;

    // One key tile j of item `cur` from stage `cs_`; the DMA of the next tile
    // of the stream (tile j+1 of cur, or tile 0 of nxt) goes to `ns_`.  KIND:
    // kMid (no key past the end), kPen (cur's second-to-last tile) or kFin
    // (cur's last tile: its DMA fetches the next item's first tile and query
    // rows; no arithmetic when it lies wholly past the end).
    auto tile = [&](const uint8_t LDS_AS *cs_, uint8_t LDS_AS *ns_, int j, auto kind_c) {
        constexpr int KIND = decltype(kind_c)::value;
        if constexpr (KIND != kFin) {
            dma(ns_, cur, j + 1);
            if constexpr (GATHER) {
                if (j + 2 < cur.np) load_ids(cur, j + 2);
                else if (nxt.valid) load_ids(nxt, 0);
            }
        } else if (nxt.valid) {
            dma(ns_, nxt, 0);
            if constexpr (GATHER) load_ids(nxt, 1);
            q_dma(nxt);
        }
        // Waves whose 32 query rows all lie past the joint sequence only move
        // their share of the tiles and meet the barriers.
        if ((KIND != kFin || j * kBN < cur.M) && cur.qt * kPkBM + wave * 32 < cur.M) {

        // S^T for 64 keys (two 32-key blocks) x this wave's 32 queries; the K
        // operands of k-step s+2 are read while step s multiplies.
        f32x16 S[2] = {f32x16{}, f32x16{}};
        bf16x8 ka[S_::KSTEPS][2];
        auto kread = [&](int s) {
#pragma unroll
            for (int mk = 0; mk < 2; ++mk)
                ka[s][mk] = *reinterpret_cast<const bf16x8 LDS_AS *>(cs_ + kaddr[s] + mk * 32 * S_::ROW);
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
        if constexpr (KIND != kMid) {
            if ((j + 1) * kBN > cur.M) {  // keys past the end of the joint sequence
                // element r of S[mk] is key 32mk + 8(r/4) + (r%4) of the tile
                // counted from this lane's first, j*kBN + 4hh
                const int lim = cur.M - j * kBN - 4 * hh;
#pragma unroll
                for (int mk = 0; mk < 2; ++mk)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (32 * mk + 8 * (r >> 2) + (r & 3) >= lim) S[mk][r] = -INFINITY;
            }
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
        auto vread = [&](int cs, bf16x8 (&dst)[S_::DT]) {
#pragma unroll
            for (int t = 0; t < S_::DT; ++t) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 LDS_AS *)(cs_ + vaddr[t][0] + cs * 16 * S_::ROW));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 LDS_AS *)(cs_ + vaddr[t][1] + cs * 16 * S_::ROW));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                dst[t] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
            }
        };
        bf16x8 va[2][S_::DT];
        vread(0, va[0]);
        // Only on an item's first tile (m_run = -inf; it goes there directly)
        // and when some probability would exceed 2^20 does the wave take the
        // exact path: tile maximum, rescale of O and l by
        // 2^((m_old - m_new)*c2), recompute.
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
            if (j != 0) {  // on an item's first tile O and l are still zero
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < S_::DT; ++t) O[t] *= alpha;
            }
            tsum = probs();
        }
        l_run += tsum;

        // O^T += V^T P^T over the tile's four 16-key k-steps, the operands of
        // step cs+1 read while step cs multiplies.
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) {
            if (cs + 1 < 4) vread(cs + 1, va[(cs + 1) & 1]);
#pragma unroll
            for (int t = 0; t < S_::DT; ++t) O[t] = mfma(va[cs & 1][t], P[cs], O[t]);
        }
        }
        // The DMA of the next tile has landed (vmcnt) and every wave is done
        // with this stage before it is refilled.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    };

    uint8_t LDS_AS *const st0 = (uint8_t LDS_AS *)stage0;
    uint8_t LDS_AS *const st1 = (uint8_t LDS_AS *)stage1;
    if constexpr (GATHER) load_qids(cur);
    q_dma(cur);
    dma(st0, cur, 0);
    if constexpr (GATHER) {
        load_ids(cur, 1);
        if (nxt.valid) load_qids(nxt);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // Every item starts in stage 0: np is even.
    for (int r = 0;;) {
        read_q();
#pragma unroll
        for (int t = 0; t < S_::DT; ++t) O[t] = f32x16{};
        m_run = -INFINITY;
        l_run = 0.f;
        int j = 0;
        for (; j + 2 < cur.np; j += 2) {
            tile(st0, st1, j, KindC<kMid>{});
            tile(st1, st0, j + 1, KindC<kMid>{});
        }
        tile(st0, st1, j, KindC<kPen>{});
        tile(st1, st0, j + 1, KindC<kFin>{});

        // Normalise and store: lane holds query q_row(cur), dims 32t + 8g +
        // 4hh + 0..3.
        const float l = halves_sum(l_run);
        const int qrow = q_row(cur);
        if (qrow < cur.M) {
            const float inv = 1.0f / l;
            if (qrow < cur.Lw) {
                uint16_t *dst = out + qtrow * rs + cur.hd;
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
                float *dst = ws + ((int64_t(cur.w) * Lt + (qrow - cur.Lw)) * H + cur.h) * D;
#pragma unroll
                for (int t = 0; t < S_::DT; ++t)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<f32x4 *>(dst + 32 * t + 8 * g + 4 * hh) =
                            f32x4{O[t][4 * g] * inv, O[t][4 * g + 1] * inv, O[t][4 * g + 2] * inv,
                                  O[t][4 * g + 3] * inv};
            }
        }
        if (!nxt.valid) break;
        ++r;
        cur = nxt;
        qtrow = qtrow_n;
        nxt = load_item(r + 1);
        qtrow_n = nxt.valid ? q_tensor_row(nxt) : -1;
        if constexpr (GATHER) {
            if (nxt.valid) load_qids(nxt);
        }
    }
#endif
}

}  // namespace

// Persistent launch: one work group per compute unit, `rounds` items each
// (items[r * n_groups + g], -1 padded).  Head dims 64 and 128.
hipError_t launch_attn_bf16_persist(int head_dim, const void *q, const void *k, const void *v,
                                    const void *tq, const void *tk, const void *tv, void *out,
                                    float *ws, const int32_t *offsets, const int32_t *ids,
                                    const int32_t *rel, const Item *items, int n_groups, int rounds,
                                    int n_heads, int text_len, float scale, hipStream_t s) {
    if (n_groups <= 0 || rounds <= 0) return hipSuccess;
    const float c2 = scale * kLog2e;
    auto U = [](const void *p) { return static_cast<const uint16_t *>(p); };
    auto launch = [&](auto kern) {
        kern<<<dim3(n_groups), dim3(64 * kPkWaves), 0, s>>>(U(q), U(k), U(v), U(tq), U(tk), U(tv),
                                                             static_cast<uint16_t *>(out), ws, offsets, ids,
                                                             rel, items, rounds, n_heads, text_len, c2);
    };
    const bool g = ids != nullptr;
    if (head_dim == 128) g ? launch(attn_bf16_persist_kernel<128, true>) : launch(attn_bf16_persist_kernel<128, false>);
    else if (head_dim == 64) g ? launch(attn_bf16_persist_kernel<64, true>) : launch(attn_bf16_persist_kernel<64, false>);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

int attn_bf16_persist_tile_m() { return kPkBM; }

}  // namespace wsp
