// Window joint attention with FP8 (OCP E4M3) queries and keys on gfx950.
//
// Same layer as attn_bf16.hip ("Window-Aligned Sequence Parallelism
// (SeedVR2)", sections "SeedVR2 integration" and "Text stream";
// "Parallelize new models with USP (text replica)", section "3. Attention
// with USP"), with the low-precision variant the page "Scaling Video Training
// with Parallelism" reports paying off in a neighbouring system: the scores
// S^T = K Q^T come from E4M3 codes (per-head scales, fp8.hip) through
// v_mfma_scale_f32_32x32x64_f8f6f4 -- four 32x32x64 products per 64-key tile
// instead of sixteen 32x32x16 -- and the K tiles move at one byte per
// element.  The softmax, P and V stay as in the bf16 kernel (float32 softmax,
// bf16 P and V, float32 accumulation), so the only new rounding is the
// quantisation of q and k; the dequantisation (amax_q/448)(amax_k/448) rides
// in the exponent scale.
//
// Layout: 8 wavefronts x 32 query rows per work group (one per CU).  A stage
// holds a K tile (64 rows x 128 bytes, 16-byte chunks XOR-swizzled by
// (row>>1)&7 so that the 32-row operand reads are bank-conflict free) and a
// V tile (64 rows x 256 bytes, swizzled as in attn_bf16.hip); two stages.
// Each K operand is 32 bytes per lane: key row 32*mk + l%32, bytes
// [64s + 32h, +32) of the head (h = l/32) -- the query operand uses the same
// byte map, so the product sums every dimension exactly once.

#include "attn_bf16_common.h"

namespace wsp {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kQ8Waves = 8;
constexpr int kQ8BM = 32 * kQ8Waves;   // query rows per work group
constexpr int kD = 128;
constexpr int kKRow = kD;              // bytes per fp8 K row
constexpr int kKTile = kBN * kKRow;    // 8 KiB
constexpr int kE8M0One = 127;          // E8M0 exponent of 1.0

__device__ __host__ constexpr int swz8(int r) { return (r >> 1) & 7; }

__device__ inline f32x16 mfma8(v8i a, v8i b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kE8M0One, 0, kE8M0One);
}

template <bool GATHER>
__global__ __launch_bounds__(64 * kQ8Waves, 1) void attn_qk8_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint8_t *__restrict__ tq, const uint8_t *__restrict__ tk, const uint16_t *__restrict__ tv,
    uint16_t *__restrict__ out, float *__restrict__ ws, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ ids, const Item *__restrict__ items, const float *__restrict__ amax_q,
    const float *__restrict__ amax_k, int H, int Lt, float c2_unit) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer resources exist only in the device pass
    using S_ = Shape<kD, kQ8Waves>;      // the V tile
    constexpr int kStage = kKTile + S_::TILE;
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStage];

    const Item it = items[blockIdx.x];
    if (it.x < 0) return;
    const int w = it.x, h = it.y >> 16, qt = it.y & 0xFFFF;
    const int64_t off = offsets[w];
    const int Lw = offsets[w + 1] - int(off);
    const int M = Lw + Lt;
    const int64_t rs = int64_t(H) * kD, hd = int64_t(h) * kD;  // elements = fp8 bytes
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;
    // Scores in log2 units: S * c2, S from the codes, c2 with both dequantisation factors.
    const float c2 = c2_unit * (amax_q[h] * (1.0f / 448.0f)) * (amax_k[h] * (1.0f / 448.0f));

    const int32_t *const wids = GATHER ? ids + off : nullptr;
    auto vrow = [&](int r) -> int64_t { return GATHER ? int64_t(wids[r]) : off + r; };

    // Query codes of this lane: bytes [64s + 32hh, +32) of its row.
    v8i Qr[2];
    const int qrow = qt * kQ8BM + wave * 32 + l32;
    {
        const int r = min(qrow, M - 1);
        const bool vid = r < Lw;
        const int64_t o = (vid ? vrow(min(r, Lw - 1)) : int64_t(r - Lw)) * rs + hd;
        const uint8_t *p = (vid ? q : tq) + o;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint4 a = *reinterpret_cast<const uint4 *>(p + 64 * s + 32 * hh);
            const uint4 b = *reinterpret_cast<const uint4 *>(p + 64 * s + 32 * hh + 16);
            Qr[s] = v8i{int(a.x), int(a.y), int(a.z), int(a.w), int(b.x), int(b.y), int(b.z), int(b.w)};
        }
    }

    // ---- DMA (buffer loads only; see attn_bf16.hip).  K: one instruction
    // per wave, rows wave*8 + lane/8, lane's 16 bytes to chunk lane%8 from
    // the row's chunk (lane%8) ^ swz8(row).  V: as attn_bf16.hip.
    const int krow_t = wave * 8 + lane / 8;                  // K row inside the tile
    const int kchunk = (lane & 7) ^ swz8(krow_t);
    const int drow0 = wave * (kBN / kQ8Waves) + lane / S_::CH;
    const int dpc = lane % S_::CH;
    int dchunk[S_::LOADS];
#pragma unroll
    for (int i = 0; i < S_::LOADS; ++i) dchunk[i] = 8 * (dpc ^ swz<kD>(drow0 + S_::ROWS_PER_LOAD * i));
    const uint32_t krow_bytes = uint32_t(rs), vrow_bytes = uint32_t(rs) * 2u;
    const int32_t id_first = GATHER ? __builtin_amdgcn_readfirstlane(wids[0]) : 0;
    const int32_t id_last = GATHER ? __builtin_amdgcn_readfirstlane(wids[Lw - 1]) : 0;
    const int64_t vrow0 = GATHER ? int64_t(id_first) : off;
    const uint32_t vrows = GATHER ? uint32_t(id_last - id_first + 1) : uint32_t(Lw);
    auto rsrc = [&](const void *base, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), kBufferFlags);
    };
    const __amdgpu_buffer_rsrc_t krs = rsrc(k + vrow0 * rs + hd, vrows * krow_bytes);
    const __amdgpu_buffer_rsrc_t vrs = rsrc(v + vrow0 * rs + hd, vrows * vrow_bytes);
    const __amdgpu_buffer_rsrc_t tkrs = rsrc(tk + hd, uint32_t(Lt) * krow_bytes);
    const __amdgpu_buffer_rsrc_t tvrs = rsrc(tv + hd, uint32_t(Lt) * vrow_bytes);
    const int kvoff = krow_t * int(krow_bytes) + 16 * kchunk;
    int dvoff[S_::LOADS];
#pragma unroll
    for (int i = 0; i < S_::LOADS; ++i)
        dvoff[i] = (drow0 + S_::ROWS_PER_LOAD * i) * int(vrow_bytes) + 2 * dchunk[i];
    int idp[S_::LOADS], idk = 0;
    auto load_ids = [&](int j) {
#pragma unroll
        for (int i = 0; i < S_::LOADS; ++i)
            idp[i] = wids[min(j * kBN + drow0 + S_::ROWS_PER_LOAD * i, Lw - 1)];
        idk = wids[min(j * kBN + krow_t, Lw - 1)];
    };
    auto dma = [&](uint8_t LDS_AS *dst, int j) {
        const int klo = wave * 8 * kKRow;
        if ((j + 1) * kBN <= Lw) {  // video rows only
            if constexpr (GATHER) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + klo), 16,
                                                         int(idk - vrow0) * int(krow_bytes) + 16 * kchunk, 0, 0, 0);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + klo), 16, kvoff,
                                                         j * kBN * int(krow_bytes), 0, 0);
            }
#pragma unroll
            for (int i = 0; i < S_::LOADS; ++i) {
                const int lo = kKTile + (wave * (kBN / kQ8Waves) + S_::ROWS_PER_LOAD * i) * S_::ROW;
                if constexpr (GATHER) {
                    const int o = int(idp[i] - vrow0) * int(vrow_bytes) + 2 * dchunk[i];
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + lo), 16, o, 0, 0, 0);
                } else {
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + lo), 16, dvoff[i],
                                                             j * kBN * int(vrow_bytes), 0, 0);
                }
            }
        } else {
            // Row by row, rows past the joint sequence clamped to its last row.
            {
                const int r = min(j * kBN + krow_t, M - 1);
                if (r < Lw) {
                    const int o = (GATHER ? int(idk - vrow0) : r) * int(krow_bytes) + 16 * kchunk;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (void LDS_AS *)(dst + klo), 16, o, 0, 0, 0);
                } else {
                    const int o = (r - Lw) * int(krow_bytes) + 16 * kchunk;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(tkrs, (void LDS_AS *)(dst + klo), 16, o, 0, 0, 0);
                    asm volatile("");  // keep the two arms apart (see attn_bf16.hip)
                }
            }
#pragma unroll
            for (int i = 0; i < S_::LOADS; ++i) {
                const int r = min(j * kBN + drow0 + S_::ROWS_PER_LOAD * i, M - 1);
                const int lo = kKTile + (wave * (kBN / kQ8Waves) + S_::ROWS_PER_LOAD * i) * S_::ROW;
                if (r < Lw) {
                    const int o = (GATHER ? int(idp[i] - vrow0) : r) * int(vrow_bytes) + 2 * dchunk[i];
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (void LDS_AS *)(dst + lo), 16, o, 0, 0, 0);
                } else {
                    const int o = (r - Lw) * int(vrow_bytes) + 2 * dchunk[i];
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(tvrs, (void LDS_AS *)(dst + lo), 16, o, 0, 0, 0);
                    asm volatile("");
                }
            }
        }
        if constexpr (GATHER) load_ids(j + 1);
    };

    // ---- LDS operand addresses inside a stage.
    //  K codes (A of S^T): row 32*mk + l32, logical chunks 4s + 2hh + e.
    int kaddr[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 2; ++e) kaddr[s][e] = l32 * kKRow + 16 * ((4 * s + 2 * hh + e) ^ swz8(l32));
    //  V^T (A of O^T) by transpose reads, as attn_bf16.hip.
    const int gi = lane & 15, ghalf = (lane >> 4) & 1;
    int vaddr[S_::DT][2];
#pragma unroll
    for (int t = 0; t < S_::DT; ++t)
#pragma unroll
        for (int B = 0; B < 2; ++B) {
            const int row = 8 * B + 4 * hh + (gi >> 2);
            const int dim = 32 * t + 16 * ghalf + 4 * (gi & 3);
            vaddr[t][B] = kKTile + row * S_::ROW + 16 * ((dim >> 3) ^ swz<kD>(row)) + 2 * (dim & 7);
        }

    f32x16 O[S_::DT];
#pragma unroll
    for (int t = 0; t < S_::DT; ++t) O[t] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    const int ntiles = (M + kBN - 1) / kBN;

    auto tile = [&](const uint8_t LDS_AS *cur, uint8_t LDS_AS *nxt, int j) {
        if (j + 1 < ntiles) dma(nxt, j + 1);

        // S^T for 64 keys x 32 queries: two key blocks x two 64-dim steps.
        v8i ka[2][2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int mk = 0; mk < 2; ++mk) {
                const uint8_t LDS_AS *base = cur + mk * 32 * kKRow;
                const u32x4 a = *reinterpret_cast<const u32x4 LDS_AS *>(base + kaddr[s][0]);
                const u32x4 b = *reinterpret_cast<const u32x4 LDS_AS *>(base + kaddr[s][1]);
                ka[s][mk] = v8i{int(a[0]), int(a[1]), int(a[2]), int(a[3]), int(b[0]), int(b[1]), int(b[2]), int(b[3])};
            }
        f32x16 S[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int mk = 0; mk < 2; ++mk) S[mk] = mfma8(ka[s][mk], Qr[s], S[mk]);
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

        // Softmax and O^T += V^T P^T exactly as attn_bf16.hip.
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
                    (s16x4 LDS_AS *)(cur + vaddr[t][0] + cs * 16 * S_::ROW));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 LDS_AS *)(cur + vaddr[t][1] + cs * 16 * S_::ROW));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                dst[t] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
            }
        };
        bf16x8 va[2][S_::DT];
        vread(0, va[0]);
        // The first tile (m_run = -inf) goes straight to the exact path.
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
#pragma unroll
        for (int cs = 0; cs < 4; ++cs) {
            if (cs + 1 < 4) vread(cs + 1, va[(cs + 1) & 1]);
#pragma unroll
            for (int t = 0; t < S_::DT; ++t) O[t] = mfma(va[cs & 1][t], P[cs], O[t]);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    };

    uint8_t LDS_AS *const st0 = (uint8_t LDS_AS *)stage0;
    uint8_t LDS_AS *const st1 = (uint8_t LDS_AS *)stage1;
    if constexpr (GATHER) load_ids(0);
    dma(st0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int j = 0; j < ntiles; j += 2) {
        tile(st0, st1, j);
        if (j + 1 < ntiles) tile(st1, st0, j + 1);
    }

    const float l = halves_sum(l_run);
    if (qrow >= M) return;
    const float inv = 1.0f / l;
    if (qrow < Lw) {
        uint16_t *dst = out + vrow(qrow) * rs + hd;
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
        float *dst = ws + ((int64_t(w) * Lt + (qrow - Lw)) * H + h) * kD;
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

int attn_qk8_tile_m() { return kQ8BM; }

hipError_t launch_attn_qk8(const void *q, const void *k, const void *v, const void *tq,
                           const void *tk, const void *tv, void *out, float *ws,
                           const int32_t *offsets, const int32_t *ids, const Item *items,
                           int n_items, const float *amax_q, const float *amax_k, int n_heads,
                           int text_len, float scale, hipStream_t s) {
    if (n_items <= 0) return hipSuccess;
    const float c2 = scale * kLog2e;
    auto B = [](const void *p) { return static_cast<const uint8_t *>(p); };
    auto U = [](const void *p) { return static_cast<const uint16_t *>(p); };
    auto launch = [&](auto kern) {
        kern<<<dim3(n_items), dim3(64 * kQ8Waves), 0, s>>>(B(q), B(k), U(v), B(tq), B(tk), U(tv),
                                                         static_cast<uint16_t *>(out), ws, offsets, ids,
                                                         items, amax_q, amax_k, n_heads, text_len, c2);
    };
    if (ids) launch(attn_qk8_kernel<true>);
    else launch(attn_qk8_kernel<false>);
    return hipGetLastError();
}

}  // namespace wsp
