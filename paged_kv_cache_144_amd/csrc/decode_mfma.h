// Paged decode attention on the matrix cores, for groups of G = 4 or 8 query heads per KV
// head (grouped-query attention) with fp16 / bf16 caches and 16-token blocks.
//
// It computes what decode_kernel computes (same work split, partials and merge records;
// "PagedAttention deep dive", donmain.dev, section on splitting the KV cache into blocks,
// for how tokens are found through the block table), but the two products of a block run
// as MFMAs instead of per-lane dot products:
//   * S^T = K Q^T with v_mfma_f32_16x16x32: the A operand is read straight from the tile
//     (lane l holds 8 consecutive elements of token row l % 16), the B operand is the G
//     query rows of the group, zero-padded to 16 and kept in registers for the segment;
//   * the accumulator layout of S^T (lane l: head l % 16, tokens 4 (l / 16) .. +3) is the A
//     operand layout of O = P V with v_mfma_f32_16x16x16, so the probabilities never leave
//     their lanes; each lane does the softmax work of its 4 tokens of one head only;
//   * V's B operand needs 4 consecutive tokens of one column per lane, so each V tile is
//     staged in the wavefront's own LDS rows and read back transposed;
//   * P is carried as hi + lo 16-bit parts (two MFMAs), as in the chunk-row kernel;
//   * masked tokens are removed by selection: their scores become -inf and their V rows
//     are zeroed before staging, so NaN in free or unused slots cannot reach the output.
#pragma once

#include "decode_impl.h"

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (DT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
    if constexpr (DT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                         __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

template <int D>
struct MfmaShape {
    static constexpr int KC = D / 32;             // 16x16x32 steps over d for S^T
    static constexpr int VB = D / 16;             // 16-column blocks of O
    static constexpr int NLD = kBlock * D * 2 / 1024;   // coalesced 1 KiB loads per V tile
    static constexpr int RS = D * 2 + 8;          // LDS bytes per staged V token row (padded)
    static constexpr int LDSW = kBlock * RS;      // LDS bytes per wavefront
};

template <int DT, int D, int G>
__global__ __launch_bounds__(kWavesPerGroup * kWave) void decode_mfma_kernel(DecodeArgs a) {
    static_assert(DT == DT_F16 || DT == DT_BF16, "16-bit caches");
    static_assert(G == 4 || G == 8, "groups of 4 or 8 query heads");
    using S = MfmaShape<D>;
    constexpr int KC = S::KC, VB = S::VB, NLD = S::NLD, RS = S::RS;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kNegBig = -3.402823466e38f;
    constexpr float kLazy = 8.f;
    __shared__ __align__(16) char lds[kWavesPerGroup * S::LDSW];

    int32_t* hdr = (int32_t*)(a.ws + a.lay.header);
    const uint32_t* cb = (const uint32_t*)(a.ws + a.lay.cb);
    const UnitInfo* unit = (const UnitInfo*)(a.ws + a.lay.unit);
    const uint32_t* wx0 = (const uint32_t*)(a.ws + a.lay.wave_x0);
    const int32_t* wu = (const int32_t*)(a.ws + a.lay.wave_u);
    float2* pml = (float2*)(a.ws + a.lay.part_ml);
    float* pacc = (float*)(a.ws + a.lay.part_acc);
    int4* tasks = (int4*)(a.ws + a.lay.tasks);
    const int32_t* empty = (const int32_t*)(a.ws + a.lay.empty);

    const int W = hdr[2], n_empty = hdr[3];
    const int wave = uniform(blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6));
    const int lane = lane_id();
    for (int i = wave; i < n_empty; i += gridDim.x * kWavesPerGroup) zero_row(a, empty[i], lane);
    if (wave >= W) return;

    const int c16 = lane % 16, q4 = lane / 16;
    char* my = lds + (threadIdx.x >> 6) * S::LDSW;
    const float qscale = a.scale * kLog2e;
    const size_t tile = (size_t)kBlock * D * 2;
    const size_t block_stride = (size_t)a.num_kv_heads * tile;
    // K: lane holds token c16, columns 32 c + 8 q4 .. +8 of each step c
    const char* kbase = (const char*)a.k_cache + (size_t)c16 * D * 2 + (size_t)q4 * 16;
    // V: coalesced; load i of lane l reads bytes 1024 i + 16 l of the tile
    const char* vbase = (const char*)a.v_cache + (size_t)lane * 16;

    const uint32_t x_start = wx0[wave];
    const uint32_t x_end = wx0[wave + 1];
    int uh = wu[wave];

    // A segment: the part of pair (u, g) inside this wavefront's share; blocks j0 .. j1-1
    // of the sequence's table row.
    struct Seg {
        int u, g, seq, len, lo_tok, j0, j1;
        uint32_t ps, pe, end;
        bool starts;     // the segment starts at the pair's first block
    };
    auto describe = [&](uint32_t xs) {
        while (cb[uh + 1] <= xs) ++uh;
        const UnitInfo ui = unit[uh];
        const uint32_t base = cb[uh];
        Seg sg;
        sg.u = uh;
        sg.g = (int)((xs - base) / (uint32_t)ui.nb);
        sg.ps = base + (uint32_t)sg.g * ui.nb;
        sg.pe = sg.ps + ui.nb;
        sg.end = x_end < sg.pe ? x_end : sg.pe;
        sg.starts = xs == sg.ps;
        sg.j0 = ui.b_lo + (int)(xs - sg.ps);
        sg.j1 = ui.b_lo + (int)(sg.end - sg.ps);
        sg.seq = ui.seq;
        sg.len = ui.len;
        sg.lo_tok = (a.window > 0 && ui.len > a.window) ? ui.len - a.window : 0;
        return sg;
    };
    // block ids c0 .. c0+63 of the segment, one per lane
    auto load_ids = [&](const Seg& sg, int c0) {
        const int n = sg.j1 - c0;
        return lane < n ? a.block_tables[(size_t)sg.seq * a.max_blocks + c0 + lane] : 0;
    };
    // B operand of S^T: query head c16 of the group (zero for c16 >= G), columns
    // 32 c + 8 q4 .. +8
    auto load_q = [&](const Seg& sg, u32x4 (&qb)[KC]) {
        const size_t qrow = ((size_t)sg.u * a.num_q_heads + (size_t)sg.g * G + c16) * D;
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < KC; ++c)
            qb[c] = c16 < G ? ld16((const char*)a.q + (qrow + 32 * c + 8 * q4) * 2) : z;
    };
    struct Tile { u32x4 k[KC], v[NLD]; };
    auto block_id = [&](int ids, int idx, bool& valid) {
        int b = __builtin_amdgcn_readlane(ids, idx);
        valid = (unsigned)b < (unsigned)a.num_blocks;
        return valid ? b : 0;
    };
    auto load_tile = [&](const Seg& sg, int b, Tile& t) {
        const size_t off = (size_t)b * block_stride + (size_t)sg.g * tile;
#pragma unroll
        for (int c = 0; c < KC; ++c) t.k[c] = ld16_stream(kbase + off + c * 64);
#pragma unroll
        for (int i = 0; i < NLD; ++i) t.v[i] = ld16_stream(vbase + off + i * 1024);
    };

    if (x_start >= x_end) return;
    Seg cur = describe(x_start);
    u32x4 qb[KC];
    load_q(cur, qb);
    int ids = load_ids(cur, cur.j0);
    Tile A, B;
    bool okA, okB;
    load_tile(cur, block_id(ids, 0, okA), A);
    bool first_segment = true;
    int bad = 0;

    for (;;) {
        // the next segment's record, queries and first block ids load while this one runs
        const bool more = cur.end < x_end;
        Seg nxt = cur;
        u32x4 qn[KC];
        int nids = 0;
        if (more) {
            nxt = describe(cur.end);
            load_q(nxt, qn);
            nids = load_ids(nxt, nxt.j0);
        }
        // a pair that starts here and continues past the share: the later shares' starts
        const bool opens_cut = cur.starts && cur.end < cur.pe;
        uint32_t next = cur.pe;
        if (opens_cut && wave + 1 + lane < W) next = wx0[wave + 1 + lane];

        f32x4 acc[VB];     // O: lane holds column 16 b + c16 of heads 4 q4 .. 4 q4 + 3
#pragma unroll
        for (int b = 0; b < VB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = kNegBig, lsum = 0.f;   // head c16, this lane's tokens
        const int len = cur.len, lo_tok = cur.lo_tok;

        auto consume = [&](Tile& tl, int j, bool valid) {
            const int t0 = j * kBlock;
            const bool edge = !valid || t0 < lo_tok || t0 + kBlock > len;   // uniform
            // stage V (rows of masked tokens zeroed) in this wavefront's LDS rows
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int byte = i * 1024 + lane * 16;
                const int tv = byte / (D * 2), col = byte % (D * 2);
                u32x4 v = tl.v[i];
                if (edge) {
                    const int t = t0 + tv;
                    const bool ok = valid && t >= lo_tok && t < len;
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    v = ok ? v : z;
                }
                char* dst = my + tv * RS + col;
                *reinterpret_cast<u32x2*>(dst) = u32x2{v.x, v.y};
                *reinterpret_cast<u32x2*>(dst + 8) = u32x2{v.z, v.w};
            }
            // S^T: lane holds head c16, tokens 4 q4 .. +3
            f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < KC; ++c) sacc = mfma_16x16x32<DT>(tl.k[c], qb[c], sacc);
            float sc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sc[r] = c16 < G ? sacc[r] * qscale : -INFINITY;
                if (edge) {
                    const int t = t0 + 4 * q4 + r;
                    const bool ok = valid && t >= lo_tok && t < len;
                    sc[r] = ok ? sc[r] : -INFINITY;
                }
            }
            // lazy rescaling, as in decode_kernel: m moves only by more than kLazy
            const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            if (__builtin_amdgcn_ballot_w64(mx > m + kLazy)) {
                float M = fmaxf(mx, __shfl_xor(mx, 16));
                M = fmaxf(M, __shfl_xor(M, 32));             // max over the head's 4 lanes
                const float mn = fmaxf(m, M);
                const float alpha = __builtin_amdgcn_exp2f(m - mn);
                m = mn;
                lsum *= alpha;
                // O rows are heads 4 q4 + r: their factor sits in lane 4 q4 + r
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = __shfl(alpha, 4 * q4 + r);
#pragma unroll
                    for (int b = 0; b < VB; ++b) acc[b][r] *= ar;
                }
            }
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[r] = __builtin_amdgcn_exp2f(sc[r] - m);
                lsum += p[r];
            }
            uint32_t h0, l0, h1, l1;
            split2<DT>(p[0], p[1], h0, l0);
            split2<DT>(p[2], p[3], h1, l1);
            const u32x2 ph = {h0, h1}, pl = {l0, l1};
            // O += P V: B operand = column 16 b + c16 of tokens 4 q4 .. +3, from LDS
            const uint16_t* vr = reinterpret_cast<const uint16_t*>(my + 4 * q4 * RS) + c16;
#pragma unroll
            for (int b = 0; b < VB; ++b) {
                const uint32_t e0 = vr[16 * b], e1 = vr[RS / 2 + 16 * b];
                const uint32_t e2 = vr[RS + 16 * b], e3 = vr[3 * RS / 2 + 16 * b];
                const u32x2 vb = {e0 | (e1 << 16), e2 | (e3 << 16)};
                acc[b] = mfma_16x16x16<DT>(ph, vb, acc[b]);
                acc[b] = mfma_16x16x16<DT>(pl, vb, acc[b]);
            }
        };

        // blocks of the segment, in chunks of 64 ids; A holds the segment's first block.
        // The load after each block's is the next block of the stream: in this chunk, the
        // next chunk, the next segment, or (at the very end) the last block again.
        int cids = ids;
        for (int c0 = cur.j0;; c0 += kWave) {
            const int n = (cur.j1 - c0) < kWave ? (cur.j1 - c0) : kWave;
            const bool last_chunk = c0 + kWave >= cur.j1;
            const int nc_ids = last_chunk ? 0 : load_ids(cur, c0 + kWave);
            auto next_block = [&](int k, bool& ok, const Seg*& sg) {
                sg = &cur;
                if (k < n) return block_id(cids, k, ok);
                if (!last_chunk) return block_id(nc_ids, 0, ok);
                if (more) {
                    sg = &nxt;
                    return block_id(nids, 0, ok);
                }
                return block_id(cids, n - 1, ok);
            };
            const Seg* sgB;
            const Seg* sgA;
            int jj = 0;
            for (;; jj += 2) {
                const int bB = next_block(jj + 1, okB, sgB);
                load_tile(*sgB, bB, B);
                bad |= !okA;
                consume(A, c0 + jj, okA);
                if (jj + 1 >= n) {
                    A = B;
                    okA = okB;
                    break;
                }
                const int bA = next_block(jj + 2, okA, sgA);
                load_tile(*sgA, bA, A);
                bad |= !okB;
                consume(B, c0 + jj + 1, okB);
                if (jj + 2 >= n) break;
            }
            if (last_chunk) break;
            cids = nc_ids;
        }

        // the head's sum over its 4 lanes; O-layout lanes fetch (m, l) of their heads
        float lt = lsum + __shfl_xor(lsum, 16);
        lt += __shfl_xor(lt, 32);
        const bool complete = cur.starts && cur.end == cur.pe;
        const int slot = first_segment ? 0 : 1;
        if (!complete && q4 == 0 && c16 < G) {
            const size_t pi = ((size_t)wave * 2 + slot) * G + c16;
            pml[pi] = make_float2(m, lt);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = 4 * q4 + r;
            const float lh = __shfl(lt, h);
            if (h < G) {
                if (complete) {
                    const float inv = lh > 0.f ? 1.f / lh : 0.f;
                    const size_t ob = ((size_t)cur.u * a.num_q_heads + (size_t)cur.g * G + h) * D + c16;
#pragma unroll
                    for (int b = 0; b < VB; ++b) store_out1(a, ob + 16 * b, acc[b][r] * inv);
                } else {
                    float* dst = pacc + (((size_t)wave * 2 + slot) * G + h) * D + c16;
#pragma unroll
                    for (int b = 0; b < VB; ++b) dst[16 * b] = acc[b][r];
                }
            }
        }
        if (opens_cut) {
            const int nc = pair_waves(wx0, W, wave, cur.pe, next, lane);
            if (lane == 0) tasks[wave + 1] = make_int4(cur.u, cur.g, nc, first_segment ? 0 : 1);
        }
        if (!more) break;
        cur = nxt;
#pragma unroll
        for (int c = 0; c < KC; ++c) qb[c] = qn[c];
        ids = nids;
        first_segment = false;
    }
    if (bad && lane == 0) atomicOr(hdr, kErrBlockId);
}

}  // namespace pa
