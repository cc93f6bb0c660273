// Paged decode attention on the matrix cores, for groups of G = 4 or 8 query heads per KV
// head (grouped-query attention) with 16-token blocks: fp16 / bf16 caches, and 8-bit caches
// with one fp16 scale per 32 values.
//
// It computes what decode_kernel computes (same work split, partials and merge records;
// "PagedAttention deep dive", donmain.dev, section on splitting the KV cache into blocks,
// for how tokens are found through the block table), but the two products of a block run
// as MFMAs instead of per-lane dot products.  The control flow (segments, prefetch,
// softmax, partials) is shared; how a tile becomes MFMA operands is a policy:
//
// 16-bit caches (MfmaKv16):
//   * S^T = K Q^T with v_mfma_f32_16x16x32: the A operand is read straight from the tile
//     (lane l holds 8 consecutive elements of token row l % 16), the B operand is the G
//     query rows of the group, zero-padded to 16 and kept in registers for the segment;
//   * the accumulator layout of S^T (lane l: head l % 16, tokens 4 (l / 16) .. +3) is the A
//     operand layout of O = P V with v_mfma_f32_16x16x16, so the probabilities never leave
//     their lanes; each lane does the softmax work of its 4 tokens of one head only;
//   * V's B operand needs 4 consecutive tokens of one column per lane, so each V tile is
//     staged in the wavefront's own LDS rows and read back transposed;
//   * P is carried as hi + lo 16-bit parts (two MFMAs), as in the chunk-row kernel.
//
// 8-bit caches (MfmaKvQ8; the format of "KV cache by model", sotaaz.com):
//   * a tile of 8-bit codes is half the bytes of a 16-bit one, so a tile holds two blocks
//     to keep as many bytes in flight per wavefront;
//   * K rows are loaded whole (each 16-byte piece of a lane lies in one row) and reach the
//     operand layout through LDS; the codes become exact fp16 integers (the flipped code
//     byte under the exponent of 1024 gives 1152 + code; the score MFMA's accumulator
//     starts at -1152 x the group's query sum, which removes the offset, or a packed
//     subtraction does where registers are short); the query is held
//     in fp16 after a power-of-two scaling per head (exact for fp16 and bf16 values), whose
//     inverse joins the softmax scale;
//   * each 16x16x32 step of S^T covers exactly one 32-column scale group, so every step
//     keeps its own accumulator and the per-(token, group) scales are applied to the four
//     partial scores of each lane before they are summed;
//   * O = P V runs on 16x16x16 bf16 MFMAs: V codes are exact in bf16 and are staged in LDS
//     as token pairs, so a lane's B operand (4 tokens of one column) is two dwords; the 16
//     columns of an MFMA lie in one scale group, so the V scales go into the A operand:
//     P x scale of the group, as hi + lo bf16 parts (16 significant bits, as for bf16
//     caches); the scale rows pass through LDS too, those of unseen tokens zeroed.
//
// Masked tokens are removed by selection in both: their scores become -inf and their V
// values zero (16-bit: rows zeroed before staging; 8-bit: scale zeroed), so NaN in free or
// unused slots cannot reach the output.
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

// ---- 16-bit caches ------------------------------------------------------------------
template <int DT, int D, int G>
struct MfmaKv16 {
    static constexpr int KC = D / 32;             // 16x16x32 steps over d for S^T
    static constexpr int NACC = D / 16;           // 16-column blocks of O
    static constexpr int NLD = kBlock * D * 2 / 1024;   // coalesced 1 KiB loads per V tile
    static constexpr int RS = D * 2 + 8;          // LDS bytes per staged V token row (padded)
    static constexpr int LDSW = kBlock * RS;      // LDS bytes per wavefront
    static constexpr int LDS_BYTES = kWavesPerGroup * LDSW;
    static constexpr size_t TILE = (size_t)kBlock * D * 2;
    static constexpr int BPT = 1;                 // blocks per tile
    static constexpr bool kNewRows = true;        // can take a step's new rows directly
    static constexpr bool kStageOut = true;       // outputs leave through LDS (see the kernel)
    static constexpr bool kLeanStream = true;     // the item stream without full waits (kernel)
    // column c16 of S^T is query head c16 (none past G); output row 4 q4 + r is head
    // 4 q4 + r, for every column block
    __device__ static int q_head(int c16) { return c16; }
    __device__ static bool q_valid(int c16) { return c16 < G; }
    __device__ static int row_head(int q4, int r) { return 4 * q4 + r; }
    __device__ static bool row_valid(int q4, int r) { return 4 * q4 + r < G; }
    __device__ static bool row_has_block(int, int, int) { return true; }

    struct Q { u32x4 b[KC]; float f; };
    struct Tile { u32x4 k[KC], v[NLD]; };
    struct Extra {};

    // K: lane holds token c16, columns 32 c + 8 q4 .. +8 of each step c.
    // V: coalesced; load i of lane l reads bytes 1024 i + 16 l of the tile.
    __device__ static size_t k_lane(int lane) {
        return (size_t)(lane % 16) * D * 2 + (size_t)(lane / 16) * 16;
    }
    __device__ static size_t v_lane(int lane) { return (size_t)lane * 16; }

    // B operand of S^T: query head c16 of the group (zero for c16 >= G), columns
    // 32 c + 8 q4 .. +8
    __device__ static void load_q(const void* q, size_t qrow, int c16, int q4, Q& r) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < KC; ++c)
            r.b[c] = c16 < G ? ld16((const char*)q + (qrow + 32 * c + 8 * q4) * 2) : z;
        r.f = 1.f;
    }
    __device__ static void prep_q(Q&) {}
    // the loads of a tile, issued over a resource of 0 bytes: zeros, no memory access (for
    // a slot nothing will consume; the same loads as load(), so the wait counts match)
    __device__ static void load_null(const char* base, Tile& t) {
        const rsrc_t r = buf_rsrc(base, 0u);
        const uint32_t o = (uint32_t)lane_id() * 16u;
#pragma unroll
        for (int c = 0; c < KC; ++c) t.k[c] = ld16_buf(r, o);
#pragma unroll
        for (int i = 0; i < NLD; ++i) t.v[i] = ld16_buf(r, o);
    }
    __device__ static void load(const char* kb, const char* vb, const size_t (&offs)[BPT],
                                Tile& t) {
        const size_t off = offs[0];
#pragma unroll
        for (int c = 0; c < KC; ++c) t.k[c] = ld16_stream(kb + off + c * 64);
#pragma unroll
        for (int i = 0; i < NLD; ++i) t.v[i] = ld16_stream(vb + off + i * 1024);
    }
    // The tile of the block holding a row's newest token (row r of the tile), with the
    // step's new rows given: the lanes that hold token row r read it from the new K and V
    // rows (kn, vn) instead of the cache, whose slot is not written yet.
    __device__ static void load_new(const char* kb, const char* vb, size_t off, const char* kn,
                                    const char* vn, int r, Tile& t) {
        constexpr int LPR = D * 2 / 16;           // lanes per token row in a V load
        constexpr int RPL = kWave / LPR;          // token rows per V load
        const int lane = lane_id();
        const char* kp = lane % 16 == r ? kn + (lane / 16) * 16 : kb + off;
#pragma unroll
        for (int c = 0; c < KC; ++c) t.k[c] = ld16_stream(kp + c * 64);
        // token row r lies in V load r / RPL, lanes LPR (r % RPL) .. +LPR
        const int ir = r / RPL;
        const char* vr = lane / LPR == r % RPL ? vn + (lane % LPR) * 16 : vb + off + ir * 1024;
#pragma unroll
        for (int i = 0; i < NLD; ++i) t.v[i] = ld16_stream(i == ir ? vr : vb + off + i * 1024);
    }
    // Stage V (rows of masked tokens zeroed) in this wavefront's LDS rows; S^T of the
    // block: lane holds head c16, tokens 4 q4 .. +3.
    template <class Ok>
    __device__ static void scores(const Tile& tl, int h, const Q& q, char* my, int t0, bool edge,
                                  Ok ok, float (&s)[4]) {
        const int lane = lane_id();
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int byte = i * 1024 + lane * 16;
            const int tv = byte / (D * 2), col = byte % (D * 2);
            u32x4 v = tl.v[i];
            if (edge) {
                const u32x4 z = {0u, 0u, 0u, 0u};
                v = ok(h, t0 + tv) ? v : z;
            }
            char* dst = my + tv * RS + col;
            *reinterpret_cast<u32x2*>(dst) = u32x2{v.x, v.y};
            *reinterpret_cast<u32x2*>(dst + 8) = u32x2{v.z, v.w};
        }
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c) sacc = mfma_16x16x32<DT>(tl.k[c], q.b[c], sacc);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = sacc[r];
    }
    // O += P V: B operand = column 16 b + c16 of tokens 4 q4 .. +3, from LDS
    template <class Ok>
    __device__ static void pv(f32x4 (&acc)[NACC], const float (&pp)[BPT][4], const Tile&, int,
                              char* my, const int (&)[BPT], const bool (&)[BPT], Ok, Extra&) {
        const int lane = lane_id(), c16 = lane % 16, q4 = lane / 16;
        const float (&p)[4] = pp[0];
        uint32_t h0, l0, h1, l1;
        split2<DT>(p[0], p[1], h0, l0);
        split2<DT>(p[2], p[3], h1, l1);
        const u32x2 ph = {h0, h1}, pl = {l0, l1};
        const uint16_t* vr = reinterpret_cast<const uint16_t*>(my + 4 * q4 * RS) + c16;
#pragma unroll
        for (int b = 0; b < NACC; ++b) {
            const uint32_t e0 = vr[16 * b], e1 = vr[RS / 2 + 16 * b];
            const uint32_t e2 = vr[RS + 16 * b], e3 = vr[3 * RS / 2 + 16 * b];
            const u32x2 vb = {e0 | (e1 << 16), e2 | (e3 << 16)};
            acc[b] = mfma_16x16x16<DT>(ph, vb, acc[b]);
            acc[b] = mfma_16x16x16<DT>(pl, vb, acc[b]);
        }
    }
    __device__ static void init(Extra&) {}
    __device__ static void rescale(Extra&, float) {}
    __device__ static void finish(f32x4 (&)[NACC], const Extra&) {}
    // acc[b] of lane c16 is column 16 b + c16
    // row r of lane quad q4, column blocks row_has_block(q4, r, b)
    // the head's row of the staged output: column 16 b + c16 = acc[b][r] x inv, as fp32 or
    // converted to the 16-bit output type
    __device__ static void stage_out(float* dst, const f32x4 (&acc)[NACC], int r, float inv,
                                     int c16, int q4) {
#pragma unroll
        for (int b = 0; b < NACC; ++b)
            if (row_has_block(q4, r, b)) dst[16 * b + c16] = acc[b][r] * inv;
    }
    __device__ static void stage_out16(int out_dtype, uint16_t* dst, const f32x4 (&acc)[NACC],
                                       int r, float inv, int c16, int q4) {
#pragma unroll
        for (int b = 0; b < NACC; ++b)
            if (row_has_block(q4, r, b)) {
                const float v = acc[b][r] * inv;
                dst[16 * b + c16] = (uint16_t)(out_dtype == PA_F16 ? f32_to_f16_bits(v)
                                                                   : f32_to_bf16_bits(v));
            }
    }
};

// ---- 8-bit caches -------------------------------------------------------------------
// Tile: 16 rows of D one-byte codes, then the scale row [16][D / 32] fp16.
template <int DT, int D, int G>
struct MfmaKvQ8 {
    static constexpr int ADT = DT == DT_Q8F16 ? DT_F16 : DT_BF16;   // query type
    static constexpr int KC = D / 32;             // steps of S^T = scale groups
    static constexpr int NACC = D / 16;           // 16-column blocks of O, two per group
    static constexpr int CPL = D / 16;            // V columns a lane loads per token row
    static constexpr int VW = CPL / 4;            // code dwords per V row and lane
    static constexpr int SW = KC / 2;             // 16-byte LDS reads of a lane's scales
    static constexpr int SCALES = kBlock * D;
    // LDS dwords per staged token pair: column c sits at dword c + 4 (c / 32) (the skew puts
    // the 16-byte writes of the 8 lanes of one pass, CPL columns apart, on distinct groups
    // of 4 of the 32 banks), and PS = 8 mod 16 keeps the one-dword reads of two lane rows
    // on distinct banks
    static constexpr int PS = (D + D / 8 + 15) / 16 * 16 + 8;
    static constexpr int SB = D / 32;             // scale-row bytes a lane loads (K or V row)
    // An 8-bit tile is half the bytes of a 16-bit one: two blocks per tile keep as many
    // bytes in flight per wavefront (head_dim 256 keeps one: its registers would not fit).
    static constexpr int BPT = D <= 128 ? 2 : 1;
    static constexpr int VBLK = kBlock / 2 * PS;  // LDS dwords of one block's staged V
    static constexpr int LDSV = BPT * VBLK * 4;   // LDS bytes of staged V per wavefront
    static constexpr int LDSS = LDSV;             // each block's K and V scale rows
    static constexpr int KS = D + 16;             // LDS bytes per staged K row (padded)
    static constexpr int LDSK = LDSS + BPT * 2 * D;     // each block's K codes
    static constexpr int LDSW = LDSK + BPT * kBlock * KS;
    static constexpr int KN = kBlock * D / 1024;  // coalesced 1 KiB loads of a block's K codes
    static constexpr int LDS_BYTES = kWavesPerGroup * LDSW;
    static constexpr size_t TILE = (size_t)(kBlock + 1) * D;
    static_assert(KC % 2 == 0, "an even number of scale groups");
    // new rows must be quantized into the cache first (pa_write_kv)
    static constexpr bool kNewRows = false;
    // Outputs are stored straight from the MFMA layout: the staging through LDS that the
    // 16-bit kernel uses needs registers this kernel does not have.
    static constexpr bool kStageOut = false;
    // The item stream keeps its register-held block ids and its copy of a tile between the
    // register sets: the scalar ids and the padding item of the 16-bit kernel spill here.
    static constexpr bool kLeanStream = false;
    // Stacked P.V, where the scale groups and heads fit the MFMA's 16 rows: A row m is
    // (scale group m / G, head m % G), so one A operand (P x the row's own V scale) serves
    // every 16-column block, and output row m is meaningful in its own group's two column
    // blocks only.  The query's columns then repeat the heads (column m holds head m % G),
    // so that S^T, the softmax and P arrive in that row order with no lane exchange.
    static constexpr bool kStacked = KC * G <= 16;
    __device__ static int q_head(int c16) { return kStacked ? c16 % G : c16; }
    __device__ static bool q_valid(int c16) { return kStacked ? c16 / G < KC : c16 < G; }
    __device__ static int row_head(int q4, int r) { return kStacked ? (4 * q4 + r) % G : 4 * q4 + r; }
    __device__ static bool row_valid(int q4, int r) {
        return kStacked ? (4 * q4 + r) / G < KC : 4 * q4 + r < G;
    }
    // column block b (scale group b / 2) of output row 4 q4 + r
    __device__ static bool row_has_block(int q4, int r, int b) {
        return !kStacked || (4 * q4 + r) / G == b / 2;
    }

    // The K code offset (+1152, below) is cancelled by the score accumulator's start where
    // the instance has registers for it (4 per scale group: the stacked instances with
    // d >= 128), else by a packed subtraction per code pair.
    static constexpr bool kBiasK = kStacked && D >= 128;
    // bias[c]: -1152 x the sum of the head's 32 (scaled) query values of scale group c
    struct Q { u32x4 b[KC]; float f; float bias[kBiasK ? KC : 1]; };
    // k: load i of lane l holds bytes 1024 i + 16 l of the block's codes (whole rows per
    // load: an MFMA operand's 8-byte pieces are read back from LDS, since loading them
    // directly would split every row into four small memory requests); v: CPL codes of
    // token 4 q4 + s; sc: SB bytes of the K scale row (lanes 0-31) or the V scale row
    // (lanes 32-63).  K, the scale rows and V are staged through LDS when consumed.
    struct Tile { u32x4 k[BPT][KN]; uint32_t v[BPT][4][VW]; uint32_t sc[BPT][(SB + 3) / 4]; };
    struct Extra {};

    __device__ static size_t k_lane(int lane) { return (size_t)lane * 16; }
    __device__ static size_t v_lane(int lane) {
        return (size_t)(lane / 16) * 4 * D + (size_t)(lane % 16) * CPL;
    }

    // B operand of S^T in fp16: query head c16 (zero for c16 >= G), columns 32 c + 8 q4 ..
    // +8, times 2^(15 - e) where 2^e bounds the head's largest |q|: every value then lies
    // below 2^15 and converts exactly.  f = 2^(e - 15) undoes the scaling.  load_q only
    // issues the loads (the next segment's queries load early); prep_q converts them once
    // the segment is the current one.
    __device__ static void load_q(const void* q, size_t qrow, int c16, int q4, Q& r) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < KC; ++c)
            r.b[c] = q_valid(c16) ? ld16((const char*)q + (qrow + 32 * c + 8 * q4) * 2) : z;
    }
    __device__ static void prep_q(Q& r) {
        float v[KC][8];
        float mx = 0.f;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            widen16<ADT>(r.b[c], v[c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[c][e]));
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));          // over the head's 4 lanes
        const int ex = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) : 0;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            uint32_t w[4];
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float a = ldexpf(v[c][e], 15 - ex), b = ldexpf(v[c][e + 1], 15 - ex);
                w[e / 2] = cvt2<DT_F16>(a, b);
                sum += a + b;
            }
            r.b[c] = u32x4{w[0], w[1], w[2], w[3]};
            if constexpr (kBiasK) {
                sum += __shfl_xor(sum, 16);
                sum += __shfl_xor(sum, 32);           // the group's 32 columns
                r.bias[c] = -1152.f * sum;
            }
        }
        r.f = ldexpf(1.f, ex - 15);
    }
    // the scale-row piece of lane l: K row bytes SB l .. (l < 32), V row bytes SB (l - 32) ..
    __device__ static const char* scale_piece(const char* kb, const char* vb, size_t off,
                                              int lane) {
        return lane < 32 ? kb - k_lane(lane) + off + SCALES + SB * lane
                         : vb - v_lane(lane) + off + SCALES + SB * (lane - 32);
    }
    // never called (kNewRows is false); present so that the shared kernel body compiles
    __device__ static void load_new(const char* kb, const char* vb, size_t off, const char*,
                                    const char*, int, Tile& t) {
        size_t offs[BPT];
#pragma unroll
        for (int h = 0; h < BPT; ++h) offs[h] = off;
        load(kb, vb, offs, t);
    }
    // the loads of a tile, issued over a resource of 0 bytes: zeros, no memory access (for
    // a slot nothing will consume; the same loads as load(), so the wait counts match)
    __device__ static void load_null(const char* base, Tile& t) {
        const rsrc_t r = buf_rsrc(base, 0u);
        const uint32_t o = (uint32_t)lane_id() * 16u;
#pragma unroll
        for (int h = 0; h < BPT; ++h) {
#pragma unroll
            for (int i = 0; i < KN; ++i) t.k[h][i] = ld16_buf(r, o);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if constexpr (VW == 1) {
                    t.v[h][s][0] = ld4_buf(r, o);
                } else if constexpr (VW == 2) {
                    const u32x2 x = ld8_buf(r, o);
                    t.v[h][s][0] = x.x; t.v[h][s][1] = x.y;
                } else {
                    const u32x4 x = ld16_buf(r, o);
                    t.v[h][s][0] = x.x; t.v[h][s][1] = x.y; t.v[h][s][2] = x.z; t.v[h][s][3] = x.w;
                }
            }
            if constexpr (SB == 2) {
                t.sc[h][0] = ld2_buf(r, o);
            } else if constexpr (SB == 4) {
                t.sc[h][0] = ld4_buf(r, o);
            } else {
                const u32x2 x = ld8_buf(r, o);
                t.sc[h][0] = x.x; t.sc[h][1] = x.y;
            }
        }
    }
    __device__ static void load(const char* kb, const char* vb, const size_t (&offs)[BPT],
                                Tile& t) {
        const int lane = lane_id();
#pragma unroll
        for (int h = 0; h < BPT; ++h) {
            const size_t off = offs[h];
#pragma unroll
            for (int i = 0; i < KN; ++i) t.k[h][i] = ld16_stream(kb + off + 1024 * i);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const char* p = vb + off + (size_t)s * D;
                if constexpr (VW == 1) {
                    t.v[h][s][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
                } else if constexpr (VW == 2) {
                    const u32x2 x = ld8_stream(p);
                    t.v[h][s][0] = x.x; t.v[h][s][1] = x.y;
                } else {
                    const u32x4 x = ld16_stream(p);
                    t.v[h][s][0] = x.x; t.v[h][s][1] = x.y; t.v[h][s][2] = x.z; t.v[h][s][3] = x.w;
                }
            }
            const char* sp = scale_piece(kb, vb, off, lane);
            if constexpr (SB == 2) {
                t.sc[h][0] = ld2_stream(sp);
            } else if constexpr (SB == 4) {
                t.sc[h][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(sp));
            } else {
                const u32x2 x = ld8_stream(sp);
                t.sc[h][0] = x.x; t.sc[h][1] = x.y;
            }
        }
    }
    // fp16 pairs (1152 + c0, 1152 + c1) from code bytes 0, 1 (lo) or 2, 3 (hi) of x, whose
    // bytes are already flipped by 0x80 (code + 128): the byte goes under 0x64.
    __device__ static uint32_t pair_lo(uint32_t x) {
        return __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
    }
    __device__ static uint32_t pair_hi(uint32_t x) {
        return __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
    }
    __device__ static int vcol(int c) { return c + 4 * (c / 32); }
    __device__ static uint32_t minus1152(uint32_t h) {
        const f16x2 k = {(_Float16)1152.f, (_Float16)1152.f};
        return __builtin_bit_cast(uint32_t, as_f16x2(h) - k);
    }
    // K rows 8 .. 15 hold each 16-byte piece with its 8-byte halves swapped (byte offset
    // XOR 8), so that the 8-byte operand reads of tokens c16 and c16 + 8, whose padded rows
    // otherwise meet on the same banks, use different bank pairs
    __device__ static int kswz(int row) { return (row & 8) ? 8 : 0; }
    // the 4 KC fp16 scales of tokens 4 q4 .. +3 of one scale row, from its staged copy;
    // (r, group g) is number r KC + g
    struct Scales { u32x4 w[SW]; };
    __device__ static void read_scales(const char* row, Scales& sc) {
        const int q4 = lane_id() / 16;
#pragma unroll
        for (int i = 0; i < SW; ++i)
            sc.w[i] = *reinterpret_cast<const u32x4*>(row + q4 * 8 * KC + 16 * i);
    }
    __device__ static float scale(const Scales& sc, int r, int g) {
        const int i = r * KC + g;
        const u32x4 w = sc.w[i / 8];
        const uint32_t d = (i / 2) % 4 == 0 ? w.x : (i / 2) % 4 == 1 ? w.y : (i / 2) % 4 == 2 ? w.z : w.w;
        return i % 2 ? f16_hi(d) : f16_lo(d);
    }
    // S^T of the block, lane: head c16, tokens 4 q4 .. +3.  Step c is scale group c.
    template <class Ok>
    __device__ static void scores(const Tile& tl, int h, const Q& q, char* my, int t0, bool,
                                  Ok ok, float (&s)[4]) {
        // stage the block's K codes and both scale rows, then read this lane's pieces
        const int lane = lane_id(), c16 = lane % 16, q4 = lane / 16;
        char* krow = my + LDSK + h * kBlock * KS;
#pragma unroll
        for (int i = 0; i < KN; ++i) {
            const int byte = 1024 * i + 16 * lane, row = byte / D;
            const u32x4 x = tl.k[h][i];
            *reinterpret_cast<u32x4*>(krow + row * KS + byte % D) =
                kswz(row) ? u32x4{x.z, x.w, x.x, x.y} : x;
        }
        char* srow = my + LDSS + h * 2 * D;
        // a V scale piece (lanes 32-63) belongs to token (lane - 32) / 2: zero for tokens the
        // row does not see, so that their V values are exact zeros whatever the slot holds
        const bool keep = lane < 32 || ok(h, t0 + (lane - 32) / 2);
        if constexpr (kStacked) {
            // K row as below; the V row group-major, [group][token], so that a lane's four
            // tokens of its own group are one 8-byte read.  Lane 32 + i holds the SB / 2
            // scales of token i / 2, groups (i % 2) SB / 2 ..
            if (lane < 32) {
                if constexpr (SB == 2)
                    *reinterpret_cast<uint16_t*>(srow + SB * lane) = (uint16_t)tl.sc[h][0];
                else if constexpr (SB == 4)
                    *reinterpret_cast<uint32_t*>(srow + SB * lane) = tl.sc[h][0];
                else
                    *reinterpret_cast<u32x2*>(srow + SB * lane) = u32x2{tl.sc[h][0], tl.sc[h][1]};
            } else {
                const int i = lane - 32, t = i / 2;
                uint16_t* vrow = reinterpret_cast<uint16_t*>(srow + D);
#pragma unroll
                for (int e = 0; e < SB / 2; ++e) {
                    const int g = (i % 2) * (SB / 2) + e;
                    const uint32_t w = tl.sc[h][e / 2];
                    vrow[g * kBlock + t] = keep ? (uint16_t)(e % 2 ? w >> 16 : w & 0xffffu) : 0;
                }
            }
        } else if constexpr (SB == 2) {
            *reinterpret_cast<uint16_t*>(srow + SB * lane) = keep ? (uint16_t)tl.sc[h][0] : 0;
        } else if constexpr (SB == 4) {
            *reinterpret_cast<uint32_t*>(srow + SB * lane) = keep ? tl.sc[h][0] : 0u;
        } else {
            *reinterpret_cast<u32x2*>(srow + SB * lane) =
                keep ? u32x2{tl.sc[h][0], tl.sc[h][1]} : u32x2{0u, 0u};
        }
        Scales ks;
        read_scales(srow, ks);
        u32x2 kp[KC];     // token c16, columns 32 c + 8 q4 .. +8
        const char* kr = krow + c16 * KS + ((8 * q4) ^ kswz(c16));
#pragma unroll
        for (int c = 0; c < KC; ++c) kp[c] = *reinterpret_cast<const u32x2*>(kr + 32 * c);
        // kBiasK: the A operand carries 1152 + code (exact fp16 integers, no subtraction);
        // the accumulator starts at -1152 x the group's query sum, which takes the offset
        // out.  The products are exact; the offset adds at most a few fp32 roundings of the
        // group's sum of |1152 q| (about 1e-5 of the raw score's scale).
        f32x4 sc[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const uint32_t x0 = kp[c].x ^ 0x80808080u, x1 = kp[c].y ^ 0x80808080u;
            if constexpr (kBiasK) {
                const u32x4 a = {pair_lo(x0), pair_hi(x0), pair_lo(x1), pair_hi(x1)};
                const float bc = q.bias[c];
                sc[c] = mfma_16x16x32<DT_F16>(a, q.b[c], f32x4{bc, bc, bc, bc});
            } else {
                const u32x4 a = {minus1152(pair_lo(x0)), minus1152(pair_hi(x0)),
                                 minus1152(pair_lo(x1)), minus1152(pair_hi(x1))};
                sc[c] = mfma_16x16x32<DT_F16>(a, q.b[c], f32x4{0.f, 0.f, 0.f, 0.f});
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float t = 0.f;
#pragma unroll
            for (int c = 0; c < KC; ++c) t = fmaf(scale(ks, r, c), sc[c][r], t);
            s[r] = t;          // the kernel applies q.f with the softmax scale
        }
    }
    // O += P V on 16x16x16 bf16 MFMAs.  V is staged as bf16 codes in token pairs: dword
    // (pair p, column c) holds tokens 2 p and 2 p + 1 of column c, so the B operand of a
    // lane (column 16 b + c16, tokens 4 q4 .. +3) is two dwords.  The A operand of the two
    // column blocks of group g is P x (V scale of group g), as hi + lo bf16 parts.  Every
    // block of the item is staged before any is read back.
    template <class Ok>
    __device__ static void pv(f32x4 (&acc)[NACC], const float (&p)[BPT][4], const Tile& tl, int,
                              char* my, const int (&)[BPT], const bool (&)[BPT], Ok, Extra&) {
        const int lane = lane_id(), c16 = lane % 16, q4 = lane / 16;
        uint32_t* lw = reinterpret_cast<uint32_t*>(my);
#pragma unroll
        for (int h = 0; h < BPT; ++h) {
#pragma unroll
            for (int pi = 0; pi < 2; ++pi) {
                uint32_t o[CPL];
#pragma unroll
                for (int w = 0; w < VW; ++w) {
                    const uint32_t y0 = tl.v[h][2 * pi][w], y1 = tl.v[h][2 * pi + 1][w];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // a code is an integer of at most 7 bits: its bf16 is exact, the
                        // high half of its fp32
                        const float f0 = (float)(int8_t)((y0 >> (8 * e)) & 0xffu);
                        const float f1 = (float)(int8_t)((y1 >> (8 * e)) & 0xffu);
                        o[4 * w + e] = __builtin_amdgcn_perm(__float_as_uint(f1),
                                                             __float_as_uint(f0), 0x07060302u);
                    }
                }
                uint32_t* dst = lw + h * VBLK + (2 * q4 + pi) * PS + vcol(CPL * c16);
#pragma unroll
                for (int i = 0; i < CPL; i += 4)
                    *reinterpret_cast<u32x4*>(dst + i) = u32x4{o[i], o[i + 1], o[i + 2], o[i + 3]};
            }
        }
        if constexpr (kStacked) {
            // A row c16 = (group c16 / G, head c16 % G): this lane's p (its column's head)
            // times the V scales of its group, tokens 4 q4 .. +3; one A for every block b
            const int gq = c16 / G < KC ? c16 / G : KC - 1;
#pragma unroll
            for (int h = 0; h < BPT; ++h) {
                const u32x2 sw = *reinterpret_cast<const u32x2*>(
                    my + LDSS + h * 2 * D + D + (gq * kBlock + 4 * q4) * 2);
                const float pg0 = p[h][0] * f16_lo(sw.x), pg1 = p[h][1] * f16_hi(sw.x);
                const float pg2 = p[h][2] * f16_lo(sw.y), pg3 = p[h][3] * f16_hi(sw.y);
                uint32_t h0, l0, h1, l1;
                split2<DT_BF16>(pg0, pg1, h0, l0);
                split2<DT_BF16>(pg2, pg3, h1, l1);
                const u32x2 ph = {h0, h1}, pl = {l0, l1};
                const uint32_t* src = lw + h * VBLK + 2 * q4 * PS + c16;
#pragma unroll
                for (int b = 0; b < NACC; ++b) {
                    const u32x2 vb = {src[vcol(16 * b)], src[PS + vcol(16 * b)]};
                    acc[b] = mfma_16x16x16<DT_BF16>(ph, vb, acc[b]);
                    acc[b] = mfma_16x16x16<DT_BF16>(pl, vb, acc[b]);
                }
            }
            return;
        }
#pragma unroll
        for (int h = 0; h < BPT; ++h) {
            Scales vs;
            read_scales(my + LDSS + h * 2 * D + D, vs);
            const uint32_t* src = lw + h * VBLK + 2 * q4 * PS + c16;
#pragma unroll
            for (int g = 0; g < KC; ++g) {
                float pg[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pg[r] = p[h][r] * scale(vs, r, g);
                }
                uint32_t h0, l0, h1, l1;
                split2<DT_BF16>(pg[0], pg[1], h0, l0);
                split2<DT_BF16>(pg[2], pg[3], h1, l1);
                const u32x2 ph = {h0, h1}, pl = {l0, l1};
#pragma unroll
                for (int bb = 0; bb < 2; ++bb) {
                    const int b = 2 * g + bb;
                    const u32x2 vb = {src[vcol(16 * b)], src[PS + vcol(16 * b)]};
                    acc[b] = mfma_16x16x16<DT_BF16>(ph, vb, acc[b]);
                    acc[b] = mfma_16x16x16<DT_BF16>(pl, vb, acc[b]);
                }
            }
        }
    }
    __device__ static void init(Extra&) {}
    __device__ static void rescale(Extra&, float) {}
    __device__ static void finish(f32x4 (&)[NACC], const Extra&) {}
    // acc[b] of lane c16 is column 16 b + c16
    // row r of lane quad q4, column blocks row_has_block(q4, r, b)
    // acc[b] of lane c16 is column 16 b + c16; row r of lane quad q4, column blocks
    // row_has_block(q4, r, b)
    __device__ static void store(const DecodeArgs& a, size_t ob, const f32x4 (&acc)[NACC],
                                 int r, float inv, int c16, int q4) {
#pragma unroll
        for (int b = 0; b < NACC; ++b)
            if (row_has_block(q4, r, b)) store_out1(a, ob + 16 * b + c16, acc[b][r] * inv);
    }
    __device__ static void store_part(float* dst, const f32x4 (&acc)[NACC], int r, int c16,
                                      int q4) {
#pragma unroll
        for (int b = 0; b < NACC; ++b)
            if (row_has_block(q4, r, b)) dst[16 * b + c16] = acc[b][r];
    }
};

template <int DT, int D, int G, bool Q8 = (DT == DT_Q8F16 || DT == DT_Q8BF16)>
struct MfmaKv;
template <int DT, int D, int G>
struct MfmaKv<DT, D, G, false> : MfmaKv16<DT, D, G> {};
template <int DT, int D, int G>
struct MfmaKv<DT, D, G, true> : MfmaKvQ8<DT, D, G> {};

// NEW: the instance that takes the step's new rows (pa_decode_write_attend); the other
// instances compile without any of that code.
template <int DT, int D, int G, bool NEW = false>
__global__ __launch_bounds__(kWavesPerGroup * kWave, D <= 128 ? 2 : 1) void decode_mfma_kernel(DecodeArgs a) {
    static_assert(G == 4 || G == 8, "groups of 4 or 8 query heads");
    using Ops = MfmaKv<DT, D, G>;
    using Q = typename Ops::Q;
    using Tile = typename Ops::Tile;
    constexpr int NACC = Ops::NACC, BPT = Ops::BPT;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kNegBig = -3.402823466e38f;
    constexpr float kLazy = 8.f;
    __shared__ __align__(16) char lds[Ops::LDS_BYTES > 0 ? Ops::LDS_BYTES : 16];

    int32_t* hdr = (int32_t*)(a.ws + a.lay.header);
    const uint32_t* cb = (const uint32_t*)(a.ws + a.lay.cb);
    const UnitInfo* unit = (const UnitInfo*)(a.ws + a.lay.unit);
    const int32_t* wcut = (const int32_t*)(a.ws + a.lay.wave_u);
    float2* pml = (float2*)(a.ws + a.lay.part_ml);
    float* pacc = (float*)(a.ws + a.lay.part_acc);
    int4* tasks = (int4*)(a.ws + a.lay.tasks);
    const int32_t* empty = (const int32_t*)(a.ws + a.lay.empty);

    const int W = hdr[2], n_empty = hdr[3];
    const int wave = uniform(blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6));
    const int lane = lane_id();
    // this wavefront's first segment, read with the header (entries from W on are unused)
    const WaveStart st = ((const WaveStart*)(a.ws + a.lay.wave_st))[wave];
    for (int i = wave; i < n_empty; i += gridDim.x * kWavesPerGroup) zero_row(a, empty[i], lane);
    if (wave >= W) return;
    if (hdr[5] != 0) {   // a group-mode plan: its records are not wave shares
        if (wave == 0 && lane == 0) atomicOr(hdr, kErrPlanMode);
        return;
    }

    const int c16 = lane % 16, q4 = lane / 16;
    char* my = Ops::LDS_BYTES > 0 ? lds + (threadIdx.x >> 6) * (Ops::LDS_BYTES / kWavesPerGroup)
                                  : lds;
    // A finished segment's output (16-bit values, or fp32 values and partials) is staged in
    // this wavefront's rows of lds_out as [G heads][D] and leaves as whole 16-byte lane
    // stores: one or two store instructions instead of one per (row, column block) of the
    // MFMA layout, each of which wrote 32-byte pieces.
    __shared__ __align__(16) float lds_out[kWavesPerGroup][Ops::kStageOut ? G * D : 4];
    float* mo = lds_out[threadIdx.x >> 6];
    const float qscale = a.scale * kLog2e;
    const size_t block_stride = (size_t)a.num_kv_heads * Ops::TILE;
    const char* kbase = (const char*)a.k_cache + Ops::k_lane(lane);
    const char* vbase = (const char*)a.v_cache + Ops::v_lane(lane);

    const uint32_t x_start = st.x0;
    const uint32_t x_end = st.x1;
    int uh = st.u;

    // the unit offsets and records are read by scalar loads (uh is wave-uniform), so that
    // describing the next segment does not wait for the tiles in flight
    auto describe = [&](uint32_t xs) {
        while (ld_scalar(cb + uh + 1) <= xs) ++uh;
        const UnitInfo ui = ld_unit(unit + uh);
        const uint32_t base = ld_scalar(cb + uh);
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
    auto load_q = [&](const Seg& sg, Q& q) {
        const size_t qrow =
            ((size_t)sg.u * a.num_q_heads + (size_t)sg.g * G + Ops::q_head(c16)) * D;
        Ops::load_q(a.q, qrow, c16, q4, q);
    };
    // An item: the next BPT blocks of the stream inside one chunk of ids (fewer at the end
    // of a chunk).  A tile always loads BPT blocks: a slot past cnt re-reads another block
    // of the item and is never consumed.  The loads are one straight sequence whatever the
    // case, so that the compiler's wait counts for the tile in use never include the tile
    // being loaded.  An empty item (cnt = 0: padding, or the end of the share) issues the
    // same loads over a resource of 0 bytes.
    // With the step's new rows given (16-bit caches, one block per tile), a row's newest
    // token (position len - 1) is not in the cache yet: the tile of the block holding it
    // (table index jl) takes that token row from new row u, KV head g (Ops::load_new).  Its
    // slot is written by the merge launch that follows.
    // nl: the segment's length when new rows are given, else 0 (then no index matches)
    constexpr bool fused = NEW && Ops::kNewRows;
    auto new_len = [&](const Seg& sg) { return fused ? sg.len : 0; };
    struct Item { int cnt; bool ok[BPT]; };
    // bid: the item's block ids (slots past cnt repeat one of them); j: the table index of
    // its first block; u, nl: its segment's unit and new_len
    auto load_item = [&](int g, const int (&bid)[BPT], int cnt, int j, int u, int nl,
                         Tile& t, Item& it) __attribute__((always_inline)) {
        size_t off[BPT];
        it.cnt = cnt;
#pragma unroll
        for (int h = 0; h < BPT; ++h) {
            bool v;
            const int b = checked_block(bid[h], a.num_blocks, v);
            it.ok[h] = v;
            off[h] = (size_t)b * block_stride + (size_t)g * Ops::TILE;
        }
        if (fused && cnt > 0 && j == (nl - 1) / kBlock && nl > 0) {   // wavefront-uniform
            const size_t noff = ((size_t)u * a.num_kv_heads + (size_t)g) * (size_t)(D * 2);
            Ops::load_new(kbase, vbase, off[0], (const char*)a.k_new + noff,
                          (const char*)a.v_new + noff, (nl - 1) % kBlock, t);
        } else {
            Ops::load(kbase, vbase, off, t);
        }
    };
    // block ids idx0 .. of a vector-loaded id register (slots past cnt repeat idx_pad)
    auto ids_of = [&](int ids, int idx0, int cnt, int idx_pad, int (&bid)[BPT])
        __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < BPT; ++h)
            bid[h] = __builtin_amdgcn_readlane(ids, h < cnt ? idx0 + h : idx_pad);
    };
    // the first BPT block ids of table entries [j, j1), by scalar loads (entries past j1
    // repeat the last): reading them out of a vector-loaded id register would make the
    // wavefront wait for the tile in flight before it could issue the next one
    auto ids_ahead = [&](int seq, int j, int j1, int (&bid)[BPT]) __attribute__((always_inline)) {
        const int32_t* row = a.block_tables + (size_t)seq * a.max_blocks;
#pragma unroll
        for (int h = 0; h < BPT; ++h) bid[h] = ld_scalar_at(row + (j + h < j1 ? j + h : j1 - 1));
    };
    // the same from an id register: ids idx0 .. for cnt slots, the rest repeat idx_pad
    auto load_item_reg = [&](int g, int ids, int idx0, int cnt, int idx_pad, int j, int u,
                             int nl, Tile& t, Item& it) __attribute__((always_inline)) {
        int bid[BPT];
        ids_of(ids, idx0, cnt, idx_pad, bid);
        load_item(g, bid, cnt, j, u, nl, t, it);
    };
    auto load_empty = [&](Tile& t, Item& it) __attribute__((always_inline)) {
        it.cnt = 0;
#pragma unroll
        for (int h = 0; h < BPT; ++h) it.ok[h] = false;
        Ops::load_null((const char*)a.k_cache, t);
    };

    if (x_start >= x_end) return;
    Seg cur = first_segment_of(st, a.window);
    Q q;
    load_q(cur, q);
    int ids = load_ids(cur, cur.j0);
    Tile A, B;
    Item iA, iB;
    {
        // the first item's blocks come with the plan's record, ahead of the ids
        size_t off[BPT];
        iA.cnt = min(BPT, cur.j1 - cur.j0);
#pragma unroll
        for (int h = 0; h < BPT; ++h) {
            const int b = checked_block(h == 0 ? st.b0 : st.b1, a.num_blocks, iA.ok[h]);
            off[h] = (size_t)b * block_stride + (size_t)cur.g * Ops::TILE;
        }
        const int nl = new_len(cur);
        if (fused && nl > 0 && cur.j0 == (nl - 1) / kBlock) {
            const size_t noff = ((size_t)cur.u * a.num_kv_heads + (size_t)cur.g) * (size_t)(D * 2);
            Ops::load_new(kbase, vbase, off[0], (const char*)a.k_new + noff,
                          (const char*)a.v_new + noff, (nl - 1) % kBlock, A);
        } else {
            Ops::load(kbase, vbase, off, A);
        }
    }
    bool first_segment = true;
    int bad = 0;

    for (;;) {
        // the next segment's record, queries and first block ids load while this one runs
        const bool more = cur.end < x_end;
        Seg nxt = cur;
        Q qn;
        int nids = 0;
        int nxt_bid[BPT];
#pragma unroll
        for (int h = 0; h < BPT; ++h) nxt_bid[h] = 0;
        if (more) {
            nxt = describe(cur.end);
            load_q(nxt, qn);
            nids = load_ids(nxt, nxt.j0);
            if constexpr (Ops::kLeanStream) ids_ahead(nxt.seq, nxt.j0, nxt.j1, nxt_bid);
        }
        Ops::prep_q(q);
        // a pair that starts here and continues past the share (only a share's last segment)
        const bool opens_cut = cur.starts && cur.end < cur.pe;

        f32x4 acc[NACC];   // O: lane holds heads 4 q4 .. 4 q4 + 3 of its columns
#pragma unroll
        for (int b = 0; b < NACC; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = kNegBig, lsum = 0.f;   // head c16, this lane's tokens
        typename Ops::Extra ex;
        Ops::init(ex);
        const int len = cur.len, lo_tok = cur.lo_tok;
        const float qs = qscale * q.f;

        // The blocks of an item are scored first, share one softmax update and then go
        // through P V together, so their independent work can interleave.
        const int nl_cur = new_len(cur);
        auto consume_item = [&](const Tile& tl, const Item& it, int j0) __attribute__((always_inline)) {
            float sc[BPT][4];
            bool valid[BPT], edge[BPT];
            int t0[BPT];
            auto ok = [&](int h, int t) { return valid[h] && t >= lo_tok && t < len; };
#pragma unroll
            for (int h = 0; h < BPT; ++h) {
                // a slot past cnt holds a re-read block: scored, then masked entirely
                t0[h] = (j0 + h) * kBlock;
                valid[h] = h < it.cnt && it.ok[h];
                edge[h] = !valid[h] || t0[h] < lo_tok || t0[h] + kBlock > len;   // uniform
                bad |= h < it.cnt && !it.ok[h];
                Ops::scores(tl, h, q, my, t0[h], edge[h], ok, sc[h]);
#pragma unroll
                for (int r = 0; r < 4; ++r) sc[h][r] = Ops::q_valid(c16) ? sc[h][r] * qs : -INFINITY;
            }
            bool any_edge = false;
#pragma unroll
            for (int h = 0; h < BPT; ++h) any_edge |= edge[h];
            if (any_edge) {
#pragma unroll
                for (int h = 0; h < BPT; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sc[h][r] = ok(h, t0[h] + 4 * q4 + r) ? sc[h][r] : -INFINITY;
            }
            // lazy rescaling, as in decode_kernel: m moves only by more than kLazy
            float mx = sc[0][0];
#pragma unroll
            for (int h = 0; h < BPT; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[h][r]);
            if (__builtin_amdgcn_ballot_w64(mx > m + kLazy)) {
                float M = fmaxf(mx, __shfl_xor(mx, 16));
                M = fmaxf(M, __shfl_xor(M, 32));             // max over the head's 4 lanes
                const float mn = fmaxf(m, M);
                const float alpha = __builtin_amdgcn_exp2f(m - mn);
                m = mn;
                lsum *= alpha;
                Ops::rescale(ex, alpha);
                // O row 4 q4 + r belongs to head row_head: its factor sits in that lane
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = __shfl(alpha, Ops::row_head(q4, r));
#pragma unroll
                    for (int b = 0; b < NACC; ++b) acc[b][r] *= ar;
                }
            }
            float p[BPT][4];
#pragma unroll
            for (int h = 0; h < BPT; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[h][r] = __builtin_amdgcn_exp2f(sc[h][r] - m);
                    lsum += p[h][r];
                }
            Ops::pv(acc, p, tl, it.cnt, my, t0, edge, ok, ex);
        };

        // blocks of the segment, in chunks of 64 ids, BPT at a time; A holds the segment's
        // first item.  The load after each item's is the next item of the stream: in this
        // chunk, the next chunk or the next segment (nothing at the very end).
        // plain copies of what the loads need (a select between fields of the two records
        // would keep both records in memory)
        const int g_cur = cur.g, g_nxt = nxt.g, j1_cur = cur.j1, nb_nxt = nxt.j1 - nxt.j0;
        const int j0_nxt = nxt.j0, u_cur = cur.u, u_nxt = nxt.u, nl_nxt = more ? new_len(nxt) : 0;
        int cids = ids;
        if constexpr (!Ops::kLeanStream) {
            for (int c0 = cur.j0;; c0 += kWave) {
                const int n = (cur.j1 - c0) < kWave ? (cur.j1 - c0) : kWave;
                const bool last_chunk = c0 + kWave >= cur.j1;
                const int nc_ids = last_chunk ? 0 : load_ids(cur, c0 + kWave);
                const int items = (n + BPT - 1) / BPT;
                // item k of this chunk, else the first item of the next chunk or of the next
                // segment; at the very end nothing (the load repeats this chunk's last
                // block).  Every case issues the same loads, so the wait counts stay exact.
                auto load_next = [&](int k, Tile& t, Item& it) __attribute__((always_inline)) {
                    if (k < items) {
                        load_item_reg(g_cur, cids, BPT * k, min(BPT, n - BPT * k), BPT * k,
                                      c0 + BPT * k, u_cur, nl_cur, t, it);
                    } else if (!last_chunk) {
                        load_item_reg(g_cur, nc_ids, 0, min(BPT, j1_cur - c0 - kWave), 0,
                                      c0 + kWave, u_cur, nl_cur, t, it);
                    } else if (more) {
                        load_item_reg(g_nxt, nids, 0, min(BPT, nb_nxt), 0, j0_nxt, u_nxt, nl_nxt,
                                      t, it);
                    } else {
                        load_item_reg(g_cur, cids, 0, 0, n - 1, -1, 0, 0, t, it);
                    }
                };
                for (int k = 0;; k += 2) {
                    load_next(k + 1, B, iB);
                    consume_item(A, iA, c0 + BPT * k);
                    if (k + 1 >= items) {
                        A = B;
                        iA = iB;
                        break;
                    }
                    load_next(k + 2, A, iA);
                    consume_item(B, iB, c0 + BPT * (k + 1));
                    if (k + 2 >= items) break;
                }
                if (last_chunk) break;
                cids = nc_ids;
            }
        } else {
            for (int c0 = cur.j0;; c0 += kWave) {
                const int n = (cur.j1 - c0) < kWave ? (cur.j1 - c0) : kWave;
                const bool last_chunk = c0 + kWave >= cur.j1;
                const int nc_ids = last_chunk ? 0 : load_ids(cur, c0 + kWave);
                int nc_bid[BPT];
#pragma unroll
                for (int h = 0; h < BPT; ++h) nc_bid[h] = 0;
                if (!last_chunk) ids_ahead(cur.seq, c0 + kWave, j1_cur, nc_bid);
                const int items = (n + BPT - 1) / BPT;
                // An odd number of items is padded with an empty one (never consumed), so that
                // the item after the chunk always lands in A: moving a tile from B to A would
                // wait for all loads in flight.
                const int items2 = (items + 1) & ~1;
                // item k of this chunk, the padding, else the first item of the next chunk or of
                // the next segment; at the very end an empty item.  Every case issues the same
                // loads, so the wait counts stay exact.
                auto load_next = [&](int k, Tile& t, Item& it) __attribute__((always_inline)) {
                    if (k < items) {
                        int bid[BPT];
                        const int cnt = min(BPT, n - BPT * k);
                        ids_of(cids, BPT * k, cnt, BPT * k, bid);
                        load_item(g_cur, bid, cnt, c0 + BPT * k, u_cur, nl_cur, t, it);
                    } else if (k < items2) {
                        load_empty(t, it);
                    } else if (!last_chunk) {
                        load_item(g_cur, nc_bid, min(BPT, j1_cur - c0 - kWave), c0 + kWave, u_cur,
                                  nl_cur, t, it);
                    } else if (more) {
                        load_item(g_nxt, nxt_bid, min(BPT, nb_nxt), j0_nxt, u_nxt, nl_nxt, t, it);
                    } else {
                        load_empty(t, it);
                    }
                };
                for (int k = 0;; k += 2) {
                    load_next(k + 1, B, iB);
                    consume_item(A, iA, c0 + BPT * k);
                    load_next(k + 2, A, iA);
                    if (k + 1 < items)   // wavefront-uniform: the padding is not consumed
                        consume_item(B, iB, c0 + BPT * (k + 1));
                    if (k + 2 >= items) break;
                }
                if (last_chunk) break;
                cids = nc_ids;
            }
        }

        Ops::finish(acc, ex);
        // the head's sum over its 4 lanes; O-layout lanes fetch (m, l) of their heads
        float lt = lsum + __shfl_xor(lsum, 16);
        lt += __shfl_xor(lt, 32);
        const bool complete = cur.starts && cur.end == cur.pe;
        const int slot = first_segment ? 0 : 1;
        const bool out16 = complete && a.out_dtype != PA_F32;
        if (!complete && q4 == 0 && c16 < G) {
            const size_t pi = ((size_t)wave * 2 + slot) * G + c16;
            pml[pi] = make_float2(m, lt);
        }
        if constexpr (Ops::kStageOut) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = Ops::row_head(q4, r);
                const float lh = __shfl(lt, h);
                if (Ops::row_valid(q4, r)) {
                    const float inv = !complete ? 1.f : lh > 0.f ? 1.f / lh : 0.f;
                    if (out16)
                        Ops::stage_out16(a.out_dtype, reinterpret_cast<uint16_t*>(mo) + h * D,
                                         acc, r, inv, c16, q4);
                    else
                        Ops::stage_out(mo + h * D, acc, r, inv, c16, q4);
                }
            }
            // the wavefront's own LDS rows, written and read back in order: no barrier
            constexpr int N = G * D;
            if (out16) {
                const size_t ob = ((size_t)cur.u * a.num_q_heads + (size_t)cur.g * G) * D;
                const uint16_t* m16 = reinterpret_cast<const uint16_t*>(mo);
#pragma unroll
                for (int i0 = 0; i0 < N; i0 += kWave * 8) {
                    const int i = i0 + lane * 8;
                    if (N % (kWave * 8) == 0 || i < N)
                        st16((uint16_t*)a.out + ob + i, *reinterpret_cast<const u32x4*>(m16 + i));
                }
            } else {
                float* dst = complete
                    ? (float*)a.out + ((size_t)cur.u * a.num_q_heads + (size_t)cur.g * G) * D
                    : pacc + ((size_t)wave * 2 + slot) * G * D;
#pragma unroll
                for (int i0 = 0; i0 < N; i0 += kWave * 4) {
                    const int i = i0 + lane * 4;
                    if (N % (kWave * 4) == 0 || i < N)
                        st16(dst + i, *reinterpret_cast<const u32x4*>(mo + i));
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = Ops::row_head(q4, r);
                const float lh = __shfl(lt, h);
                if (Ops::row_valid(q4, r)) {
                    if (complete) {
                        const float inv = lh > 0.f ? 1.f / lh : 0.f;
                        const size_t ob =
                            ((size_t)cur.u * a.num_q_heads + (size_t)cur.g * G + h) * D;
                        Ops::store(a, ob, acc, r, inv, c16, q4);
                    } else {
                        Ops::store_part(pacc + (((size_t)wave * 2 + slot) * G + h) * D, acc, r,
                                        c16, q4);
                    }
                }
            }
        }
        if (opens_cut) {   // the plan counted the shares the pair spans
            const int nc = ld_scalar(wcut + wave);
            if (lane == 0) tasks[wave + 1] = make_int4(cur.u, cur.g, nc, first_segment ? 0 : 1);
        }
        if (!more) break;
        cur = nxt;
        q = qn;
        ids = nids;
        first_segment = false;
    }
    if (bad && lane == 0) atomicOr(hdr, kErrBlockId);
}

}  // namespace pa
