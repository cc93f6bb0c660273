// Paged decode attention kernel (wavefront-64, gfx950).
//
// What it computes: for each (query row u, KV head g) pair, the softmax-weighted sum of the
// V rows of the tokens the row sees, with scores scale * <q, K_t>, for the G query heads
// g*G .. g*G+G-1 that read KV head g.  K and V are reached through the block table:
// token t of the row's sequence sits in physical block block_tables[seq][t / 16], offset
// t % 16 ("PagedAttention deep dive", donmain.dev, section on splitting the KV cache into
// blocks).  A sliding window drops whole blocks before the window and masks the rest
// (sotaaz.com, section on layer kinds).  KV reads are not shared between sequences, so
// this is a streaming read of the cache bounded by HBM bandwidth (velog.io "Batching
// strategies", section 2.3).
//
// How, on CDNA4:
//   * one wavefront is one worker; it owns an equal share of the linear block space laid
//     out by the plan kernel and walks the pairs that share covers;
//   * a (block, KV head) tile is 16 x d elements, contiguous; load i of a lane reads bytes
//     [1024 i + 16 lane, +16) of the tile, so each load instruction of the wavefront reads
//     1 KiB of consecutive bytes.  Lane l therefore holds PE consecutive elements of token
//     (i * TPI + l / LPT), columns (l % LPT) * PE .. +PE;
//   * each tile is read once for all G query heads of the group;
//   * the dot product over d is a within-row DPP reduction over LPT lanes;
//   * the LPT-lane rows of the wavefront (TPI of them) each keep their own running max,
//     sum and output for the tokens they hold, so the hot loop needs no cross-row traffic;
//     rows are combined once per segment with the log-sum-exp rule;
//   * the next block's K and V are loaded before the current block is consumed;
//   * block ids come from one coalesced load of up to 64 table entries (one per lane),
//     broadcast with readlane; an id outside the pool sets an error bit and masks the
//     block instead of being dereferenced;
//   * masked tokens are removed by selection (score -inf, V zeroed), never by a zero
//     weight, so NaN in free or unused slots cannot reach the output;
//   * 8-bit caches ("KV cache by model", sotaaz.com: one scale per 32 values) are decoded
//     in registers: codes become fp16 values 1152 + code by placing the flipped code byte
//     under the exponent bits of 1024 (exact), the score is a packed fp16 dot product with
//     q (held in fp16 after a per-lane power-of-two scaling, exact), minus 1152 * sum(q),
//     times the group's scale; V codes are converted byte by byte to fp32 (code + 128) and
//     the 128 * sum of weights is taken off once per segment;
//   * a pair cut by share boundaries leaves one partial (max, sum, unnormalised output)
//     per wavefront; the wavefront holding the pair's first block also leaves a merge task
//     (pair, number of partials) for the merge kernel, which combines them with the
//     log-sum-exp rule.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// How a cache dtype's tiles are loaded and consumed.  Lane l of a load holds PE elements
// of token (i * TPI + l / LPT), columns (l % LPT) * PE .. +PE.
template <int DT, int D, int G, int BS, bool Q8 = (DT == DT_Q8F16 || DT == DT_Q8BF16)>
struct KvOps;

// fp32 / fp16 / bf16 caches: 16-byte lane loads, 1 KiB per load instruction; a tile is
// BS tokens (the block size).
template <int DT, int D, int G, int BS>
struct KvOps<DT, D, G, BS, false> {
    static constexpr bool kNewRows = true;       // can take a step's new rows directly
    static constexpr int EB = Elem<DT>::bytes;
    static constexpr int QB = EB;                // bytes per query element
    static constexpr int PE = Elem<DT>::per16;   // elements per 16-byte lane load
    static constexpr int LPT = D / PE;           // lanes holding one token row
    static constexpr int TPI = kWave / LPT;      // tokens per load instruction
    static constexpr int NLD = BS / TPI;         // load instructions per tile
    static constexpr int TILE = BS * D * EB;     // bytes of one (block, head) tile
    static_assert(LPT >= 8 && LPT <= 64 && (LPT & (LPT - 1)) == 0, "row width");
    static_assert(NLD >= 1 && NLD * 1024 == TILE, "tile covered by whole-wave loads");

    struct Tile { u32x4 k[NLD], v[NLD]; };
    struct Q { uint32_t v[G][4]; };
    typedef Q QRaw;                              // the query as loaded is the query used
    struct Extra {};

    __device__ static size_t lane_off(int lane) { return (size_t)lane * 16; }
    // this lane's slice of query row q_row (element index of its first element)
    __device__ static void load_q(const char* q, size_t elem, int gi, Q& r) {
        const u32x4 t = ld16(q + elem * QB);
        r.v[gi][0] = t.x; r.v[gi][1] = t.y; r.v[gi][2] = t.z; r.v[gi][3] = t.w;
    }
    __device__ static void prep_q(const QRaw& r, Q& q) { q = r; }
    // the tile at byte offset off of both caches; bytes = TILE reads it, bytes = 0 issues
    // the same loads without touching memory (zeros)
    __device__ static void load_buf(const char* kc, const char* vc, size_t off, uint32_t bytes,
                                    uint32_t lo, Tile& t) {
        const rsrc_t rk = buf_rsrc(kc + off, bytes), rv = buf_rsrc(vc + off, bytes);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            t.k[i] = ld16_buf(rk, lo + i * 1024);
            t.v[i] = ld16_buf(rv, lo + i * 1024);
        }
    }
    // this lane's share of q . k for each load and head (summed over the row afterwards)
    __device__ static void partial_scores(const Q& q, const Tile& t, float sc[G][NLD]) {
#pragma unroll
        for (int i = 0; i < NLD; ++i)
#pragma unroll
            for (int gi = 0; gi < G; ++gi) sc[gi][i] = dot16<DT>(q.v[gi], t.k[i]);
    }
    __device__ static void mask_v(Tile& t, int i, bool ok) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        t.v[i] = ok ? t.v[i] : z;
    }
    __device__ static void init(Extra&) {}
    __device__ static void rescale(Extra&, int, float) {}
    __device__ static void accumulate(float (&acc)[G][PE], const float (&p)[G][NLD],
                                      const Tile& t, Extra&) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            float vf[PE];
            widen16<DT>(t.v[i], vf);
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
#pragma unroll
                for (int e = 0; e < PE; ++e) acc[gi][e] = fmaf(p[gi][i], vf[e], acc[gi][e]);
        }
    }
    __device__ static void finish(float (&)[G][PE], const Extra&) {}
};

// 8-bit caches: each (block, head) tile is 16 rows of D one-byte codes followed by one row
// holding the 16 tokens' fp16 scales ([16][D / 32]).  A lane loads PE codes of a token row
// (16 bytes for G <= 4, 8 bytes for G = 8, whose accumulators would not fit twice as many
// columns) and the 2-byte scale of their group.
template <int DT, int D, int G, int BS>
struct KvOps<DT, D, G, BS, true> {
    static_assert(BS == kBlock, "8-bit tiles hold 16 tokens");
    // new rows must be quantized into the cache first (pa_write_kv)
    static constexpr bool kNewRows = false;
    static constexpr int EB = 1;
    static constexpr int ADT = DT == DT_Q8F16 ? DT_F16 : DT_BF16;   // query / new-row type
    static constexpr int QB = 2;
    static constexpr int PE = G <= 4 ? 16 : 8;
    static constexpr int NW = PE / 4;                  // code dwords per lane and load
    static constexpr int LPT = D / PE;
    static constexpr int TPI = kWave / LPT;
    static constexpr int NLD = kBlock / TPI;
    static constexpr int GROUPS = D / kQ8Group;
    static constexpr int SCALES = kBlock * D;          // offset of the scale row
    static constexpr int TILE = SCALES + D;            // 17 * D bytes
    static_assert(LPT >= 4 && LPT <= 32 && (LPT & (LPT - 1)) == 0, "row width");
    static_assert(NLD * kWave * PE == SCALES, "codes covered by whole-wave loads");

    typedef uint32_t CodeVec __attribute__((ext_vector_type(NW)));
    struct Tile { CodeVec k[NLD], v[NLD]; uint32_t ks[NLD], vs[NLD]; };
    // q in fp16 scaled by 2^e per lane and head, 1152 * sum of those values, 2^-e
    struct Q { uint32_t v[G][PE / 2]; float off[G]; float inv[G]; };
    struct QRaw { u32x4 r[G][PE / 8]; };   // the 16-bit query elements as loaded
    struct Extra { float corr[G]; };   // sum of weight * scale, per head

    __device__ static size_t lane_off(int lane) { return (size_t)lane * PE; }
    // byte offset in the tile of the scale of lane's first load
    __device__ static uint32_t scale_at(int lane) {
        const int row = lane / LPT, col = lane % LPT;
        return SCALES + (uint32_t)(row * GROUPS + col * PE / kQ8Group) * 2;
    }
    __device__ static void load_q(const char* q, size_t elem, int gi, QRaw& r) {
#pragma unroll
        for (int j = 0; j < PE / 8; ++j) r.r[gi][j] = ld16(q + (elem + 8 * j) * QB);
    }
    __device__ static void prep_q(const QRaw& raw, Q& r) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) prep_head(raw, gi, r);
    }
    __device__ static void prep_head(const QRaw& raw, int gi, Q& r) {
        float f[PE];
#pragma unroll
        for (int j = 0; j < PE / 8; ++j) widen16<ADT>(raw.r[gi][j], f + 8 * j);
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < PE; ++e) mx = fmaxf(mx, fabsf(f[e]));
        // 2^(15 - e) with mx < 2^e: the scaled values lie below 2^15 and convert to fp16
        // exactly (fp16 and bf16 values both fit in fp16's 11-bit significand)
        const int ex = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) : 0;
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < PE; e += 2) {
            const float a = ldexpf(f[e], 15 - ex), b = ldexpf(f[e + 1], 15 - ex);
            r.v[gi][e / 2] = f32_to_f16_bits(a) | (f32_to_f16_bits(b) << 16);
            sum += a + b;
        }
        r.off[gi] = 1152.f * sum;
        r.inv[gi] = ldexpf(1.f, ex - 15);
    }
    // as for 16-bit tiles: bytes = TILE reads the tile, bytes = 0 reads nothing
    __device__ static CodeVec ld_codes(rsrc_t r, uint32_t off) {
        if constexpr (NW == 2)
            return __builtin_bit_cast(CodeVec, ld8_buf(r, off));
        else
            return __builtin_bit_cast(CodeVec, ld16_buf(r, off));
    }
    __device__ static void load_buf(const char* kc, const char* vc, size_t off, uint32_t bytes,
                                    uint32_t lo, Tile& t) {
        const rsrc_t rk = buf_rsrc(kc + off, bytes), rv = buf_rsrc(vc + off, bytes);
        const uint32_t so = scale_at(lane_id());
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            t.k[i] = ld_codes(rk, lo + i * (kWave * PE));
            t.v[i] = ld_codes(rv, lo + i * (kWave * PE));
            t.ks[i] = ld2_buf(rk, so + i * TPI * GROUPS * 2);
            t.vs[i] = ld2_buf(rv, so + i * TPI * GROUPS * 2);
        }
    }
    // fp16 pair (1152 + c0, 1152 + c1) from two code bytes of w (already flipped by 0x80)
    __device__ static uint32_t pair_lo(uint32_t w) {
        return (w & 0xffu) | ((w & 0xff00u) << 8) | 0x64006400u;
    }
    __device__ static uint32_t pair_hi(uint32_t w) {
        return ((w >> 16) & 0xffu) | ((w >> 8) & 0xff0000u) | 0x64006400u;
    }
    __device__ static void words(const CodeVec& c, uint32_t (&w)[NW]) {
        if constexpr (NW == 2) {
            w[0] = c.x; w[1] = c.y;
        } else {
            w[0] = c.x; w[1] = c.y; w[2] = c.z; w[3] = c.w;
        }
    }
    __device__ static void partial_scores(const Q& q, const Tile& t, float sc[G][NLD]) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            uint32_t w[NW];
            words(t.k[i], w);
            uint32_t h[PE / 2];
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                const uint32_t x = w[j] ^ 0x80808080u;
                h[2 * j] = pair_lo(x);
                h[2 * j + 1] = pair_hi(x);
            }
            const float ks = f16_lo(t.ks[i]);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < PE / 2; ++j)
                    s = __builtin_amdgcn_fdot2(as_f16x2(q.v[gi][j]), as_f16x2(h[j]), s, false);
                sc[gi][i] = (s - q.off[gi]) * (q.inv[gi] * ks);
            }
        }
    }
    __device__ static void mask_v(Tile& t, int i, bool ok) { t.vs[i] = ok ? t.vs[i] : 0u; }
    __device__ static void init(Extra& x) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) x.corr[gi] = 0.f;
    }
    __device__ static void rescale(Extra& x, int gi, float alpha) { x.corr[gi] *= alpha; }
    __device__ static void accumulate(float (&acc)[G][PE], const float (&p)[G][NLD],
                                      const Tile& t, Extra& x) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            uint32_t w[NW];
            words(t.v[i], w);
            float u[PE];
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                const uint32_t y = w[j] ^ 0x80808080u;
#pragma unroll
                for (int e = 0; e < 4; ++e) u[4 * j + e] = (float)((y >> (8 * e)) & 0xffu);
            }
            const float vs = f16_lo(t.vs[i]);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                const float wv = p[gi][i] * vs;
                x.corr[gi] += wv;
#pragma unroll
                for (int e = 0; e < PE; ++e) acc[gi][e] = fmaf(wv, u[e], acc[gi][e]);
            }
        }
    }
    // sum_t w_t (c_t + 128) - 128 sum_t w_t = sum_t w_t c_t
    __device__ static void finish(float (&acc)[G][PE], const Extra& x) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int e = 0; e < PE; ++e) acc[gi][e] = fmaf(-128.f, x.corr[gi], acc[gi][e]);
    }
};

template <int PE>
__device__ __forceinline__ void store_row(const DecodeArgs& a, size_t idx, const float* v) {
    if (a.out_dtype == PA_F32) {
        float* o = (float*)a.out + idx;
#pragma unroll
        for (int e = 0; e < PE; e += 4) {
            u32x4 w = {__float_as_uint(v[e]), __float_as_uint(v[e + 1]),
                       __float_as_uint(v[e + 2]), __float_as_uint(v[e + 3])};
            st16(o + e, w);
        }
    } else {
        uint32_t w[PE / 2];
#pragma unroll
        for (int e = 0; e < PE; e += 2) {
            uint32_t lo, hi;
            if (a.out_dtype == PA_F16) {
                lo = f32_to_f16_bits(v[e]);
                hi = f32_to_f16_bits(v[e + 1]);
            } else {
                lo = f32_to_bf16_bits(v[e]);
                hi = f32_to_bf16_bits(v[e + 1]);
            }
            w[e / 2] = lo | (hi << 16);
        }
        uint16_t* o = (uint16_t*)a.out + idx;
        if constexpr (PE % 8 == 0) {
#pragma unroll
            for (int j = 0; j < PE / 8; ++j) {
                u32x4 x = {w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
                st16(o + 8 * j, x);
            }
        } else {
            *reinterpret_cast<uint2*>(o) = make_uint2(w[0], w[1]);
        }
    }
}

// One wavefront zeroes one output row (a multiple of 16 bytes).
__device__ inline void zero_row(const DecodeArgs& a, int row, int lane) {
    const int ob = a.out_dtype == PA_F32 ? 4 : 2;
    const size_t bytes = (size_t)a.num_q_heads * a.head_dim * ob;
    char* p = (char*)a.out + (size_t)row * bytes;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (size_t o = (size_t)lane * 16; o < bytes; o += kWave * 16) st16(p + o, z);
}

__device__ __forceinline__ void store_out1(const DecodeArgs& a, size_t idx, float v) {
    if (a.out_dtype == PA_F32) {
        ((float*)a.out)[idx] = v;
    } else if (a.out_dtype == PA_F16) {
        ((uint16_t*)a.out)[idx] = (uint16_t)f32_to_f16_bits(v);
    } else {
        ((uint16_t*)a.out)[idx] = (uint16_t)f32_to_bf16_bits(v);
    }
}

// One round of loads for at most R contributors: every contributor's (max, sum) and output
// slice load together (lane c < nc holds contributor c's (max, sum), every lane its columns
// of each output), so the task, that round and the store are the only dependent steps.
// Indices past nc re-read contributor 0 and get weight 0: no branches, so every load goes
// out before the first wait.
template <int D, int G, int R>
__device__ void merge_round(const DecodeArgs& a, int u, int g, int w_first, int nc,
                            int first_slot, int gi, const float2* pml, const float* pacc,
                            int lane) {
    constexpr int KD = (D + kWave - 1) / kWave;
    auto part = [&](int c) {
        return ((size_t)(w_first + c) * 2 + (c == 0 ? first_slot : 0)) * G + gi;
    };
    const float2 mine = pml[part(lane < nc ? lane : 0)];
    float val[R][KD];
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const float* src = pacc + part(t < nc ? t : 0) * D;
#pragma unroll
        for (int k = 0; k < KD; ++k)
            val[t][k] = (D % 64 == 0 || lane + 64 * k < D) ? src[lane + 64 * k] : 0.f;
    }
    const float M = wave_max(lane < nc ? mine.x : -3.402823466e38f);
    const float f = lane < nc ? __builtin_amdgcn_exp2f(mine.x - M) : 0.f;
    const float den = wave_sum(f * mine.y);
    float num[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) num[k] = 0.f;
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const float ft = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), t));
#pragma unroll
        for (int k = 0; k < KD; ++k) num[k] += ft * val[t][k];
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const size_t obase = ((size_t)u * a.num_q_heads + (size_t)g * G + gi) * D;
#pragma unroll
    for (int k = 0; k < KD; ++k)
        if (D % 64 == 0 || lane + 64 * k < D) store_out1(a, obase + lane + 64 * k, num[k] * inv);
}

// Combine the partials of head gi of pair (u, g) left by wavefronts w_first ..
// w_first + nc - 1 (slot first_slot for the first, slot 0 for the others):
//   out = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c,   M = max_c m_c   (m in log2 units)
// Up to 8 contributors (every cut pair of evenly long sequences) take one round of 8 loads;
// up to 32 (the long pairs of a skewed length mix, cut over many wavefronts) one round of
// 32 (d <= 128); more take rounds of four.
template <int D, int G>
__device__ void merge_pair(const DecodeArgs& a, int u, int g, int w_first, int nc,
                           int first_slot, int gi, const float2* pml, const float* pacc,
                           int lane) {
    constexpr int KD = (D + kWave - 1) / kWave;
    if (nc <= 8) {
        merge_round<D, G, 8>(a, u, g, w_first, nc, first_slot, gi, pml, pacc, lane);
        return;
    }
    if constexpr (D <= 128) {
        if (nc <= 32) {
            merge_round<D, G, 32>(a, u, g, w_first, nc, first_slot, gi, pml, pacc, lane);
            return;
        }
    }
    {
        float M = -3.402823466e38f;
        for (int c0 = 0; c0 < nc; c0 += kWave) {
            const int c = c0 + lane;
            if (c < nc) {
                const int v = w_first + c, slot = c == 0 ? first_slot : 0;
                M = fmaxf(M, pml[((size_t)v * 2 + slot) * G + gi].x);
            }
        }
        M = wave_max(M);
        float den = 0.f, num[KD];
#pragma unroll
        for (int k = 0; k < KD; ++k) num[k] = 0.f;
        for (int c0 = 0; c0 < nc; c0 += kWave) {
            const int c = c0 + lane;
            float f = 0.f;
            if (c < nc) {
                const int v = w_first + c, slot = c == 0 ? first_slot : 0;
                const float2 ml = pml[((size_t)v * 2 + slot) * G + gi];
                f = __builtin_amdgcn_exp2f(ml.x - M);
                den += f * ml.y;
            }
            const int n = nc - c0 < kWave ? nc - c0 : kWave;
            // four contributors per round, all loads issued before any use
            for (int j = 0; j < n; j += 4) {
                float fj[4], val[4][KD];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int jj = j + t < n ? j + t : j;        // in range; weight 0 below
                    fj[t] = j + t < n
                                ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), jj))
                                : 0.f;
                    const int v = w_first + c0 + jj, slot = c0 + jj == 0 ? first_slot : 0;
                    const float* src = pacc + (((size_t)v * 2 + slot) * G + gi) * D;
#pragma unroll
                    for (int k = 0; k < KD; ++k)
                        val[t][k] = lane + 64 * k < D ? src[lane + 64 * k] : 0.f;
                }
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int k = 0; k < KD; ++k) num[k] += fj[t] * val[t][k];
            }
        }
        den = wave_sum(den);
        const float inv = den > 0.f ? 1.f / den : 0.f;
        const size_t obase = ((size_t)u * a.num_q_heads + (size_t)g * G + gi) * D;
#pragma unroll
        for (int k = 0; k < KD; ++k)
            if (lane + 64 * k < D) store_out1(a, obase + lane + 64 * k, num[k] * inv);
    }
}

// A segment: the part of pair (u, g) inside a wavefront's share; blocks j0 .. j1-1 of the
// sequence's table row.
struct Seg {
    int u, g, seq, len, lo_tok, j0, j1;
    uint32_t ps, pe, end;
    bool starts;     // the segment starts at the pair's first block
};
// the first segment of a share, from the plan's record
__device__ inline Seg first_segment_of(const WaveStart& st, int window) {
    Seg sg;
    sg.u = st.u;
    sg.g = st.g;
    sg.seq = st.seq;
    sg.len = st.len;
    sg.lo_tok = (window > 0 && st.len > window) ? st.len - window : 0;
    sg.j0 = st.j0;
    sg.j1 = st.j1;
    sg.ps = st.ps;
    sg.pe = st.pe;
    sg.end = st.x1 < st.pe ? st.x1 : st.pe;
    sg.starts = st.x0 == st.ps;
    return sg;
}
// a wavefront's first-segment record with every field wave-uniform (the record is read by
// vector loads; as uniform values its fields, and the branches on them, stay scalar)
__device__ inline WaveStart uniform_start(const WaveStart& r) {
    WaveStart st;
    st.x0 = (uint32_t)uniform((int)r.x0);
    st.x1 = (uint32_t)uniform((int)r.x1);
    st.u = uniform(r.u);
    st.g = uniform(r.g);
    st.ps = (uint32_t)uniform((int)r.ps);
    st.pe = (uint32_t)uniform((int)r.pe);
    st.j0 = uniform(r.j0);
    st.j1 = uniform(r.j1);
    st.seq = uniform(r.seq);
    st.len = uniform(r.len);
    st.b0 = uniform(r.b0);
    st.b1 = uniform(r.b1);
    return st;
}
// a unit record by scalar loads, one field at a time
__device__ inline UnitInfo ld_unit(const UnitInfo* p) {
    const int32_t* f = reinterpret_cast<const int32_t*>(p);
    UnitInfo ui;
    ui.b_lo = ld_scalar(f);
    ui.nb = ld_scalar(f + 1);
    ui.len = ld_scalar(f + 2);
    ui.seq = ld_scalar(f + 3);
    return ui;
}
// a block id from the table, checked: outside [0, num_blocks) it reads block 0 and is masked
__device__ inline int checked_block(int b, int num_blocks, bool& valid) {
    valid = (unsigned)b < (unsigned)num_blocks;
    return valid ? b : 0;
}

// NEW: the instance that takes the step's new rows (pa_decode_write_attend); the other
// instances compile without any of that code.
template <int DT, int D, int G, int BS = kBlock, bool NEW = false>
__global__ __launch_bounds__(kWavesPerGroup * kWave) void decode_kernel(DecodeArgs a) {
    using S = KvOps<DT, D, G, BS>;
    constexpr int PE = S::PE, LPT = S::LPT, TPI = S::TPI, NLD = S::NLD;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kNegBig = -3.402823466e38f;
    constexpr float kLazy = 8.f;

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
    const WaveStart st = uniform_start(((const WaveStart*)(a.ws + a.lay.wave_st))[wave]);
    // rows with nothing to read are zeros (shared out among all launched wavefronts)
    for (int i = wave; i < n_empty; i += gridDim.x * kWavesPerGroup) zero_row(a, empty[i], lane);
    if (wave >= W) return;
    if (hdr[5] != 0) {   // a group-mode plan: its records are not wave shares
        if (wave == 0 && lane == 0) atomicOr(hdr, kErrPlanMode);
        return;
    }

    const int row = lane / LPT;        // which token of each load this lane holds
    const int col = lane % LPT;        // which PE-element column
    const float qscale = a.scale * kLog2e;
    const size_t head_stride = S::TILE;
    const size_t block_stride = (size_t)a.num_kv_heads * S::TILE;

    const uint32_t x_start = st.x0;
    const uint32_t x_end = st.x1;
    int uh = uniform(st.u);
    if (x_start >= x_end) return;

    // the unit offsets and records are read by scalar loads (uh is wave-uniform), so that
    // describing the next segment does not wait for the tiles in flight
    auto describe = [&](uint32_t xs) {
        while (ld_scalar(cb + uh + 1) <= xs) ++uh;       // skip finished / empty units
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
    // this lane's slice of the segment's G query rows, as loaded
    auto load_q = [&](const Seg& sg, typename S::QRaw& r) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            const size_t qi = ((size_t)sg.u * a.num_q_heads + (size_t)sg.g * G + gi) * D + col * PE;
            S::load_q((const char*)a.q, qi, gi, r);
        }
    };
    auto block_id = [&](int ids, int idx, bool& valid) {
        int b = __builtin_amdgcn_readlane(ids, idx);
        valid = (unsigned)b < (unsigned)a.num_blocks;
        return valid ? b : 0;
    };
    // live = false: the loads are issued (every step then waits for the same count) but
    // read nothing
    auto load_tile = [&](int g, int b, bool live, typename S::Tile& t) {
        S::load_buf((const char*)a.k_cache, (const char*)a.v_cache,
                    (size_t)b * block_stride + (size_t)g * head_stride,
                    live ? (uint32_t)S::TILE : 0u, (uint32_t)S::lane_off(lane), t);
    };
    // With the step's new rows given, a row's newest token (position len - 1) is not in the
    // cache yet: the tiles are read with it masked out, and the segment that reaches the
    // pair's last block adds it from new row u, KV head g (its slot is written by the merge
    // launch that follows).  Lane (row, col) holds bytes 16 col .. +16 of that row.  The
    // loads go out when the segment starts, ahead of its tiles.
    constexpr int RB = D * S::EB;                  // bytes of one token row
    constexpr bool fused = NEW && S::kNewRows;
    auto load_new = [&](const Seg& sg, u32x4& kn, u32x4& vn) {
        const size_t off = ((size_t)sg.u * a.num_kv_heads + (size_t)sg.g) * RB + col * 16;
        kn = ld16((const char*)a.k_new + off);
        vn = ld16((const char*)a.v_new + off);
    };

    // The tiles stream without a break: the load after each block's is the next block of
    // this 64-id chunk, else the first of the next chunk, else the first of the next
    // segment, whose record, queries and first ids load while this segment runs.
    Seg cur = first_segment_of(st, a.window);
    typename S::QRaw qr;
    load_q(cur, qr);
    int ids = load_ids(cur, cur.j0);
    typename S::Tile A, B;
    bool okA, okB;
    load_tile(cur.g, checked_block(st.b0, a.num_blocks, okA), true, A);
    bool first_segment = true;
    int bad = 0;

    for (;;) {
        const bool more = cur.end < x_end;
        Seg nxt = cur;
        typename S::QRaw qn;
        int nids = 0;
        if (more) {
            nxt = describe(cur.end);
            load_q(nxt, qn);
            nids = load_ids(nxt, nxt.j0);
        }
        typename S::Q qv;
        S::prep_q(qr, qv);
        const bool takes_new = fused && cur.end == cur.pe && cur.len > 0;
        u32x4 kn = {0u, 0u, 0u, 0u}, vn = {0u, 0u, 0u, 0u};
        if constexpr (fused)
            if (takes_new) load_new(cur, kn, vn);   // wavefront-uniform
        // a pair cut after this segment and starting in it (only a share's last segment)
        const bool opens_cut = cur.starts && cur.end < cur.pe;

        typename S::Extra ex;
        S::init(ex);
        float m[G], l[G], acc[G][PE];
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            m[gi] = kNegBig;
            l[gi] = 0.f;
#pragma unroll
            for (int e = 0; e < PE; ++e) acc[gi][e] = 0.f;
        }
        const int lo_tok = cur.lo_tok;
        // positions at or past lim are masked; with new rows the newest is not in the tiles
        const int lim_tiles = fused ? cur.len - 1 : cur.len;

        // the tokens t0 + i * TPI + row of tile tl, those in [lo_tok, lim) taken
        auto consume = [&](typename S::Tile& tl, int t0, int lim, bool valid) {
            float sc[G][NLD];
            S::partial_scores(qv, tl, sc);
#pragma unroll
            for (int i = 0; i < NLD; ++i)
#pragma unroll
                for (int gi = 0; gi < G; ++gi) sc[gi][i] = group_sum<LPT>(sc[gi][i]) * qscale;
            if (!valid || t0 < lo_tok || t0 + BS > lim) {   // wavefront-uniform
#pragma unroll
                for (int i = 0; i < NLD; ++i) {
                    const int t = t0 + i * TPI + row;
                    const bool ok = valid && t >= lo_tok && t < lim;
#pragma unroll
                    for (int gi = 0; gi < G; ++gi) sc[gi][i] = ok ? sc[gi][i] : -INFINITY;
                    S::mask_v(tl, i, ok);
                }
            }
            // Lazy rescaling: the running max m only moves when a score exceeds it by more
            // than kLazy (weights then stay below 2^kLazy); the sum and the output use the
            // same m, so the result is unchanged.  The test is wavefront-uniform.
            float mx[G];
            bool grow = false;
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                mx[gi] = sc[gi][0];
#pragma unroll
                for (int i = 1; i < NLD; ++i) mx[gi] = fmaxf(mx[gi], sc[gi][i]);
                grow |= mx[gi] > m[gi] + kLazy;
            }
            if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
                for (int gi = 0; gi < G; ++gi) {
                    const float mn = fmaxf(m[gi], mx[gi]);
                    const float alpha = __builtin_amdgcn_exp2f(m[gi] - mn);
                    m[gi] = mn;
                    l[gi] *= alpha;
#pragma unroll
                    for (int e = 0; e < PE; ++e) acc[gi][e] *= alpha;
                    S::rescale(ex, gi, alpha);
                }
            }
            float p[G][NLD];
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                float sum = 0.f;
#pragma unroll
                for (int i = 0; i < NLD; ++i) {
                    p[gi][i] = __builtin_amdgcn_exp2f(sc[gi][i] - m[gi]);
                    sum += p[gi][i];
                }
                l[gi] += sum;
            }
            S::accumulate(acc, p, tl, ex);
        };

        // plain copies of what the loads need (a select between fields of the two records
        // would keep both records in memory)
        const int g_cur = cur.g, g_nxt = nxt.g, j1_cur = cur.j1;
        // The first block id of the next chunk and of the next segment come by scalar loads:
        // reading them out of a vector-loaded id register at the chunk's end would make the
        // wavefront wait for the tile in flight before issuing the next one.
        const int32_t* bt_cur = a.block_tables + (size_t)cur.seq * a.max_blocks;
        const int nxt_b =
            more ? ld_scalar_at(a.block_tables + (size_t)nxt.seq * a.max_blocks + nxt.j0) : 0;
        int cids = ids;
        for (int c0 = cur.j0;; c0 += kWave) {
            const int n = (j1_cur - c0) < kWave ? (j1_cur - c0) : kWave;
            const bool last_chunk = c0 + kWave >= j1_cur;
            const int nc_ids = last_chunk ? 0 : load_ids(cur, c0 + kWave);
            const int nc_b = last_chunk ? 0 : ld_scalar_at(bt_cur + c0 + kWave);
            // An odd chunk is padded with an empty block (loads of 0 bytes, never consumed),
            // so that the block after the chunk always lands in A: moving a tile from B to A
            // would wait for all loads in flight.
            const int n2 = (n + 1) & ~1;
            // block k of this chunk, the padding, else the next chunk's or next segment's
            // first block; at the very end the same loads read nothing.  Every case issues
            // the same loads, so the wait counts stay exact.
            auto load_next = [&](int k, typename S::Tile& t, bool& ok) {
                if (k < n) {
                    load_tile(g_cur, block_id(cids, k, ok), true, t);
                } else if (k < n2) {
                    ok = false;
                    load_tile(g_cur, 0, false, t);
                } else if (!last_chunk) {
                    load_tile(g_cur, checked_block(nc_b, a.num_blocks, ok), true, t);
                } else if (more) {
                    load_tile(g_nxt, checked_block(nxt_b, a.num_blocks, ok), true, t);
                } else {
                    ok = false;
                    load_tile(g_cur, 0, false, t);
                }
            };
            for (int k = 0;; k += 2) {
                load_next(k + 1, B, okB);
                bad |= !okA;
                consume(A, (c0 + k) * BS, lim_tiles, okA);
                load_next(k + 2, A, okA);
                if (k + 1 < n) {   // wavefront-uniform: the padding is not consumed
                    bad |= !okB;
                    consume(B, (c0 + k + 1) * BS, lim_tiles, okB);
                }
                if (k + 2 >= n) break;
            }
            if (last_chunk) break;
            cids = nc_ids;
        }
        S::finish(acc, ex);

        // combine the TPI rows of the wavefront (log-sum-exp), then write
        const bool complete = cur.starts && cur.end == cur.pe;
        const int slot = first_segment ? 0 : 1;
        const int u = cur.u, g = cur.g;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            float M = m[gi];
#pragma unroll
            for (int msk = LPT; msk < kWave; msk <<= 1) M = fmaxf(M, __shfl_xor(M, msk));
            const float f = __builtin_amdgcn_exp2f(m[gi] - M);
            float lt = l[gi] * f;
#pragma unroll
            for (int e = 0; e < PE; ++e) acc[gi][e] *= f;
#pragma unroll
            for (int msk = LPT; msk < kWave; msk <<= 1) {
                lt += __shfl_xor(lt, msk);
#pragma unroll
                for (int e = 0; e < PE; ++e) acc[gi][e] += __shfl_xor(acc[gi][e], msk);
            }
            if constexpr (fused) {
                if (takes_new) {   // wavefront-uniform: the newest token, one more term
                    const float sn = group_sum<LPT>(dot16<DT>(qv.v[gi], kn)) * qscale;
                    const float mn = fmaxf(M, sn);
                    const float fo = __builtin_amdgcn_exp2f(M - mn);
                    const float fn = __builtin_amdgcn_exp2f(sn - mn);
                    float vf[PE];
                    widen16<DT>(vn, vf);
                    lt = fmaf(lt, fo, fn);
#pragma unroll
                    for (int e = 0; e < PE; ++e) acc[gi][e] = fmaf(acc[gi][e], fo, fn * vf[e]);
                    M = mn;
                }
            }
            if (row == 0) {
                if (complete) {
                    const float inv = lt > 0.f ? 1.f / lt : 0.f;
                    float o[PE];
#pragma unroll
                    for (int e = 0; e < PE; ++e) o[e] = acc[gi][e] * inv;
                    store_row<PE>(a, ((size_t)u * a.num_q_heads + (size_t)g * G + gi) * D + col * PE, o);
                } else {
                    const size_t pi = ((size_t)wave * 2 + slot) * G + gi;
                    if (col == 0) pml[pi] = make_float2(M, lt);
                    float* dst = pacc + pi * D + col * PE;
#pragma unroll
                    for (int e = 0; e < PE; e += 4) {
                        u32x4 w4 = {__float_as_uint(acc[gi][e]), __float_as_uint(acc[gi][e + 1]),
                                    __float_as_uint(acc[gi][e + 2]), __float_as_uint(acc[gi][e + 3])};
                        st16(dst + e, w4);
                    }
                }
            }
        }
        if (opens_cut) {
            // this wavefront holds the pair's first block: leave its merge task (the plan
            // counted the shares the pair spans)
            const int nc = ld_scalar(wcut + wave);
            if (lane == 0) tasks[wave + 1] = make_int4(u, g, nc, first_segment ? 0 : 1);
        }
        if (!more) break;
        cur = nxt;
        qr = qn;
        ids = nids;
        first_segment = false;
    }
    if (bad && lane == 0) atomicOr(hdr, kErrBlockId);
}

}  // namespace pa
