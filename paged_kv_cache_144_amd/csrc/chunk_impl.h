// Chunked-prefill rows on the matrix cores (gfx950 MFMA 32x32x16, fp16 / bf16 in, fp32
// accumulate).
//
// A prompt chunk of n rows at context length L sits at positions L - n .. L - 1; row r
// attends to positions [lo_r, L - n + r] (causal; lo_r > 0 only under a sliding window).
// Chunked prefill mixes such chunks with decode rows in one batch (duolabs.co.kr, section on
// paging-based KV management); K/V are gathered through the block table as for decode
// ("PagedAttention deep dive", donmain.dev, section on splitting the KV cache into blocks).
// Unlike decode rows, the rows of a chunk share their K/V, so the work is a dense
// contraction: Q tile x K tile and P x V tile, done here with MFMA.
//
// Mapping.  One workgroup = (chunk tile of QT rows, KV head g); its 4 wavefronts each own 32
// "M-rows" (query row, query head of the group), QT = 4 * 32 / G.  The context is walked in
// steps of 32 tokens (two blocks).  Each step, the workgroup stages the step's K and V in
// LDS (16-byte coalesced loads; tokens past the sequence, before the window or in a block
// with an invalid id are staged as zeros, so no NaN reaches a product), both row-major.
// Then every wavefront computes
//     S^T[32 tokens][32 M-rows] = K . Q^T            (D/16 MFMAs, K operand from LDS)
// applies the causal / window mask by selection (only on steps that straddle a row's edge),
// runs the online softmax per M-row (each lane owns one M-row column; partner lane l^32
// holds the other half of the step's tokens), and
//     O^T[d][M-row] += V^T . P^T                     (2 * D/32 fp16 MFMAs)
// where P^T comes straight from the S^T accumulator registers in the MFMA B-operand order
// and the V^T operand is two LDS transpose reads in the matching token order.  P and V
// enter that product in fp16 for both cache types: bf16 V is converted as it is staged,
// exactly wherever |v| lies in fp16's range.  A bf16 value beyond that range becomes an
// infinity, which leaves non-finite accumulators; the workgroup then computes its tile
// again in a second pass that stages V as bf16 and carries P as hi + lo bf16 parts (two
// MFMAs per product).  The running max is raised only when a row's new maximum exceeds it
// by more than 2^8 (weights stay <= 256), so the accumulators are rescaled on few steps.
// The next steps' global loads are in flight while the current step computes (LDS double
// buffer, one barrier per step).
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (DT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Lane l's value and lane (l ^ 32)'s (gfx950 v_permlane32_swap: the two halves of the
// wavefront trade places), one of each per lane in some order: enough for a max or a sum
// over the two halves without an LDS round trip.
__device__ __forceinline__ float2 with_partner(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// gfx950 LDS transpose read of 4 x 16-bit elements (ds_read_b64_tr_b16)
__device__ __forceinline__ u32x2 tr_read(const char* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
}

template <int D>
struct ChunkShape {
    static constexpr int MW = 32;                 // M-rows per wavefront
    static constexpr int STEP = 32;               // tokens per step
    static constexpr int ROWB = D * 2 + 16;       // LDS bytes per staged K token row (padded)
    // LDS bytes per staged V token row: padded so that the row stride is 16 dwords mod 64,
    // which keeps the transpose reads of the P.V operand (below) off shared banks
    static constexpr int ROWV = D * 2 + 4 * ((16 - D / 2 % 64 + 64) % 64);
    static constexpr int KREG = STEP * ROWB;
    static constexpr int VREG = STEP * ROWV;
    static constexpr int THREADS = kWavesPerGroup * kWave;
    static constexpr int KPIECES = STEP * D / 8;        // 16-byte pieces of K per step
    static constexpr int VPIECES = STEP * D / 8;        // 16-byte pieces of V per step
    static constexpr int KPT = (KPIECES + THREADS - 1) / THREADS;
    static constexpr int VPT = (VPIECES + THREADS - 1) / THREADS;
};

template <int DT, int D, int G>
// d <= 128: two workgroups per CU.  d = 256 needs more than 256 VGPRs: one wavefront per
// SIMD (512 registers).  Its fp16 instances spill nothing; the bf16 ones, which also hold the
// second pass, spill 2-4 registers (12-20 bytes of scratch memory per lane).
__global__ __launch_bounds__(kWavesPerGroup * kWave, D <= 128 ? 2 : 1) void chunk_kernel(DecodeArgs a) {
    using S = ChunkShape<D>;
    constexpr int KS = D / 16, DT32 = D / 32, QR = S::MW / G;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kNegBig = -3.402823466e38f;
    __shared__ __attribute__((aligned(16))) char lds_k[2][S::KREG];
    __shared__ __attribute__((aligned(16))) char lds_v[2][S::VREG];
    __shared__ int lds_vover;                  // a staged bf16 V value is beyond fp16's range
    constexpr bool kConvV = DT == DT_BF16;

    const int32_t* hdr = (const int32_t*)(a.ws + a.lay.header);
    const int2* tiles = (const int2*)(a.ws + a.lay.tiles);
    // Workgroup i of a.max_tiles * Hkv takes tile position i / Hkv for KV head i % Hkv: the
    // tiles in use come first, and as workgroups are dispatched round-robin over the XCDs,
    // every tile of a chunk that reads one KV head's K/V runs on the same XCD and shares its
    // L2 (when Hkv is a multiple of the XCD count).  The second half of the positions takes
    // the tiles in reverse order: a chunk's tiles grow longer with their rows, and the two
    // workgroups that share a CU (positions t and t + NT / 2 when one round holds them all)
    // then pair a long tile with a short one, which evens the work per CU.
    const int nt = hdr[4];
    const int tpos = (int)blockIdx.x / a.num_kv_heads;
    const int g = (int)blockIdx.x - tpos * a.num_kv_heads;
    if (tpos >= nt) return;                                // whole workgroup leaves together
    const int half = (nt + 1) / 2;
    const int tile = tpos < half ? tpos : nt - 1 - (tpos - half);
    const int2 tl = tiles[tile];
    const int s = tl.x, r0 = tl.y;
    const int L = a.seq_lens[s];
    const int rs = a.query_start_loc[s];
    const int n = a.query_start_loc[s + 1] - rs;
    const int QT = kWavesPerGroup * QR;

    const int tid = threadIdx.x, lane = tid & 63;
    __builtin_assume(tid < S::THREADS);
    // the wavefront index as a scalar, so that its row and token bounds below are scalars
    // and the steps it skips or masks branch on the scalar unit
    const int wave = uniform(tid >> 6);
    const int j = lane & 31, h = lane >> 5;
    // the V row this lane names in the P.V transpose reads (see the product below)
    const int v_lane = (4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * S::ROWV +
                       (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

    // this lane's M-row (column of S^T and O^T)
    const int m = wave * S::MW + j;
    const int qrow = r0 + m / G, gi = m % G;
    const bool row_ok = qrow < n;
    const int qrow_c = row_ok ? qrow : n - 1;
    const int pos = L - n + qrow_c;                                   // this row's position
    const int lo = (a.window > 0 && pos - a.window + 1 > 0) ? pos - a.window + 1 : 0;

    // the workgroup's token range [t_first, p_last]
    const int r_last = (r0 + QT < n ? r0 + QT : n) - 1;
    const int p_last = L - n + r_last, p_first = L - n + r0;
    const int lo_first = (a.window > 0 && p_first - a.window + 1 > 0) ? p_first - a.window + 1 : 0;
    const int t_first = (lo_first / S::STEP) * S::STEP;
    const int nsteps = p_last >= t_first ? (p_last - t_first) / S::STEP + 1 : 0;
    // wavefront-uniform bounds of its rows, to skip steps none of them sees
    const int wr_last = min(r0 + (wave + 1) * QR, n) - 1;
    const int wp_last = L - n + wr_last;
    const int wlo_first = (a.window > 0) ? max(0, L - n + r0 + wave * QR - a.window + 1) : 0;
    // a step needs no mask when every row of the wavefront exists and sees all its tokens
    const bool w_rows_full = r0 + (wave + 1) * QR <= n;
    const int wp_first = L - n + r0 + wave * QR;
    const int wlo_last = (a.window > 0) ? max(0, wp_last - a.window + 1) : 0;
    // A range [lo, hi] of step starts, kept as lo and hi - lo so that a test is one unsigned
    // compare; an empty range (hi < lo, or !ok) holds no step start.
    struct Span {
        uint32_t lo, n;
        __device__ bool has(int t) const { return (uint32_t)t - lo <= n; }
    };
    auto make_span = [](int lo, int hi, bool ok) {
        return ok && hi >= lo ? Span{(uint32_t)lo, (uint32_t)(hi - lo)} : Span{1u << 30, 0u};
    };
    // the steps some row of the wavefront sees: t0 <= wp_last and t0 + STEP > wlo_first
    const Span w_steps = make_span(wlo_first - (S::STEP - 1), wp_last, true);
    // the steps every row of the wavefront sees whole: all its rows exist,
    // t0 + STEP - 1 <= wp_first and t0 >= wlo_last
    const Span w_full = make_span(wlo_last, wp_first - (S::STEP - 1), w_rows_full);

    // Q^T operand: 8 elements at d = 16 ks + 8 h of this lane's row and head
    u32x4 qb[KS];
    {
        const char* qp = (const char*)a.q +
            (((size_t)(rs + qrow_c) * a.num_q_heads + (size_t)g * G + gi) * D) * 2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qb[ks] = ld16(qp + (16 * ks + 8 * h) * 2);
            // a negative scale is carried by Q's signs (exact for 16-bit values), so the
            // softmax below always scales by a non-negative factor
            if (a.scale < 0.f) qb[ks] ^= 0x80008000u;
        }
    }

    f32x16 acc[DT32];
    // m_run: the running max (log2 units), the same in the two lanes of an M-row;
    // l_run: this lane's part of the weight sum (its half of each step's tokens), the two
    // parts added once at the end
    float m_run, l_run;
    const float qscale = fabsf(a.scale) * kLog2e;

    const int32_t* bt = a.block_tables + (size_t)s * a.max_blocks;
    const size_t tile_bytes = (size_t)kBlock * D * 2;
    const size_t block_stride = (size_t)a.num_kv_heads * tile_bytes;

    // staging.  K and V piece c -> token c / (D/8), 16-byte column c % (D/8), both
    // row-major in LDS.
    // two register sets: the loads of the next two steps are in flight during a step.
    // Every lane issues the same loads in every case (a position outside the row range or
    // in a block with an invalid id reads the cache's first bytes instead, and the masked
    // store zeroes it), so that the compiler's wait counts for one register set never
    // include the other set's loads.  What the store needs to know of the set's step is
    // scalar: its first token, which of its two blocks are staged, and whether all of its
    // tokens are.
    // flags: bit 0 / 1 the step's first / second block is staged, bit 2 all its tokens are
    struct Stage {
        u32x4 k[S::KPT], v[S::VPT];
        int t0, flags;
    };
    Stage sg[2];
    // Block ids are uniform over the workgroup: scalar loads, counted apart from the vector
    // loads.  The table row is read in range only: a step's first token lies before L (the
    // steps past the last repeat it), and its second block is read only when it starts
    // before L (else the first block's entry is read again, and not used).
    typedef const __attribute__((address_space(4))) int32_t* ConstIds;
    const ConstIds btc = (ConstIds)bt;
    const uint64_t goff = (uint64_t)g * tile_bytes;
    // A step's two block ids (-1: the block is outside the row's range).  (Fetching them a
    // step early measured slower: scalar loads share the LDS wait counter, so the next
    // step's first products then wait for them too.)
    struct StepIds {
        int t0, id0, id1;
    };
    auto step_ids = [&](int t0) {
        const uint32_t b0 = (uint32_t)t0 / kBlock;
        const bool two = t0 + kBlock < L;
        const int r0 = btc[b0], r1 = btc[two ? b0 + 1 : b0];
        return StepIds{t0, t0 + kBlock > lo_first ? r0 : -1,
                       two && t0 + 2 * kBlock > lo_first ? r1 : -1};
    };
    // the steps inside the row range, t0 >= lo_first and t0 + STEP <= L, when every block
    // id the tile reads is in the pool (set by the check before the loop)
    Span in_steps = make_span(0, -1, false);
    // The step's loads: scalar base offsets of its two blocks (the cache's first tile for a
    // block outside the row's range or with an invalid id); each lane's pieces sit at a
    // fixed 32-bit offset from one of them.  A step inside the row's range, [lo_first, L),
    // with valid ids (the common case) takes a short scalar path: two table entries, two
    // products, all its tokens staged.
    auto stage_load = [&](int t0, Stage& st) {
        uint64_t base[2];
        st.t0 = t0;
        if (in_steps.has(t0)) {
            const uint32_t b0 = (uint32_t)t0 / kBlock;
            const int id0 = btc[b0], id1 = btc[b0 + 1];
            st.flags = 7;
            base[0] = (uint64_t)(uint32_t)id0 * (uint32_t)block_stride + goff;
            base[1] = (uint64_t)(uint32_t)id1 * (uint32_t)block_stride + goff;
        } else {
            const StepIds ids = step_ids(t0);
            const int id0 = ids.id0, id1 = ids.id1;
            const bool ok0 = (uint32_t)id0 < (uint32_t)a.num_blocks;
            const bool ok1 = (uint32_t)id1 < (uint32_t)a.num_blocks;
            st.flags = (int)ok0 | (int)ok1 << 1 |
                       (int)(ok0 && ok1 && t0 >= lo_first && t0 + S::STEP <= L) << 2;
            base[0] = ok0 ? (uint64_t)(uint32_t)id0 * (uint32_t)block_stride + goff : 0;
            base[1] = ok1 ? (uint64_t)(uint32_t)id1 * (uint32_t)block_stride + goff : 0;
        }
#pragma unroll
        for (int i = 0; i < S::KPT; ++i) {
            const int c = (tid + i * S::THREADS) % S::KPIECES;
            const int tau = c / (D / 8);
            const uint32_t lane_off = (uint32_t)((tau % kBlock) * D * 2 + (c % (D / 8)) * 16);
            st.k[i] = ld16_stream((const char*)a.k_cache + base[tau / kBlock] + lane_off);
        }
#pragma unroll
        for (int i = 0; i < S::VPT; ++i) {
            const int c = (tid + i * S::THREADS) % S::VPIECES;
            const int tau = c / (D / 8);
            const uint32_t lane_off = (uint32_t)((tau % kBlock) * D * 2 + (c % (D / 8)) * 16);
            st.v[i] = ld16_stream((const char*)a.v_cache + base[tau / kBlock] + lane_off);
        }
    };
    // bf16 V -> fp16, rounded to nearest: exact for |v| in fp16's normal range, within
    // 2^-25 below it; |v| >= 65520 becomes an infinity (caught after the pass, below).
    auto v_to_f16 = [&](const u32x4& x) {
        u32x4 y;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float lo = __uint_as_float(x[w] << 16);
            const float hi = __uint_as_float(x[w] & 0xffff0000u);
            y[w] = cvt2<DT_F16>(lo, hi);
        }
        return y;
    };
    // A step whose tokens are all staged (the common case) stores without the per-piece
    // selects: the store body is instantiated with and without masks, chosen by a scalar
    // branch.  Cc: the fp16 pass (bf16 V converted) or the bf16 pass.
    auto stage_store = [&](auto Cc, int buf, const Stage& st) {
        constexpr bool kConv = decltype(Cc)::value && kConvV;
        auto put = [&](auto masked_c) {
            constexpr bool kMasked = decltype(masked_c)::value;
            const u32x4 z = {0u, 0u, 0u, 0u};
            // token tau of the step is staged: its block is, and it lies in [lo_first, L)
            auto pick = [&](int tau, const u32x4& x) {
                if constexpr (kMasked) {
                    const int t = st.t0 + tau;
                    const bool on = (st.flags >> (tau / kBlock) & 1) && t < L && t >= lo_first;
                    return on ? x : z;
                } else {
                    return x;
                }
            };
#pragma unroll
            for (int i = 0; i < S::KPT; ++i) {
                const int c = tid + i * S::THREADS;
                if (c < S::KPIECES)
                    st16(&lds_k[buf][(c / (D / 8)) * S::ROWB + (c % (D / 8)) * 16],
                         pick(c / (D / 8), st.k[i]));
            }
#pragma unroll
            for (int i = 0; i < S::VPT; ++i) {
                const int c = tid + i * S::THREADS;
                if (c < S::VPIECES) {
                    u32x4 x = pick(c / (D / 8), st.v[i]);
                    if constexpr (kConv) x = v_to_f16(x);
                    st16(&lds_v[buf][(c / (D / 8)) * S::ROWV + (c % (D / 8)) * 16], x);
                }
            }
        };
        if (st.flags & 4)
            put(std::false_type{});
        else
            put(std::true_type{});
    };

    // loads past the last step repeat the last step (never staged: the same loads in every
    // case keep the wait counts exact)
    const int t_last = t_first + (nsteps > 0 ? nsteps - 1 : 0) * S::STEP;
    // A block id outside the pool sets the error bit (its tokens are staged as zeros).  The
    // ids the steps read, blocks t_first / 16 .. t_last / 16 + 1 that start before L and
    // end after lo_first, are checked once here, spread over the workgroup's threads.
    {
        bool bad = false;
        for (int b = t_first / kBlock + tid; b <= t_last / kBlock + 1; b += S::THREADS)
            if (kBlock * b < L && kBlock * b + kBlock > lo_first)
                bad |= (uint32_t)bt[b] >= (uint32_t)a.num_blocks;
        if (bad) atomicOr((int32_t*)(a.ws + a.lay.header), kErrBlockId);
        const bool ids_ok = __builtin_amdgcn_readfirstlane(__syncthreads_or(bad)) == 0;
        in_steps = make_span(lo_first, L - S::STEP, ids_ok);
    }
    auto step_t = [&](int st) { return min(t_first + st * S::STEP, t_last); };
    // step st computes from LDS buffer st & 1 while steps st+1 (register set (st+1) & 1)
    // and st+2 are loading; then st+1 goes to LDS and step st+3 starts loading into the
    // set st+1 used.  P = (st + 1) & 1 is a compile-time constant.
    auto body = [&](auto Cc, auto Pc, int st) {
        constexpr int P = decltype(Pc)::value;
        constexpr bool kF16PV = DT == DT_F16 || decltype(Cc)::value;
        const int buf = st & 1, t0 = t_first + st * S::STEP;
        if (w_steps.has(t0)) {                                  // wavefront-uniform
            const char* kl = lds_k[buf];
            const char* vl = lds_v[buf];
            // S^T = K . Q^T (raw dot products)
            f32x16 sc;
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[r] = 0.f;
            if constexpr (KS <= 8) {
                // the step's K operands are all read before the first product (the
                // scheduling barrier keeps them there), so that the chain waits for one
                // LDS latency, not one per product.  d = 256 has no registers to spare.
                u32x4 ka[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    ka[ks] = ld16(kl + j * S::ROWB + (16 * ks + 8 * h) * 2);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) sc = mfma32<DT>(ka[ks], qb[ks], sc);
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const u32x4 ka = ld16(kl + j * S::ROWB + (16 * ks + 8 * h) * 2);
                    sc = mfma32<DT>(ka, qb[ks], sc);
                }
            }
            // The V^T operand of the P.V product for tokens 16 k2 .. 16 k2 + 15 and columns
            // 32 dt .. 32 dt + 31 (the transpose reads are described at the product below).
            // Where registers allow (d <= 128), the first half is read before the softmax,
            // so that its LDS latency passes during the exponentials.
            auto v_operand = [&](int k2, int dt) {
                const char* p0 = vl + v_lane + (16 * k2) * S::ROWV + 64 * dt;
                const u32x2 t0 = tr_read(p0), t1 = tr_read(p0 + 8 * S::ROWV);
                return u32x4{t0.x, t0.y, t1.x, t1.y};
            };
            constexpr bool kEarlyV = KS <= 8;
            u32x4 va0[DT32];
            if constexpr (kEarlyV) {
#pragma unroll
                for (int dt = 0; dt < DT32; ++dt) va0[dt] = v_operand(0, dt);
            }
            // element r of this lane is token t0 + 8 (r/4) + 4 h + r%4 of its M-row
            const bool full = w_full.has(t0);
            float p16[16];
            // element r is visible: it lies in this lane's visible token range of the step,
            // [tlo, thi] as offsets 0..31 (both less 4 h, so that element r compares a
            // constant).  Where registers allow (d <= 128), only masked steps compute the
            // range; at d = 256 every step does, which keeps that instance from spilling.
            auto range = [&](int& tlo_h, int& thi_h) {
                tlo_h = (row_ok ? max(lo - t0, 0) : 32) - 4 * h;
                thi_h = (row_ok ? min(pos - t0, 31) : -1) - 4 * h;
            };
            int tlo_e = 0, thi_e = 0;
            if constexpr (KS > 8) range(tlo_e, thi_e);
            auto vis = [&](int r) {
                int tlo_h = tlo_e, thi_h = thi_e;
                if constexpr (KS <= 8) range(tlo_h, thi_h);
                const int tt = 8 * (r / 4) + (r % 4);
                return tt >= tlo_h && tt <= thi_h;
            };
            // the weights p = 2^(s qscale - m_run) with the running max as it stands, and
            // this lane's sum of them
            auto weights = [&]() {
                if (full) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        p16[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], qscale, -m_run));
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        p16[r] = vis(r) ? __builtin_amdgcn_exp2f(fmaf(sc[r], qscale, -m_run))
                                        : 0.f;
                }
                float ps = p16[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) ps += p16[r];
                return ps;
            };
            float psum = weights();
            // The running max is raised only when the step's maximum exceeds it by more than
            // 8 (log2), and then some weight exceeds 2^8: steps where no lane's sum reaches
            // 2^8 (the common case, and the first step always does: m_run starts at the
            // lowest float) need neither the maximum nor the exchange with the partner lane.
            if (__ballot(psum >= 256.f)) {                     // wavefront-uniform
                float mx = -INFINITY;
                if (full) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, vis(r) ? sc[r] : -INFINITY);
                }
                {
                    const float2 pm = with_partner(mx);
                    mx = fmaxf(pm.x, pm.y);
                }
                const float mxs = mx > -INFINITY ? mx * qscale : -INFINITY;
                if (__ballot(mxs > m_run + 8.f)) {             // wavefront-uniform
                    const float mn = fmaxf(m_run, mxs);
                    const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
                    m_run = mn;
                    l_run *= alpha;
#pragma unroll
                    for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
                    psum = weights();
                }
            }
            l_run += psum;
            // P^T operands: K-step k2 covers tokens 16 k2 .. 16 k2 + 15; element kk of lane
            // (j, h) is token 16 k2 + (kk < 4 ? 4 h + kk : 8 + 4 h + kk - 4) = p16[8 k2 + kk].
            // fp16 pass: P rounded to nearest fp16 (2^-11 relative; p <= 2^8 here).  bf16
            // pass: P = hi + lo bf16 parts (about 16 significant bits).
            u32x4 pb[2], pl[2];
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const float* pp = p16 + 8 * k2;
                if constexpr (kF16PV) {
                    const u32x4 th = {cvt2<DT_F16>(pp[0], pp[1]), cvt2<DT_F16>(pp[2], pp[3]),
                                      cvt2<DT_F16>(pp[4], pp[5]), cvt2<DT_F16>(pp[6], pp[7])};
                    pb[k2] = th;
                } else {
                    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
                    split2<DT>(pp[0], pp[1], h0, l0);
                    split2<DT>(pp[2], pp[3], h1, l1);
                    split2<DT>(pp[4], pp[5], h2, l2);
                    split2<DT>(pp[6], pp[7], h3, l3);
                    const u32x4 th = {h0, h1, h2, h3}, tl2 = {l0, l1, l2, l3};
                    pb[k2] = th;
                    pl[k2] = tl2;
                }
            }
            // O^T += V^T . P^T.  Lane (j, h) needs column j of tokens 16 k2 + 4 h .. +3 and
            // 16 k2 + 8 + 4 h .. +3, in that order: two LDS transpose reads (each lane of a
            // 16-lane group names one 4-element row; lane 4a+b receives element b of the rows
            // named by lanes a, a+4, a+8, a+12) over V staged row-major.  Lane s of a group
            // names token 4 h + s/4 at columns 4 (s%4) of its group's 16-column half.
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
                for (int dt = 0; dt < DT32; ++dt) {
                    const u32x4 va = k2 == 0 && kEarlyV ? va0[dt] : v_operand(k2, dt);
                    if constexpr (kF16PV) {
                        acc[dt] = mfma32<DT_F16>(va, pb[k2], acc[dt]);
                    } else {
                        acc[dt] = mfma32<DT>(va, pb[k2], acc[dt]);
                        acc[dt] = mfma32<DT>(va, pl[k2], acc[dt]);
                    }
                }
            }
        }
        if (st + 1 < nsteps) stage_store(Cc, buf ^ 1, sg[P]);
        stage_load(step_t(st + 3), sg[P]);
        __syncthreads();
    };
    // one pass over the tile's steps
    auto pass = [&](auto Cc) {
#pragma unroll
        for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
        m_run = kNegBig;
        l_run = 0.f;
        stage_load(step_t(0), sg[0]);
        if (nsteps > 0) stage_store(Cc, 0, sg[0]);
        stage_load(step_t(1), sg[1]);
        stage_load(step_t(2), sg[0]);
        __syncthreads();
        for (int st = 0; st < nsteps; st += 2) {
            body(Cc, std::integral_constant<int, 1>{}, st);
            if (st + 1 < nsteps) body(Cc, std::integral_constant<int, 0>{}, st + 1);
        }
    };
    if (tid == 0) lds_vover = 0;
    __syncthreads();
    pass(std::true_type{});
    if constexpr (kConvV) {
        // A staged bf16 value beyond fp16's range became an infinity, and every product it
        // entered left an infinite or NaN (0 x inf) accumulator in each wavefront that
        // computed its step; finite accumulators stay far below the float range, so the
        // sum of |acc| is finite exactly when none is.  Such a tile is computed again with
        // V kept in bf16.  (A NaN in V also takes that pass; its output is NaN either way.)
        float sa = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) sa += fabsf(acc[dt][r]);
        if (!(sa < INFINITY)) lds_vover = 1;
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(lds_vover) != 0) pass(std::false_type{});
    }

    // out[row][head][d]: lane holds O^T[d = 32 dt + 8 (r/4) + 4 h + r%4][its M-row]
    // the row's weight sum: this lane's part and its partner's (taken by every lane)
    const float2 lp = with_partner(l_run);
    const float l_row = lp.x + lp.y;
    if (row_ok) {
        const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
        const size_t obase = ((size_t)(rs + qrow) * a.num_q_heads + (size_t)g * G + gi) * D;
#pragma unroll
        for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d0 = 32 * dt + 8 * q4 + 4 * h;
                const float o0 = acc[dt][4 * q4] * inv, o1 = acc[dt][4 * q4 + 1] * inv;
                const float o2 = acc[dt][4 * q4 + 2] * inv, o3 = acc[dt][4 * q4 + 3] * inv;
                if (a.out_dtype == PA_F32) {
                    const u32x4 w = {__float_as_uint(o0), __float_as_uint(o1),
                                     __float_as_uint(o2), __float_as_uint(o3)};
                    st16((float*)a.out + obase + d0, w);
                } else {
                    const uint32_t w0 = a.out_dtype == PA_F16
                        ? f32_to_f16_bits(o0) | (f32_to_f16_bits(o1) << 16)
                        : f32_to_bf16_bits(o0) | (f32_to_bf16_bits(o1) << 16);
                    const uint32_t w1 = a.out_dtype == PA_F16
                        ? f32_to_f16_bits(o2) | (f32_to_f16_bits(o3) << 16)
                        : f32_to_bf16_bits(o2) | (f32_to_bf16_bits(o3) << 16);
                    *reinterpret_cast<uint2*>((uint16_t*)a.out + obase + d0) = make_uint2(w0, w1);
                }
            }
    }
}

}  // namespace pa
