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
// steps of 32 tokens (two blocks).  Each step, the workgroup stages the steps' K and V rows
// in LDS (16-byte coalesced loads; tokens past the sequence, before the window or in a
// block with an invalid id are staged as zeros, so no NaN reaches a product), then every
// wavefront computes
//     S^T[32 tokens][32 M-rows] = K . Q^T            (D/16 MFMAs, K operand from LDS)
// applies the causal / window mask by selection, runs the online softmax per M-row (each
// lane owns one M-row column: a running max and sum, partner lane l^32 holds the rest), and
//     O^T[d][M-row] += V^T . P^T                     (4 * D/32 MFMAs: P = hi + lo)
// where P^T comes straight from the S^T accumulator registers in the MFMA B-operand order
// and V^T is gathered from LDS in the matching token order.  The next step's global loads
// are in flight while the current step computes (LDS double buffer, one barrier per step).
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (DT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ uint32_t to16(float x) {
    if constexpr (DT == DT_BF16) return f32_to_bf16_bits(x);
    else return f32_to_f16_bits(x);
}
template <int DT>
__device__ __forceinline__ float from16(uint32_t b) {
    if constexpr (DT == DT_BF16) return __uint_as_float(b << 16);
    else return f16_lo(b);
}

// P as the sum of two 16-bit numbers: hi = round(p), lo = round(p - hi).  Two MFMAs with
// hi and lo carry P to about 16 significant bits; one 16-bit P alone (2^-9 relative for
// bf16) would put up to ~1e-2 absolute error on rows that see only a few tokens.
template <int DT>
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const uint32_t ha = to16<DT>(a), hb = to16<DT>(b);
    hi = ha | (hb << 16);
    lo = to16<DT>(a - from16<DT>(ha)) | (to16<DT>(b - from16<DT>(hb)) << 16);
}

template <int D>
struct ChunkShape {
    static constexpr int MW = 32;                 // M-rows per wavefront
    static constexpr int STEP = 32;               // tokens per step
    static constexpr int ROWB = D * 2 + 16;       // LDS bytes per staged token row (padded)
    static constexpr int REGION = STEP * ROWB;    // one staged K or V step
    static constexpr int CHUNKS = STEP * D * 2 / 16;            // 16-byte pieces per region
    static constexpr int PER_THREAD = CHUNKS / (kWavesPerGroup * kWave);
    static_assert(CHUNKS % (kWavesPerGroup * kWave) == 0, "staging split");
};

template <int DT, int D, int G>
__global__ __launch_bounds__(kWavesPerGroup * kWave) void chunk_kernel(DecodeArgs a) {
    using S = ChunkShape<D>;
    constexpr int KS = D / 16, DT32 = D / 32, QR = S::MW / G;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kNegBig = -3.402823466e38f;
    __shared__ __attribute__((aligned(16))) char lds[2][2][S::REGION];

    const int32_t* hdr = (const int32_t*)(a.ws + a.lay.header);
    const int2* tiles = (const int2*)(a.ws + a.lay.tiles);
    if ((int)blockIdx.x >= hdr[4]) return;                 // whole workgroup leaves together
    const int2 tl = tiles[blockIdx.x];
    const int s = tl.x, r0 = tl.y, g = blockIdx.y;
    const int L = a.seq_lens[s];
    const int rs = a.query_start_loc[s];
    const int n = a.query_start_loc[s + 1] - rs;
    const int QT = kWavesPerGroup * QR;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 31, h = lane >> 5;

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

    // Q^T operand: 8 elements at d = 16 ks + 8 h of this lane's row and head
    u32x4 qb[KS];
    {
        const char* qp = (const char*)a.q +
            (((size_t)(rs + qrow_c) * a.num_q_heads + (size_t)g * G + gi) * D) * 2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qb[ks] = ld16(qp + (16 * ks + 8 * h) * 2);
    }

    f32x16 acc[DT32];
#pragma unroll
    for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    float m_run = kNegBig, l_run = 0.f;
    const float qscale = a.scale * kLog2e;

    const int32_t* bt = a.block_tables + (size_t)s * a.max_blocks;
    const size_t tile_bytes = (size_t)kBlock * D * 2;
    const size_t block_stride = (size_t)a.num_kv_heads * tile_bytes;
    const int nblk_seq = (L + kBlock - 1) / kBlock;

    // staging: thread piece c -> token c / (D/8), 16-byte column c % (D/8)
    u32x4 sk[S::PER_THREAD], sv[S::PER_THREAD];
    int bad = 0;
    auto stage_load = [&](int t0) {
#pragma unroll
        for (int i = 0; i < S::PER_THREAD; ++i) {
            const int c = tid + i * kWavesPerGroup * kWave;
            const int tt = c / (D / 8), col = c % (D / 8);
            const int t = t0 + tt;
            const u32x4 z = {0u, 0u, 0u, 0u};
            sk[i] = z;
            sv[i] = z;
            if (t < L && t >= lo_first && t / kBlock < nblk_seq) {
                const int b = bt[t / kBlock];
                if ((unsigned)b < (unsigned)a.num_blocks) {
                    const size_t off = (size_t)b * block_stride + (size_t)g * tile_bytes +
                                       (size_t)(t % kBlock) * D * 2 + col * 16;
                    sk[i] = ld16_stream((const char*)a.k_cache + off);
                    sv[i] = ld16_stream((const char*)a.v_cache + off);
                } else {
                    bad = 1;
                }
            }
        }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < S::PER_THREAD; ++i) {
            const int c = tid + i * kWavesPerGroup * kWave;
            const int tt = c / (D / 8), col = c % (D / 8);
            st16(&lds[buf][0][tt * S::ROWB + col * 16], sk[i]);
            st16(&lds[buf][1][tt * S::ROWB + col * 16], sv[i]);
        }
    };

    if (nsteps > 0) {
        stage_load(t_first);
        stage_store(0);
    }
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1, t0 = t_first + st * S::STEP;
        if (st + 1 < nsteps) stage_load(t0 + S::STEP);
        if (t0 <= wp_last && t0 + S::STEP > wlo_first) {      // wavefront-uniform
            const char* kl = lds[buf][0];
            const char* vl = lds[buf][1];
            // S^T = K . Q^T
            f32x16 sc;
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 ka = ld16(kl + j * S::ROWB + (16 * ks + 8 * h) * 2);
                sc = mfma32<DT>(ka, qb[ks], sc);
            }
            // mask (selection), online softmax for this lane's M-row
            float sv16[16];
            float mx = kNegBig;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int t = t0 + 8 * (r / 4) + 4 * h + (r % 4);
                const bool ok = row_ok && t >= lo && t <= pos;
                sv16[r] = ok ? sc[r] * qscale : -INFINITY;
                mx = fmaxf(mx, sv16[r]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mn = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
            m_run = mn;
            float p16[16], psum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p16[r] = __builtin_amdgcn_exp2f(sv16[r] - mn);
                psum += p16[r];
            }
            psum += __shfl_xor(psum, 32);
            l_run = fmaf(l_run, alpha, psum);
#pragma unroll
            for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
            // P^T operands: K-step k2 covers tokens 16 k2 .. 16 k2 + 15; element kk of lane
            // (j, h) is token 16 k2 + (kk < 4 ? 4 h + kk : 8 + 4 h + kk - 4) = p16[8 k2 + kk]
            u32x4 pb[2], pl[2];
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const float* pp = p16 + 8 * k2;
                uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
                split2<DT>(pp[0], pp[1], h0, l0);
                split2<DT>(pp[2], pp[3], h1, l1);
                split2<DT>(pp[4], pp[5], h2, l2);
                split2<DT>(pp[6], pp[7], h3, l3);
                const u32x4 th = {h0, h1, h2, h3}, tl = {l0, l1, l2, l3};
                pb[k2] = th;
                pl[k2] = tl;
            }
            // O^T += V^T . P^T; the V^T operand takes the same token order
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int ta = 16 * k2 + 4 * h, tb = 16 * k2 + 8 + 4 * h;
#pragma unroll
                for (int dt = 0; dt < DT32; ++dt) {
                    const int dcol = (32 * dt + j) * 2;
                    const uint16_t* v0 = (const uint16_t*)(vl + ta * S::ROWB + dcol);
                    const uint16_t* v1 = (const uint16_t*)(vl + tb * S::ROWB + dcol);
                    constexpr int RW = S::ROWB / 2;
                    const u32x4 va = {(uint32_t)v0[0] | ((uint32_t)v0[RW] << 16),
                                      (uint32_t)v0[2 * RW] | ((uint32_t)v0[3 * RW] << 16),
                                      (uint32_t)v1[0] | ((uint32_t)v1[RW] << 16),
                                      (uint32_t)v1[2 * RW] | ((uint32_t)v1[3 * RW] << 16)};
                    acc[dt] = mfma32<DT>(va, pb[k2], acc[dt]);
                    acc[dt] = mfma32<DT>(va, pl[k2], acc[dt]);
                }
            }
        }
        if (st + 1 < nsteps) stage_store(buf ^ 1);
        __syncthreads();
    }
    if (bad) atomicOr((int32_t*)(a.ws + a.lay.header), kErrBlockId);

    // out[row][head][d]: lane holds O^T[d = 32 dt + 8 (r/4) + 4 h + r%4][its M-row]
    if (row_ok) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
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
