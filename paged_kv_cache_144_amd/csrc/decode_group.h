// Paged decode attention in group mode, for sliding-window decode batches: each (row, KV
// head) pair is split among S workgroups of kWavesPerGroup wavefronts, S chosen so that the
// batch's pairs fill the compute units.
//
// A sliding-window layer only sees the last W tokens of a sequence ("KV cache by model",
// sotaaz.com, section on layer kinds), so every pair spans at most W / 16 + 1 blocks and a
// fixed number of wavefronts per pair is balanced by construction.  Wavefront i of the pair
// takes the i-th of its 4 S parts (the plan writes it as its share), streams it exactly as
// decode_kernel does (same tile policies, masking by selection, lazy rescaling), and leaves
// its (max, sum, output) in LDS; after one barrier wavefront 0 of each workgroup combines its
// group's parts with the log-sum-exp rule.  With S = 1 it writes the row.  With S > 1 it
// writes the workgroup's part to the workspace and counts itself in the pair's arrival
// counter (agent-scope release / acquire); the last of the S workgroups to arrive combines
// the S parts in a fixed order, writes the row and resets the counter for the next call.
// No merge launch follows: a window's few hundred pairs would otherwise pay for a whole
// launch.
//
// NEW: the instance that takes the step's new rows (pa_decode_write_attend): the newest
// token comes from the new rows (its slot is not written yet) and the wavefront that took
// it writes it into its slot after its last tile.
#pragma once

#include "decode_impl.h"

namespace pa {

template <int DT, int D, int G, bool NEW = false>
__global__ __launch_bounds__(kWavesPerGroup * kWave) void decode_group_kernel(DecodeArgs a) {
    constexpr int GW = kWavesPerGroup;
    using S = KvOps<DT, D, G, kBlock>;
    constexpr int BS = kBlock;
    constexpr int PE = S::PE, LPT = S::LPT, TPI = S::TPI, NLD = S::NLD;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kNegBig = -3.402823466e38f;
    constexpr float kLazy = 8.f;
    constexpr bool fused = NEW && S::kNewRows;
    constexpr int RB = D * S::EB;                  // bytes of one token row
    __shared__ float group_lds[GW * G * (D + 2)];  // [wavefront][head][max, sum, D outputs]

    int32_t* hdr = (int32_t*)(a.ws + a.lay.header);
    const int32_t* empty = (const int32_t*)(a.ws + a.lay.empty);
    const int W = hdr[2], n_empty = hdr[3];
    const int wi = threadIdx.x >> 6;
    const int wave = uniform(blockIdx.x * GW + wi);
    const int lane = lane_id();
    const int row = lane / LPT, col = lane % LPT;
    const WaveStart st = ((const WaveStart*)(a.ws + a.lay.wave_st))[wave];
    // rows with nothing to read are zeros (shared out among all launched wavefronts)
    for (int i = wave; i < n_empty; i += gridDim.x * GW) zero_row(a, empty[i], lane);
    // nothing planned (W = 0: the plan found bad row ranges), or a plan for another mode:
    // the same for every workgroup, so no wavefront reaches the barrier below
    const int split = a.group_mode;                // workgroups per pair
    if (W != (int)gridDim.x * GW || hdr[5] != split) {
        if (W > 0 && wave == 0 && lane == 0) atomicOr(hdr, kErrPlanMode);
        return;
    }

    const float qscale = a.scale * kLog2e;
    const size_t head_stride = S::TILE;
    const size_t block_stride = (size_t)a.num_kv_heads * S::TILE;
    const int n = st.j1 - st.j0;                   // this wavefront's blocks: 0 .. 64
    const int len = st.len, g = st.g;
    const int lo_tok = (a.window > 0 && len > a.window) ? len - a.window : 0;
    // the newest token, when the new rows are given: taken by the wavefront holding the
    // pair's last block, masked out of the tiles
    const bool takes_new = fused && n > 0 && st.x1 == st.pe && len > 0;
    const int lim = fused ? len - 1 : len;

    float m[G], l[G], acc[G][PE];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        m[gi] = kNegBig;
        l[gi] = 0.f;
#pragma unroll
        for (int e = 0; e < PE; ++e) acc[gi][e] = 0.f;
    }
    typename S::Q qv;
    u32x4 kn = {0u, 0u, 0u, 0u}, vn = {0u, 0u, 0u, 0u};
    int bad = 0;
    if (n > 0) {   // wavefront-uniform
        typename S::QRaw qr;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            const size_t qi = ((size_t)st.u * a.num_q_heads + (size_t)g * G + gi) * D + col * PE;
            S::load_q((const char*)a.q, qi, gi, qr);
        }
        const int ids =
            lane < n ? a.block_tables[(size_t)st.seq * a.max_blocks + st.j0 + lane] : 0;
        if constexpr (fused) {
            if (takes_new) {
                const size_t off = ((size_t)st.u * a.num_kv_heads + (size_t)g) * RB + col * 16;
                kn = ld16((const char*)a.k_new + off);
                vn = ld16((const char*)a.v_new + off);
            }
        }
        auto load_tile = [&](int b, bool live, typename S::Tile& t) {
            S::load_buf((const char*)a.k_cache, (const char*)a.v_cache,
                        (size_t)b * block_stride + (size_t)g * head_stride,
                        live ? (uint32_t)S::TILE : 0u, (uint32_t)S::lane_off(lane), t);
        };
        auto block_id = [&](int idx, bool& valid) {
            const int b = __builtin_amdgcn_readlane(ids, idx);
            valid = (unsigned)b < (unsigned)a.num_blocks;
            return valid ? b : 0;
        };
        // block k of the share, else (past the end) the same loads reading nothing, so that
        // every step waits for the same count
        auto load_next = [&](int k, typename S::Tile& t, bool& ok) {
            if (k < n) {
                load_tile(block_id(k, ok), true, t);
            } else {
                ok = false;
                load_tile(0, false, t);
            }
        };
        typename S::Tile A, B;
        bool okA, okB;
        load_tile(checked_block(st.b0, a.num_blocks, okA), true, A);
        S::prep_q(qr, qv);
        typename S::Extra ex;
        S::init(ex);

        // the tokens t0 + i * TPI + row of tile tl, those in [lo_tok, lim) taken
        auto consume = [&](typename S::Tile& tl, int t0, bool valid) {
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
            // lazy rescaling: m only moves when a score exceeds it by more than kLazy
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

        // two tiles in flight: the next block's loads go out before the current one is used
        // (deeper rings measured slower: more loads queue on the compute unit)
        for (int k = 0;; k += 2) {
            load_next(k + 1, B, okB);
            bad |= !okA;
            consume(A, (st.j0 + k) * BS, okA);
            if (k + 1 >= n) break;
            load_next(k + 2, A, okA);
            bad |= !okB;
            consume(B, (st.j0 + k + 1) * BS, okB);
            if (k + 2 >= n) break;
        }
        S::finish(acc, ex);
    }

    // combine the TPI rows of the wavefront (log-sum-exp), fold in the newest token, and
    // leave the result in this wavefront's LDS slots (an empty share leaves max = kNegBig,
    // sum 0, output 0)
    float* my = group_lds + wi * G * (D + 2);
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
            float* sl = my + gi * (D + 2);
            if (col == 0) {
                sl[0] = M;
                sl[1] = lt;
            }
#pragma unroll
            for (int e = 0; e < PE; ++e) sl[2 + col * PE + e] = acc[gi][e];
        }
    }
    if constexpr (fused) {
        // the newest token into its slot, after this wavefront's last tile load
        if (takes_new && row == 0) {
            const int b = a.block_tables[(size_t)st.seq * a.max_blocks + (len - 1) / BS];
            if ((unsigned)b < (unsigned)a.num_blocks) {
                const size_t at = (size_t)b * block_stride + (size_t)g * head_stride +
                                  (size_t)((len - 1) % BS) * RB + (size_t)col * 16;
                st16((char*)a.k_cache + at, kn);
                st16((char*)a.v_cache + at, vn);
            }
        }
    }
    if (bad && lane == 0) atomicOr(hdr, kErrBlockId);
    __syncthreads();   // every wavefront of the group reaches it
    if (wi != 0) return;

    // wavefront 0 combines the group's parts of pair blockIdx.x / split; the lanes of token
    // row 0 hold the output columns
    float Mg[G], lg[G], og[G][PE];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        float Mk[GW];
        Mg[gi] = kNegBig;
#pragma unroll
        for (int k = 0; k < GW; ++k) {
            Mk[k] = group_lds[(k * G + gi) * (D + 2)];
            Mg[gi] = fmaxf(Mg[gi], Mk[k]);
        }
        lg[gi] = 0.f;
#pragma unroll
        for (int e = 0; e < PE; ++e) og[gi][e] = 0.f;
#pragma unroll
        for (int k = 0; k < GW; ++k) {
            const float* sl = group_lds + (k * G + gi) * (D + 2);
            const float f = __builtin_amdgcn_exp2f(Mk[k] - Mg[gi]);
            lg[gi] = fmaf(f, sl[1], lg[gi]);
#pragma unroll
            for (int e = 0; e < PE; ++e) og[gi][e] = fmaf(f, sl[2 + col * PE + e], og[gi][e]);
        }
    }
    const int pair = (int)blockIdx.x / split;
    if (split > 1) {
        // publish this group's part, then count it in the pair's arrival counter; the last
        // group to arrive combines all parts of the pair
        float2* pml = (float2*)(a.ws + a.lay.part_ml);
        float* pacc = (float*)(a.ws + a.lay.part_acc);
        int32_t* arrivals = (int32_t*)(a.ws + a.lay.tasks);
        if (row == 0) {
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                const size_t pi = (size_t)blockIdx.x * G + gi;
                if (col == 0) pml[pi] = make_float2(Mg[gi], lg[gi]);
                float* dst = pacc + pi * D + col * PE;
#pragma unroll
                for (int e = 0; e < PE; e += 4) {
                    u32x4 w = {__float_as_uint(og[gi][e]), __float_as_uint(og[gi][e + 1]),
                               __float_as_uint(og[gi][e + 2]), __float_as_uint(og[gi][e + 3])};
                    st16(dst + e, w);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        int before = 0;
        if (lane == 0)
            before = __hip_atomic_fetch_add(arrivals + pair, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        before = __builtin_amdgcn_readfirstlane(before);
        if (before != split - 1) return;            // another group of the pair is still out
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (lane == 0)
            __hip_atomic_store(arrivals + pair, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (row == 0) {
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                // the pair's parts in a fixed order (the result does not depend on which
                // group arrived last)
                Mg[gi] = kNegBig;
                for (int k = 0; k < split; ++k)
                    Mg[gi] = fmaxf(Mg[gi], pml[((size_t)pair * split + k) * G + gi].x);
                lg[gi] = 0.f;
#pragma unroll
                for (int e = 0; e < PE; ++e) og[gi][e] = 0.f;
                for (int k = 0; k < split; ++k) {
                    const size_t pi = ((size_t)pair * split + k) * G + gi;
                    const float2 ml = pml[pi];
                    const float f = __builtin_amdgcn_exp2f(ml.x - Mg[gi]);
                    lg[gi] = fmaf(f, ml.y, lg[gi]);
                    const float* src = pacc + pi * D + col * PE;
#pragma unroll
                    for (int e = 0; e < PE; e += 4) {
                        const u32x4 w = ld16(src + e);
                        og[gi][e] = fmaf(f, __uint_as_float(w[0]), og[gi][e]);
                        og[gi][e + 1] = fmaf(f, __uint_as_float(w[1]), og[gi][e + 1]);
                        og[gi][e + 2] = fmaf(f, __uint_as_float(w[2]), og[gi][e + 2]);
                        og[gi][e + 3] = fmaf(f, __uint_as_float(w[3]), og[gi][e + 3]);
                    }
                }
            }
        }
    }
    if (row == 0) {
        const int u = pair / a.num_kv_heads, gg = pair % a.num_kv_heads;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            const float inv = lg[gi] > 0.f ? 1.f / lg[gi] : 0.f;
#pragma unroll
            for (int e = 0; e < PE; ++e) og[gi][e] *= inv;
            store_row<PE>(a, ((size_t)u * a.num_q_heads + (size_t)gg * G + gi) * D + col * PE,
                          og[gi]);
        }
    }
}

}  // namespace pa
