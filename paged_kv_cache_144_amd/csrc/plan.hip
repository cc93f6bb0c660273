// Plan kernel of pa_decode (one workgroup).
//
// Validates lengths and row ranges, turns every decode query row into a decode unit, lays
// all (unit, KV head) pairs end to end in one linear space of KV blocks, and cuts that
// space into equal shares, one per wavefront worker of the decode kernel.  A pair that fits
// inside one share is finished by that wavefront; a pair cut by share boundaries leaves
// partial (max, sum, unnormalised output) results that the last of its wavefronts combines
// with the log-sum-exp rule.  Equal shares keep every worker busy for the same number of
// blocks whatever the length mix (log-normal lengths differ by three orders of magnitude).
// Rows of chunks (several query rows) go to the chunk kernel's tile list instead.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ void unit_range(int32_t len, int32_t window, int32_t bs,
                                           int32_t& b_lo, int32_t& nb) {
    // a row at length len sees positions [lo, len); with a window only the last `window`
    if (len <= 0) {
        b_lo = 0;
        nb = 0;
        return;
    }
    const int32_t lo = (window > 0 && len > window) ? len - window : 0;
    b_lo = lo / bs;
    nb = (len + bs - 1) / bs - b_lo;
}

// A sequence is accepted when 0 <= L <= min(max_seq_len, block_size * max_blocks).  Rows that would
// sit before position 0 (more rows than context) see nothing and give zeros.
__device__ __forceinline__ bool len_ok(const DecodeArgs& a, int L) {
    return L >= 0 && L <= a.max_seq_len && (int64_t)L <= (int64_t)a.max_blocks * a.block_size;
}


// Inclusive scan of one value per thread over the workgroup (Hillis-Steele in LDS).
__device__ uint32_t block_scan(uint32_t* buf, uint32_t v) {
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const uint32_t add = tid >= off ? buf[tid - off] : 0u;
        __syncthreads();
        buf[tid] += add;
        __syncthreads();
    }
    return buf[tid];
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(DecodeArgs a) {
    int32_t* hdr = (int32_t*)(a.ws + a.lay.header);
    uint32_t* cb = (uint32_t*)(a.ws + a.lay.cb);
    uint32_t* cw = (uint32_t*)(a.ws + a.lay.cw);
    UnitInfo* unit = (UnitInfo*)(a.ws + a.lay.unit);
    uint32_t* wx0 = (uint32_t*)(a.ws + a.lay.wave_x0);
    int32_t* wu = (int32_t*)(a.ws + a.lay.wave_u);
    int32_t* empty = (int32_t*)(a.ws + a.lay.empty);
    int2* tiles = (int2*)(a.ws + a.lay.tiles);
    int4* tasks = (int4*)(a.ws + a.lay.tasks);
    WaveStart* wst = (WaveStart*)(a.ws + a.lay.wave_st);

    __shared__ uint32_t s_blk[kPlanThreads], s_til[kPlanThreads], s_pr[kPlanThreads];
    __shared__ int s_err, s_bad, s_empty;
    const int tid = threadIdx.x;
    if (tid == 0) { s_err = 0; s_bad = 0; s_empty = 0; }
    __syncthreads();

    const int B = a.num_seqs, U = a.total_q_rows;
    const int per = (B + kPlanThreads - 1) / kPlanThreads;
    const int s0 = min(B, tid * per), s1 = min(B, s0 + per);
    const int QT = a.chunk_rows;
    const uint32_t H = (uint32_t)a.num_kv_heads;

    // pass 1: validate; count decode blocks, (row, KV head) pairs with blocks, chunk tiles
    uint32_t my_blk = 0, my_til = 0, my_pr = 0;
    int err = 0, bad = 0;
    for (int s = s0; s < s1; ++s) {
        int r0 = s, r1 = s + 1;
        if (a.query_start_loc) { r0 = a.query_start_loc[s]; r1 = a.query_start_loc[s + 1]; }
        if (r0 < 0 || r1 < r0 || r1 > U || (s == 0 && r0 != 0) || (s == B - 1 && r1 != U)) {
            bad = 1;
            continue;
        }
        const int n = r1 - r0, L = a.seq_lens[s];
        if (!len_ok(a, L)) {
            err |= kErrSeqLen;
            continue;
        }
        if (QT > 0 && n >= 2) {          // a chunk: rows go to the MFMA kernel
            my_til += (uint32_t)((n + QT - 1) / QT);
            continue;
        }
        for (int r = 0; r < n; ++r) {
            int32_t b_lo, nb;
            unit_range(L - n + r + 1, a.window, a.block_size, b_lo, nb);
            my_blk += (uint32_t)nb * H;                          // one pair per KV head
            if (nb > 0) my_pr += H;
        }
    }
    if (bad) atomicOr(&s_bad, 1);
    if (err) atomicOr(&s_err, err);
    const uint32_t blk_incl = block_scan(s_blk, my_blk);
    const uint32_t til_incl = block_scan(s_til, my_til);
    const uint32_t pr_incl = block_scan(s_pr, my_pr);
    const uint32_t T = s_blk[kPlanThreads - 1];
    const uint32_t NT = s_til[kPlanThreads - 1];
    const uint32_t NP = s_pr[kPlanThreads - 1];

    // W wavefronts, at least min_blocks blocks each (when there are that many), at most
    // max_waves.  W <= T / min_blocks + 1 makes T / W >= min_blocks / 2 for T >= min_blocks,
    // so consecutive share starts in the weighted space lie at least 4 T / W - 1 quarter
    // blocks apart; a pair cost C with C + 4 below that keeps every share non-empty (a
    // share start at offset o of a pair maps to the pair's first block while o <= C).
    int W = 0;
    uint32_t C = 0;
    if (a.group_mode) {
        W = a.max_waves;   // 4 group_mode wavefronts per (row, KV head), empty or not
    } else if (T > 0) {
        const uint32_t mb = (uint32_t)a.min_blocks;
        W = (int)((T + mb - 1) / mb);
        W = W < 1 ? 1 : (W > a.max_waves ? a.max_waves : W);
        // Whole rounds of one workgroup per compute unit: a partial round would put a
        // second workgroup on a few units, whose shared bandwidth then sets the kernel's
        // length (fewer, longer shares keep every property below).
        if (W < a.max_waves && a.wave_round > 0 && W > a.wave_round)
            W = W / a.wave_round * a.wave_round;
        const uint32_t room = (uint32_t)(4ull * T / (uint32_t)W);
        C = (uint32_t)a.pair_cost;
        if (W > 1) C = room >= C + 5 ? C : (room > 5 ? room - 5 : 0);
    }
    const uint32_t TW = 4u * T + C * NP;
    const uint32_t wt_incl = 4u * blk_incl + C * pr_incl;
    const uint32_t my_wt = 4u * my_blk + C * my_pr;
    if (s_bad || NT > (uint32_t)a.max_tiles) {
        // row ranges cannot be trusted (or would overflow the tile list): no unit, no write
        if (tid == 0) {
            hdr[0] = s_err | kErrSeqLen;
            hdr[1] = 0; hdr[2] = 0; hdr[3] = 0; hdr[4] = 0; hdr[5] = a.group_mode;
        }
        return;
    }

    // pass 2: units, their offsets in the linear block space, chunk tiles
    uint32_t off = blk_incl - my_blk, toff = til_incl - my_til, woff = wt_incl - my_wt;
    for (int s = s0; s < s1; ++s) {
        int r0 = s, r1 = s + 1;
        if (a.query_start_loc) { r0 = a.query_start_loc[s]; r1 = a.query_start_loc[s + 1]; }
        const int n = r1 - r0, L = a.seq_lens[s];
        const bool ok = len_ok(a, L);
        const bool chunk = ok && QT > 0 && n >= 2;
        if (chunk) {
            // the rows' unit records are written by all threads below; here the tiles and
            // the sequence's offset (no decode blocks: every row keeps the same offset)
            for (int q0 = 0; q0 < n; q0 += QT) tiles[toff++] = make_int2(s, q0);
            cb[r0] = off;
            cw[r0] = woff;
            continue;
        }
        for (int r = 0; r < n; ++r) {
            UnitInfo ui{0, 0, 0, s};
            if (ok) {
                ui.len = max(0, L - n + r + 1);
                unit_range(ui.len, a.window, a.block_size, ui.b_lo, ui.nb);
            }
            unit[r0 + r] = ui;
            cb[r0 + r] = off;
            cw[r0 + r] = woff;
            off += (uint32_t)ui.nb * H;
            if (ui.nb > 0) woff += (4u * (uint32_t)ui.nb + C) * H;
        }
    }
    if (tid == 0) {
        cb[U] = T;
        cw[U] = TW;
    }
    __syncthreads();
    // rows of chunk sequences: marked for the chunk kernel, offset of their first row
    for (int i = tid; i < (int)NT * QT; i += kPlanThreads) {
        const int2 tl = tiles[i / QT];
        const int rs = a.query_start_loc[tl.x];
        const int n = a.query_start_loc[tl.x + 1] - rs;
        const int r = tl.y + i % QT;
        if (r < n) {
            const int u = rs + r;
            unit[u] = UnitInfo{-1, 0, 0, tl.x};
            if (u != rs) {
                cb[u] = cb[rs];
                cw[u] = cw[rs];
            }
        }
    }

    __syncthreads();

    // every task slot the merge kernel may look at starts empty (in group mode: every
    // pair's arrival counter starts at zero)
    for (int w = tid; w <= a.max_waves; w += kPlanThreads) tasks[w] = make_int4(0, 0, 0, 0);
    // rows with nothing to read (empty context, or rejected lengths) get zeros later
    for (int u = tid; u < U; u += kPlanThreads)
        if (unit[u].nb == 0 && unit[u].b_lo >= 0) empty[atomicAdd(&s_empty, 1)] = u;
    // The shares cut the weighted space evenly: wavefront w's share starts at weighted
    // position y(w) = floor(w TW / W), where a pair weighs 4 nb + C quarter blocks (its
    // blocks plus the fixed cost of starting a segment).  y(w) falls inside unit u exactly
    // when ceil(cw[u] W / TW) <= w < ceil(cw[u+1] W / TW); these ranges tile [0, W).  A
    // position in a pair's first C quarters maps to the pair's first block, one further on
    // to the next whole block.  Consecutive y differ by at least 31 >= C + 4, so every share
    // holds at least one block and the shares are consecutive.
    for (int u = tid; u < U && W > 0 && !a.group_mode; u += kPlanThreads) {
        const uint64_t c0 = cw[u], c1 = cw[u + 1];
        if (c1 == c0) continue;
        const uint64_t w0 = (c0 * (uint64_t)W + TW - 1) / TW;
        uint64_t w1 = (c1 * (uint64_t)W + TW - 1) / TW;
        if (w1 > (uint64_t)W) w1 = W;
        const uint32_t nb = (uint32_t)unit[u].nb, pw = 4u * nb + C;
        for (uint64_t w = w0; w < w1; ++w) {
            const uint32_t y = (uint32_t)((w * TW) / (uint64_t)W) - (uint32_t)c0;
            const uint32_t g = y / pw, o = y - g * pw;
            uint32_t k = o <= C ? 0u : (o - C + 3) / 4;
            k = k < nb ? k : nb;
            wx0[w] = cb[u] + g * nb + k;
            wu[w] = u;
        }
    }
    // group mode: wavefront i of the N = 4 group_mode wavefronts of pair (u, g) takes blocks
    // [i nb / N, (i + 1) nb / N) of the pair (an empty share when the pair has fewer blocks);
    // the pairs' arrival counters live in the task slots zeroed above
    for (int w = tid; w < W && a.group_mode; w += kPlanThreads) {
        const int N = kWavesPerGroup * a.group_mode, pr = w / N, i = w % N;
        const int u = pr / (int)H, g = pr % (int)H;
        const UnitInfo ui = unit[u];
        const uint32_t nb = ui.nb > 0 ? (uint32_t)ui.nb : 0u;
        const uint32_t ps = cb[u] + (uint32_t)g * nb;
        WaveStart st{};
        st.x0 = ps + (uint32_t)i * nb / N;
        st.x1 = ps + (uint32_t)(i + 1) * nb / N;
        st.u = u;
        st.g = g;
        st.ps = ps;
        st.pe = ps + nb;
        st.j0 = ui.b_lo + (int32_t)(st.x0 - ps);
        st.j1 = ui.b_lo + (int32_t)(st.x1 - ps);
        st.seq = ui.seq;
        st.len = ui.len;
        if (st.x1 > st.x0) {
            const int32_t* bt = a.block_tables + (size_t)ui.seq * a.max_blocks;
            st.b0 = bt[st.j0];
            st.b1 = st.j0 + 1 < st.j1 ? bt[st.j0 + 1] : st.b0;
        }
        wst[w] = st;
        wx0[w] = st.x0;
        wu[w] = u;
    }
    __syncthreads();
    if (tid == 0) wx0[W] = T;
    __syncthreads();
    // each share's first segment, as the decode kernels would find it from wx0 and wu
    for (int w = tid; w < W && !a.group_mode; w += kPlanThreads) {
        const uint32_t x0 = wx0[w], x1 = wx0[w + 1];
        int u = wu[w];
        while (cb[u + 1] <= x0) ++u;                 // skip finished / empty units
        const UnitInfo ui = unit[u];
        const uint32_t nb = (uint32_t)ui.nb, base = cb[u];
        const uint32_t g = (x0 - base) / nb;
        const uint32_t ps = base + g * nb, pe = ps + nb;
        const uint32_t end = x1 < pe ? x1 : pe;
        WaveStart st;
        st.x0 = x0;
        st.x1 = x1;
        st.u = u;
        st.g = (int32_t)g;
        st.ps = ps;
        st.pe = pe;
        st.j0 = ui.b_lo + (int32_t)(x0 - ps);
        st.j1 = ui.b_lo + (int32_t)(end - ps);
        st.seq = ui.seq;
        st.len = ui.len;
        const int32_t* bt = a.block_tables + (size_t)ui.seq * a.max_blocks;
        st.b0 = bt[st.j0];
        st.b1 = st.j0 + 1 < st.j1 ? bt[st.j0 + 1] : st.b0;
        wst[w] = st;
        // A pair that starts inside this share and runs past its end is cut: its first
        // wavefront writes its merge task, whose contributor count is the number of shares
        // that start before the pair's end.  Only the share's last segment can open such a
        // pair.  The count replaces the unit index in wu (read above, by this thread only).
        int nc = 0;
        {
            int ul = u;
            while (cb[ul + 1] <= x1 - 1) ++ul;       // the unit of the share's last block
            const uint32_t nbl = (uint32_t)unit[ul].nb, bl = cb[ul];
            const uint32_t psl = bl + (x1 - 1 - bl) / nbl * nbl, pel = psl + nbl;
            if (psl >= x0 && pel > x1) {
                // first share index past w that starts at or after pel (wx0[W] = T >= pel)
                int lo = w + 1, hi = W;
                while (lo < hi) {
                    const int mid = (lo + hi) / 2;
                    if (wx0[mid] < pel) lo = mid + 1; else hi = mid;
                }
                nc = lo - w;
            }
        }
        wu[w] = nc;
    }
    if (tid == 0) {
        hdr[0] = s_err; hdr[1] = (int32_t)T; hdr[2] = W; hdr[3] = s_empty; hdr[4] = (int32_t)NT;
        hdr[5] = a.group_mode;
    }
}

hipError_t launch_plan(const DecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
