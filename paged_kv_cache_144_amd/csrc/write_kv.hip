// pa_write_kv: scatter each new token's K and V rows into the cache slot its block table
// assigned.  "vLLM and PagedAttention" notes (ghkdgus29.github.io), section on basic
// decoding: a new token's KV entry goes after the existing ones in its logical block,
// which the manager has mapped to a physical block.
//
// One thread moves 16 bytes of one (token, KV head) row of K and the same 16 bytes of V.
// A row is head_dim * elem_bytes bytes (128 .. 1024), so consecutive threads read and write
// consecutive 16-byte pieces: both sides are fully coalesced.  Slots are int64; a negative
// slot, or one past the pool, is skipped, so no write ever leaves the pool.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Index type I: 32-bit when the number of 16-byte pieces fits, which avoids emulated 64-bit
// divisions.  The K and V pieces are loaded before the slot is known (their source is always
// in range), so the slot load and the data loads are in flight together.  Block sizes are
// powers of two (8, 16, 32): the slot splits into block and row with a shift and a mask.
template <typename I>
__global__ __launch_bounds__(256) void write_kv_kernel(
    const char* __restrict__ k, const char* __restrict__ v, const int64_t* __restrict__ slots,
    I n_chunks, int chunks_per_row, int hkv, int bs_log2, int64_t pool_slots,
    char* __restrict__ kc, char* __restrict__ vc) {
    const I stride = (I)gridDim.x * blockDim.x;
    for (I i = (I)blockIdx.x * blockDim.x + threadIdx.x; i < n_chunks; i += stride) {
        const I row = i / (I)chunks_per_row;          // (token, head) row
        const int c = (int)(i - row * (I)chunks_per_row);
        const I tok = row / (I)hkv;
        const int h = (int)(row - tok * (I)hkv);
        const size_t src = (size_t)i * 16;
        const u32x4 kx = ld16(k + src), vx = ld16(v + src);
        const int64_t slot = slots[tok];
        if (slot < 0 || slot >= pool_slots) continue;
        const int64_t blk = slot >> bs_log2, off = slot & ((1 << bs_log2) - 1);
        const int64_t dst = (((blk * hkv + h) << bs_log2) + off) * chunks_per_row * 16 + c * 16;
        st16(kc + dst, kx);
        st16(vc + dst, vx);
    }
}

// 8-bit caches ("KV cache by model", sotaaz.com: one scale per 32 values).  One thread
// quantizes one group of 32 consecutive values of one (token, head) row: scale = the
// group's largest |x| / 127 (fp32), rounded to fp16 (held at 65504 if it would overflow);
// code = round-half-to-even(x / scale) clamped to [-127, 127], both divisions IEEE fp32.
// Codes go to the token's row of its (block, head) tile, the scale to the tile's scale row.
template <int ADT>
__device__ __forceinline__ void quantize_group(const char* src, char* codes, char* scale) {
    float x[kQ8Group];
#pragma unroll
    for (int j = 0; j < kQ8Group / 8; ++j) widen16<ADT>(ld16(src + 16 * j), x + 8 * j);
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < kQ8Group; ++e) amax = fmaxf(amax, fabsf(x[e]));
    uint32_t sb = f32_to_f16_bits(amax / 127.f);
    if ((sb & 0x7fffu) == 0x7c00u) sb = 0x7bffu;              // overflow: largest fp16
    const float s = f16_lo(sb);
    uint32_t w[kQ8Group / 4];
#pragma unroll
    for (int j = 0; j < kQ8Group / 4; ++j) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float c = s > 0.f ? __builtin_rintf(x[4 * j + b] / s) : 0.f;
            c = fminf(fmaxf(c, -127.f), 127.f);
            word |= ((uint32_t)(int)c & 0xffu) << (8 * b);
        }
        w[j] = word;
    }
    st16(codes, u32x4{w[0], w[1], w[2], w[3]});
    st16(codes + 16, u32x4{w[4], w[5], w[6], w[7]});
    *reinterpret_cast<uint16_t*>(scale) = (uint16_t)sb;
}

template <int ADT>
__global__ __launch_bounds__(256) void write_kv_q8_kernel(
    const char* __restrict__ k, const char* __restrict__ v, const int64_t* __restrict__ slots,
    int64_t n_groups, int groups_per_row, int hkv, int d, int64_t pool_slots,
    char* __restrict__ kc, char* __restrict__ vc) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_groups; i += stride) {
        const int64_t row = i / groups_per_row;       // (token, head) row
        const int gr = (int)(i - row * groups_per_row);
        const int64_t tok = row / hkv;
        const int h = (int)(row - tok * hkv);
        const int64_t slot = slots[tok];
        if (slot < 0 || slot >= pool_slots) continue;
        const int64_t blk = slot / kBlock, off = slot % kBlock;
        const int64_t tile = (blk * hkv + h) * (int64_t)(kBlock + 1) * d;
        const int64_t code_off = tile + off * d + gr * kQ8Group;
        const int64_t scale_off = tile + (int64_t)kBlock * d + (off * groups_per_row + gr) * 2;
        const int64_t src = i * kQ8Group * 2;
        quantize_group<ADT>(k + src, kc + code_off, kc + scale_off);
        quantize_group<ADT>(v + src, vc + code_off, vc + scale_off);
    }
}

hipError_t launch_write_kv_q8(const void* k, const void* v, const int64_t* slots, int32_t n,
                              void* kc, void* vc, int32_t nb, int32_t hkv, int32_t d,
                              int act_dtype, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int groups_per_row = d / kQ8Group;
    const int64_t n_groups = (int64_t)n * hkv * groups_per_row;
    int64_t blocks = (n_groups + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    auto fn = act_dtype == DT_F16 ? write_kv_q8_kernel<DT_F16> : write_kv_q8_kernel<DT_BF16>;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(256), 0, stream, (const char*)k,
                       (const char*)v, slots, n_groups, groups_per_row, hkv, d,
                       (int64_t)nb * kBlock, (char*)kc, (char*)vc);
    return hipGetLastError();
}

hipError_t launch_write_kv(const void* k, const void* v, const int64_t* slots, int32_t n,
                           void* kc, void* vc, int32_t nb, int32_t bs, int32_t hkv, int32_t d,
                           int32_t elem_bytes, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int chunks_per_row = d * elem_bytes / 16;
    const int64_t n_chunks = (int64_t)n * hkv * chunks_per_row;
    int64_t blocks = (n_chunks + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    int bs_log2 = 0;
    while ((1 << bs_log2) < bs) ++bs_log2;
    if ((1 << bs_log2) != bs) return hipErrorInvalidValue;   // 8, 16 or 32 only
    // 32-bit indices while the grid-stride loop cannot overflow them
    if (n_chunks + (int64_t)blocks * 256 < ((int64_t)1 << 31)) {
        hipLaunchKernelGGL(write_kv_kernel<int32_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const char*)k, (const char*)v, slots, (int32_t)n_chunks,
                           chunks_per_row, hkv, bs_log2, (int64_t)nb * bs, (char*)kc, (char*)vc);
    } else {
        hipLaunchKernelGGL(write_kv_kernel<int64_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const char*)k, (const char*)v, slots, n_chunks, chunks_per_row, hkv,
                           bs_log2, (int64_t)nb * bs, (char*)kc, (char*)vc);
    }
    return hipGetLastError();
}

}  // namespace pa
