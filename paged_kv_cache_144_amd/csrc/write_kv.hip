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

__global__ __launch_bounds__(256) void write_kv_kernel(
    const char* __restrict__ k, const char* __restrict__ v, const int64_t* __restrict__ slots,
    int64_t n_chunks, int chunks_per_row, int hkv, int64_t pool_slots, char* __restrict__ kc,
    char* __restrict__ vc) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_chunks; i += stride) {
        const int64_t row = i / chunks_per_row;       // (token, head) row
        const int c = (int)(i - row * chunks_per_row);
        const int64_t tok = row / hkv;
        const int h = (int)(row - tok * hkv);
        const int64_t slot = slots[tok];
        if (slot < 0 || slot >= pool_slots) continue;
        const int64_t blk = slot / kBlock, off = slot % kBlock;
        const int64_t dst = (((blk * hkv + h) * kBlock + off) * chunks_per_row + c) * 16;
        const int64_t src = i * 16;
        st16(kc + dst, ld16(k + src));
        st16(vc + dst, ld16(v + src));
    }
}

hipError_t launch_write_kv(const void* k, const void* v, const int64_t* slots, int32_t n,
                           void* kc, void* vc, int32_t nb, int32_t hkv, int32_t d,
                           int32_t elem_bytes, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int chunks_per_row = d * elem_bytes / 16;
    const int64_t n_chunks = (int64_t)n * hkv * chunks_per_row;
    int64_t blocks = (n_chunks + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(write_kv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const char*)k, (const char*)v, slots, n_chunks, chunks_per_row, hkv,
                       (int64_t)nb * kBlock, (char*)kc, (char*)vc);
    return hipGetLastError();
}

}  // namespace pa
