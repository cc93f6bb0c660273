// pa_copy_blocks: the device half of copy-on-write.  "vLLM and PagedAttention" notes
// (ghkdgus29.github.io), section on parallel sampling: when samples that share a block
// write different tokens into it, the block is copied and each sample keeps its own.
//
// One workgroup per (copy, KV head).  The rows a copy moves, rows 0 .. entries-1 of one
// (block, head) tile, are one contiguous run of entries * row_bytes bytes in both blocks, so
// the workgroup moves 16-byte pieces of K and then of V with consecutive threads on
// consecutive addresses.  An 8-bit tile also carries a row of scales after its 16 code
// rows; the entries' scales (scale_bytes each, a multiple of 4) are copied in 4-byte
// pieces.  A triple with an id outside the pool, or a row count outside [0, block_size], is
// skipped and reported; nothing outside the two tiles is touched.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ kc,
                                                          char* __restrict__ vc,
                                                          const int32_t* __restrict__ copies,
                                                          int nb, int hkv, int bs,
                                                          int row_bytes, int scale_bytes,
                                                          int32_t* err) {
    const int c = blockIdx.x, h = blockIdx.y;
    const int src = copies[3 * c], dst = copies[3 * c + 1], rows = copies[3 * c + 2];
    if (src < 0 || src >= nb || dst < 0 || dst >= nb || rows < 0 || rows > bs) {
        if (err && h == 0 && threadIdx.x == 0) atomicOr(err, kErrBlockId);
        return;
    }
    const int64_t tile = (int64_t)bs * (row_bytes + scale_bytes);
    const int64_t from = ((int64_t)src * hkv + h) * tile;
    const int64_t to = ((int64_t)dst * hkv + h) * tile;
    const int n = rows * (row_bytes / 16);
    for (int i = threadIdx.x; i < 2 * n; i += blockDim.x) {
        char* base = i < n ? kc : vc;
        const int j = i < n ? i : i - n;
        st16(base + to + (int64_t)j * 16, ld16(base + from + (int64_t)j * 16));
    }
    if (scale_bytes) {
        const int64_t so = (int64_t)bs * row_bytes;
        const int m = rows * (scale_bytes / 4);
        for (int i = threadIdx.x; i < 2 * m; i += blockDim.x) {
            char* base = i < m ? kc : vc;
            const int j = i < m ? i : i - m;
            *reinterpret_cast<uint32_t*>(base + to + so + (int64_t)j * 4) =
                *reinterpret_cast<const uint32_t*>(base + from + so + (int64_t)j * 4);
        }
    }
}

// Swapping: one workgroup per (pair, KV head) moves the whole tile (16-byte pieces of K,
// then of V) from one pool to another; either may be pinned host memory, reached over the
// host link.
__global__ __launch_bounds__(256) void swap_blocks_kernel(const char* __restrict__ sk,
                                                          const char* __restrict__ sv,
                                                          char* __restrict__ dk,
                                                          char* __restrict__ dv,
                                                          const int32_t* __restrict__ pairs,
                                                          int src_nb, int dst_nb, int hkv,
                                                          int tile_bytes, int32_t* err) {
    const int c = blockIdx.x, h = blockIdx.y;
    const int src = pairs[2 * c], dst = pairs[2 * c + 1];
    if (src < 0 || src >= src_nb || dst < 0 || dst >= dst_nb) {
        if (err && h == 0 && threadIdx.x == 0) atomicOr(err, kErrBlockId);
        return;
    }
    const int64_t from = ((int64_t)src * hkv + h) * tile_bytes;
    const int64_t to = ((int64_t)dst * hkv + h) * tile_bytes;
    const int n = tile_bytes / 16;
    for (int i = threadIdx.x; i < 2 * n; i += blockDim.x) {
        const bool k = i < n;
        const int64_t j = (int64_t)(k ? i : i - n) * 16;
        st16((k ? dk : dv) + to + j, ld16((k ? sk : sv) + from + j));
    }
}

hipError_t launch_swap_blocks(const void* sk, const void* sv, void* dk, void* dv,
                              const int32_t* pairs, int32_t n, int32_t src_nb, int32_t dst_nb,
                              int32_t hkv, int32_t tile_bytes, int32_t* err,
                              hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(swap_blocks_kernel, dim3((unsigned)n, (unsigned)hkv), dim3(256), 0,
                       stream, (const char*)sk, (const char*)sv, (char*)dk, (char*)dv, pairs,
                       src_nb, dst_nb, hkv, tile_bytes, err);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(void* kc, void* vc, const int32_t* copies, int32_t n,
                              int32_t nb, int32_t hkv, int32_t bs, int32_t row_bytes,
                              int32_t scale_bytes, int32_t* err, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n, (unsigned)hkv), dim3(256), 0,
                       stream, (char*)kc, (char*)vc, copies, nb, hkv, bs, row_bytes,
                       scale_bytes, err);
    return hipGetLastError();
}

}  // namespace pa
