// Dispatch of the paged decode kernel over (cache dtype, head_dim, group).
#include <cstdlib>

#include "decode_impl.h"

namespace pa {

const void* decode_kernel_ptr_f32(int head_dim, int group);
const void* decode_kernel_ptr_f16(int head_dim, int group);
const void* decode_kernel_ptr_bf16(int head_dim, int group);
const void* decode_kernel_ptr_q8(int dtype, int head_dim, int group);
const void* decode_kernel_ptr_mfma(int dtype, int head_dim, int group);
const void* decode_kernel_ptr_mfma_q8(int dtype, int head_dim, int group);
const void* decode_kernel_ptr_f16_bs(int head_dim, int group, int block_size);
const void* decode_kernel_ptr_bf16_bs(int head_dim, int group, int block_size);
const void* chunk_kernel_ptr_f16(int head_dim, int group);
const void* chunk_kernel_ptr_bf16(int head_dim, int group);

// Groups of 4 or 8 query heads with 16-token blocks take the matrix-core kernel
// (PA_DECODE_MFMA=0 selects the per-lane kernel instead).
bool decode_uses_mfma(int dtype, int group, int block_size) {
    if (block_size != kBlock || dtype == DT_F32 || (group != 4 && group != 8)) return false;
    const char* e = std::getenv("PA_DECODE_MFMA");
    return !(e && e[0] == '0');
}

const void* decode_kernel_ptr(int dtype, int head_dim, int group, int block_size) {
    if (decode_uses_mfma(dtype, group, block_size)) {
        if (dtype == DT_Q8F16 || dtype == DT_Q8BF16)
            return decode_kernel_ptr_mfma_q8(dtype, head_dim, group);
        return decode_kernel_ptr_mfma(dtype, head_dim, group);
    }
    if (block_size != kBlock) {
        switch (dtype) {
            case DT_F16: return decode_kernel_ptr_f16_bs(head_dim, group, block_size);
            case DT_BF16: return decode_kernel_ptr_bf16_bs(head_dim, group, block_size);
            default: return nullptr;   // fp32 and 8-bit caches: 16-token blocks only
        }
    }
    switch (dtype) {
        case DT_F32: return decode_kernel_ptr_f32(head_dim, group);
        case DT_F16: return decode_kernel_ptr_f16(head_dim, group);
        case DT_BF16: return decode_kernel_ptr_bf16(head_dim, group);
        case DT_Q8F16:
        case DT_Q8BF16: return decode_kernel_ptr_q8(dtype, head_dim, group);
        default: return nullptr;
    }
}

const void* chunk_kernel_ptr(int dtype, int head_dim, int group, int block_size) {
    if (block_size != kBlock) return nullptr;   // other block sizes: chunk rows decode
    switch (dtype) {
        case DT_F16: return chunk_kernel_ptr_f16(head_dim, group);
        case DT_BF16: return chunk_kernel_ptr_bf16(head_dim, group);
        default: return nullptr;   // fp32 and 8-bit caches: chunk rows take the decode kernel
    }
}

hipError_t launch_chunk(const DecodeArgs& a, int dtype, hipStream_t stream) {
    if (a.chunk_rows <= 0 || a.max_tiles <= 0) return hipSuccess;
    const void* fn = chunk_kernel_ptr(dtype, a.head_dim, a.group, a.block_size);
    if (!fn) return hipErrorInvalidDeviceFunction;
    void* args[] = {(void*)&a};
    return hipLaunchKernel(fn, dim3(a.max_tiles * a.num_kv_heads), dim3(kWavesPerGroup * kWave),
                           args, 0, stream);
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream) {
    const void* fn = decode_kernel_ptr(dtype, a.head_dim, a.group, a.block_size);
    if (!fn) return hipErrorInvalidDeviceFunction;
    int groups = (a.max_waves + kWavesPerGroup - 1) / kWavesPerGroup;
    if (groups < 1) groups = 1;   // at least one group: it also zeroes rows with nothing to read
    void* args[] = {(void*)&a};
    return hipLaunchKernel(fn, dim3(groups), dim3(kWavesPerGroup * kWave), args, 0, stream);
}

// Merge kernel: one wavefront per (share boundary w >= 1, head of the group).  It reads
// the task of boundary w, if any, and combines that pair's partials for its head.  The
// decode kernel rewrites the same tasks on every call with the same plan and the plan
// zeroes every task slot, so tasks are read-only here.
template <int D, int G>
__global__ __launch_bounds__(kWavesPerGroup * kWave) void merge_kernel(DecodeArgs a) {
    const int4* tasks = (const int4*)(a.ws + a.lay.tasks);
    const float2* pml = (const float2*)(a.ws + a.lay.part_ml);
    const float* pacc = (const float*)(a.ws + a.lay.part_acc);
    const int q = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
    const int w = q / G + 1, gi = q % G;
    const int W = ((const int32_t*)(a.ws + a.lay.header))[2];
    if (w >= W) return;
    const int4 t = tasks[w];
    if (t.z <= 0) return;
    merge_pair<D, G>(a, t.x, t.y, w - 1, t.z, t.w, gi, pml, pacc, lane_id());
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t stream) {
    const void* fn = nullptr;
#define PA_CASE(D, G) \
    if (a.head_dim == D && a.group == G) fn = (const void*)&merge_kernel<D, G>;
#define PA_CASES(D) PA_CASE(D, 1) PA_CASE(D, 2) PA_CASE(D, 4) PA_CASE(D, 8)
    PA_CASES(64) PA_CASES(128) PA_CASES(256)
#undef PA_CASES
#undef PA_CASE
    if (!fn) return hipErrorInvalidDeviceFunction;
    if (a.max_waves <= 1) return hipSuccess;
    const int groups = ((a.max_waves - 1) * a.group + kWavesPerGroup - 1) / kWavesPerGroup;
    void* args[] = {(void*)&a};
    return hipLaunchKernel(fn, dim3(groups), dim3(kWavesPerGroup * kWave), args, 0, stream);
}

}  // namespace pa
