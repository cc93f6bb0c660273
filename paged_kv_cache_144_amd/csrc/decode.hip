// Dispatch of the paged decode kernel over (cache dtype, head_dim, group).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

const void* decode_kernel_ptr_f32(int head_dim, int group);
const void* decode_kernel_ptr_f16(int head_dim, int group);
const void* decode_kernel_ptr_bf16(int head_dim, int group);
const void* chunk_kernel_ptr_f16(int head_dim, int group);
const void* chunk_kernel_ptr_bf16(int head_dim, int group);

const void* decode_kernel_ptr(int dtype, int head_dim, int group) {
    switch (dtype) {
        case DT_F32: return decode_kernel_ptr_f32(head_dim, group);
        case DT_F16: return decode_kernel_ptr_f16(head_dim, group);
        case DT_BF16: return decode_kernel_ptr_bf16(head_dim, group);
        default: return nullptr;
    }
}

const void* chunk_kernel_ptr(int dtype, int head_dim, int group) {
    switch (dtype) {
        case DT_F16: return chunk_kernel_ptr_f16(head_dim, group);
        case DT_BF16: return chunk_kernel_ptr_bf16(head_dim, group);
        default: return nullptr;   // fp32 caches: chunk rows take the decode kernel
    }
}

hipError_t launch_chunk(const DecodeArgs& a, int dtype, hipStream_t stream) {
    if (a.chunk_rows <= 0 || a.max_tiles <= 0) return hipSuccess;
    const void* fn = chunk_kernel_ptr(dtype, a.head_dim, a.group);
    if (!fn) return hipErrorInvalidDeviceFunction;
    void* args[] = {(void*)&a};
    return hipLaunchKernel(fn, dim3(a.max_tiles, a.num_kv_heads), dim3(kWavesPerGroup * kWave),
                           args, 0, stream);
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream) {
    const void* fn = decode_kernel_ptr(dtype, a.head_dim, a.group);
    if (!fn) return hipErrorInvalidDeviceFunction;
    const int groups = (a.max_waves + kWavesPerGroup - 1) / kWavesPerGroup;
    if (groups == 0) return hipSuccess;
    void* args[] = {(void*)&a};
    return hipLaunchKernel(fn, dim3(groups), dim3(kWavesPerGroup * kWave), args, 0, stream);
}

}  // namespace pa
