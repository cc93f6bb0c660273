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
const void* decode_kernel_ptr_f32_new(int head_dim, int group);
const void* decode_kernel_ptr_f16_new(int head_dim, int group);
const void* decode_kernel_ptr_bf16_new(int head_dim, int group);
const void* decode_kernel_ptr_f16_bs_new(int head_dim, int group, int block_size);
const void* decode_kernel_ptr_bf16_bs_new(int head_dim, int group, int block_size);
const void* decode_kernel_ptr_mfma_new(int dtype, int head_dim, int group);
const void* decode_group_ptr_f32(int head_dim, int group, bool new_rows);
const void* decode_group_ptr_f16(int head_dim, int group, bool new_rows);
const void* decode_group_ptr_bf16(int head_dim, int group, bool new_rows);
const void* decode_group_ptr_q8(int dtype, int head_dim, int group);
const void* chunk_kernel_ptr_f16(int head_dim, int group);
const void* chunk_kernel_ptr_bf16(int head_dim, int group);

// Groups of 4 or 8 query heads with 16-token blocks take the matrix-core kernel
// (PA_DECODE_MFMA=0 selects the per-lane kernel instead).
bool decode_uses_mfma(int dtype, int group, int block_size) {
    if (block_size != kBlock || dtype == DT_F32 || (group != 4 && group != 8)) return false;
    const char* e = std::getenv("PA_DECODE_MFMA");
    return !(e && e[0] == '0');
}

const void* decode_kernel_ptr(int dtype, int head_dim, int group, int block_size,
                              bool new_rows) {
    const bool q8 = dtype == DT_Q8F16 || dtype == DT_Q8BF16;
    if (new_rows && q8) return nullptr;   // 8-bit rows are quantized by pa_write_kv first
    if (decode_uses_mfma(dtype, group, block_size)) {
        if (q8) return decode_kernel_ptr_mfma_q8(dtype, head_dim, group);
        return new_rows ? decode_kernel_ptr_mfma_new(dtype, head_dim, group)
                        : decode_kernel_ptr_mfma(dtype, head_dim, group);
    }
    if (block_size != kBlock) {
        switch (dtype) {
            case DT_F16:
                return new_rows ? decode_kernel_ptr_f16_bs_new(head_dim, group, block_size)
                                : decode_kernel_ptr_f16_bs(head_dim, group, block_size);
            case DT_BF16:
                return new_rows ? decode_kernel_ptr_bf16_bs_new(head_dim, group, block_size)
                                : decode_kernel_ptr_bf16_bs(head_dim, group, block_size);
            default: return nullptr;   // fp32 and 8-bit caches: 16-token blocks only
        }
    }
    if (new_rows) {
        switch (dtype) {
            case DT_F32: return decode_kernel_ptr_f32_new(head_dim, group);
            case DT_F16: return decode_kernel_ptr_f16_new(head_dim, group);
            case DT_BF16: return decode_kernel_ptr_bf16_new(head_dim, group);
            default: return nullptr;
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

const void* decode_group_ptr(int dtype, int head_dim, int group, bool new_rows) {
    switch (dtype) {
        case DT_F32: return decode_group_ptr_f32(head_dim, group, new_rows);
        case DT_F16: return decode_group_ptr_f16(head_dim, group, new_rows);
        case DT_BF16: return decode_group_ptr_bf16(head_dim, group, new_rows);
        case DT_Q8F16:
        case DT_Q8BF16: return new_rows ? nullptr : decode_group_ptr_q8(dtype, head_dim, group);
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
    const void* fn = a.group_mode ? decode_group_ptr(dtype, a.head_dim, a.group, a.k_new)
                                  : decode_kernel_ptr(dtype, a.head_dim, a.group, a.block_size,
                                                      a.k_new);
    if (!fn) return hipErrorInvalidDeviceFunction;
    void* args[] = {(void*)&a};
    if (a.group_mode) {
        // group_mode workgroups per pair, one wave record each wavefront
        const int groups = a.max_waves / kWavesPerGroup > 0 ? a.max_waves / kWavesPerGroup : 1;
        return hipLaunchKernel(fn, dim3(groups), dim3(kWavesPerGroup * kWave), args, 0, stream);
    }
    int groups = (a.max_waves + kWavesPerGroup - 1) / kWavesPerGroup;
    if (groups < 1) groups = 1;   // at least one group: it also zeroes rows with nothing to read
    return hipLaunchKernel(fn, dim3(groups), dim3(kWavesPerGroup * kWave), args, 0, stream);
}

// With a step's new rows given (pa_decode_write_attend): thread t of the slot-write groups
// copies 16 bytes of one new K or V row into the slot of position len - 1 of its sequence
// ("vLLM and PagedAttention" notes, basic decoding: the new token goes after the existing
// ones, in the block the manager mapped).  The decode kernel of the same call took those
// rows from the new rows directly, so nothing reads the slots before they are written.
// An id outside the pool is skipped (the decode kernel sets the error bit for it).
__device__ void write_new_rows(const DecodeArgs& a, long t) {
    const int pieces = a.row_bytes / 16;
    const long per_seq = 2L * a.num_kv_heads * pieces;
    if (t >= per_seq * a.num_seqs) return;
    const int s = (int)(t / per_seq);
    const int r = (int)(t % per_seq);
    const int kv = r / (a.num_kv_heads * pieces);          // 0: K, 1: V
    const int g = (r / pieces) % a.num_kv_heads, c = r % pieces;
    // The row piece loads beside the sequence's length, so that the store waits for two
    // dependent loads (length, then table entry), not three.  (The empty asm takes the
    // piece where it is loaded: the compiler would otherwise sink the load past the
    // checks, next to the store.)
    const size_t src = ((size_t)s * a.num_kv_heads + g) * a.row_bytes + (size_t)c * 16;
    const char* from = (const char*)(kv ? a.v_new : a.k_new);
    u32x4 row = ld16(from + src);
    const int L = a.seq_lens[s];
    asm volatile("" : "+v"(row));
    if (L <= 0 || L > a.max_seq_len || (long)L > (long)a.max_blocks * a.block_size) return;
    const int j = (L - 1) / a.block_size;
    const int b = a.block_tables[(size_t)s * a.max_blocks + j];
    if ((unsigned)b >= (unsigned)a.num_blocks) return;
    const size_t tile = (size_t)a.block_size * a.row_bytes;
    const size_t dst = ((size_t)b * a.num_kv_heads + g) * tile +
                       (size_t)((L - 1) % a.block_size) * a.row_bytes + (size_t)c * 16;
    char* to = (char*)(kv ? a.v_cache : a.k_cache);
    st16(to + dst, row);
}

// Merge kernel: one wavefront per (share boundary w >= 1, head of the group).  It reads
// the task of boundary w, if any, and combines that pair's partials for its head.  The
// decode kernel rewrites the same tasks on every call with the same plan and the plan
// zeroes every task slot, so tasks are read-only here.  With new rows given, the groups
// after the merge groups write them into their slots.
template <int D, int G>
__global__ __launch_bounds__(kWavesPerGroup * kWave) void merge_kernel(DecodeArgs a, int merge_groups) {
    if ((int)blockIdx.x >= merge_groups) {
        write_new_rows(a, (long)(blockIdx.x - merge_groups) * blockDim.x + threadIdx.x);
        return;
    }
    const int4* tasks = (const int4*)(a.ws + a.lay.tasks);
    const float2* pml = (const float2*)(a.ws + a.lay.part_ml);
    const float* pacc = (const float*)(a.ws + a.lay.part_acc);
    const int q = uniform(blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6));
    const int w = q / G + 1, gi = q % G;
    const int32_t* hdr = (const int32_t*)(a.ws + a.lay.header);
    // The header's fields and the task slot are read together by scalar loads (w is
    // wave-uniform; the slot index is clamped to the last of the max_waves + 1 slots, as the
    // grid is rounded up to whole workgroups): one wait before the partials are loaded.
    const int32_t* slot = (const int32_t*)(tasks + (w < a.max_waves ? w : a.max_waves));
    const int4 t = make_int4(ld_scalar(slot), ld_scalar(slot + 1), ld_scalar(slot + 2),
                             ld_scalar(slot + 3));
    const int W = ld_scalar(hdr + 2), group_mode = ld_scalar(hdr + 5);
    if (w >= W || group_mode != 0) return;   // (a group-mode plan holds no merge tasks)
    if (t.z <= 0) return;
    merge_pair<D, G>(a, t.x, t.y, w - 1, t.z, t.w, gi, pml, pacc, lane_id());
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t stream) {
    if (a.group_mode) return hipSuccess;   // combined inside the decode launch
    const void* fn = nullptr;
#define PA_CASE(D, G) \
    if (a.head_dim == D && a.group == G) fn = (const void*)&merge_kernel<D, G>;
#define PA_CASES(D) PA_CASE(D, 1) PA_CASE(D, 2) PA_CASE(D, 4) PA_CASE(D, 8)
    PA_CASES(64) PA_CASES(128) PA_CASES(256)
#undef PA_CASES
#undef PA_CASE
    if (!fn) return hipErrorInvalidDeviceFunction;
    int groups = a.max_waves > 1
                     ? ((a.max_waves - 1) * a.group + kWavesPerGroup - 1) / kWavesPerGroup
                     : 0;
    const int merge_groups = groups;
    if (a.k_new) {   // the slot-write groups: 16 bytes per thread, K and V
        const long threads = 2L * a.num_seqs * a.num_kv_heads * (a.row_bytes / 16);
        groups += (int)((threads + kWavesPerGroup * kWave - 1) / (kWavesPerGroup * kWave));
    }
    if (groups == 0) return hipSuccess;
    void* args[] = {(void*)&a, (void*)&merge_groups};
    return hipLaunchKernel(fn, dim3(groups), dim3(kWavesPerGroup * kWave), args, 0, stream);
}

}  // namespace pa
