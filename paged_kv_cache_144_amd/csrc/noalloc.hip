// pa_decode_noalloc: pa_decode with its workspace in a fixed device array, for callers that
// cannot allocate device memory (code under stream capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// The array lives in this file.  In host code its name is only a stand-in for the symbol, so
// the entry point looks up the array's device address with hipGetSymbolAddress on its first
// call on each device (with that device current) and hands that address to pa_decode as the
// workspace.  Every call on one device shares that device's array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa.h"

namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte lines");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// The array's device address on the current device, looked up once per device.
pa_status scratch_address(void** out) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return PA_ERR_LAUNCH;
        }
        addr[dev] = p;
    }
    *out = addr[dev];
    return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_noalloc(void* out, pa_dtype out_dtype, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const pa_cache_desc* desc, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                       const int32_t* query_start_loc, int32_t num_seqs,
                                       int32_t total_q_rows, int32_t max_seq_len,
                                       int32_t num_q_heads, float scale, int32_t window,
                                       void* stream) {
    // shapes whose workspace exceeds the array are refused before anything is touched
    const size_t need =
        pa_decode_workspace_size(desc, num_seqs, total_q_rows, num_q_heads, max_seq_len);
    if (need > kScratchBytes) return PA_ERR_WORKSPACE;
    void* ws = nullptr;
    const pa_status st = scratch_address(&ws);
    if (st != PA_OK) return st;
    // pa_decode validates the remaining arguments; its plan kernel writes every part of the
    // workspace the attention reads (headers, shares, zeroed merge records), so what an
    // earlier call left in the array never matters
    return pa_decode(out, out_dtype, q, k_cache, v_cache, desc, block_tables,
                     max_blocks_per_seq, seq_lens, query_start_loc, num_seqs, total_q_rows,
                     max_seq_len, num_q_heads, scale, window, ws, kScratchBytes, stream);
}
