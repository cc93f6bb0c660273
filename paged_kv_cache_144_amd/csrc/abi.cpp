// The exported C ABI (declared in include/pa.h): argument validation, kernel selection,
// workspace sizing and launches on the caller's stream.  No device memory is allocated or
// freed here and no call synchronizes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <map>
#include <mutex>
#include <utility>

#include "pa.h"
#include "pa_internal.h"

namespace {

using pa::DecodeArgs;

// element types of q, new rows and outputs
bool dtype_ok(int dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }
int dtype_bytes(int dt) { return dt == PA_F32 ? 4 : 2; }
// cache types: the element types, or 8-bit codes with a scale per 32 values
bool is_q8(int dt) { return dt == PA_Q8_F16 || dt == PA_Q8_BF16; }
bool cache_dtype_ok(int dt) { return dtype_ok(dt) || is_q8(dt); }
// the type of q and of new K / V rows for a cache type
int act_dtype(int dt) { return dt == PA_Q8_F16 ? PA_F16 : dt == PA_Q8_BF16 ? PA_BF16 : dt; }
// bytes of one token's row of one (block, head) tile, and of its scales (8-bit tiles)
int64_t row_bytes(const pa_cache_desc* d) {
    return is_q8(d->dtype) ? d->head_dim : (int64_t)d->head_dim * dtype_bytes(d->dtype);
}
int64_t scale_bytes(const pa_cache_desc* d) {
    return is_q8(d->dtype) ? 2 * (d->head_dim / pa::kQ8Group) : 0;
}

pa_status check_desc(const pa_cache_desc* d) {
    if (!d) return PA_ERR_NULL;
    if (!cache_dtype_ok(d->dtype)) return PA_ERR_DTYPE;
    if (d->num_blocks <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 || d->block_size <= 0)
        return PA_ERR_SHAPE;
    // 16-token blocks for every type; 8 and 32 for the 16-bit types
    const bool bs16 = d->dtype == PA_F16 || d->dtype == PA_BF16;
    if (d->block_size != pa::kBlock && !(bs16 && (d->block_size == 8 || d->block_size == 32)))
        return PA_ERR_UNSUPPORTED;
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

// Compute units of the current device (0 on failure).
int cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus;
}

// Resident decode wavefronts on the current device for one kernel instance.
int resident_waves(const void* fn) {
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    auto key = std::make_pair(dev, fn);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0, groups = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&groups, fn, pa::kWavesPerGroup * pa::kWave,
                                                     0) != hipSuccess)
        return 0;
    if (groups < 1) groups = 1;
    const int waves = cus * groups * pa::kWavesPerGroup;
    cache[key] = waves;
    return waves;
}

struct Plan {
    const void* fn = nullptr;
    int group = 0;
    int max_waves = 0;
    int wave_round = 0;   // wavefronts of one workgroup on every compute unit
    int chunk_rows = 0;   // query rows per chunk tile; 0 = chunk rows run as decode rows
    int max_tiles = 0;
    int pair_cost = pa::kPairCost;
    int min_blocks = pa::kMinBlocksPerWave;
    pa::Layout lay{};
};

pa_status plan_shape(const pa_cache_desc* desc, int32_t num_seqs, int32_t total_q_rows,
                     int32_t num_q_heads, bool one_row_per_seq, Plan& p) {
    pa_status st = check_desc(desc);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || total_q_rows < 0 || num_q_heads <= 0) return PA_ERR_SHAPE;
    if (num_q_heads % desc->num_kv_heads) return PA_ERR_SHAPE;
    p.group = num_q_heads / desc->num_kv_heads;
    p.fn = pa::decode_kernel_ptr(desc->dtype, desc->head_dim, p.group, desc->block_size);
    if (!p.fn) return PA_ERR_UNSUPPORTED;
    p.max_waves = resident_waves(p.fn);
    if (p.max_waves <= 0) return PA_ERR_LAUNCH;
    // The per-lane kernel with 16- and 32-bit caches keeps one workgroup per compute unit:
    // its light work per byte needs no second workgroup to keep the memory busy, and fewer,
    // longer shares cut fewer pairs.  8-bit caches, which decode their codes on the vector
    // ALU, and the matrix-core kernel keep every resident wavefront.
    const bool q8 = desc->dtype == PA_Q8_F16 || desc->dtype == PA_Q8_BF16;
    if (!q8 && !pa::decode_uses_mfma(desc->dtype, p.group, desc->block_size))
        p.max_waves = std::min(p.max_waves, cu_count() * pa::kWavesPerGroup);
    if ((desc->dtype == PA_Q8_F16 || desc->dtype == PA_Q8_BF16) &&
        pa::decode_uses_mfma(desc->dtype, p.group, desc->block_size))
        p.pair_cost = pa::kPairCostQ8Mfma;
    p.wave_round = cu_count() * pa::kWavesPerGroup;
    // tuning / testing knob: fewer decode wavefronts than the device keeps resident
    if (const char* e = std::getenv("PA_DECODE_WAVES")) {
        const int v = std::atoi(e);
        if (v > 0 && v < p.max_waves) p.max_waves = v;
    }
    // tuning knob: the fixed cost of a pair in the wave split, in quarter blocks
    if (const char* e = std::getenv("PA_PAIR_COST")) {
        const int v = std::atoi(e);
        if (v >= 0 && v <= pa::kMaxPairCost) p.pair_cost = v;
    }
    // tuning knob: the smallest share of KV blocks a decode wavefront is given
    if (const char* e = std::getenv("PA_MIN_BLOCKS")) {
        const int v = std::atoi(e);
        if (v >= pa::kMinBlocksFloor && v <= 256) p.min_blocks = v;
    }
    // chunk rows (sequences with several query rows) take the MFMA kernel when one exists
    // for this shape; PA_CHUNK_KERNEL=0 sends them through the decode kernel instead
    const char* ck = std::getenv("PA_CHUNK_KERNEL");
    const bool chunk_off = ck && ck[0] == '0';
    if (!one_row_per_seq && !chunk_off &&
        pa::chunk_kernel_ptr(desc->dtype, desc->head_dim, p.group, desc->block_size)) {
        p.chunk_rows = pa::chunk_tile_rows(p.group);
        // sum over sequences of ceil(n_s / QT) <= rows / QT + sequences
        p.max_tiles = total_q_rows / p.chunk_rows + num_seqs + 1;
    }
    p.lay = pa::layout(total_q_rows, p.max_waves, p.max_tiles, p.group, desc->head_dim);
    return PA_OK;
}

// Group mode for a batch of num_seqs decode rows (one query row each) under a sliding window
// of `window` tokens: the workgroups per (row, KV head) pair, or 0 for the wave split.
// A sliding-window layer bounds every pair by its window (sotaaz.com, "KV cache by model",
// section on layer kinds: such a layer only needs the last W tokens), so a fixed number of
// wavefronts per pair is balanced; they combine in LDS and through a per-pair arrival
// counter, with no merge launch.  Small batches split each pair among S = CUs / pairs
// workgroups, so that every compute unit streams one; below 4 the split's cross-workgroup
// handoff (an L2 write-back and invalidate at agent scope) costs more than it saves and S
// is 1.  S is raised where a wavefront's share would pass one 64-entry chunk of block ids
// and lowered where shares would fall under two blocks.  The per-lane kernel with 16-token blocks only; the
// workspace must hold one record per wavefront.  PA_GROUP_MODE=0 keeps the wave split (for
// A/Bs); PA_GROUP_SPLIT=S fixes the split (for sweeps).
int group_split(const pa_cache_desc* desc, const Plan& p, int32_t num_seqs, int32_t window) {
    const char* gm = std::getenv("PA_GROUP_MODE");
    if ((gm && gm[0] == '0') || window <= 0 || desc->block_size != pa::kBlock) return 0;
    if (num_seqs <= 0 || pa::decode_uses_mfma(desc->dtype, p.group, desc->block_size)) return 0;
    if (!pa::decode_group_ptr(desc->dtype, desc->head_dim, p.group, false)) return 0;
    constexpr int WB = pa::kWavesPerGroup;
    const int64_t win_blocks = ((int64_t)window + desc->block_size - 1) / desc->block_size + 1;
    const int64_t pairs = (int64_t)num_seqs * desc->num_kv_heads;
    int64_t s = cu_count() / pairs;
    if (s < 4) s = 1;
    if (s > win_blocks / (2 * WB)) s = win_blocks / (2 * WB);
    const int64_t need = (win_blocks + 64 * WB - 1) / (64 * WB);
    if (s < need) s = need;
    if (s < 1) s = 1;
    if (s > pa::kGroupMaxSplit) s = pa::kGroupMaxSplit;
    if (const char* e = std::getenv("PA_GROUP_SPLIT")) {
        const int v = std::atoi(e);
        if (v >= 1 && v <= pa::kGroupMaxSplit && v >= need) s = v;
    }
    if (win_blocks > 64 * WB * s) return 0;
    if (WB * s * pairs > p.max_waves) return 0;
    return (int)s;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
    switch (s) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "null pointer";
        case PA_ERR_SHAPE: return "inconsistent or negative sizes";
        case PA_ERR_DTYPE: return "unsupported dtype";
        case PA_ERR_UNSUPPORTED: return "no kernel for this head_dim / group / block size";
        case PA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case PA_ERR_LAUNCH: return "HIP launch error";
        case PA_ERR_OUT_OF_BLOCKS: return "not enough free blocks";
        case PA_ERR_SHARED_BLOCK: return "copy-on-write would read a block with pending writes";
        case PA_ERR_BAD_SEQ: return "unknown or non-empty sequence";
        case PA_ERR_ADMISSION: return "no new request while sequences are swapped out";
    }
    return "unknown status";
}

pa_status pa_write_kv(const void* k, const void* v, const int64_t* slot_mapping,
                      int32_t num_tokens, void* k_cache, void* v_cache,
                      const pa_cache_desc* desc, void* stream) {
    pa_status st = check_desc(desc);
    if (st != PA_OK) return st;
    if (num_tokens < 0) return PA_ERR_SHAPE;
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
    hipError_t e =
        is_q8(desc->dtype)
            ? pa::launch_write_kv_q8(k, v, slot_mapping, num_tokens, k_cache, v_cache,
                                     desc->num_blocks, desc->num_kv_heads, desc->head_dim,
                                     act_dtype(desc->dtype), (hipStream_t)stream)
            : pa::launch_write_kv(k, v, slot_mapping, num_tokens, k_cache, v_cache,
                                  desc->num_blocks, desc->block_size, desc->num_kv_heads,
                                  desc->head_dim, dtype_bytes(desc->dtype), (hipStream_t)stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (bytes == 0) return PA_OK;
    if (!buf || !sink) return PA_ERR_NULL;
    if ((bytes & 15u) || ((uintptr_t)buf & 15u)) return PA_ERR_SHAPE;
    return pa::launch_stream_read(buf, bytes, sink, (hipStream_t)stream) == hipSuccess
               ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const pa_cache_desc* desc,
                         const int32_t* copies, int32_t num_copies, int32_t* error_word,
                         void* stream) {
    if (!desc) return PA_ERR_NULL;
    if (!cache_dtype_ok(desc->dtype)) return PA_ERR_DTYPE;
    if (desc->num_blocks <= 0 || desc->num_kv_heads <= 0 || desc->num_kv_heads > 65535 ||
        desc->head_dim <= 0 || desc->block_size <= 0 || num_copies < 0)
        return PA_ERR_SHAPE;
    const int64_t rb = row_bytes(desc), sb = scale_bytes(desc);
    if (rb % 16 || sb % 4 || (rb + sb) * desc->block_size > INT32_MAX / 2 ||
        (is_q8(desc->dtype) && (desc->head_dim % pa::kQ8Group || desc->block_size != pa::kBlock)))
        return PA_ERR_UNSUPPORTED;
    if (num_copies == 0) return PA_OK;
    if (!k_cache || !v_cache || !copies) return PA_ERR_NULL;
    hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, copies, num_copies,
                                          desc->num_blocks, desc->num_kv_heads,
                                          desc->block_size, (int32_t)rb, (int32_t)sb,
                                          error_word, (hipStream_t)stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// The address a kernel uses for p: device memory as is, pinned host memory through its
// device mapping.  Anything else (pageable host memory) is refused.
pa_status kernel_address(const void* p, const void** out) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();   // do not leave the failed query as the last error
        return PA_ERR_UNSUPPORTED;
    }
    if (attr.type == hipMemoryTypeDevice) {
        *out = p;
        return PA_OK;
    }
    if (attr.type == hipMemoryTypeHost && attr.devicePointer) {
        // the same offset into the allocation, through its device mapping
        *out = (const char*)attr.devicePointer + ((const char*)p - (const char*)attr.hostPointer);
        return PA_OK;
    }
    return PA_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

pa_status pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                         const pa_cache_desc* desc, int32_t src_blocks, int32_t dst_blocks,
                         const int32_t* pairs, int32_t n, int32_t* error_word, void* stream) {
    if (!desc) return PA_ERR_NULL;
    if (!cache_dtype_ok(desc->dtype)) return PA_ERR_DTYPE;
    if (desc->num_kv_heads <= 0 || desc->num_kv_heads > 65535 || desc->head_dim <= 0 ||
        desc->block_size <= 0 || src_blocks < 0 || dst_blocks < 0 || n < 0)
        return PA_ERR_SHAPE;
    const int64_t tile = desc->block_size * (row_bytes(desc) + scale_bytes(desc));
    if (tile % 16 || tile > INT32_MAX / 2 ||
        (is_q8(desc->dtype) && (desc->head_dim % pa::kQ8Group || desc->block_size != pa::kBlock)))
        return PA_ERR_UNSUPPORTED;
    if (n == 0) return PA_OK;
    if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return PA_ERR_NULL;
    const void *sk, *sv, *dk, *dv;
    pa_status st;
    if ((st = kernel_address(src_k, &sk)) != PA_OK || (st = kernel_address(src_v, &sv)) != PA_OK ||
        (st = kernel_address(dst_k, &dk)) != PA_OK || (st = kernel_address(dst_v, &dv)) != PA_OK)
        return st;
    hipError_t e = pa::launch_swap_blocks(sk, sv, (void*)dk, (void*)dv, pairs, n, src_blocks,
                                          dst_blocks, desc->num_kv_heads, (int32_t)tile,
                                          error_word, (hipStream_t)stream);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

const char* pa_decode_kernel_name(const pa_cache_desc* desc, int32_t num_q_heads,
                                  int32_t num_seqs, int32_t window) {
    if (check_desc(desc) != PA_OK || num_q_heads <= 0 || num_q_heads % desc->num_kv_heads ||
        num_seqs < 0)
        return nullptr;
    const int group = num_q_heads / desc->num_kv_heads;
    if (!pa::decode_kernel_ptr(desc->dtype, desc->head_dim, group, desc->block_size))
        return nullptr;
    if (window > 0) {
        Plan p;
        if (plan_shape(desc, num_seqs, num_seqs, num_q_heads, true, p) != PA_OK) return nullptr;
        if (group_split(desc, p, num_seqs, window) > 0) return "decode_group_kernel";
    }
    return pa::decode_uses_mfma(desc->dtype, group, desc->block_size) ? "decode_mfma_kernel"
                                                                      : "decode_kernel";
}

size_t pa_decode_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                int32_t total_q_rows, int32_t num_q_heads,
                                int32_t max_seq_len) {
    Plan p;
    if (max_seq_len < 0) return 0;
    // sized for query_start_loc != NULL (the larger case)
    if (plan_shape(desc, num_seqs, total_q_rows, num_q_heads, false, p) != PA_OK) return 0;
    return p.lay.total;
}

}  // extern "C"

namespace {

// Profiling hooks: hipEvents recorded around the decode / chunk kernel launches
// (caller-owned).
hipEvent_t g_prof_before = nullptr, g_prof_after = nullptr;
hipEvent_t g_chunk_before = nullptr, g_chunk_after = nullptr;

pa_status build_args(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                     const void* v_cache, const pa_cache_desc* desc,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                     int32_t total_q_rows, int32_t max_seq_len, int32_t num_q_heads,
                     float scale, int32_t window, void* workspace, size_t workspace_bytes,
                     bool need_attend_ptrs, DecodeArgs& a, bool& nothing) {
    Plan p;
    nothing = false;
    pa_status st = plan_shape(desc, num_seqs, total_q_rows, num_q_heads, !query_start_loc, p);
    if (st != PA_OK) return st;
    if (!dtype_ok(out_dtype)) return PA_ERR_DTYPE;
    if (max_seq_len < 0 || max_blocks_per_seq < 0) return PA_ERR_SHAPE;
    if (!query_start_loc && total_q_rows != num_seqs) return PA_ERR_SHAPE;
    if (total_q_rows == 0) {
        nothing = true;
        return PA_OK;
    }
    if (num_seqs == 0) return PA_ERR_SHAPE;   // rows without sequences
    if (!block_tables || !seq_lens) return PA_ERR_NULL;
    if (need_attend_ptrs && (!out || !q || !k_cache || !v_cache)) return PA_ERR_NULL;
    if (max_blocks_per_seq == 0) return PA_ERR_SHAPE;
    // the linear block space and its weighted copy (4 per block plus the pair cost) are
    // indexed with 32-bit offsets
    if ((uint64_t)total_q_rows * (uint64_t)desc->num_kv_heads *
            (4ull * (uint64_t)max_blocks_per_seq + pa::kMaxPairCost) >= (1ull << 32))
        return PA_ERR_SHAPE;
    if (!workspace || ((uintptr_t)workspace & 255u)) return PA_ERR_WORKSPACE;
    if (workspace_bytes < p.lay.total) return PA_ERR_WORKSPACE;

    a = DecodeArgs{};
    a.out = out;
    a.out_dtype = out_dtype;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.query_start_loc = query_start_loc;
    a.num_blocks = desc->num_blocks;
    a.num_kv_heads = desc->num_kv_heads;
    a.head_dim = desc->head_dim;
    a.block_size = desc->block_size;
    a.num_q_heads = num_q_heads;
    a.group = p.group;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.total_q_rows = total_q_rows;
    a.max_seq_len = max_seq_len;
    a.window = window > 0 ? window : 0;
    a.scale = scale;
    a.max_waves = p.max_waves;
    a.wave_round = p.wave_round;
    a.chunk_rows = p.chunk_rows;
    a.max_tiles = p.max_tiles;
    a.pair_cost = p.pair_cost;
    a.min_blocks = p.min_blocks;
    a.ws = (char*)workspace;
    a.lay = p.lay;
    // sliding-window decode batches: one workgroup per (row, KV head) pair
    const int split = query_start_loc ? 0 : group_split(desc, p, num_seqs, window);
    if (split > 0) {
        a.group_mode = split;
        a.max_waves = pa::kWavesPerGroup * split * num_seqs * desc->num_kv_heads;
    }
    return PA_OK;
}

pa_status run_attend(const DecodeArgs& a, int dtype, hipStream_t s) {
    if (g_prof_before && hipEventRecord(g_prof_before, s) != hipSuccess) return PA_ERR_LAUNCH;
    if (pa::launch_decode(a, dtype, s) != hipSuccess) return PA_ERR_LAUNCH;
    if (g_prof_after && hipEventRecord(g_prof_after, s) != hipSuccess) return PA_ERR_LAUNCH;
    if (pa::launch_merge(a, s) != hipSuccess) return PA_ERR_LAUNCH;
    if (a.chunk_rows > 0 && g_chunk_before && hipEventRecord(g_chunk_before, s) != hipSuccess)
        return PA_ERR_LAUNCH;
    if (pa::launch_chunk(a, dtype, s) != hipSuccess) return PA_ERR_LAUNCH;
    if (a.chunk_rows > 0 && g_chunk_after && hipEventRecord(g_chunk_after, s) != hipSuccess)
        return PA_ERR_LAUNCH;
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_plan(const pa_cache_desc* desc, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens,
                         const int32_t* query_start_loc, int32_t num_seqs,
                         int32_t total_q_rows, int32_t max_seq_len, int32_t num_q_heads,
                         int32_t window, void* workspace, size_t workspace_bytes,
                         void* stream) {
    DecodeArgs a;
    bool nothing;
    pa_status st = build_args(nullptr, PA_F32, nullptr, nullptr, nullptr, desc, block_tables,
                              max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                              total_q_rows, max_seq_len, num_q_heads, 0.f, window, workspace,
                              workspace_bytes, false, a, nothing);
    if (st != PA_OK || nothing) return st;
    return pa::launch_plan(a, (hipStream_t)stream) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_decode_attend(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                           const void* v_cache, const pa_cache_desc* desc,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, const int32_t* query_start_loc,
                           int32_t num_seqs, int32_t total_q_rows, int32_t max_seq_len,
                           int32_t num_q_heads, float scale, int32_t window, void* workspace,
                           size_t workspace_bytes, void* stream) {
    DecodeArgs a;
    bool nothing;
    pa_status st = build_args(out, out_dtype, q, k_cache, v_cache, desc, block_tables,
                              max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                              total_q_rows, max_seq_len, num_q_heads, scale, window, workspace,
                              workspace_bytes, true, a, nothing);
    if (st != PA_OK || nothing) return st;
    return run_attend(a, desc->dtype, (hipStream_t)stream);
}

pa_status pa_decode_write_attend(void* out, pa_dtype out_dtype, const void* q, const void* k_new,
                                 const void* v_new, void* k_cache, void* v_cache,
                                 const pa_cache_desc* desc, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
                                 float scale, int32_t window, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    if (!desc) return PA_ERR_NULL;
    if (is_q8(desc->dtype)) return PA_ERR_UNSUPPORTED;   // new rows are quantized first
    DecodeArgs a;
    bool nothing;
    pa_status st = build_args(out, out_dtype, q, k_cache, v_cache, desc, block_tables,
                              max_blocks_per_seq, seq_lens, nullptr, num_seqs, num_seqs,
                              max_seq_len, num_q_heads, scale, window, workspace,
                              workspace_bytes, true, a, nothing);
    if (st != PA_OK || nothing) return st;
    if (!k_new || !v_new) return PA_ERR_NULL;
    a.k_new = k_new;
    a.v_new = v_new;
    a.row_bytes = (int32_t)row_bytes(desc);
    return run_attend(a, desc->dtype, (hipStream_t)stream);
}

pa_status pa_decode_noalloc(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                            const void* v_cache, const pa_cache_desc* desc,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, const int32_t* query_start_loc,
                            int32_t num_seqs, int32_t total_q_rows, int32_t max_seq_len,
                            int32_t num_q_heads, float scale, int32_t window, void* stream) {
    // shapes whose workspace exceeds the array are refused before anything is touched
    const size_t need =
        pa_decode_workspace_size(desc, num_seqs, total_q_rows, num_q_heads, max_seq_len);
    if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
    void* ws = nullptr;
    size_t bytes = 0;
    const pa_status st = pa::noalloc_scratch(&ws, &bytes);
    if (st != PA_OK) return st;
    // pa_decode validates the remaining arguments; its plan kernel writes every part of the
    // workspace the attention reads (headers, shares, zeroed merge records), so what an
    // earlier call left in the array never matters
    return pa_decode(out, out_dtype, q, k_cache, v_cache, desc, block_tables,
                     max_blocks_per_seq, seq_lens, query_start_loc, num_seqs, total_q_rows,
                     max_seq_len, num_q_heads, scale, window, ws, bytes, stream);
}

pa_status pa_decode(void* out, pa_dtype out_dtype, const void* q, const void* k_cache,
                    const void* v_cache, const pa_cache_desc* desc,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
                    int32_t total_q_rows, int32_t max_seq_len, int32_t num_q_heads, float scale,
                    int32_t window, void* workspace, size_t workspace_bytes, void* stream) {
    DecodeArgs a;
    bool nothing;
    pa_status st = build_args(out, out_dtype, q, k_cache, v_cache, desc, block_tables,
                              max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                              total_q_rows, max_seq_len, num_q_heads, scale, window, workspace,
                              workspace_bytes, true, a, nothing);
    if (st != PA_OK || nothing) return st;
    hipStream_t s = (hipStream_t)stream;
    if (pa::launch_plan(a, s) != hipSuccess) return PA_ERR_LAUNCH;
    return run_attend(a, desc->dtype, s);
}

void pa_set_decode_profile_events(void* before, void* after) {
    g_prof_before = (hipEvent_t)before;
    g_prof_after = (hipEvent_t)after;
}

void pa_set_chunk_profile_events(void* before, void* after) {
    g_chunk_before = (hipEvent_t)before;
    g_chunk_after = (hipEvent_t)after;
}

}  // extern "C"
