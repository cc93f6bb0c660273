// Internal declarations shared by the host ABI (abi.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pa.h"

namespace pa {

constexpr int kBlock = 16;          // default tokens per KV block (8 and 32 also have
                                    // decode kernels for 16-bit caches)
constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kWavesPerGroup = 4;   // decode workgroup = 4 independent wavefront workers
constexpr int kMinBlocksPerWave = 12;  // default smallest share of KV blocks per wavefront
constexpr int kMinBlocksFloor = 4;     // the plan needs shares of at least 4 blocks
constexpr int kPairCost = 14;       // default fixed cost per pair in quarter blocks: the
                                    // dependent loads that start a segment
// The 8-bit matrix-core decode kernel reads half the bytes per block, so a pair's fixed
// cost weighs more against its blocks there.
constexpr int kPairCostQ8Mfma = 22;
// The plan lowers the pair cost where shares are short (consecutive share starts lie at
// least 4 T / W - 1 quarter blocks apart), so any cost up to this bound keeps every share
// non-empty.
constexpr int kMaxPairCost = 27;
constexpr int kQ8Group = 32;        // values per scale in 8-bit caches

// Group mode: each (row, KV head) pair is split among at most kGroupMaxSplit workgroups of
// kWavesPerGroup wavefronts; a wavefront takes at most 64 blocks (one chunk of block ids),
// so a window may span at most 64 kWavesPerGroup kGroupMaxSplit blocks.
constexpr int kGroupMaxSplit = 8;

// Error bits written to the first word of the workspace.
constexpr int kErrBlockId = 1;
constexpr int kErrSeqLen = 2;
constexpr int kErrPlanMode = 4;   // the plan was made for the other decode mode

// One decode unit per query row: what the row reads, derived once per call by the plan
// kernel.  A chunk row r of a sequence with n rows and length L is the decode row of
// length L - n + r + 1 (causal mask), so every row is a unit of the same kind.
struct UnitInfo {
    int32_t b_lo;   // first logical block the row reads (-1: row done by the chunk kernel)
    int32_t nb;     // number of blocks it reads (0: nothing to read)
    int32_t len;    // tokens visible to the row (positions < len)
    int32_t seq;    // block-table row
};

// The first segment of a wavefront's share, laid out by the plan so that the wavefront can
// issue its queries', block ids' and first tile's loads right after reading it (instead of
// finding its pair through the share start, the unit offsets and the unit record first).
struct WaveStart {
    uint32_t x0, x1;   // the share: linear blocks [x0, x1)
    int32_t u, g;      // its first pair (unit, KV head)
    uint32_t ps, pe;   // that pair's linear blocks [ps, pe)
    int32_t j0, j1;    // the first segment's table entries [j0, j1)
    int32_t seq, len;  // the unit's table row and visible length
    int32_t b0, b1;    // block ids at j0 and j0 + 1 (b0 again when j1 = j0 + 1)
};
static_assert(sizeof(WaveStart) == 48, "three 16-byte loads");

// Workspace layout (all offsets 256-byte aligned); U = query rows, W = wavefront workers:
//   header   int32[64]: [0] error bits, [1] total blocks T, [2] active waves,
//                       [3] rows with nothing to read (their output is zeros),
//                       [4] chunk-row tiles, [5] the plan's group_mode
//   cb       uint32[U+1]   linear offset of pair (u, kv head 0); pair (u, g) starts at
//                          cb[u] + g * nb(u) and spans nb(u) blocks
//   cw       uint32[U+1]   the same in the weighted space the wave shares cut evenly: a
//                          pair weighs 4 nb(u) + pair_cost (quarter blocks)
//   unit     UnitInfo[U]
//   empty    int32[U]      the rows with nothing to read
//   wave_x0  uint32[W+1]   first linear block of each wave's share
//   wave_u   int32[W]      unit holding that block, while the plan runs; then the number of
//                          shares of the cut pair that the share's last segment opens (0:
//                          none), which the decode kernels read for the pair's merge task
//   wave_st  WaveStart[Wmax+4]  each wavefront's first segment (every launched
//                          wavefront reads its entry before it checks w < W)
//   tiles    int2[Tmax]    chunk-row tiles (sequence, first row) for the MFMA kernel
//   tasks    int4[W+1]     merge task of the cut pair whose first share boundary is w:
//                          (unit, KV head, contributing wavefronts, slot of the first);
//                          zeroed by the plan, written by the pair's first wavefront;
//                          in group mode int32 per pair: the arrival counter of its
//                          workgroups (zeroed by the plan, reset by the last arrival)
//   part_ml  float2[W*2*G]       partial (max, sum) per wave, slot, head of the group
//                                (group mode: per workgroup and head)
//   part_acc float[W*2*G*d]      partial unnormalised output
struct Layout {
    size_t header, cb, cw, unit, empty, wave_x0, wave_u, wave_st, tiles, tasks, part_ml, part_acc,
        total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline Layout layout(int num_rows, int max_waves, int max_tiles, int group, int head_dim) {
    Layout L{};
    size_t o = 0;
    L.header = o;   o = align256(o + 64 * sizeof(int32_t));
    L.cb = o;       o = align256(o + (size_t)(num_rows + 1) * sizeof(uint32_t));
    L.cw = o;       o = align256(o + (size_t)(num_rows + 1) * sizeof(uint32_t));
    L.unit = o;     o = align256(o + (size_t)num_rows * sizeof(UnitInfo));
    L.empty = o;    o = align256(o + (size_t)num_rows * sizeof(int32_t));
    L.wave_x0 = o;  o = align256(o + (size_t)(max_waves + 1) * sizeof(uint32_t));
    L.wave_u = o;   o = align256(o + (size_t)max_waves * sizeof(int32_t));
    L.wave_st = o;  o = align256(o + (size_t)(max_waves + 4) * sizeof(WaveStart));
    L.tiles = o;    o = align256(o + (size_t)max_tiles * 2 * sizeof(int32_t));
    L.tasks = o;    o = align256(o + (size_t)(max_waves + 1) * 4 * sizeof(int32_t));
    L.part_ml = o;  o = align256(o + (size_t)max_waves * 2 * group * 2 * sizeof(float));
    L.part_acc = o; o = align256(o + (size_t)max_waves * 2 * group * head_dim * sizeof(float));
    L.total = o;
    return L;
}

// Everything one pa_decode call hands to its kernels.
struct DecodeArgs {
    void* out;
    int out_dtype;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    const int32_t* query_start_loc;   // may be null
    // This step's new K / V rows, [rows][num_kv_heads][head_dim] in the cache dtype, or null.
    // When set (decode rows only: one row per sequence), the decode kernels take the token
    // at position len - 1 of row u from row u here instead of the cache, and the merge
    // launch that follows writes each row into its slot: a decode step's slot write costs
    // no launch of its own.  row_bytes: bytes of one K or V row (head_dim x element size).
    const void* k_new;
    const void* v_new;
    int32_t row_bytes;
    int32_t num_blocks, block_size, num_kv_heads, head_dim, num_q_heads, group;
    int32_t max_blocks, num_seqs, total_q_rows, max_seq_len, window;
    float scale;
    int32_t max_waves;                // decode wavefront workers launched
    int32_t wave_round;               // wavefronts of one workgroup on every compute unit
    int32_t chunk_rows;               // query rows per chunk tile (0: chunk rows decode)
    int32_t max_tiles;                // chunk tiles the work list holds
    int32_t pair_cost;                // fixed cost of a (row, KV head) pair, quarter blocks
    int32_t min_blocks;               // smallest share of blocks a wavefront is given
    // Group mode (sliding-window decode batches on the per-lane kernel): one workgroup of
    // group_mode workgroups per (row, KV head) pair (0: off), wavefront i of the pair's
    // 4 group_mode taking the i-th part of its blocks; they combine in LDS and through the
    // pair's arrival counter, so no merge launch follows.  max_waves is then
    // kWavesPerGroup x group_mode x rows x KV heads.
    int32_t group_mode;
    char* ws;
    Layout lay;
};

// The fixed workspace of pa_decode_noalloc on the current device (noalloc.hip): its device
// address and size, looked up on the first call on each device.
pa_status noalloc_scratch(void** out, size_t* bytes);

// launchers (each enqueues on `stream`, returns hipSuccess or the launch error)
hipError_t launch_write_kv(const void* k, const void* v, const int64_t* slots, int32_t n,
                           void* kc, void* vc, int32_t nb, int32_t bs, int32_t hkv, int32_t d,
                           int32_t elem_bytes, hipStream_t stream);
hipError_t launch_write_kv_q8(const void* k, const void* v, const int64_t* slots, int32_t n,
                              void* kc, void* vc, int32_t nb, int32_t hkv, int32_t d,
                              int act_dtype, hipStream_t stream);
hipError_t launch_copy_blocks(void* kc, void* vc, const int32_t* copies, int32_t n,
                              int32_t nb, int32_t hkv, int32_t bs, int32_t row_bytes,
                              int32_t scale_bytes, int32_t* err, hipStream_t stream);
hipError_t launch_swap_blocks(const void* sk, const void* sv, void* dk, void* dv,
                              const int32_t* pairs, int32_t n, int32_t src_nb, int32_t dst_nb,
                              int32_t hkv, int32_t tile_bytes, int32_t* err,
                              hipStream_t stream);
hipError_t launch_plan(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream);
hipError_t launch_merge(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_chunk(const DecodeArgs& a, int dtype, hipStream_t stream);

// The decode kernel instance for (dtype, head_dim, group), or null if none is built;
// new_rows: the instance that takes the step's new rows (pa_decode_write_attend).
const void* decode_kernel_ptr(int dtype, int head_dim, int group, int block_size,
                              bool new_rows = false);
// The group-mode decode kernel instance (16-token blocks), or null.
const void* decode_group_ptr(int dtype, int head_dim, int group, bool new_rows);
// Whether that instance is the matrix-core decode kernel (decode_mfma_kernel).
bool decode_uses_mfma(int dtype, int group, int block_size);
// The chunk-row MFMA kernel instance, or null (then chunk rows run as decode rows).
const void* chunk_kernel_ptr(int dtype, int head_dim, int group, int block_size);
// Query rows one chunk tile covers: 4 wavefronts x 32 (row, head) pairs / group.
inline int chunk_tile_rows(int group) { return kWavesPerGroup * 32 / group; }

}  // namespace pa
