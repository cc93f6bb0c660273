/*
 * pa.h - paged KV-cache attention for AMD Instinct MI355X (gfx950): the C ABI.
 *
 * The KV cache is one pool of fixed 16-token blocks; each sequence owns a block table that
 * maps its logical blocks to physical ones, as a page table maps pages ("PagedAttention
 * deep dive", donmain.dev, section on splitting the KV cache into blocks; the pool is one
 * region reserved up front and a physical block is an index into it: velog.io "Batching
 * strategies", section 5, on why continuous batching needs PagedAttention).  This library
 * writes new tokens' K/V into the slots the tables assign and computes decode / chunk-row
 * attention by gathering K/V through the tables.  It also exports a host block ledger that
 * produces the tables and slots.
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are HIP device pointers; (host) are host pointers.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Device work is
 *     enqueued on it; no call synchronizes, allocates or frees device memory, and no
 *     pointer is kept after a call returns.  The caller owns every buffer.
 *   - Errors are returned as pa_status; nothing is launched when a host-checkable
 *     precondition fails.  Device-resident values the host cannot see (block ids, lengths)
 *     are range-checked on the device: an out-of-range value is never dereferenced, it sets
 *     a bit in the workspace's error word (see pa_decode) and the affected tokens are
 *     treated as absent.
 *
 * Cache layout (the pages fix only "a pool of fixed-size blocks"; this layout is this
 * library's choice): k_cache and v_cache are each [num_blocks][num_kv_heads][16][head_dim]
 * in the cache dtype, row-major, so each (block, KV head) tile of 16 x head_dim is one
 * contiguous run of bytes.  8-bit caches add a row of scales to each tile (see pa_dtype).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  PA_Q8_F16 and PA_Q8_BF16 are cache types only: an 8-bit cache with one
 * fp16 scale per 32 values, whose queries and new K / V rows are fp16 (PA_Q8_F16) or bf16
 * (PA_Q8_BF16).  Source: "KV cache by model" (sotaaz.com), planning notes of the
 * full-attention section - an 8-bit cache keeps a scale for every 32 values and takes
 * 53.1% of a 16-bit one.
 *
 * 8-bit cache layout: k_cache and v_cache are each [num_blocks][num_kv_heads][17][head_dim]
 * bytes.  Rows 0-15 of a (block, head) tile hold the int8 codes of the block's 16 tokens;
 * row 16 holds their scales, [16][head_dim / 32] fp16.  A value decodes as scale * code.
 * pa_write_kv quantizes each group of 32 consecutive values of a new row: scale = the
 * group's largest |x| / 127 in fp32, rounded to fp16 (held at 65504 if it would overflow);
 * code = round-half-to-even(x / scale) in fp32, clamped to [-127, 127]; an all-zero group
 * gets scale 0 and codes 0.  (The pages give the group size and the scale's 2 bytes; the
 * rest is this library's choice.) */
typedef enum pa_dtype {
    PA_F32 = 0,
    PA_F16 = 1,
    PA_BF16 = 2,
    PA_Q8_F16 = 3,
    PA_Q8_BF16 = 4
} pa_dtype;

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL = -1,           /* a required pointer is NULL                              */
    PA_ERR_SHAPE = -2,          /* inconsistent or negative sizes                          */
    PA_ERR_DTYPE = -3,          /* unknown dtype, or an unsupported dtype combination      */
    PA_ERR_UNSUPPORTED = -4,    /* head_dim / group size / block size with no kernel       */
    PA_ERR_WORKSPACE = -5,      /* workspace NULL, too small or not 256-byte aligned       */
    PA_ERR_LAUNCH = -6,         /* the HIP runtime reported an error                       */
    PA_ERR_OUT_OF_BLOCKS = -7,  /* ledger: not enough free blocks (nothing was taken)      */
    PA_ERR_SHARED_BLOCK = -8,   /* ledger: a copy-on-write or swap-out would read a block  *
                                 * that has writes pending in the current batch            */
    PA_ERR_BAD_SEQ = -9,        /* ledger: unknown sequence, or one that must be empty     */
    PA_ERR_ADMISSION = -10      /* ledger: a new request while sequences are swapped out   */
} pa_status;

/* Describes one layer's KV pool.  block_size must be 16 for the kernels (the pages'
 * default block size); the host ledger accepts any positive block size. */
typedef struct pa_cache_desc {
    int32_t num_blocks;     /* NB: physical blocks in the pool                      */
    int32_t block_size;     /* tokens per block (16)                                 */
    int32_t num_kv_heads;   /* Hkv                                                   */
    int32_t head_dim;       /* d: 64, 128 or 256                                     */
    pa_dtype dtype;         /* element type of k_cache / v_cache (and of q)          */
} pa_cache_desc;

/* Supported by the kernels: dtype F32, F16, BF16, Q8_F16, Q8_BF16; head_dim 64, 128, 256;
 * group size G = num_q_heads / num_kv_heads in {1, 2, 4, 8}; block_size 16.  Where an
 * entry point says "cache dtype" for q, k or v, an 8-bit cache means its fp16 / bf16
 * activation type. */

/* ------------------------------------------------------------------ slot write
 * pa_write_kv - scatter each new token's K and V into the slot its block table assigns.
 * Source: "vLLM and PagedAttention" notes (ghkdgus29.github.io), section on basic
 * decoding - new tokens' KV entries go after the existing ones in the sequence's logical
 * block, in the physical block the manager mapped it to.
 *
 *   k, v          (device) [num_tokens][num_kv_heads][head_dim], cache dtype.
 *   slot_mapping  (device) int64 [num_tokens]; slot = physical_block * 16 + offset.
 *                 A negative slot means "skip this token" (padding, or a token outside a
 *                 sliding window).  A slot >= num_blocks * 16 is skipped as well.
 *   k_cache, v_cache (device) the pool, layout above; written in place.
 *   desc          (host) pool description.
 * The copy is bit-exact.  Two tokens mapped to the same slot leave one of them (which one
 * is unspecified).  Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED,
 * PA_ERR_LAUNCH. */
pa_status pa_write_kv(const void* k, const void* v, const int64_t* slot_mapping,
                      int32_t num_tokens, void* k_cache, void* v_cache,
                      const pa_cache_desc* desc, void* stream);

/* ------------------------------------------------------------------ attention
 * pa_decode_workspace_size - bytes of device workspace pa_decode needs for this shape on
 * the current device (it depends on how many wavefronts the device keeps resident).
 * Returns 0 for unsupported arguments. */
size_t pa_decode_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                int32_t total_q_rows, int32_t num_q_heads,
                                int32_t max_seq_len);

/*
 * pa_decode - attention of each query row over its sequence's cached K/V, gathered through
 * the block table.  Sources: "PagedAttention deep dive" (donmain.dev), section on
 * splitting the KV cache into blocks (the kernel follows the table and gathers the
 * blocks); velog.io "Batching strategies", section 2.3 (KV reads are per sequence and not
 * shared by batching: this is a bandwidth-bound read of the cache); sotaaz.com "KV cache
 * by model", section on layer kinds (a sliding-window layer only sees the most recent W
 * tokens); duolabs.co.kr "vLLM vs Ollama", section on paging-based KV management (chunked
 * prefill mixes prompt chunks with decodes in one batch).
 *
 * For sequence s with context length L = seq_lens[s] (this step's tokens included; their
 * K/V must already be written) and n query rows, row r sits at position p = L - n + r and
 * attends to positions [lo, p], lo = 0, or lo = max(0, p - window + 1) when window > 0.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).  With
 * x_t = scale * <q, K_t>:  out = sum_t softmax(x)_t V_t.  An empty range gives zeros.
 *
 *   out           (device) [total_q_rows][num_q_heads][head_dim] in out_dtype
 *                 (PA_F32 recommended; F16/BF16 give the fp32 result rounded to nearest
 *                 even).
 *   q             (device) [total_q_rows][num_q_heads][head_dim], cache dtype.
 *   k_cache, v_cache, desc   the pool (device) and its description (host).
 *   block_tables  (device) int32 [num_seqs][max_blocks_per_seq]; only entries of blocks
 *                 that hold an attended position are read (others may hold anything).
 *   seq_lens      (device) int32 [num_seqs].
 *   query_start_loc (device) int32 [num_seqs + 1] row offsets, or NULL for one row per
 *                 sequence.  Sequences with one row take the decode kernel; sequences with
 *                 more rows (chunked prefill, causal within the chunk) take the chunk-row
 *                 kernel in the same call.
 *   max_seq_len   host-side upper bound of seq_lens (sequences above it, or above
 *                 16 * max_blocks_per_seq, are rejected on the device: zero output and an
 *                 error bit).
 *   scale         softmax scale (usually 1/sqrt(head_dim)).
 *   window        <= 0: full attention; > 0: sliding window of that many tokens.
 *   workspace     (device) at least pa_decode_workspace_size(...) bytes, 256-byte aligned.
 *                 Its first 4 bytes receive the call's device error bits: 1 = a block id
 *                 outside [0, num_blocks) was met, 2 = a sequence length or row count was
 *                 out of range, 4 = pa_decode_attend was given a plan made for the other
 *                 decode mode (a different window; nothing computed).  Concurrent calls
 *                 must not share a workspace.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE,
 * PA_ERR_LAUNCH.
 */
/* Tuning knob: the environment variable PA_DECODE_WAVES, when set to a positive number
 * below the device's resident count, caps the decode wavefront workers (for sweeps and
 * tests; a workspace sized without it is large enough). */
pa_status pa_decode(void* out, pa_dtype out_dtype, const void* q,
                    const void* k_cache, const void* v_cache, const pa_cache_desc* desc,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, const int32_t* query_start_loc,
                    int32_t num_seqs, int32_t total_q_rows, int32_t max_seq_len,
                    int32_t num_q_heads, float scale, int32_t window,
                    void* workspace, size_t workspace_bytes, void* stream);

/* pa_decode_write_attend - one decode step of one layer in one launch: the slot write of
 * each sequence's new token and the attention, for batches of one query row per sequence.
 * Source: "vLLM and PagedAttention" notes (ghkdgus29.github.io), section on basic decoding
 * (the new token's KV goes into the slot after the existing ones, in the block the manager
 * mapped), and "PagedAttention deep dive" (donmain.dev), section on splitting the KV cache
 * into blocks (attention gathers the blocks through the table).
 *
 * The result equals pa_write_kv of row s of k_new / v_new into the slot
 * block_tables[s][(L - 1) / bs] * bs + (L - 1) % bs, L = seq_lens[s] (nothing for L = 0),
 * followed by pa_decode_attend.  The newest token is taken from k_new / v_new directly and
 * the attention's own launches write it into the cache (the launch that combines cut
 * pairs, or in group mode the wavefront that holds the pair's last block), so the slot
 * write costs no launch of its own.
 *
 *   k_new, v_new  (device) [num_seqs][num_kv_heads][head_dim], cache dtype.
 *   k_cache, v_cache  (device) the pool; the new tokens' slots are written.
 *   The other arguments are pa_decode_attend's with query_start_loc = NULL and
 *   total_q_rows = num_seqs; the workspace must hold a plan from pa_decode_plan with those
 *   values.  A sequence's newest slot must lie in a block no other sequence of the batch
 *   reads (the ledger's copy-on-write guarantees it).
 * Errors: as pa_decode_attend; PA_ERR_UNSUPPORTED for 8-bit caches (their new rows are
 * quantized by pa_write_kv first). */
pa_status pa_decode_write_attend(void* out, pa_dtype out_dtype, const void* q, const void* k_new,
                                 const void* v_new, void* k_cache, void* v_cache,
                                 const pa_cache_desc* desc, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
                                 float scale, int32_t window, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* pa_decode_noalloc - pa_decode for callers that cannot allocate device memory: code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc.  It takes the same
 * arguments as pa_decode minus the workspace: its workspace is a fixed array of
 * PA_NOALLOC_SCRATCH_BYTES bytes in the library's device memory, one per device the library
 * runs on, held until the process ends.  The call allocates and frees nothing; on its first
 * call on a device it looks up that device's array (hipGetSymbolAddress).
 *   - Shapes whose pa_decode_workspace_size exceeds PA_NOALLOC_SCRATCH_BYTES are refused
 *     with PA_ERR_WORKSPACE before anything is launched.
 *   - Every call on one device shares that device's array, which keeps the last call's
 *     contents (each call's own plan rewrites everything its kernels read).  Calls whose
 *     work overlaps on one device (other streams, other threads) race: serialize them.
 *   - The error bits that pa_decode leaves in its workspace are not readable here.
 * Errors as pa_decode, and PA_ERR_LAUNCH if the array's address cannot be found. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_decode_noalloc(void* out, pa_dtype out_dtype, const void* q,
                            const void* k_cache, const void* v_cache, const pa_cache_desc* desc,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, const int32_t* query_start_loc,
                            int32_t num_seqs, int32_t total_q_rows, int32_t max_seq_len,
                            int32_t num_q_heads, float scale, int32_t window, void* stream);

/* pa_decode_plan + pa_decode_attend = pa_decode, split so that one plan serves every layer
 * of a step: the plan depends only on block_tables, seq_lens, query_start_loc, the shapes
 * and the window, which all layers of a step share (the CPU ships one set of tables per
 * step: velog.io "Batching strategies", section 5, one step's flow).  Both take the same
 * arguments as pa_decode; pa_decode_attend must be given the values pa_decode_plan was
 * given on the same workspace (scale, q, caches and out may differ), and the plan stays
 * valid until the workspace is planned again.  pa_decode_plan ignores out, q and the caches.
 * Errors as pa_decode. */
pa_status pa_decode_plan(const pa_cache_desc* desc, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens,
                         const int32_t* query_start_loc, int32_t num_seqs,
                         int32_t total_q_rows, int32_t max_seq_len, int32_t num_q_heads,
                         int32_t window, void* workspace, size_t workspace_bytes,
                         void* stream);
pa_status pa_decode_attend(void* out, pa_dtype out_dtype, const void* q,
                           const void* k_cache, const void* v_cache,
                           const pa_cache_desc* desc, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                           const int32_t* query_start_loc, int32_t num_seqs,
                           int32_t total_q_rows, int32_t max_seq_len, int32_t num_q_heads,
                           float scale, int32_t window, void* workspace,
                           size_t workspace_bytes, void* stream);

/* pa_decode_kernel_name - the name of the decode kernel pa_decode launches for a batch of
 * num_seqs decode rows (one query row per sequence, query_start_loc NULL) of this pool and
 * query-head count under `window` (0: none):
 *   "decode_mfma_kernel"  the matrix-core kernel, for groups of 4 or 8 query heads per KV
 *                         head with 16-token blocks and 16-bit or 8-bit caches;
 *   "decode_group_kernel" the per-lane kernel in group mode, one workgroup per (row, KV
 *                         head) pair, for sliding-window batches on the per-lane kernel
 *                         with 16-token blocks whose windows span at most 256 or 512
 *                         blocks (sotaaz.com, "KV cache by model", layer kinds);
 *   "decode_kernel"       the per-lane kernel otherwise;
 * NULL for unsupported arguments.  For reports that name the kernel a profile timed.
 * Static storage; launches nothing (with window > 0 it queries the device's occupancy, so
 * a device must be present). */
const char* pa_decode_kernel_name(const pa_cache_desc* desc, int32_t num_q_heads,
                                  int32_t num_seqs, int32_t window);

/* Profiling hook: when set (non-NULL), every later pa_decode / pa_decode_attend records the
 * hipEvent_t `before` just before its decode-kernel launch and `after` just after it, on
 * the call's stream, so a caller can time that kernel alone.  The events are the caller's;
 * NULL, NULL switches the hook off.  Process-wide, not thread-safe. */
void pa_set_decode_profile_events(void* before, void* after);

/* The same hook around the chunk-row kernel launch (calls whose sequences include chunks
 * of several query rows and whose cache dtype is F16 or BF16). */
void pa_set_chunk_profile_events(void* before, void* after);

/* pa_stream_read - read a device buffer once, contiguously, with the 16-byte non-temporal
 * loads the attention kernels use, and write (practically) nothing.  It measures the plain
 * read rate of the device, the ceiling that the paged kernels' KV-read rates are set
 * against ("PagedAttention deep dive", donmain.dev: decoding is bound by reading the KV
 * cache).  Not part of the attention path.
 *
 *   buf     (device) the buffer, 16-byte aligned; only read.
 *   bytes   a multiple of 16; 0 launches nothing.
 *   sink    (device) one uint32; receives a word only if the XOR of all words read equals
 *           0x9e3779b9 (so that the loads cannot be removed); otherwise untouched.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (misaligned or bytes % 16 != 0), PA_ERR_LAUNCH. */
pa_status pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Human-readable name of a status code (static storage). */
const char* pa_status_string(pa_status s);

/* ------------------------------------------------------------------ block copy
 * pa_copy_blocks - carry out a batch of copy-on-write copies on the device.  Source: "vLLM
 * and PagedAttention" notes (ghkdgus29.github.io), section on parallel sampling - when
 * samples sharing a block write different tokens into it, the block is copied.
 *
 *   k_cache, v_cache (device) the pool, layout above; written in place.
 *   desc          (host) pool description (any block_size here).
 *   copies        (device) int32 [num_copies][3]: (src_block, dst_block, entries).  For
 *                 every KV head, rows 0 .. entries-1 of block src (K and V) are copied to the
 *                 same rows of block dst; rows entries.. of dst are not touched.
 *   num_copies    >= 0; 0 launches nothing.
 *   error_word    (device, nullable) int32; a triple with a block id outside
 *                 [0, num_blocks) or entries outside [0, block_size] is skipped and sets
 *                 bit 0 (value 1) here.
 * All triples are applied at once: the destinations must be distinct and no destination
 * may be the source of another triple of the same call (pa_pool_take_copies batches obey
 * this); otherwise the contents of the blocks concerned are unspecified, but nothing
 * outside them is read or written.  The copy is bit-exact.  Errors: PA_ERR_NULL,
 * PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_LAUNCH. */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const pa_cache_desc* desc,
                         const int32_t* copies, int32_t num_copies, int32_t* error_word,
                         void* stream);

/* ------------------------------------------------------------------ block swap
 * pa_swap_blocks - copy whole blocks between two pools with the same tile shape, for
 * swapping ("vLLM and PagedAttention" notes, scheduling section: evicted KV blocks go to
 * CPU memory and come back when there is room).  Either pool may be pinned host memory
 * (allocated with hipHostMalloc, e.g. a torch tensor with pin_memory=True): the kernel
 * reads or writes it directly over the host link.
 *
 *   src_k, src_v  the pool read: src_blocks blocks of num_kv_heads tiles (device or pinned
 *                 host).
 *   dst_k, dst_v  the pool written: dst_blocks blocks (device or pinned host).
 *   desc          (host) tile shape (block_size, num_kv_heads, head_dim, dtype; its
 *                 num_blocks is not used).
 *   pairs         (device) int32 [n][2]: (src block, dst block).
 *   error_word    (device, nullable) int32; a pair with an id out of range is skipped and
 *                 sets bit 0 (value 1).
 * All pairs are applied at once: destinations must be distinct and no pool may be both
 * read and written by one call.  The copy is bit-exact.  Errors: PA_ERR_NULL,
 * PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED (a pointer that is neither device memory
 * nor pinned host memory), PA_ERR_LAUNCH. */
pa_status pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                         const pa_cache_desc* desc, int32_t src_blocks, int32_t dst_blocks,
                         const int32_t* pairs, int32_t n, int32_t* error_word, void* stream);

/* ------------------------------------------------------------------ host block ledger
 * A host-only ledger of one pool's blocks (no device memory).  Sources: "PagedAttention
 * deep dive" (donmain.dev), sections on splitting the KV cache into blocks (a block is
 * taken only when the sequence's last block is full, from anywhere in the pool) and on
 * waste falling under 4% (only the last block can be partly empty); "vLLM and
 * PagedAttention" notes (ghkdgus29.github.io), sections on basic decoding (filled counts,
 * freeing at the end), parallel sampling (reference counts of shared blocks) and
 * scheduling (all-or-nothing per sequence).
 *
 * Policy where the pages are silent: free blocks leave the pool first-in first-out,
 * starting from `free_order` (or 0..num_blocks-1); a block whose count drops to zero goes
 * to the back of the queue, in logical-block order.  A handle is not thread-safe. */
typedef struct pa_pool pa_pool;

/* free_order (host, nullable): the order in which blocks are first handed out; a
 * permutation of a subset of [0, num_blocks) (blocks left out are never handed out). */
pa_status pa_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                         int32_t free_order_len, pa_pool** out);
void pa_pool_destroy(pa_pool* p);

/* Keep only the last `window` tokens of `seq` (0 = keep all).  Must precede the first
 * append.  Creates `seq` if it is unknown (PA_ERR_ADMISSION while sequences are swapped
 * out).  Later appends release blocks that fall wholly before the window (their table
 * entries become -1) and report slot -1 for positions that are not kept. */
pa_status pa_seq_set_window(pa_pool* p, int64_t seq, int32_t window);

/* Append n_tokens to `seq` (created on first use) and write each token's slot
 * (block * block_size + offset, or -1) to slots_out (host, n_tokens entries, nullable).
 *
 * Copy-on-write ("vLLM and PagedAttention" notes, ghkdgus29.github.io, section on parallel
 * sampling; "PagedAttention deep dive", section on block sharing): if the first token lands
 * in the sequence's partly filled last block while another sequence also references that
 * block, the append first takes a fresh block, records the copy (old block, fresh block,
 * entries the old block holds) in the pool's copy batch, and drops one reference from the
 * old block; the sequence's table then points at the fresh block.  The last holder of a
 * block writes in place.  The copy is taken before any new block of the same append.
 *
 * Batches: pa_pool_take_copies ends a batch.  The caller carries out a batch's swap-outs
 * (pa_swap_blocks), copies (pa_copy_blocks), swap-ins and slot writes (pa_write_kv), in
 * that order, before the next batch's.  Because each kind runs all at once, an append
 * whose copy would read a block with writes pending in the current batch (slots, a copy
 * or a swap-in into it) fails with PA_ERR_SHARED_BLOCK, and blocks released while work on
 * them is pending are not handed out again before the batch ends.
 *
 * All or nothing: PA_ERR_OUT_OF_BLOCKS if the free blocks do not suffice for the copy and
 * the new blocks, PA_ERR_SHARED_BLOCK as above, PA_ERR_BAD_SEQ for a swapped-out
 * sequence, PA_ERR_ADMISSION for an unknown `seq` while any sequence is swapped out (see
 * the swapping section below); nothing changes on error. */
pa_status pa_seq_append(pa_pool* p, int64_t seq, int32_t n_tokens, int64_t* slots_out);

/* `dst` (new or empty) becomes a second sample of `src` (parallel sampling): the same
 * length, window and physical blocks, each block one reference more.  Blocks released by a
 * window stay -1 in the copy of the table. */
pa_status pa_seq_fork(pa_pool* p, int64_t dst, int64_t src);

/* ---- swapping (ghkdgus29.github.io, "vLLM and PagedAttention" notes, scheduling section:
 * eviction takes all of a sequence's blocks or none, the victim is the sequence that
 * arrived last, and swapping moves the evicted blocks to CPU memory until GPU memory frees
 * up).  The host swap space is a pool of host blocks, ids 0 .. num_host_blocks-1, handed
 * out first-in first-out; the caller owns its memory (pinned host tiles laid out like the
 * device pool's) and moves the data with pa_swap_blocks.
 *
 * Batch order: a batch's swap-outs run first, then its copies (pa_copy_blocks), then its
 * swap-ins, then its slot writes; pa_pool_take_copies ends the batch.  A block or host
 * block freed while work on it is pending in the batch joins its free queue only when the
 * batch ends.
 *
 * pa_pool_set_host_blocks: size the host swap space (PA_ERR_BAD_SEQ while host blocks are
 * in use).
 * pa_pool_latest_resident: the victim - the resident sequence holding device blocks that
 * arrived last (a sequence arrives when it is first created); PA_ERR_BAD_SEQ if none.
 * pa_seq_swap_out: move the blocks `seq` holds alone (reference count 1) to host blocks;
 * blocks it shares stay on the device, still referenced.  Writes (device, host) int32
 * pairs to pairs (host, 2 * cap entries), *n their number.  All or nothing:
 * PA_ERR_OUT_OF_BLOCKS if host blocks are short, PA_ERR_SHARED_BLOCK if one of the blocks
 * has writes pending in the batch, PA_ERR_SHAPE if cap < *n; nothing changes on error.
 * The sequence's table entries for moved blocks become -1; until its swap-in it cannot
 * append, fork or share.  pa_seq_free releases its host blocks too.
 * pa_seq_swap_in: bring it back; writes (host, device) pairs; all or nothing
 * (PA_ERR_OUT_OF_BLOCKS if free device blocks are short). */
pa_status pa_pool_set_host_blocks(pa_pool* p, int32_t num_host_blocks);
int32_t pa_pool_num_host_free(const pa_pool* p);
pa_status pa_pool_latest_resident(const pa_pool* p, int64_t* seq);
pa_status pa_seq_swap_out(pa_pool* p, int64_t seq, int32_t* pairs, int32_t cap, int32_t* n);
pa_status pa_seq_swap_in(pa_pool* p, int64_t seq, int32_t* pairs, int32_t cap, int32_t* n);

/* End the current copy batch: write its copies, in the order they were recorded, as
 * (src_block, dst_block, entries) int32 triples to out (host, 3 * cap entries) and start a
 * new batch.  *n receives the number of copies.  PA_ERR_SHAPE if cap is too small (nothing
 * is taken; *n tells how many there are). */
pa_status pa_pool_take_copies(pa_pool* p, int32_t* out, int32_t cap, int32_t* n);
int32_t pa_pool_num_pending_copies(const pa_pool* p);

/* `dst` (new or empty) begins with the first n_tokens of `src`, pointing at the same
 * physical blocks (each gets one more reference): a shared system prompt ("PagedAttention
 * deep dive", section on block sharing).  An unknown dst is a new request:
 * PA_ERR_ADMISSION while sequences are swapped out.  A prefix that ends inside a block shares that
 * block too; the first append of either sequence into it copies it (see pa_seq_append). */
pa_status pa_seq_share_prefix(pa_pool* p, int64_t dst, int64_t src, int32_t n_tokens);

/* Drop `seq`: one reference less on each of its blocks; blocks reaching zero are free. */
pa_status pa_seq_free(pa_pool* p, int64_t seq);

/* Copy seq's block table (entries -1 for released blocks) into out (host, cap entries);
 * *n receives its length.  PA_ERR_SHAPE if cap is too small (nothing copied). */
pa_status pa_seq_block_table(const pa_pool* p, int64_t seq, int32_t* out, int32_t cap,
                             int32_t* n);

/* Block tables of num_seqs sequences as one row-major [num_seqs][max_blocks] int32 array
 * (host), ready to upload; entries past a table's end and released entries get `fill`. */
pa_status pa_pool_block_tables(const pa_pool* p, const int64_t* seqs, int32_t num_seqs,
                               int32_t max_blocks, int32_t fill, int32_t* out);

int32_t pa_seq_len(const pa_pool* p, int64_t seq);          /* -1 if unknown          */
int32_t pa_pool_num_free(const pa_pool* p);
int32_t pa_block_refcount(const pa_pool* p, int32_t block);  /* 0 if free or unknown   */

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
