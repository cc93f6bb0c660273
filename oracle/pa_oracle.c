/*
 * CPU oracle for paged KV-cache attention: plain fp64, slow on purpose.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark may load this library.  It shares no code, header or table with the HIP
 * library, and the library never calls it.
 *
 * What it computes is the plain definition of the method:
 *   - Slot write.  A new token's K and V go to the slot the block table assigns:
 *     block = slot / block_size, offset = slot % block_size ("vLLM and PagedAttention",
 *     ghkdgus29.github.io, section on basic decoding: new KV entries are placed after the
 *     existing ones in the logical block).  A negative slot is skipped.  Bit copy.
 *   - Attention.  Paging changes only where the bytes sit, so the result is ordinary
 *     attention over each sequence's logical (contiguous) K/V, reached by following the
 *     block table like a page table ("PagedAttention deep dive", donmain.dev, section on
 *     splitting the KV cache into blocks: the kernel gathers the blocks the table lists).
 *     For query row r of sequence s (n rows, context length L counting this step's
 *     tokens) the position is p = L - n + r and the attended range is [lo, p], lo = 0 or,
 *     with a window W > 0, max(0, p - W + 1) (a sliding layer sees only the last W
 *     tokens: sotaaz.com, section on layer kinds).  Query head h reads KV head
 *     h / (Hq / Hkv).  With x_t = scale * <q, K_t>, m = max x_t, w_t = exp(x_t - m):
 *     out = sum_t w_t V_t / sum_t w_t.  An empty range gives zeros.
 *
 * Cache layout (the pages only fix "one contiguous pool of fixed-size blocks"):
 *   k_cache, v_cache = [num_blocks][num_kv_heads][block_size][head_dim], row-major.
 * Element types: 0 = float32, 1 = IEEE binary16, 2 = bfloat16; every stored value is
 * widened to double exactly (decoded from its bit fields below).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_OK = 0, OR_ERR_ARG = -1, OR_ERR_BLOCK = -2, OR_ERR_SLOT = -3, OR_ERR_MEM = -4 };

static int elem_size(int dt) { return dt == OR_F32 ? 4 : 2; }

/* binary16: sign, 5-bit exponent (bias 15), 10-bit fraction */
static double f16_to_double(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 0x1f, f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^(1-15-10) */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25); /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper half of a binary32 */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return (double)x;
}

static double load(const void *base, size_t i, int dt) {
    if (dt == OR_F32) {
        float x;
        memcpy(&x, (const char *)base + 4 * i, 4);
        return (double)x;
    }
    uint16_t h;
    memcpy(&h, (const char *)base + 2 * i, 2);
    return dt == OR_F16 ? f16_to_double(h) : bf16_to_double(h);
}

/* ------------------------------------------------------------------ slot write */
int oracle_write_kv(const void *k, const void *v, const int64_t *slots, int64_t num_tokens,
                    void *k_cache, void *v_cache, int32_t num_blocks, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t dtype) {
    if (!k || !v || !slots || !k_cache || !v_cache || block_size <= 0) return OR_ERR_ARG;
    size_t row = (size_t)head_dim * elem_size(dtype);
    for (int64_t j = 0; j < num_tokens; ++j) {
        int64_t s = slots[j];
        if (s < 0) continue;
        int64_t blk = s / block_size, off = s % block_size;
        if (blk >= num_blocks) return OR_ERR_SLOT;
        for (int h = 0; h < num_kv_heads; ++h) {
            size_t src = ((size_t)j * num_kv_heads + h) * row;
            size_t dst = (((size_t)blk * num_kv_heads + h) * block_size + off) * row;
            memcpy((char *)k_cache + dst, (const char *)k + src, row);
            memcpy((char *)v_cache + dst, (const char *)v + src, row);
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------ attention core */
/* out[d] = softmax_t(scale * <q, K_t>) . V_t over the n rows listed in krows / vrows. */
static void attend(double *out, const double *q, const void *const *krows,
                   const void *const *vrows, int64_t n, int d, int dt, double scale, double *x) {
    for (int i = 0; i < d; ++i) out[i] = 0.0;
    if (n <= 0) return;
    double m = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += q[i] * load(krows[t], (size_t)i, dt);
        x[t] = scale * acc;
        if (x[t] > m) m = x[t];
    }
    double den = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        double w = exp(x[t] - m);
        den += w;
        for (int i = 0; i < d; ++i) out[i] += w * load(vrows[t], (size_t)i, dt);
    }
    for (int i = 0; i < d; ++i) out[i] /= den;
}

/* Shared driver: mode 0 = paged (through block tables), mode 1 = contiguous. */
static int attention_driver(int mode, double *out, const void *q, const void *kbase,
                            const void *vbase, int32_t dtype, int32_t num_blocks,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            const int32_t *block_tables, int32_t max_blocks,
                            const int64_t *tok_off, const int32_t *first_pos,
                            const int32_t *seq_lens, const int32_t *query_start_loc,
                            int32_t num_seqs, int32_t num_q_heads, double scale, int32_t window,
                            int32_t num_threads) {
    if (!out || !q || !kbase || !vbase || !seq_lens || num_kv_heads <= 0 ||
        num_q_heads % num_kv_heads)
        return OR_ERR_ARG;
    const int group = num_q_heads / num_kv_heads;
    const int d = head_dim;
    const size_t esz = (size_t)elem_size(dtype);
    int64_t max_len = 1;
    for (int s = 0; s < num_seqs; ++s)
        if (seq_lens[s] > max_len) max_len = seq_lens[s];
    int err = OR_OK;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)max_len);
        double *qd = (double *)malloc(sizeof(double) * (size_t)d);
        const void **kr = (const void **)malloc(sizeof(void *) * (size_t)max_len);
        const void **vr = (const void **)malloc(sizeof(void *) * (size_t)max_len);
        if (!x || !qd || !kr || !vr) {
#pragma omp atomic write
            err = OR_ERR_MEM;
        }
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int s = 0; s < num_seqs; ++s) {
            for (int h = 0; h < num_q_heads; ++h) {
                if (!x || !qd || !kr || !vr) continue;
                const int L = seq_lens[s];
                const int r0 = query_start_loc ? query_start_loc[s] : s;
                const int nrows = query_start_loc ? query_start_loc[s + 1] - query_start_loc[s] : 1;
                const int g = h / group;
                for (int r = 0; r < nrows; ++r) {
                    const int64_t p = (int64_t)L - nrows + r;
                    int64_t lo = 0;
                    if (window > 0 && p - window + 1 > 0) lo = p - window + 1;
                    int64_t n = p - lo + 1;
                    if (n < 0) n = 0;
                    int bad = 0;
                    for (int64_t t = lo; t <= p; ++t) {
                        size_t idx;
                        if (mode == 0) {
                            int64_t lb = t / block_size;
                            int32_t blk = lb < max_blocks ? block_tables[(size_t)s * max_blocks + lb] : -1;
                            if (blk < 0 || blk >= num_blocks) { bad = 1; break; }
                            idx = (((size_t)blk * num_kv_heads + g) * block_size + (size_t)(t % block_size)) * d;
                        } else {
                            int64_t row = tok_off[s] + (t - first_pos[s]);
                            if (t < first_pos[s]) { bad = 1; break; }
                            idx = ((size_t)row * num_kv_heads + g) * d;
                        }
                        kr[t - lo] = (const char *)kbase + idx * esz;
                        vr[t - lo] = (const char *)vbase + idx * esz;
                    }
                    if (bad) {
#pragma omp atomic write
                        err = OR_ERR_BLOCK;
                        continue;
                    }
                    const size_t qrow = ((size_t)(r0 + r) * num_q_heads + h) * d;
                    for (int i = 0; i < d; ++i) qd[i] = load(q, qrow + i, dtype);
                    attend(out + qrow, qd, kr, vr, n, d, dtype, scale, x);
                }
            }
        }
        free(x);
        free(qd);
        free(kr);
        free(vr);
    }
    return err;
}

/* Paged attention; out is [rows][num_q_heads][head_dim] doubles. */
int oracle_paged_attention(double *out, const void *q, const void *k_cache, const void *v_cache,
                           int32_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, const int32_t *block_tables,
                           int32_t max_blocks, const int32_t *seq_lens,
                           const int32_t *query_start_loc, int32_t num_seqs, int32_t num_q_heads,
                           double scale, int32_t window, int32_t num_threads) {
    if (!block_tables) return OR_ERR_ARG;
    return attention_driver(0, out, q, k_cache, v_cache, dtype, num_blocks, num_kv_heads,
                            head_dim, block_size, block_tables, max_blocks, NULL, NULL, seq_lens,
                            query_start_loc, num_seqs, num_q_heads, scale, window, num_threads);
}

/* Contiguous attention over logical per-sequence arrays k_log / v_log = [N][Hkv][d]:
 * token t of sequence s sits at row tok_off[s] + (t - first_pos[s]). */
int oracle_contiguous_attention(double *out, const void *q, const void *k_log, const void *v_log,
                                int32_t dtype, int32_t num_kv_heads, int32_t head_dim,
                                const int64_t *tok_off, const int32_t *first_pos,
                                const int32_t *seq_lens, const int32_t *query_start_loc,
                                int32_t num_seqs, int32_t num_q_heads, double scale,
                                int32_t window, int32_t num_threads) {
    if (!tok_off || !first_pos) return OR_ERR_ARG;
    return attention_driver(1, out, q, k_log, v_log, dtype, 0, num_kv_heads, head_dim, 1, NULL,
                            0, tok_off, first_pos, seq_lens, query_start_loc, num_seqs,
                            num_q_heads, scale, window, num_threads);
}

/* Exact widening of stored elements (exported so tests can pin the decoders). */
int oracle_widen(double *out, const void *src, int64_t n, int32_t dtype) {
    for (int64_t i = 0; i < n; ++i) out[i] = load(src, (size_t)i, dtype);
    return OR_OK;
}
