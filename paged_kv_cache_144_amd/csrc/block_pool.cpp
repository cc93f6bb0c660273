// Host block ledger: which physical block each logical block of each sequence lives in.
//
// Sources: "PagedAttention deep dive" (donmain.dev) - blocks are taken one at a time, only
// when a sequence's last block is full, from anywhere in the pool (section on splitting the
// KV cache into blocks); only the last block can be partly filled (section on waste under
// 4%); several tables may point at one block (section on block sharing).
// "vLLM and PagedAttention" notes (ghkdgus29.github.io) - the manager counts the entries
// in each block and frees them when the request ends (basic decoding), counts the
// sequences referencing a block and copies a shared block when samples write different
// tokens into it, while earlier blocks stay shared (parallel sampling), and evicts all of
// a sequence or none of it, the latest arrival first, moving its blocks to CPU memory until
// there is room again, and takes no new request while any sequence sits in CPU memory
// (scheduling, Swapping among the restoring strategies).  A sliding-window layer keeps only
// its last W tokens (sotaaz.com, section on layer kinds).
//
// Admission: a call that would create a sequence for a new request (append, share_prefix,
// set_window on an unknown id) returns PA_ERR_ADMISSION while a sequence is swapped out.
// A fork is a further sample of a request already taken and stays allowed.
//
// Batches: the caller carries out one batch's work in the order swap-outs, copies,
// swap-ins, slot writes (each kind all at once) and ends the batch with
// pa_pool_take_copies.  So a copy or a swap-out may not read a block with writes pending
// in the batch, and a block (or host block) freed while work on it is pending joins its
// free queue only when the batch ends.
//
// The CPU side owns this ledger and ships block tables to the GPU each step (velog.io,
// "Batching strategies", section 5: the scheduler and block manager run on the CPU).
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

struct Seq {
    std::vector<int32_t> blocks;  // logical -> physical; -1 = released / never held / on host
    std::vector<int32_t> host;    // while swapped out: host block per logical block, or -1
    int64_t len = 0;              // tokens appended so far
    int32_t window = 0;           // 0 = keep everything
    int64_t arrival = 0;          // creation order
    bool swapped = false;
};

}  // namespace

struct pa_pool {
    int32_t num_blocks = 0;
    int32_t bs = 16;
    std::deque<int32_t> free_q;        // first-in first-out
    std::vector<int32_t> ref;          // per physical block
    std::unordered_map<int64_t, Seq> seqs;
    // Copy-on-write batch: copies recorded since the last take, as (src, dst, entries)
    // triples, and the blocks that received slots or a copy in that time.  A copy may not
    // read such a block: the batch's copies run all at once, before the batch's writes.
    std::vector<int32_t> pending;
    std::vector<uint8_t> touched;
    std::vector<int32_t> touched_list;
    // Blocks a pending copy reads, and blocks freed while work on them is pending: those
    // join the free queue when the batch ends, so no batch reads and writes one block in
    // two roles.
    std::vector<uint8_t> copy_src;
    std::vector<int32_t> copy_src_list;
    std::vector<int32_t> quarantine;
    // host swap space
    int32_t num_host = 0;
    std::deque<int32_t> host_free;
    std::vector<int32_t> host_quarantine;
    int64_t clock = 0;
    int64_t num_swapped = 0;           // sequences whose blocks are in host memory

    // a new request waits while any sequence is swapped out
    bool admission_closed(int64_t seq) const {
        return num_swapped > 0 && seqs.find(seq) == seqs.end();
    }
    bool busy(int32_t b) const { return touched[b] || copy_src[b]; }
    void release(int32_t b) {
        if (--ref[b] != 0) return;
        if (busy(b))
            quarantine.push_back(b);
        else
            free_q.push_back(b);
    }
    void touch(int32_t b) {
        if (!touched[b]) {
            touched[b] = 1;
            touched_list.push_back(b);
        }
    }
    void mark_copy_src(int32_t b) {
        if (!copy_src[b]) {
            copy_src[b] = 1;
            copy_src_list.push_back(b);
        }
    }
    // the sequence, created (with the next arrival stamp) if it does not exist
    Seq& create(int64_t seq) {
        auto it = seqs.find(seq);
        if (it != seqs.end()) return it->second;
        Seq& s = seqs[seq];
        s.arrival = ++clock;
        return s;
    }
    void end_batch() {
        pending.clear();
        for (int32_t b : touched_list) touched[b] = 0;
        touched_list.clear();
        for (int32_t b : copy_src_list) copy_src[b] = 0;
        copy_src_list.clear();
        for (int32_t b : quarantine) free_q.push_back(b);
        quarantine.clear();
        for (int32_t h : host_quarantine) host_free.push_back(h);
        host_quarantine.clear();
    }
};

extern "C" {

pa_status pa_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                         int32_t free_order_len, pa_pool** out) {
    if (!out) return PA_ERR_NULL;
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0) return PA_ERR_SHAPE;
    pa_pool* p = new (std::nothrow) pa_pool();
    if (!p) return PA_ERR_SHAPE;
    p->num_blocks = num_blocks;
    p->bs = block_size;
    p->ref.assign(num_blocks, 0);
    p->touched.assign(num_blocks, 0);
    p->copy_src.assign(num_blocks, 0);
    if (free_order) {
        if (free_order_len < 0 || free_order_len > num_blocks) {
            delete p;
            return PA_ERR_SHAPE;
        }
        std::vector<char> seen(num_blocks, 0);
        for (int32_t i = 0; i < free_order_len; ++i) {
            int32_t b = free_order[i];
            if (b < 0 || b >= num_blocks || seen[b]) {
                delete p;
                return PA_ERR_SHAPE;
            }
            seen[b] = 1;
            p->free_q.push_back(b);
        }
    } else {
        for (int32_t b = 0; b < num_blocks; ++b) p->free_q.push_back(b);
    }
    *out = p;
    return PA_OK;
}

void pa_pool_destroy(pa_pool* p) { delete p; }

pa_status pa_seq_set_window(pa_pool* p, int64_t seq, int32_t window) {
    if (!p) return PA_ERR_NULL;
    if (window < 0) return PA_ERR_SHAPE;
    if (p->admission_closed(seq)) return PA_ERR_ADMISSION;
    Seq& s = p->create(seq);
    if (s.len != 0 || s.swapped) return PA_ERR_BAD_SEQ;
    s.window = window;
    return PA_OK;
}

pa_status pa_seq_append(pa_pool* p, int64_t seq, int32_t n_tokens, int64_t* slots_out) {
    if (!p) return PA_ERR_NULL;
    if (n_tokens < 0) return PA_ERR_SHAPE;
    {
        auto it = p->seqs.find(seq);
        if (it != p->seqs.end() && it->second.swapped) return PA_ERR_BAD_SEQ;
    }
    if (p->admission_closed(seq)) return PA_ERR_ADMISSION;
    Seq& s = p->create(seq);
    const int64_t bs = p->bs;
    const int64_t cur = s.len, end = cur + n_tokens;
    // first position that is still kept after this append
    const int64_t keep_from = (s.window > 0 && end - s.window > 0) ? end - s.window : 0;
    const int64_t first_kept_blk = keep_from / bs;
    const int64_t blocks_after = (end + bs - 1) / bs;
    const int64_t held = (int64_t)s.blocks.size();

    // a token written into the current, partly filled last block while another sequence
    // holds it: that block is copied first (copy-on-write)
    int64_t cow = -1;
    if (n_tokens > 0 && cur % bs != 0) {
        const int64_t last = cur / bs;
        if (last >= first_kept_blk && s.blocks[last] >= 0 && p->ref[s.blocks[last]] > 1) {
            if (p->touched[s.blocks[last]]) return PA_ERR_SHARED_BLOCK;
            cow = last;
        }
    }
    // blocks to open (logical ids held..blocks_after-1 that hold a kept position, plus the
    // copy) versus blocks available (free now, plus held blocks this append releases)
    int64_t need = cow >= 0 ? 1 : 0;
    for (int64_t i = held; i < blocks_after; ++i)
        if (i >= first_kept_blk) ++need;
    int64_t avail = (int64_t)p->free_q.size();
    const int64_t rel_end = first_kept_blk < held ? first_kept_blk : held;
    for (int64_t i = 0; i < rel_end; ++i)
        if (s.blocks[i] >= 0 && p->ref[s.blocks[i]] == 1 && !p->busy(s.blocks[i])) ++avail;
    if (need > avail) return PA_ERR_OUT_OF_BLOCKS;

    for (int64_t i = 0; i < rel_end; ++i) {
        if (s.blocks[i] >= 0) {
            p->release(s.blocks[i]);
            s.blocks[i] = -1;
        }
    }
    if (cow >= 0) {
        const int32_t old = s.blocks[cow];
        const int32_t b = p->free_q.front();
        p->free_q.pop_front();
        p->ref[b] = 1;
        --p->ref[old];
        p->mark_copy_src(old);
        s.blocks[cow] = b;
        p->pending.push_back(old);
        p->pending.push_back(b);
        p->pending.push_back((int32_t)(cur - cow * bs));
        p->touch(b);
    }
    for (int64_t i = held; i < blocks_after; ++i) {
        if (i >= first_kept_blk) {
            int32_t b = p->free_q.front();
            p->free_q.pop_front();
            p->ref[b] = 1;
            s.blocks.push_back(b);
        } else {
            s.blocks.push_back(-1);
        }
    }
    s.len = end;
    for (int64_t pos = cur; pos < end; ++pos) {
        int64_t slot = -1;
        if (pos >= keep_from) {
            const int32_t b = s.blocks[pos / bs];
            p->touch(b);
            slot = (int64_t)b * bs + pos % bs;
        }
        if (slots_out) slots_out[pos - cur] = slot;
    }
    return PA_OK;
}

pa_status pa_seq_fork(pa_pool* p, int64_t dst, int64_t src) {
    if (!p) return PA_ERR_NULL;
    auto dit = p->seqs.find(dst);
    if (dit != p->seqs.end() &&
        (dit->second.len != 0 || !dit->second.blocks.empty() || dit->second.swapped))
        return PA_ERR_BAD_SEQ;
    auto it = p->seqs.find(src);
    if (it == p->seqs.end() || dst == src || it->second.swapped) return PA_ERR_BAD_SEQ;
    for (int32_t b : it->second.blocks)
        if (b >= 0) ++p->ref[b];
    const Seq& from = it->second;
    std::vector<int32_t> blocks = from.blocks;
    const int64_t len = from.len;
    const int32_t window = from.window;
    Seq& d = p->create(dst);
    d.blocks = std::move(blocks);
    d.len = len;
    d.window = window;
    return PA_OK;
}

int32_t pa_pool_num_pending_copies(const pa_pool* p) {
    return p ? (int32_t)(p->pending.size() / 3) : 0;
}

pa_status pa_pool_take_copies(pa_pool* p, int32_t* out, int32_t cap, int32_t* n) {
    if (!p || !n) return PA_ERR_NULL;
    const int32_t count = (int32_t)(p->pending.size() / 3);
    *n = count;
    if (count > cap) return PA_ERR_SHAPE;
    if (count && !out) return PA_ERR_NULL;
    for (size_t i = 0; i < p->pending.size(); ++i) out[i] = p->pending[i];
    p->end_batch();
    return PA_OK;
}

pa_status pa_pool_set_host_blocks(pa_pool* p, int32_t num_host_blocks) {
    if (!p) return PA_ERR_NULL;
    if (num_host_blocks < 0) return PA_ERR_SHAPE;
    if ((int32_t)p->host_free.size() != p->num_host || !p->host_quarantine.empty())
        return PA_ERR_BAD_SEQ;   // host blocks in use
    p->num_host = num_host_blocks;
    p->host_free.clear();
    for (int32_t h = 0; h < num_host_blocks; ++h) p->host_free.push_back(h);
    return PA_OK;
}

int32_t pa_pool_num_host_free(const pa_pool* p) { return p ? (int32_t)p->host_free.size() : 0; }

pa_status pa_pool_latest_resident(const pa_pool* p, int64_t* seq) {
    if (!p || !seq) return PA_ERR_NULL;
    const Seq* best = nullptr;
    int64_t best_id = 0;
    for (const auto& kv : p->seqs) {
        const Seq& s = kv.second;
        if (s.swapped) continue;
        bool any = false;
        for (int32_t b : s.blocks) any = any || b >= 0;
        if (!any) continue;
        if (!best || s.arrival > best->arrival) {
            best = &s;
            best_id = kv.first;
        }
    }
    if (!best) return PA_ERR_BAD_SEQ;
    *seq = best_id;
    return PA_OK;
}

pa_status pa_seq_swap_out(pa_pool* p, int64_t seq, int32_t* pairs, int32_t cap, int32_t* n) {
    if (!p || !n) return PA_ERR_NULL;
    *n = 0;
    auto it = p->seqs.find(seq);
    if (it == p->seqs.end() || it->second.swapped) return PA_ERR_BAD_SEQ;
    Seq& s = it->second;
    int32_t count = 0;
    for (int32_t b : s.blocks) {
        if (b >= 0 && p->ref[b] == 1) {
            if (p->touched[b]) return PA_ERR_SHARED_BLOCK;   // writes pending
            ++count;
        }
    }
    if (count > (int32_t)p->host_free.size()) return PA_ERR_OUT_OF_BLOCKS;
    *n = count;
    if (count > cap) return PA_ERR_SHAPE;
    if (count && !pairs) return PA_ERR_NULL;
    s.host.assign(s.blocks.size(), -1);
    int32_t k = 0;
    for (size_t i = 0; i < s.blocks.size(); ++i) {
        const int32_t b = s.blocks[i];
        if (b < 0 || p->ref[b] != 1) continue;
        const int32_t h = p->host_free.front();
        p->host_free.pop_front();
        pairs[2 * k] = b;
        pairs[2 * k + 1] = h;
        ++k;
        s.host[i] = h;
        p->release(b);
        s.blocks[i] = -1;
    }
    s.swapped = true;
    ++p->num_swapped;
    return PA_OK;
}

pa_status pa_seq_swap_in(pa_pool* p, int64_t seq, int32_t* pairs, int32_t cap, int32_t* n) {
    if (!p || !n) return PA_ERR_NULL;
    *n = 0;
    auto it = p->seqs.find(seq);
    if (it == p->seqs.end() || !it->second.swapped) return PA_ERR_BAD_SEQ;
    Seq& s = it->second;
    int32_t count = 0;
    for (int32_t h : s.host) count += h >= 0;
    if (count > (int32_t)p->free_q.size()) return PA_ERR_OUT_OF_BLOCKS;
    *n = count;
    if (count > cap) return PA_ERR_SHAPE;
    if (count && !pairs) return PA_ERR_NULL;
    int32_t k = 0;
    for (size_t i = 0; i < s.host.size(); ++i) {
        const int32_t h = s.host[i];
        if (h < 0) continue;
        const int32_t b = p->free_q.front();
        p->free_q.pop_front();
        p->ref[b] = 1;
        s.blocks[i] = b;
        pairs[2 * k] = h;
        pairs[2 * k + 1] = b;
        ++k;
        p->touch(b);
        p->host_quarantine.push_back(h);
    }
    s.host.clear();
    s.swapped = false;
    --p->num_swapped;
    return PA_OK;
}

pa_status pa_seq_share_prefix(pa_pool* p, int64_t dst, int64_t src, int32_t n_tokens) {
    if (!p) return PA_ERR_NULL;
    if (n_tokens < 0) return PA_ERR_SHAPE;
    auto it = p->seqs.find(src);
    if (it == p->seqs.end() || dst == src || it->second.swapped) return PA_ERR_BAD_SEQ;
    if (n_tokens > it->second.len) return PA_ERR_SHAPE;
    auto dit = p->seqs.find(dst);
    if (dit != p->seqs.end() &&
        (dit->second.len != 0 || !dit->second.blocks.empty() || dit->second.swapped))
        return PA_ERR_BAD_SEQ;
    if (p->admission_closed(dst)) return PA_ERR_ADMISSION;
    const int64_t nblk = (n_tokens + p->bs - 1) / p->bs;
    const std::vector<int32_t>& sb = it->second.blocks;
    for (int64_t i = 0; i < nblk; ++i)
        if (sb[i] < 0) return PA_ERR_BAD_SEQ;
    std::vector<int32_t> blocks(sb.begin(), sb.begin() + nblk);
    for (int32_t b : blocks) ++p->ref[b];
    Seq& d = p->create(dst);
    d.blocks = std::move(blocks);
    d.len = n_tokens;
    return PA_OK;
}

pa_status pa_seq_free(pa_pool* p, int64_t seq) {
    if (!p) return PA_ERR_NULL;
    auto it = p->seqs.find(seq);
    if (it == p->seqs.end()) return PA_ERR_BAD_SEQ;
    for (int32_t b : it->second.blocks)
        if (b >= 0) p->release(b);
    for (int32_t h : it->second.host)
        if (h >= 0) p->host_quarantine.push_back(h);
    if (it->second.swapped) --p->num_swapped;
    p->seqs.erase(it);
    return PA_OK;
}

pa_status pa_seq_block_table(const pa_pool* p, int64_t seq, int32_t* out, int32_t cap,
                             int32_t* n) {
    if (!p || !n) return PA_ERR_NULL;
    auto it = p->seqs.find(seq);
    if (it == p->seqs.end()) return PA_ERR_BAD_SEQ;
    const std::vector<int32_t>& b = it->second.blocks;
    *n = (int32_t)b.size();
    if ((int64_t)b.size() > cap) return PA_ERR_SHAPE;
    if (!out && !b.empty()) return PA_ERR_NULL;
    for (size_t i = 0; i < b.size(); ++i) out[i] = b[i];
    return PA_OK;
}

pa_status pa_pool_block_tables(const pa_pool* p, const int64_t* seqs, int32_t num_seqs,
                               int32_t max_blocks, int32_t fill, int32_t* out) {
    if (!p || (!seqs && num_seqs) || (!out && num_seqs && max_blocks)) return PA_ERR_NULL;
    if (num_seqs < 0 || max_blocks < 0) return PA_ERR_SHAPE;
    for (int32_t i = 0; i < num_seqs; ++i) {
        auto it = p->seqs.find(seqs[i]);
        if (it == p->seqs.end()) return PA_ERR_BAD_SEQ;
        if ((int64_t)it->second.blocks.size() > max_blocks) return PA_ERR_SHAPE;
    }
    for (int32_t i = 0; i < num_seqs; ++i) {
        const std::vector<int32_t>& b = p->seqs.find(seqs[i])->second.blocks;
        int32_t* row = out + (size_t)i * max_blocks;
        for (int32_t j = 0; j < max_blocks; ++j) {
            int32_t v = j < (int32_t)b.size() ? b[j] : -1;
            row[j] = v < 0 ? fill : v;
        }
    }
    return PA_OK;
}

int32_t pa_seq_len(const pa_pool* p, int64_t seq) {
    if (!p) return -1;
    auto it = p->seqs.find(seq);
    return it == p->seqs.end() ? -1 : (int32_t)it->second.len;
}

int32_t pa_pool_num_free(const pa_pool* p) { return p ? (int32_t)p->free_q.size() : 0; }

int32_t pa_block_refcount(const pa_pool* p, int32_t block) {
    if (!p || block < 0 || block >= p->num_blocks) return 0;
    return p->ref[block];
}

}  // extern "C"
