// Host block manager for the paged KV cache: allocates fixed 16-token blocks
// on demand, lets sequences share blocks by reference counting (fork for
// parallel sampling / beam search), copies a shared, partly filled block on
// the first write into it (copy-on-write), and emits the block table rows and
// slot_mapping entries the GPU calls take.
//
// What it follows: the ai-maas.com vLLM article (先看浪费在哪里: blocks are
// requested and returned on demand instead of reserving max_len per request)
// and the ipipp.com vLLM/PagedAttention article (section 二: 16-token blocks,
// a per-sequence block table, blocks shared between sequences with reference
// counts and copied when a shared block is written).
//
// Allocation is deterministic: free blocks form a stack that starts as
// [num_blocks-1, ..., 1, 0] (block 0 is handed out first); a block returns to
// the top of the stack when its last reference goes (a freed sequence
// releases its blocks in table order).
//
// A copy-on-write queues a copy (src -> dst) for the caller to run on the GPU
// before the new tokens are written.  Until the caller takes it, the copy pins
// both blocks (a pin is not a reference: it does not make dst look shared),
// so neither can be handed out again while the copy is pending.
#include "../../include/pkv.h"

#include <cstdint>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pkv_internal.h"

struct pkv_block_manager {
    struct Seq {
        std::vector<int32_t> blocks;
        int64_t len = 0;
    };
    int32_t num_blocks = 0;
    int32_t max_blocks_per_seq = 0;
    std::vector<int32_t> free_stack;  // top = back
    std::vector<int32_t> refcount;    // sequences whose table holds the block
    std::vector<int32_t> pins;        // pending copies that read or write the block
    std::unordered_map<int64_t, Seq> seqs;
    std::vector<std::pair<int32_t, int32_t>> copies;  // (src, dst) not yet taken

    int32_t pop_free() {
        const int32_t b = free_stack.back();
        free_stack.pop_back();
        refcount[b] = 1;
        return b;
    }
    void maybe_free(int32_t b) {
        if (refcount[b] == 0 && pins[b] == 0) free_stack.push_back(b);
    }
    void release(int32_t b) {
        --refcount[b];
        maybe_free(b);
    }
    void unpin(int32_t b) {
        --pins[b];
        maybe_free(b);
    }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t max_blocks_per_seq) {
    if (num_blocks < 0 || max_blocks_per_seq < 0 || int64_t(num_blocks) * pkv::kBlockTokens >= (int64_t(1) << 31))
        return nullptr;
    pkv_block_manager* m = new (std::nothrow) pkv_block_manager;
    if (!m) return nullptr;
    m->num_blocks = num_blocks;
    m->max_blocks_per_seq = max_blocks_per_seq;
    m->refcount.assign(size_t(num_blocks), 0);
    m->pins.assign(size_t(num_blocks), 0);
    m->free_stack.reserve(size_t(num_blocks));
    for (int32_t b = num_blocks - 1; b >= 0; --b) m->free_stack.push_back(b);
    return m;
}

void pkv_bm_destroy(pkv_block_manager* m) { delete m; }

int pkv_bm_add(pkv_block_manager* m, int64_t seq_id) {
    if (!m || m->seqs.count(seq_id)) return PKV_ERR_INVALID_ARG;
    m->seqs.emplace(seq_id, pkv_block_manager::Seq{});
    return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* m, int64_t parent, int64_t child) {
    if (!m || parent == child || m->seqs.count(child)) return PKV_ERR_INVALID_ARG;
    auto it = m->seqs.find(parent);
    if (it == m->seqs.end()) return PKV_ERR_INVALID_ARG;
    pkv_block_manager::Seq c = it->second;
    for (int32_t b : c.blocks) ++m->refcount[b];
    m->seqs.emplace(child, std::move(c));
    return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* m, int64_t seq_id, int32_t n, int32_t* slots_out) {
    if (!m || n < 0 || (n > 0 && !slots_out)) return PKV_ERR_INVALID_ARG;
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PKV_ERR_INVALID_ARG;
    pkv_block_manager::Seq& sq = it->second;
    const int64_t len1 = sq.len + n;
    const int64_t nb1 = (len1 + pkv::kBlockTokens - 1) / pkv::kBlockTokens;
    if (nb1 > m->max_blocks_per_seq) return PKV_ERR_OUT_OF_BLOCKS;
    // blocks needed: the new ones, plus a private copy of a shared, partly filled last block
    const bool cow = n > 0 && sq.len % pkv::kBlockTokens != 0 && m->refcount[sq.blocks.back()] > 1;
    const int64_t need = (nb1 - int64_t(sq.blocks.size())) + (cow ? 1 : 0);
    if (need > int64_t(m->free_stack.size())) return PKV_ERR_OUT_OF_BLOCKS;  // nothing changed
    if (cow) {
        const int32_t src = sq.blocks.back();
        const int32_t dst = m->pop_free();
        ++m->pins[src];
        ++m->pins[dst];
        m->release(src);
        sq.blocks.back() = dst;
        m->copies.emplace_back(src, dst);
    }
    while (int64_t(sq.blocks.size()) < nb1) sq.blocks.push_back(m->pop_free());
    for (int32_t i = 0; i < n; ++i) {
        const int64_t p = sq.len + i;
        slots_out[i] = sq.blocks[size_t(p / pkv::kBlockTokens)] * pkv::kBlockTokens + int32_t(p % pkv::kBlockTokens);
    }
    sq.len = len1;
    return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* m, int64_t seq_id) {
    if (!m) return PKV_ERR_INVALID_ARG;
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PKV_ERR_INVALID_ARG;
    for (int32_t b : it->second.blocks) m->release(b);
    m->seqs.erase(it);
    return PKV_OK;
}

int pkv_bm_table(const pkv_block_manager* m, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                 int32_t* table_out, int32_t* lens_out) {
    if (!m || n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || !table_out || !lens_out))) return PKV_ERR_INVALID_ARG;
    for (int32_t r = 0; r < n; ++r) {
        auto it = m->seqs.find(seq_ids[r]);
        if (it == m->seqs.end() || int64_t(it->second.blocks.size()) > max_blocks) return PKV_ERR_INVALID_ARG;
    }
    for (int32_t r = 0; r < n; ++r) {
        const pkv_block_manager::Seq& sq = m->seqs.find(seq_ids[r])->second;
        int32_t* row = table_out + int64_t(r) * max_blocks;
        for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < int32_t(sq.blocks.size()) ? sq.blocks[size_t(j)] : -1;
        lens_out[r] = int32_t(sq.len);
    }
    return PKV_OK;
}

int32_t pkv_bm_take_copies(pkv_block_manager* m, int32_t* src_out, int32_t* dst_out, int32_t max_copies) {
    if (!m || max_copies < 0 || (max_copies > 0 && (!src_out || !dst_out))) return -1;
    // the oldest pending copies, stopping before one that reads a block an
    // earlier copy of this batch writes (the batch runs in parallel)
    int32_t k = 0;
    while (k < max_copies && size_t(k) < m->copies.size()) {
        const int32_t src = m->copies[size_t(k)].first;
        bool chained = false;
        for (int32_t i = 0; i < k; ++i) chained = chained || dst_out[i] == src;
        if (chained) break;
        src_out[k] = src;
        dst_out[k] = m->copies[size_t(k)].second;
        ++k;
    }
    m->copies.erase(m->copies.begin(), m->copies.begin() + k);
    for (int32_t i = 0; i < k; ++i) {
        m->unpin(src_out[i]);
        m->unpin(dst_out[i]);
    }
    return k;
}

int pkv_bm_stats(const pkv_block_manager* m, int64_t* out) {
    if (!m || !out) return PKV_ERR_INVALID_ARG;
    int64_t tokens = 0;  // tokens held by the used blocks, a shared block counted once
    std::vector<int32_t> fill(size_t(m->num_blocks), 0);
    for (const auto& kv : m->seqs) {
        const auto& sq = kv.second;
        for (size_t j = 0; j < sq.blocks.size(); ++j) {
            const int64_t in_block = sq.len - int64_t(j) * pkv::kBlockTokens;
            const int32_t t = int32_t(in_block < pkv::kBlockTokens ? in_block : pkv::kBlockTokens);
            int32_t& f = fill[size_t(sq.blocks[j])];
            f = t > f ? t : f;
        }
    }
    for (int32_t f : fill) tokens += f;
    out[0] = int64_t(m->free_stack.size());
    out[1] = int64_t(m->num_blocks) - int64_t(m->free_stack.size());
    out[2] = int64_t(m->seqs.size());
    out[3] = tokens;
    out[4] = int64_t(m->copies.size());
    return PKV_OK;
}

}  // extern "C"
