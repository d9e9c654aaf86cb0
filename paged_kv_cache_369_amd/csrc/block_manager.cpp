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
//
// Automatic prefix caching (bytelighting wiki "vLLM", paragraph on APC; the
// ai-maas.com article's note that repeated prefixes are computed once and
// shared): when enabled, every block a sequence with known token ids fills is
// registered in a table under a chained hash of its content (the parent
// block's hash mixed with the block's 16 token ids).  A new sequence added
// with its prompt reuses the longest run of registered full blocks matching
// its prompt's first blocks.  A match is exact: the candidate's tokens must
// equal the prompt's and its parent must be the block matched one step
// earlier (at the generation it had when the candidate registered), so the
// hash only narrows the search.  A registered block whose last reference goes
// stays in the table as evictable; blocks are evicted least recently released
// first, and only when no block that was never registered is free.
#include "../../include/pkv.h"

#include <cstdint>
#include <list>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pkv_internal.h"

struct pkv_block_manager {
    struct Seq {
        std::vector<int32_t> blocks;
        int64_t len = 0;
        // prefix caching: whether every token id is known, the chained hash of
        // the last full block, and the token ids of the partly filled last block
        bool tracked = false;
        uint64_t chain = 0;
        int32_t reg_parent = -1;  // the registered block with the same content as the last full block (-1: none)
        uint64_t reg_gen = 0;     // its generation then
        std::vector<int32_t> tail;
    };
    int32_t num_blocks = 0;
    int32_t max_blocks_per_seq = 0;
    std::vector<int32_t> free_stack;  // top = back
    std::vector<int32_t> refcount;    // sequences whose table holds the block
    std::vector<int32_t> pins;        // pending copies that read or write the block
    std::unordered_map<int64_t, Seq> seqs;
    std::vector<std::pair<int32_t, int32_t>> copies;  // (src, dst) not yet taken

    // prefix cache (empty unless enabled)
    bool caching = false;
    std::vector<uint8_t> cached;        // block is registered in the table
    std::vector<uint64_t> bhash;        // its chained hash
    std::vector<int32_t> parent;        // block matched before it (-1: first block of a prompt)
    std::vector<uint64_t> parent_gen;   // generation of that parent at registration
    std::vector<uint64_t> gen;          // registration generation (0: not registered)
    std::vector<int32_t> btokens;       // [block][16] token ids of a registered block
    std::unordered_multimap<uint64_t, int32_t> table;
    std::list<int32_t> lru;             // registered blocks without references, oldest first
    std::vector<std::list<int32_t>::iterator> lru_pos;
    std::vector<uint8_t> in_lru;
    uint64_t next_gen = 0;
    int64_t hits = 0, lookups = 0, evictions = 0;

    int32_t free_count() const { return int32_t(free_stack.size() + lru.size()); }

    void unregister(int32_t b) {
        auto range = table.equal_range(bhash[size_t(b)]);
        for (auto it = range.first; it != range.second; ++it)
            if (it->second == b) {
                table.erase(it);
                break;
            }
        cached[size_t(b)] = 0;
        gen[size_t(b)] = 0;
    }
    int32_t pop_free() {
        int32_t b;
        if (!free_stack.empty()) {
            b = free_stack.back();
            free_stack.pop_back();
        } else {  // evict the least recently released registered block
            b = lru.front();
            lru.pop_front();
            in_lru[size_t(b)] = 0;
            unregister(b);
            ++evictions;
        }
        refcount[b] = 1;
        return b;
    }
    void maybe_free(int32_t b) {
        if (refcount[b] != 0 || pins[b] != 0) return;
        if (caching && cached[size_t(b)]) {
            lru_pos[size_t(b)] = lru.insert(lru.end(), b);
            in_lru[size_t(b)] = 1;
        } else {
            free_stack.push_back(b);
        }
    }
    void acquire_cached(int32_t b) {  // a hit: one more reference to a registered block
        if (refcount[b] == 0 && in_lru[size_t(b)]) {
            lru.erase(lru_pos[size_t(b)]);
            in_lru[size_t(b)] = 0;
        }
        ++refcount[b];
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

namespace {

// Chained content hash of a block: the parent's hash mixed with the block's
// token ids, each step a 64-bit finaliser (splitmix64's).  Only narrows the
// search; matches are checked exactly.
uint64_t mix64(uint64_t x) {
    x += 0x9e3779b97f4a7c15ull;
    x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
    x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
    return x ^ (x >> 31);
}

constexpr uint64_t kRootHash = 0x243f6a8885a308d3ull;

uint64_t block_hash(uint64_t parent_hash, const int32_t* tokens) {
    uint64_t h = mix64(parent_hash);
    for (int i = 0; i < pkv::kBlockTokens; ++i) h = mix64(h ^ uint64_t(uint32_t(tokens[i])));
    return h;
}

// The registered block holding `tokens` after parent block `par` (-1: none), or -1.
int32_t find_cached(const pkv_block_manager* m, uint64_t h, int32_t par, const int32_t* tokens) {
    auto range = m->table.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
        const int32_t b = it->second;
        if (m->parent[size_t(b)] != par) continue;
        if (par >= 0 && m->parent_gen[size_t(b)] != m->gen[size_t(par)]) continue;
        bool same = true;
        for (int i = 0; i < pkv::kBlockTokens && same; ++i)
            same = m->btokens[size_t(b) * pkv::kBlockTokens + size_t(i)] == tokens[i];
        if (same) return b;
    }
    return -1;
}

// Sequence sq's block j (index in its table) just filled with `tokens`:
// register it under the registered block equivalent to its predecessor,
// unless that same content is registered there already (then that block is
// the equivalent one for the next step).
void register_full(pkv_block_manager* m, pkv_block_manager::Seq& sq, size_t j, const int32_t* tokens) {
    const uint64_t h = block_hash(sq.chain, tokens);
    sq.chain = h;
    const int32_t b = sq.blocks[j];
    const int32_t par = j > 0 ? sq.reg_parent : -1;
    if (j > 0 && par < 0) return;  // the predecessor's content is not registered: neither is this
    if (par >= 0 && m->gen[size_t(par)] != sq.reg_gen) {  // the predecessor was evicted since
        sq.reg_parent = -1;
        return;
    }
    const int32_t same = find_cached(m, h, par, tokens);
    if (same >= 0) {
        sq.reg_parent = same;
        sq.reg_gen = m->gen[size_t(same)];
        return;
    }
    if (m->cached[size_t(b)]) {  // registered under another chain (cannot happen for a private block)
        sq.reg_parent = -1;
        return;
    }
    sq.reg_parent = b;
    m->cached[size_t(b)] = 1;
    m->bhash[size_t(b)] = h;
    m->parent[size_t(b)] = par;
    m->parent_gen[size_t(b)] = par >= 0 ? m->gen[size_t(par)] : 0;
    m->gen[size_t(b)] = ++m->next_gen;
    sq.reg_gen = m->gen[size_t(b)];
    for (int i = 0; i < pkv::kBlockTokens; ++i) m->btokens[size_t(b) * pkv::kBlockTokens + size_t(i)] = tokens[i];
    m->table.emplace(h, b);
}

}  // namespace

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
    pkv_block_manager::Seq sq;
    sq.tracked = m->caching;  // an empty sequence: every token id (none) is known
    sq.chain = kRootHash;
    m->seqs.emplace(seq_id, std::move(sq));
    return PKV_OK;
}

int pkv_bm_enable_prefix_caching(pkv_block_manager* m) {
    if (!m || !m->seqs.empty() || !m->copies.empty()) return PKV_ERR_INVALID_ARG;
    if (m->caching) return PKV_OK;
    const size_t nb = size_t(m->num_blocks);
    m->caching = true;
    m->cached.assign(nb, 0);
    m->bhash.assign(nb, 0);
    m->parent.assign(nb, -1);
    m->parent_gen.assign(nb, 0);
    m->gen.assign(nb, 0);
    m->btokens.assign(nb * pkv::kBlockTokens, 0);
    m->lru_pos.assign(nb, m->lru.end());
    m->in_lru.assign(nb, 0);
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

}  // extern "C"

namespace {

int append_impl(pkv_block_manager* m, int64_t seq_id, int32_t n, const int32_t* tokens, int32_t* slots_out) {
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
    if (need > int64_t(m->free_count())) return PKV_ERR_OUT_OF_BLOCKS;  // nothing changed
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
    if (m->caching && sq.tracked && n > 0) {
        if (!tokens) {
            sq.tracked = false;  // token ids unknown from here on: nothing more of it is registered
        } else {
            for (int32_t i = 0; i < n; ++i) {
                sq.tail.push_back(tokens[i]);
                if (int32_t(sq.tail.size()) == pkv::kBlockTokens) {
                    register_full(m, sq, size_t((sq.len + i) / pkv::kBlockTokens), sq.tail.data());
                    sq.tail.clear();
                }
            }
        }
    }
    sq.len = len1;
    return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_bm_append(pkv_block_manager* m, int64_t seq_id, int32_t n, int32_t* slots_out) {
    return append_impl(m, seq_id, n, nullptr, slots_out);
}

int pkv_bm_append_tokens(pkv_block_manager* m, int64_t seq_id, const int32_t* tokens, int32_t n,
                         int32_t* slots_out) {
    if (n > 0 && !tokens) return PKV_ERR_INVALID_ARG;
    return append_impl(m, seq_id, n, tokens, slots_out);
}

int pkv_bm_add_prompt(pkv_block_manager* m, int64_t seq_id, const int32_t* tokens, int32_t n, int32_t* slots_out,
                      int32_t* cached_out) {
    if (!m || !m->caching || n < 0 || (n > 0 && (!tokens || !slots_out)) || !cached_out || m->seqs.count(seq_id))
        return PKV_ERR_INVALID_ARG;
    const int64_t nb = (int64_t(n) + pkv::kBlockTokens - 1) / pkv::kBlockTokens;
    if (nb > m->max_blocks_per_seq) return PKV_ERR_OUT_OF_BLOCKS;
    // the longest run of registered full blocks matching the prompt's first
    // blocks, leaving the last prompt token to be computed
    const int32_t eligible = n > 0 ? (n - 1) / pkv::kBlockTokens : 0;
    std::vector<int32_t> hit;
    uint64_t chain = kRootHash;
    int32_t in_lru = 0;
    for (int32_t j = 0; j < eligible; ++j) {
        const uint64_t h = block_hash(chain, tokens + int64_t(j) * pkv::kBlockTokens);
        const int32_t b = find_cached(m, h, j > 0 ? hit.back() : -1, tokens + int64_t(j) * pkv::kBlockTokens);
        if (b < 0) break;
        hit.push_back(b);
        in_lru += m->in_lru[size_t(b)] ? 1 : 0;
        chain = h;
    }
    const int64_t need = nb - int64_t(hit.size());
    if (need > int64_t(m->free_count()) - in_lru) return PKV_ERR_OUT_OF_BLOCKS;  // nothing changed
    m->lookups += eligible;
    m->hits += int64_t(hit.size());
    pkv_block_manager::Seq sq;
    sq.tracked = true;
    sq.chain = chain;
    sq.reg_parent = hit.empty() ? -1 : hit.back();
    sq.reg_gen = hit.empty() ? 0 : m->gen[size_t(hit.back())];
    for (int32_t b : hit) {
        m->acquire_cached(b);
        sq.blocks.push_back(b);
    }
    while (int64_t(sq.blocks.size()) < nb) sq.blocks.push_back(m->pop_free());
    const int32_t cached = int32_t(hit.size()) * pkv::kBlockTokens;
    for (int32_t p = cached; p < n; ++p)
        slots_out[p - cached] = sq.blocks[size_t(p / pkv::kBlockTokens)] * pkv::kBlockTokens + p % pkv::kBlockTokens;
    for (int32_t p = cached; p < n; ++p) {
        sq.tail.push_back(tokens[p]);
        if (int32_t(sq.tail.size()) == pkv::kBlockTokens) {
            register_full(m, sq, size_t(p / pkv::kBlockTokens), sq.tail.data());
            sq.tail.clear();
        }
    }
    sq.len = n;
    m->seqs.emplace(seq_id, std::move(sq));
    *cached_out = cached;
    return PKV_OK;
}

int pkv_bm_cache_stats(const pkv_block_manager* m, int64_t* out) {
    if (!m || !out) return PKV_ERR_INVALID_ARG;
    out[0] = int64_t(m->table.size());
    out[1] = int64_t(m->lru.size());
    out[2] = m->lookups;
    out[3] = m->hits;
    out[4] = m->evictions;
    return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* m, int64_t seq_id) {
    if (!m) return PKV_ERR_INVALID_ARG;
    auto it = m->seqs.find(seq_id);
    if (it == m->seqs.end()) return PKV_ERR_INVALID_ARG;
    const std::vector<int32_t>& bl = it->second.blocks;
    if (m->caching) {  // the deepest block first, so a cached prefix is evicted from its end
        for (size_t k = bl.size(); k-- > 0;) m->release(bl[k]);
    } else {
        for (int32_t b : bl) m->release(b);
    }
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
    out[0] = int64_t(m->free_count());
    out[1] = int64_t(m->num_blocks) - int64_t(m->free_count());
    out[2] = int64_t(m->seqs.size());
    out[3] = tokens;
    out[4] = int64_t(m->copies.size());
    return PKV_OK;
}

}  // extern "C"
