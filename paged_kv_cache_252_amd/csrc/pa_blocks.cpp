// Host-side block manager: free list, reference counts, block tables, growth,
// fork, free, copy-on-write decisions, slots, and a content-addressed cache of
// full blocks.
//
// Sources (web pages, by title and section):
//   [ZQ] "How does PagedAttention enable prefix sharing across requests and
//        what data structure makes it cheap?" -- answer, TL;DR.
//   [KG] "Day 28: PagedAttention" -- "Growth Needs Only Another Free Block",
//        "Prefix Sharing Is a Natural Extension", "Shared Blocks Must Not Be
//        Changed in Place".
//
// Everything is O(1) per token except the prefix lookup, which hashes each
// prompt block once.  Every mutating call first checks that it can finish
// (ids known, enough blocks), so a failed call leaves the state untouched.

#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_blocks.h"
#include "pa_internal.h"

namespace {

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

uint64_t fnv_bytes(uint64_t h, const unsigned char* p, size_t n) {
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= kFnvPrime;
    }
    return h;
}

uint64_t block_key(uint64_t parent, const int32_t* tokens, int32_t n) {
    unsigned char buf[8];
    for (int i = 0; i < 8; ++i) buf[i] = static_cast<unsigned char>(parent >> (8 * i));
    uint64_t h = fnv_bytes(kFnvOffset, buf, 8);
    for (int32_t t = 0; t < n; ++t) {
        const uint32_t v = static_cast<uint32_t>(tokens[t]);
        unsigned char b[4] = {static_cast<unsigned char>(v), static_cast<unsigned char>(v >> 8),
                              static_cast<unsigned char>(v >> 16), static_cast<unsigned char>(v >> 24)};
        h = fnv_bytes(h, b, 4);
    }
    return h;
}

struct Seq {
    std::vector<int32_t> table;   // logical block -> physical block
    int64_t len = 0;              // reserved positions
    std::vector<int32_t> tokens;  // token ids (prefix cache only)
    uint64_t parent = 0;          // key of the last full block (the salt before the first)
};

}  // namespace

struct pa_bm {
    int32_t num_blocks = 0;
    int32_t bs = 0;
    bool cache = false;
    uint64_t salt = 0;
    int64_t next_id = 0;
    std::vector<int32_t> refcount;
    std::vector<int32_t> free_list;               // LIFO: back() is handed out next
    std::unordered_map<int64_t, Seq> seqs;

    // prefix cache: key -> block; per block its key, parent key, tokens, and an
    // intrusive LRU list of cached blocks whose count is zero (oldest at head)
    std::unordered_map<uint64_t, int32_t> by_key;
    std::vector<uint8_t> cached;                  // block is registered
    std::vector<uint64_t> key, parent_key;
    std::vector<int32_t> key_tokens;              // [num_blocks][bs]
    std::vector<int32_t> lru_prev, lru_next;
    int32_t lru_head = -1, lru_tail = -1;
    int64_t lru_size = 0;

    int64_t available() const { return static_cast<int64_t>(free_list.size()) + lru_size; }

    void lru_push(int32_t b) {
        lru_prev[b] = lru_tail;
        lru_next[b] = -1;
        if (lru_tail >= 0) lru_next[lru_tail] = b; else lru_head = b;
        lru_tail = b;
        ++lru_size;
    }
    void lru_remove(int32_t b) {
        if (lru_prev[b] >= 0) lru_next[lru_prev[b]] = lru_next[b]; else lru_head = lru_next[b];
        if (lru_next[b] >= 0) lru_prev[lru_next[b]] = lru_prev[b]; else lru_tail = lru_prev[b];
        --lru_size;
    }

    // Callers have checked available() first.
    int32_t take() {
        int32_t b;
        if (!free_list.empty()) {
            b = free_list.back();
            free_list.pop_back();
        } else {                                  // evict the oldest unused cached block
            b = lru_head;
            lru_remove(b);
            by_key.erase(key[b]);
            cached[b] = 0;
        }
        refcount[b] = 1;
        return b;
    }

    void release(int32_t b) {
        if (--refcount[b] == 0) {
            if (cache && cached[b]) lru_push(b); else free_list.push_back(b);
        }
    }

    // Block b now holds the full block `tokens` after parent key `parent`.
    // Returns its key; registers it unless that key is taken.
    uint64_t register_block(int32_t b, uint64_t parent, const int32_t* tokens) {
        const uint64_t k = block_key(parent, tokens, bs);
        if (by_key.emplace(k, b).second) {
            cached[b] = 1;
            key[b] = k;
            parent_key[b] = parent;
            std::memcpy(&key_tokens[static_cast<size_t>(b) * bs], tokens, sizeof(int32_t) * bs);
        }
        return k;
    }

    // The cached block for (parent, tokens), or -1; *k receives the key.
    int32_t lookup(uint64_t parent, const int32_t* tokens, uint64_t* k) const {
        *k = block_key(parent, tokens, bs);
        auto it = by_key.find(*k);
        if (it == by_key.end()) return -1;
        const int32_t b = it->second;
        if (parent_key[b] != parent ||
            std::memcmp(&key_tokens[static_cast<size_t>(b) * bs], tokens, sizeof(int32_t) * bs) != 0)
            return -1;                            // a different block with the same hash
        return b;
    }

    int64_t slot(const Seq& s, int64_t pos) const {
        return static_cast<int64_t>(s.table[pos / bs]) * bs + pos % bs;
    }
};

using pa::fail;
using pa::ok;

extern "C" {

uint64_t pa_bm_block_key(uint64_t parent, const int32_t* tokens, int32_t n) {
    if (tokens == nullptr || n < 0) n = 0;
    return block_key(parent, tokens, n);
}

int pa_bm_create(int64_t num_blocks, int32_t block_size, uint32_t flags, uint64_t salt,
                 pa_bm_t** out) {
    if (out == nullptr) return fail(PA_ERR_NULL, "out is NULL");
    *out = nullptr;
    if (num_blocks < 1 || num_blocks > INT32_MAX)
        return fail(PA_ERR_SHAPE, "num_blocks %lld outside [1, 2^31-1]", (long long)num_blocks);
    if (block_size < 1 || block_size > 4096)
        return fail(PA_ERR_SHAPE, "block_size %d outside [1, 4096]", block_size);
    if (flags & ~PA_BM_PREFIX_CACHE) return fail(PA_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
    pa_bm* bm = new (std::nothrow) pa_bm;
    if (bm == nullptr) return fail(PA_ERR_NO_SPACE, "out of host memory");
    try {
        bm->num_blocks = static_cast<int32_t>(num_blocks);
        bm->bs = block_size;
        bm->cache = (flags & PA_BM_PREFIX_CACHE) != 0;
        bm->salt = salt;
        bm->refcount.assign(num_blocks, 0);
        bm->free_list.resize(num_blocks);
        for (int64_t i = 0; i < num_blocks; ++i)
            bm->free_list[i] = static_cast<int32_t>(num_blocks - 1 - i);
        if (bm->cache) {
            bm->cached.assign(num_blocks, 0);
            bm->key.assign(num_blocks, 0);
            bm->parent_key.assign(num_blocks, 0);
            bm->key_tokens.assign(static_cast<size_t>(num_blocks) * block_size, 0);
            bm->lru_prev.assign(num_blocks, -1);
            bm->lru_next.assign(num_blocks, -1);
        }
    } catch (const std::bad_alloc&) {
        delete bm;
        return fail(PA_ERR_NO_SPACE, "out of host memory for %lld blocks", (long long)num_blocks);
    }
    *out = bm;
    return ok();
}

void pa_bm_destroy(pa_bm_t* bm) { delete bm; }

int64_t pa_bm_num_free(const pa_bm_t* bm) { return bm ? bm->available() : -1; }

int64_t pa_bm_num_cached(const pa_bm_t* bm) {
    return bm ? static_cast<int64_t>(bm->by_key.size()) : -1;
}

static int pa_bm_add_impl(pa_bm_t* bm, const int32_t* tokens, int64_t num_tokens, int64_t* seq_id,
              int64_t* num_cached_tokens) {
    if (bm == nullptr || seq_id == nullptr) return fail(PA_ERR_NULL, "manager or seq_id is NULL");
    if (num_tokens < 0 || num_tokens > INT32_MAX)
        return fail(PA_ERR_SHAPE, "num_tokens %lld outside [0, 2^31-1]", (long long)num_tokens);
    if (bm->cache && tokens == nullptr && num_tokens > 0)
        return fail(PA_ERR_NULL, "the prefix cache needs the prompt's token ids");
    const int32_t bs = bm->bs;
    const int64_t n_blocks = (num_tokens + bs - 1) / bs;
    const int64_t n_full = num_tokens / bs;

    // Leading cache hits ([ZQ] TL;DR): look up block by block, stop at the first miss.
    std::vector<int32_t> hits;
    std::vector<uint64_t> hit_keys;
    uint64_t parent = bm->salt;
    if (bm->cache) {
        for (int64_t i = 0; i < n_full; ++i) {
            uint64_t k;
            const int32_t b = bm->lookup(parent, tokens + i * bs, &k);
            if (b < 0) break;
            hits.push_back(b);
            hit_keys.push_back(k);
            parent = k;
        }
    }
    int64_t revived = 0;
    for (int32_t b : hits) revived += bm->refcount[b] == 0 ? 1 : 0;
    const int64_t need = n_blocks - static_cast<int64_t>(hits.size());
    if (need > bm->available() - revived)
        return fail(PA_ERR_NO_SPACE, "the prompt needs %lld blocks, %lld are free",
                    (long long)need, (long long)(bm->available() - revived));

    Seq s;
    s.table.reserve(n_blocks);
    s.parent = bm->salt;
    for (size_t i = 0; i < hits.size(); ++i) {
        const int32_t b = hits[i];
        if (bm->refcount[b] == 0) bm->lru_remove(b);
        ++bm->refcount[b];
        s.table.push_back(b);
        s.parent = hit_keys[i];
    }
    for (int64_t i = static_cast<int64_t>(hits.size()); i < n_blocks; ++i) {
        const int32_t b = bm->take();
        s.table.push_back(b);
        if (bm->cache && i < n_full) s.parent = bm->register_block(b, s.parent, tokens + i * bs);
    }
    s.len = num_tokens;
    if (bm->cache) s.tokens.assign(tokens, tokens + num_tokens);
    const int64_t id = bm->next_id++;
    bm->seqs.emplace(id, std::move(s));
    *seq_id = id;
    if (num_cached_tokens) *num_cached_tokens = static_cast<int64_t>(hits.size()) * bs;
    return ok();
}

static int pa_bm_fork_impl(pa_bm_t* bm, int64_t parent, int64_t* child) {
    if (bm == nullptr || child == nullptr) return fail(PA_ERR_NULL, "manager or child is NULL");
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "unknown sequence %lld", (long long)parent);
    Seq s = it->second;                           // the same blocks, by pointer
    for (int32_t b : s.table) ++bm->refcount[b];
    const int64_t id = bm->next_id++;
    bm->seqs.emplace(id, std::move(s));
    *child = id;
    return ok();
}

int pa_bm_free(pa_bm_t* bm, int64_t seq_id) {
    if (bm == nullptr) return fail(PA_ERR_NULL, "manager is NULL");
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "unknown sequence %lld", (long long)seq_id);
    const std::vector<int32_t>& t = it->second.table;
    for (size_t i = t.size(); i-- > 0;) bm->release(t[i]);
    bm->seqs.erase(it);
    return ok();
}

static int pa_bm_append_impl(pa_bm_t* bm, const int64_t* seq_ids, const int32_t* tokens, int32_t n,
                 int64_t* slots, int64_t* cow_pairs, int32_t* num_cow) {
    if (bm == nullptr || num_cow == nullptr) return fail(PA_ERR_NULL, "manager or num_cow is NULL");
    if (n < 0) return fail(PA_ERR_SHAPE, "n %d < 0", n);
    *num_cow = 0;
    if (n == 0) return ok();
    if (seq_ids == nullptr || slots == nullptr || cow_pairs == nullptr)
        return fail(PA_ERR_NULL, "seq_ids, slots or cow_pairs is NULL");
    if (bm->cache && tokens == nullptr) return fail(PA_ERR_NULL, "the prefix cache needs token ids");
    const int32_t bs = bm->bs;

    // Dry run: resolve ids and count the blocks the step takes, following the
    // same rules in the same order as the real pass below.
    struct Sim { Seq* s; int64_t len; bool last_private; };
    std::unordered_map<int64_t, Sim> sim;
    std::unordered_map<int32_t, int32_t> dropped;   // shared block -> references given up
    std::vector<Seq*> resolved(n);
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
        auto f = sim.find(seq_ids[i]);
        if (f == sim.end()) {
            auto it = bm->seqs.find(seq_ids[i]);
            if (it == bm->seqs.end())
                return fail(PA_ERR_NOT_FOUND, "unknown sequence %lld at index %d", (long long)seq_ids[i], i);
            if (it->second.len >= INT32_MAX)
                return fail(PA_ERR_SHAPE, "sequence %lld is at 2^31-1 positions", (long long)seq_ids[i]);
            f = sim.emplace(seq_ids[i], Sim{&it->second, it->second.len, false}).first;
        }
        Sim& m = f->second;
        resolved[i] = m.s;
        if (m.len % bs == 0) {
            ++need;
            m.last_private = true;
        } else if (!m.last_private) {
            const int32_t last = m.s->table.back();
            int32_t& d = dropped[last];
            if (bm->refcount[last] - d > 1) {
                ++need;
                ++d;
            }
            m.last_private = true;
        }
        ++m.len;
    }
    if (need > bm->available())
        return fail(PA_ERR_NO_SPACE, "the step needs %lld blocks, %lld are free", (long long)need,
                    (long long)bm->available());

    int32_t ncow = 0;
    for (int32_t i = 0; i < n; ++i) {
        Seq& s = *resolved[i];
        if (s.len % bs == 0) {                    // growth ([KG] "Growth Needs Only Another Free Block")
            s.table.push_back(bm->take());
        } else {
            const int32_t last = s.table.back();
            if (bm->refcount[last] > 1) {         // copy-on-write ([ZQ] answer)
                const int32_t dst = bm->take();
                --bm->refcount[last];
                s.table.back() = dst;
                cow_pairs[2 * ncow] = last;
                cow_pairs[2 * ncow + 1] = dst;
                ++ncow;
            }
        }
        slots[i] = bm->slot(s, s.len);
        ++s.len;
        if (bm->cache) {
            s.tokens.push_back(tokens[i]);
            if (s.len % bs == 0)
                s.parent = bm->register_block(s.table.back(), s.parent, s.tokens.data() + (s.len - bs));
        }
    }
    *num_cow = ncow;
    return ok();
}

int pa_bm_slots(const pa_bm_t* bm, int64_t seq_id, int64_t start, int64_t count, int64_t* slots) {
    if (bm == nullptr) return fail(PA_ERR_NULL, "manager is NULL");
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "unknown sequence %lld", (long long)seq_id);
    const Seq& s = it->second;
    if (start < 0 || count < 0 || start + count > s.len)
        return fail(PA_ERR_SHAPE, "positions [%lld, %lld) outside the reserved [0, %lld)",
                    (long long)start, (long long)(start + count), (long long)s.len);
    if (count > 0 && slots == nullptr) return fail(PA_ERR_NULL, "slots is NULL");
    for (int64_t p = 0; p < count; ++p) slots[p] = bm->slot(s, start + p);
    return ok();
}

static int pa_bm_tables_impl(const pa_bm_t* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                 int32_t* tables, int32_t* lens) {
    if (bm == nullptr) return fail(PA_ERR_NULL, "manager is NULL");
    if (n < 0 || max_blocks < 1) return fail(PA_ERR_SHAPE, "n %d or max_blocks %d out of range", n, max_blocks);
    if (n == 0) return ok();
    if (seq_ids == nullptr || tables == nullptr) return fail(PA_ERR_NULL, "seq_ids or tables is NULL");
    std::vector<const Seq*> rs(n);
    for (int32_t i = 0; i < n; ++i) {
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end())
            return fail(PA_ERR_NOT_FOUND, "unknown sequence %lld at index %d", (long long)seq_ids[i], i);
        if (it->second.table.size() > static_cast<size_t>(max_blocks) || it->second.len > INT32_MAX)
            return fail(PA_ERR_SHAPE, "sequence %lld has %zu blocks (max_blocks %d)",
                        (long long)seq_ids[i], it->second.table.size(), max_blocks);
        rs[i] = &it->second;
    }
    for (int32_t i = 0; i < n; ++i) {
        int32_t* row = tables + static_cast<int64_t>(i) * max_blocks;
        const std::vector<int32_t>& t = rs[i]->table;
        std::memcpy(row, t.data(), sizeof(int32_t) * t.size());
        for (int32_t j = static_cast<int32_t>(t.size()); j < max_blocks; ++j) row[j] = -1;
        if (lens) lens[i] = static_cast<int32_t>(rs[i]->len);
    }
    return ok();
}

int pa_bm_seq_info(const pa_bm_t* bm, int64_t seq_id, int64_t* length, int64_t* num_blocks) {
    if (bm == nullptr) return fail(PA_ERR_NULL, "manager is NULL");
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "unknown sequence %lld", (long long)seq_id);
    if (length) *length = it->second.len;
    if (num_blocks) *num_blocks = static_cast<int64_t>(it->second.table.size());
    return ok();
}

int pa_bm_refcount(const pa_bm_t* bm, int64_t block, int32_t* refcount) {
    if (bm == nullptr || refcount == nullptr) return fail(PA_ERR_NULL, "manager or refcount is NULL");
    if (block < 0 || block >= bm->num_blocks)
        return fail(PA_ERR_SHAPE, "block %lld outside [0, %d)", (long long)block, bm->num_blocks);
    *refcount = bm->refcount[block];
    return ok();
}

}  // extern "C"

// Host memory exhaustion inside a container operation must not cross the C
// boundary as an exception: it is reported as PA_ERR_NO_SPACE, after which
// the manager may hold a partly applied operation and should be destroyed.
template <typename F>
static int guarded(const char* fn, F&& f) {
    try {
        return f();
    } catch (const std::bad_alloc&) {
        return fail(PA_ERR_NO_SPACE, "%s: out of host memory", fn);
    } catch (...) {
        return fail(PA_ERR_NO_SPACE, "%s: unexpected host failure", fn);
    }
}

extern "C" {

int pa_bm_add(pa_bm_t* bm, const int32_t* tokens, int64_t num_tokens, int64_t* seq_id,
              int64_t* num_cached_tokens) {
    return guarded("pa_bm_add", [&] { return pa_bm_add_impl(bm, tokens, num_tokens, seq_id, num_cached_tokens); });
}

int pa_bm_fork(pa_bm_t* bm, int64_t parent, int64_t* child) {
    return guarded("pa_bm_fork", [&] { return pa_bm_fork_impl(bm, parent, child); });
}

int pa_bm_append(pa_bm_t* bm, const int64_t* seq_ids, const int32_t* tokens, int32_t n,
                 int64_t* slots, int64_t* cow_pairs, int32_t* num_cow) {
    return guarded("pa_bm_append",
                   [&] { return pa_bm_append_impl(bm, seq_ids, tokens, n, slots, cow_pairs, num_cow); });
}

int pa_bm_tables(const pa_bm_t* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                 int32_t* tables, int32_t* lens) {
    return guarded("pa_bm_tables", [&] { return pa_bm_tables_impl(bm, seq_ids, n, max_blocks, tables, lens); });
}

}  // extern "C"
