/* pa_blocks.h -- host-side block manager of the paged KV cache.
 *
 * The bookkeeping on either side of the device path: the pool of free
 * physical blocks, a reference count per block, per-request block tables,
 * growth by one block, fork (sharing every block by pointer), free, the
 * copy-on-write decision, the slot of each new token, and a content-addressed
 * cache of full blocks for prefix reuse.  It moves no data: it returns the
 * slots to pass to pa_write_kv, the (src, dst) pairs to pass to
 * pa_copy_blocks, and the tables and lengths to upload for pa_decode.
 *
 * Sources (web pages, cited by title and section):
 *   [ZQ] zenaique.com, "How does PagedAttention enable prefix sharing across
 *        requests and what data structure makes it cheap?" -- the answer, the
 *        TL;DR and "Most common mistake".
 *   [KG] kgptalkie.com, "Day 28: PagedAttention" -- "Split the Cache Into
 *        Fixed Blocks", "The Block Table Is the Map", "Growth Needs Only
 *        Another Free Block", "Prefix Sharing Is a Natural Extension",
 *        "Shared Blocks Must Not Be Changed in Place".
 *
 * Conventions (all calls):
 *  - Every pointer is a HOST pointer.  Nothing here touches the GPU, so the
 *    manager also runs where no GPU is present.
 *  - Return value: PA_OK or a pa_status_t from pa.h.  On error the manager's
 *    state is exactly as before the call and pa_last_error() says why.
 *  - A manager is not thread-safe: calls on one manager must not overlap.
 *    Different managers are independent.
 *  - Sequence ids are assigned by the manager (0, 1, 2, ... in creation
 *    order) and never reused.
 *  - Physical blocks are handed out from a LIFO free list that starts as
 *    0, 1, 2, ...: a released block is the next one reused.  Any free block
 *    would be correct; the fixed order makes runs repeatable.
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_bm pa_bm_t;   /* opaque */

/* pa_bm_create flags */
#define PA_BM_PREFIX_CACHE 1u   /* keep a hash table of full blocks ([ZQ] TL;DR): a new
                                   request's leading full blocks that are in the table are
                                   shared instead of allocated.  A block is keyed by a
                                   64-bit FNV-1a hash of (parent block's key, its token
                                   ids), and a hit also compares the stored parent key and
                                   token ids, so a hash collision cannot share a wrong
                                   block.  Cached blocks whose count drops to zero stay
                                   reusable and are evicted oldest first, only when no
                                   never-cached block is free. */

/* A manager for a pool of num_blocks (>= 1, < 2^31) blocks of block_size
 * (1..4096) token positions.  `salt` is mixed into the first block's key: requests
 * may share cached blocks only under the same salt (use it for whatever besides
 * token ids decides the cached values -- model, adapter, position rules, cache
 * settings: [KG] "Shared Blocks Must Not Be Changed in Place").  *out receives the
 * manager; release it with pa_bm_destroy.  Errors: PA_ERR_NULL, PA_ERR_SHAPE,
 * PA_ERR_UNSUPPORTED (unknown flag bits). */
int pa_bm_create(int64_t num_blocks, int32_t block_size, uint32_t flags, uint64_t salt,
                 pa_bm_t** out);

/* Frees the manager (NULL is ignored). */
void pa_bm_destroy(pa_bm_t* bm);

/* Blocks available to new allocations: free blocks plus unused cached blocks
 * (-1 for a NULL manager). */
int64_t pa_bm_num_free(const pa_bm_t* bm);

/* Blocks currently registered in the prefix cache (0 without PA_BM_PREFIX_CACHE;
 * -1 for a NULL manager). */
int64_t pa_bm_num_cached(const pa_bm_t* bm);

/* Admits a request whose prompt has num_tokens (>= 0) tokens and reserves its
 * positions: ceil(num_tokens / block_size) blocks ([KG] "Growth Needs Only Another
 * Free Block").  With PA_BM_PREFIX_CACHE, `tokens` (num_tokens int32 ids) is
 * required: the prompt is hashed block by block and each leading full block found
 * in the cache is shared (its count goes up) until the first miss; the prompt's
 * other full blocks are registered as they are allocated, so the caller must
 * write their keys and values (pa_write_kv at pa_bm_slots) before any later call
 * reads them.  Without the flag `tokens` is ignored and may be NULL.
 * *seq_id receives the new request; *num_cached_tokens (may be NULL) the number of
 * leading prompt positions whose keys and values are already in the cache (a
 * multiple of block_size; their prefill can be skipped).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_NO_SPACE (state unchanged). */
int pa_bm_add(pa_bm_t* bm, const int32_t* tokens, int64_t num_tokens, int64_t* seq_id,
              int64_t* num_cached_tokens);

/* A new request sharing every block of `parent` by pointer ([ZQ] answer; the
 * fan-out of sampling branches).  Each block's count goes up by one.
 * Errors: PA_ERR_NULL, PA_ERR_NOT_FOUND. */
int pa_bm_fork(pa_bm_t* bm, int64_t parent, int64_t* child);

/* The request finishes: one reference to each of its blocks is dropped, last
 * block first; a block whose count reaches zero becomes free (or, if cached,
 * reusable until evicted) ([KG] "Shared Blocks Must Not Be Changed in Place").
 * The id becomes unknown.  Errors: PA_ERR_NOT_FOUND. */
int pa_bm_free(pa_bm_t* bm, int64_t seq_id);

/* One decode step: reserves the next position of each of the n (>= 0) requests
 * seq_ids[0..n) in that order (a request listed twice gets two positions).  For
 * each: at a block boundary one more block is taken; inside a block that other
 * requests still reference, copy-on-write gives this request a fresh block and
 * the pair (shared, fresh) is reported, to be copied before the token is written
 * ([ZQ] answer; [KG] "Shared Blocks Must Not Be Changed in Place").
 * slots[i] (n int64, out) is the flat slot (block * block_size + offset) of the
 * i-th new token; cow_pairs (2n int64, out) receives *num_cow (out) pairs
 * {src, dst}, in order.  With PA_BM_PREFIX_CACHE, `tokens` (n int32 ids) is
 * required and a block filled by its last token is registered in the cache.
 * All blocks needed are counted first: if the pool cannot supply them the call
 * returns PA_ERR_NO_SPACE and changes nothing.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_NOT_FOUND, PA_ERR_NO_SPACE. */
int pa_bm_append(pa_bm_t* bm, const int64_t* seq_ids, const int32_t* tokens, int32_t n,
                 int64_t* slots, int64_t* cow_pairs, int32_t* num_cow);

/* Flat slots of positions [start, start + count) of a request, which must lie
 * within its reserved length ([KG] "Follow One Token Address").
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_NOT_FOUND. */
int pa_bm_slots(const pa_bm_t* bm, int64_t seq_id, int64_t start, int64_t count,
                int64_t* slots);

/* Block tables and lengths of n requests in the layout pa_decode reads:
 * tables is [n][max_blocks] int32 (out), entries past a request's blocks set to
 * -1; lens is [n] int32 (out, may be NULL).  Errors: PA_ERR_NULL, PA_ERR_SHAPE
 * (a request has more than max_blocks blocks or more than 2^31-1 positions),
 * PA_ERR_NOT_FOUND. */
int pa_bm_tables(const pa_bm_t* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                 int32_t* tables, int32_t* lens);

/* Length (reserved positions) and block count of one request (either output may
 * be NULL).  Errors: PA_ERR_NOT_FOUND. */
int pa_bm_seq_info(const pa_bm_t* bm, int64_t seq_id, int64_t* length, int64_t* num_blocks);

/* Reference count of one physical block (0 for free and unused cached blocks).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (block out of range). */
int pa_bm_refcount(const pa_bm_t* bm, int64_t block, int32_t* refcount);

/* The key of one full block: 64-bit FNV-1a over `parent` (8 bytes,
 * little-endian) followed by the n token ids (4 bytes each, little-endian).  A
 * request's first block uses the manager's salt as its parent.  Exposed so a
 * caller can precompute keys; no manager is needed. */
uint64_t pa_bm_block_key(uint64_t parent, const int32_t* tokens, int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H */
