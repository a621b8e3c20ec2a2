/*
 * pa.h -- C ABI of libpagedkv: decode attention over a paged KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [ZQ] zenaique.com, "How does PagedAttention enable prefix sharing across
 *        requests and what data structure makes it cheap?" (answer, TL;DR,
 *        "Most common mistake").
 *   [KG] kgptalkie.com, "Day 28: PagedAttention".
 *
 * The KV cache of one attention layer lives in fixed-size physical blocks
 * ([KG] "Split the Cache Into Fixed Blocks").  A request reaches its tokens
 * through a block table: the token at logical position p is in logical
 * block p / block_size at offset p % block_size, and the table names the
 * physical block ([KG] "The Block Table Is the Map", "Follow One Token
 * Address").  Requests that share a prefix name the same physical blocks;
 * copy-on-write copies only a block that diverges ([ZQ] answer, "Most common
 * mistake"; [KG] "Shared Blocks Must Not Be Changed in Place").
 *
 * ---------------------------------------------------------------------------
 * Conventions for every call
 * ---------------------------------------------------------------------------
 *  - Pointers named *_cache, q, out, k_new, v_new, block_tables,
 *    context_lens, slot_mapping, block_pairs, seq_ids, positions, workspace
 *    are DEVICE pointers (memory of the current HIP device).  Descriptor
 *    structs and scalars are host values.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on `stream` and returns; nothing
 *    synchronises unless PA_VALIDATE=1 is set in the environment (below).
 *  - The caller owns all memory.  The library allocates no device memory,
 *    keeps no pointer after a call returns and holds no global mutable state
 *    except a thread-local error message -- and, for pa_decode_step_noalloc
 *    only, one static device array per GPU (see there).
 *  - Return value: PA_OK (0) or a pa_status_t error.  On error nothing was
 *    enqueued and pa_last_error() describes the problem.  Device-side
 *    contract violations (a block id outside [0, num_blocks), a context
 *    length above max_context_len, duplicate write slots, a copy destination
 *    that is also a source) are not detected in normal runs; the kernels
 *    clamp every such index so no access leaves the buffers, and the
 *    results are then unspecified.  With PA_VALIDATE=1 the library copies
 *    the index arrays to the host (a synchronising copy) and rejects such
 *    calls with PA_ERR_VALIDATE before launching.
 *
 * ---------------------------------------------------------------------------
 * Cache layout (one layer; K and V are separate buffers)
 * ---------------------------------------------------------------------------
 *  The pages leave the bytes of a block to the implementation ([KG] "Split
 *  the Cache Into Fixed Blocks").  This library fixes them so that a block's
 *  keys feed the gfx950 matrix cores straight from 16-byte loads:
 *
 *    x = 16 / sizeof(element)           (8 for bf16, 4 for f32)
 *    T = 16 if block_size is a multiple of 16, else block_size
 *        (positions per tile; a block holds block_size / T tiles)
 *    S = block_stride (or Hkv * block_size * D when it is 0)
 *    for offset t in the block: tile u = t / T, position p = t % T, and
 *    R = b * S + h * block_size * D + u * T * D  (the tile's region)
 *    K element (block b, kv head h, offset t, dim d) at index
 *        R + ((d / x) * T + p) * x + d % x
 *    V element (block b, kv head h, offset t, dim d) at index
 *        R + d * T + p
 *
 *  i.e. each block of K is [Hkv][tiles][D/x][T][x] and each block of V is
 *  [Hkv][tiles][D][T]; for block sizes up to 16 that is [Hkv][D/x][bs][x]
 *  and [Hkv][D][bs].  A (block, head) region is contiguous, and so is each
 *  16-position tile in it (4 KiB of K and 4 KiB of V at D 128, bf16), which
 *  is what one MFMA step consumes.  Both buffers must be 16-byte aligned
 *  and S * sizeof(element) a multiple of 16.
 *
 *  Recommended allocation: one buffer of [num_blocks][2][Hkv * block_size *
 *  D] elements with k_cache = its start, v_cache = start + Hkv * block_size
 *  * D and S = 2 * Hkv * block_size * D, so a block's keys and values of all
 *  heads sit in one contiguous region (measured on MI355X: 4-7% more decode
 *  bandwidth than two separate dense buffers).
 *
 *  Queries, outputs and new-token K/V are plain row-major
 *  [tokens][heads][D].  Query head hq reads KV head hq / (Hq / Hkv).
 */
#ifndef PAGED_KV_PA_H
#define PAGED_KV_PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 5   /* 4: PA_DECODE_PREFIX_RUNS; 5: PA_DECODE_APPEND_TILES */

typedef enum {
    PA_F32 = 0,   /* IEEE binary32 */
    PA_BF16 = 1,  /* bfloat16 */
} pa_dtype_t;

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL = 1,         /* a required pointer is NULL */
    PA_ERR_SHAPE = 2,        /* a size is negative, zero where it must not be, or inconsistent */
    PA_ERR_DTYPE = 3,        /* unknown dtype */
    PA_ERR_ALIGN = 4,        /* a buffer is not 16-byte aligned */
    PA_ERR_UNSUPPORTED = 5,  /* a combination outside the compiled set */
    PA_ERR_WORKSPACE = 6,    /* workspace missing or smaller than pa_decode_workspace_bytes */
    PA_ERR_HIP = 7,          /* the HIP runtime reported an error (launch or query) */
    PA_ERR_VALIDATE = 8,     /* PA_VALIDATE=1 found an index outside its range */
    PA_ERR_NO_SPACE = 9,     /* block manager: not enough free blocks (nothing was changed) */
    PA_ERR_NOT_FOUND = 10,   /* block manager: unknown sequence id */
} pa_status_t;

/* Shape of one layer's paged KV cache. */
typedef struct {
    int64_t num_blocks;    /* physical blocks in each of the K and V buffers, >= 1 */
    int32_t block_size;    /* token positions per block: 1..256 (MFMA decode: 8, 16, 32
                              or 64; the grouped, prefix-run and prefill kernels: 16) */
    int32_t num_kv_heads;  /* Hkv >= 1 */
    int32_t head_dim;      /* D: 16, 32, 64, 128 or 256 (MFMA decode: bf16 64, 128 or 256,
                              fp32 64 or 128; the grouped, prefix-run and prefill kernels:
                              bf16 128) */
    int32_t dtype;         /* pa_dtype_t of K, V, q, out, k_new, v_new */
    int64_t block_stride;  /* elements from block b to block b+1 in k_cache and in v_cache;
                              0 means dense (Hkv * block_size * head_dim) */
} pa_cache_desc_t;

/* pa_decode flags */
#define PA_DECODE_GROUP_SHARED 2u  /* consecutive requests may share leading blocks (a common
                                      prompt or prefix): the fast path then processes up to
                                      16 / (Hq/Hkv) consecutive requests per wave and reads a
                                      block they all name only once.  The output bits equal
                                      the ungrouped ones: every request still sees its
                                      tiles in logical order with the same partitions and
                                      the same arithmetic. */
#define PA_DECODE_PREFIX_RUNS 4u   /* long runs of consecutive requests share their leading
                                      blocks (one prefix, many requests).  A partition that
                                      all 4 * 16/(Hq/Hkv) requests of a chunk share is decoded
                                      for all of them at once by four waves that copy each
                                      tile to LDS once; the other partitions are decoded one
                                      request per wave in the same launch.  Output bits equal
                                      one request per wave.  Used on the fast path with
                                      16 % (Hq/Hkv) == 0 and at least two partitions, except
                                      in pa_decode_step with copy-on-write sources; elsewhere
                                      ignored (PA_DECODE_GROUP_SHARED then applies if set). */
#define PA_DECODE_STREAM_KV 1u  /* read K/V with non-temporal loads, which keeps them from
                                   displacing other cache contents.  A cache hint only:
                                   results are identical.  Measured on MI355X: +6..13% when
                                   no block is read by two waves of the call (unshared
                                   batches, or shared blocks decoded with
                                   PA_DECODE_GROUP_SHARED, which reads each once per group);
                                   -10% for a prefix shared by many requests decoded one
                                   request per wave, whose repeat reads must hit the caches */
#define PA_DECODE_APPEND_TILES 8u  /* pa_decode_append / pa_decode_step on the MFMA path with
                                      block size 16, 32 or 64: the wave that appends a
                                      request's token writes the 16-position tile holding it
                                      back whole, token included, once it has read the tile
                                      (full-line stores), instead of storing the token's K
                                      chunks and V elements on their own (the V column of a
                                      dim-major tile lands in partial sectors).  A store-pattern
                                      choice only: cache bytes and output are identical.
                                      Applied without the flag when num_seqs * Hkv >= 1024;
                                      measured on MI355X: -3.6% step time at 2,048 appends,
                                      +2% at 256, where the tile stores come at the end of the
                                      longest walks.  Ignored by pa_decode and elsewhere. */

/* Version of this ABI (PA_ABI_VERSION of the library that was built). */
int pa_abi_version(void);

/* Static name of a status code. */
const char* pa_status_string(int status);

/* Detail for the last non-OK return on this thread ("" if none). */
const char* pa_last_error(void);

/*
 * pa_write_kv -- scatter new tokens' keys and values into the cache.
 *
 * For every token t with slot_mapping[t] >= 0, writes k_new[t][h][:] and
 * v_new[t][h][:] for every KV head h at block slot / block_size, offset
 * slot % block_size ([KG] "Follow One Token Address": the flat slot is
 * physical_block * block_size + offset).  A negative slot marks a padding
 * token and is skipped.  Bytes are copied unchanged.
 *
 *   c            cache descriptor (host)
 *   k_cache      [num_blocks] blocks in the K layout above (written)
 *   v_cache      [num_blocks] blocks in the V layout above (written)
 *   k_new, v_new [num_tokens][Hkv][D], dtype c->dtype
 *   slot_mapping int64 [num_tokens]; valid slots are < num_blocks * block_size
 *                and unique (a duplicate slot is a race; the winner is unspecified)
 *   num_tokens   >= 0 (0 enqueues nothing)
 */
int pa_write_kv(const pa_cache_desc_t* c, void* k_cache, void* v_cache, const void* k_new,
                const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                void* stream);

/*
 * pa_copy_blocks -- copy-on-write block copies.
 *
 * For each pair i, copies the whole physical block block_pairs[2i] (src) to
 * block_pairs[2i+1] (dst): every head, every slot, K and V ([ZQ] answer: a
 * diverging request gets a fresh block; [KG] "Shared Blocks Must Not Be
 * Changed in Place": a private copy is made before the shared part changes;
 * [ZQ] "Most common mistake": only that block is copied).  Destinations
 * must be distinct and no destination may be a source of the same call.
 *
 *   block_pairs  int64 [num_pairs][2] = {src, dst}, each in [0, num_blocks)
 *   num_pairs    >= 0 (0 enqueues nothing)
 */
int pa_copy_blocks(const pa_cache_desc_t* c, void* k_cache, void* v_cache,
                   const int64_t* block_pairs, int32_t num_pairs, void* stream);

/*
 * pa_slot_mapping -- address translation on the device.
 *
 * slot_mapping[t] = block_tables[s][p / block_size] * block_size + p % block_size
 * with s = seq_ids[t] (or t when seq_ids is NULL) and p = positions[t]
 * ([KG] "Follow One Token Address").  A negative position gives -1; so does
 * a position past the table (p / block_size >= max_blocks_per_seq), a
 * sequence index outside [0, num_seqs) or a negative table entry.
 *
 *   block_tables int32 [num_seqs][max_blocks_per_seq]
 *   seq_ids      int32 [num_tokens] or NULL
 *   positions    int32 [num_tokens]
 *   slot_mapping int64 [num_tokens] (written)
 */
int pa_slot_mapping(int32_t block_size, const int32_t* block_tables, int32_t num_seqs,
                    int32_t max_blocks_per_seq, const int32_t* seq_ids,
                    const int32_t* positions, int32_t num_tokens, int64_t* slot_mapping,
                    void* stream);

/*
 * pa_gather_kv -- the contiguous history of one request.
 *
 * Walks block_table in logical order and writes the first context_len
 * tokens' keys and values as row-major [context_len][Hkv][D] ([KG] "Batching
 * Becomes More Flexible": the kernel reads the request's table and gathers
 * its history).  A copy, bit for bit; used to check address translation in
 * isolation.
 *
 *   block_table  int32 [ceil(context_len / block_size)] (device)
 *   k_out, v_out [context_len][Hkv][D], dtype c->dtype (written)
 */
int pa_gather_kv(const pa_cache_desc_t* c, const void* k_cache, const void* v_cache,
                 const int32_t* block_table, int32_t context_len, void* k_out, void* v_out,
                 void* stream);

/*
 * Partition length, in tokens, that pa_decode uses for split-K when
 * partition_tokens = 0.  It depends only on these host scalars and the
 * device's compute-unit count, never on block placement, so outputs are
 * bit-identical whatever the physical block ids.
 */
int32_t pa_decode_partition_tokens(const pa_cache_desc_t* c, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_context_len);

/*
 * Bytes of workspace pa_decode needs for these sizes (0 when every request
 * fits one partition): the fp32 partial results of every partition,
 * S * Hq * ceil(max_context_len / partition) * (D + 2) floats.
 * partition_tokens as for pa_decode (0 = automatic).
 */
size_t pa_decode_workspace_bytes(const pa_cache_desc_t* c, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_context_len,
                                 int32_t partition_tokens);

/*
 * pa_decode -- one decode query per request against its paged history.
 *
 * For request i and query head hq, with h = hq / (Hq / Hkv) and
 * L = context_lens[i]:
 *     s_t = scale * <q[i][hq], K_i[t][h]>          for t = 0 .. L-1
 *     out[i][hq] = sum_t softmax(s)_t * V_i[t][h]
 * where K_i[t], V_i[t] are found through block_tables[i] as in
 * pa_slot_mapping ([KG] "Follow One Token Address", closing sentence: the
 * table only locates keys and values, the decode attention over them is the
 * usual one; "The Contiguous Allocation Problem": paging changes placement,
 * not the attention formula).  The query sees positions [0, L): the cache holds the current
 * token's K/V (written by pa_write_kv) and nothing later.  L = 0 gives a
 * zero output.  Positions at or past L are never read into the result, so
 * stale or NaN bytes there do not matter.
 *
 * Arithmetic: fp32 accumulation; bf16 outputs are rounded to nearest even.
 * Long histories are split into partitions of partition_tokens positions
 * whose partial softmax states are merged in a fixed order, so results are
 * deterministic and independent of physical block placement.
 *
 *   q             [num_seqs][num_q_heads][D], dtype c->dtype
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]
 *   context_lens  int32 [num_seqs], 0 <= L <= max_context_len and
 *                 L <= max_blocks_per_seq * block_size
 *   num_q_heads   a multiple of Hkv, with Hq / Hkv <= 16
 *   max_context_len  host int >= every L (sizes the launch; no device->host sync)
 *   scale         softmax scale (1/sqrt(D) for standard attention)
 *   out           [num_seqs][num_q_heads][D], dtype c->dtype (written)
 *   workspace     device scratch of >= pa_decode_workspace_bytes(...) bytes,
 *                 16-byte aligned, any contents (may be NULL when the size
 *                 is 0).  Calls in flight at the same time must not share a
 *                 workspace.
 *   partition_tokens  0 = automatic; otherwise a multiple of block_size in
 *                 [block_size, 1024] (the MFMA path -- block size 8, 16, 32 or 64;
 *                 bf16 at head_dim 64, 128 or 256, fp32 at 64 or 128 -- also needs a
 *                 multiple of 16 and at most 64 blocks: 512 positions at block size 8)
 *   flags         0 or an OR of PA_DECODE_STREAM_KV (a cache hint; results are the
 *                 same), PA_DECODE_GROUP_SHARED and PA_DECODE_PREFIX_RUNS
 *                 (PA_DECODE_APPEND_TILES is accepted and has no effect here)
 */
int pa_decode(const pa_cache_desc_t* c, const void* k_cache, const void* v_cache,
              const void* q, const int32_t* block_tables, const int32_t* context_lens,
              int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
              int32_t max_context_len, float scale, void* out, void* workspace,
              size_t workspace_bytes, int32_t partition_tokens, uint32_t flags,
              void* stream);

/*
 * pa_decode_append -- one decode step: append each request's newest token,
 * then attend.
 *
 * Same result as pa_write_kv of k_new[i] / v_new[i] at the slot of position
 * context_lens[i] - 1 of request i (translated through block_tables as in
 * pa_slot_mapping), followed by pa_decode with the same arguments: the new
 * token is the query's own position, the last one it sees ([KG] "Follow One
 * Token Address": the newest query attends to the history including itself;
 * "Growth Needs Only Another Free Block": the engine has already given the
 * request a block with room for it).  Requests with L = 0 append nothing.
 * On the fast path one kernel does both: the wave of each request's last
 * partition stores the token and uses it directly, so no separate write
 * launch or read-back is needed.
 *
 * The block that receives the token must be private to the request (a
 * shared block is first copied with pa_copy_blocks, [ZQ] answer; [KG]
 * "Shared Blocks Must Not Be Changed in Place").
 *
 *   k_cache, v_cache  written at the appended slots
 *   k_new, v_new      [num_seqs][Hkv][D], dtype c->dtype, 16-byte aligned
 *   flags             as for pa_decode, plus PA_DECODE_APPEND_TILES
 *   other arguments   as for pa_decode
 */
int pa_decode_append(const pa_cache_desc_t* c, void* k_cache, void* v_cache, const void* k_new,
                     const void* v_new, const void* q, const int32_t* block_tables,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                     int32_t max_blocks_per_seq, int32_t max_context_len, float scale, void* out,
                     void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                     uint32_t flags, void* stream);

/*
 * pa_decode_step -- one decode step with its copy-on-write copies folded in.
 *
 * Exactly pa_copy_blocks of the pairs {cow_src[i], B_i} for every request i
 * with cow_src[i] >= 0, where B_i = block_tables[i][(L_i - 1) / block_size]
 * is the block that holds the request's newest position, followed by
 * pa_decode_append ([ZQ] answer and [KG] "Shared Blocks Must Not Be Changed
 * in Place": a request that writes into a shared block gets a fresh copy of
 * it first; the block manager's pa_bm_append reports exactly such pairs).
 * With block size 16 on the MFMA path the wave that reads the request's last
 * block reads it from cow_src[i] and writes it back whole, new token
 * included, to B_i: the copy and the token write become full-line stores and
 * the block is read once.  Other shapes copy first with a kernel of their own.
 *
 * Arguments: as pa_decode_append, plus
 *   cow_src   [num_seqs] int32 device array (may be NULL = no copies):
 *             the source block of request i's copy, or -1.  Each B_i with a
 *             copy must be distinct and must not be another request's source;
 *             out-of-range sources are skipped (PA_VALIDATE=1 rejects them).
 */
int pa_decode_step(const pa_cache_desc_t* c, void* k_cache, void* v_cache, const void* k_new,
                   const void* v_new, const int32_t* cow_src, const void* q,
                   const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                   int32_t num_q_heads, int32_t max_blocks_per_seq, int32_t max_context_len,
                   float scale, void* out, void* workspace, size_t workspace_bytes,
                   int32_t partition_tokens, uint32_t flags, void* stream);

/*
 * pa_decode_step_noalloc -- pa_decode_step without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, results and errors as pa_decode_step, minus workspace and
 * workspace_bytes.  The split-K partials go to a static device array inside
 * the library (PA_DECODE_NOALLOC_MAX_BYTES bytes on every GPU the library
 * runs on, held from module load until the process ends).  The call itself
 * allocates nothing; its first call on a device looks up that device's
 * address of the array.
 *   - A call whose partials need more than PA_DECODE_NOALLOC_MAX_BYTES (what
 *     pa_decode_workspace_bytes reports for the same shape and partition)
 *     returns PA_ERR_WORKSPACE and enqueues nothing.
 *   - Every call on one GPU shares that GPU's array, and it keeps the last
 *     call's contents (the kernels need no cleared memory).  Calls that
 *     overlap on one GPU (different streams, or threads without ordering)
 *     race on it: serialise them.
 */
#define PA_DECODE_NOALLOC_MAX_BYTES ((size_t)64 << 20)
int pa_decode_step_noalloc(const pa_cache_desc_t* c, void* k_cache, void* v_cache,
                           const void* k_new, const void* v_new, const int32_t* cow_src,
                           const void* q, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                           int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                           void* out, int32_t partition_tokens, uint32_t flags, void* stream);

/*
 * pa_prefill -- several new query tokens per request against the paged
 * history: a chunk of a prompt whose earlier part is cached (e.g. found by
 * the prefix cache), a chunked prefill, or several tokens checked at once.
 *
 * Request i's query tokens are rows q_start[i] .. q_start[i+1]-1 of q, n_i of
 * them.  They are the request's last n_i positions and their K/V are already
 * in the cache (pa_write_kv), counted in L = context_lens[i]; token j sits at
 * position L - n_i + j and, for query head hq with h = hq / (Hq / Hkv), gives
 *     s_t = scale * <q[row][hq], K_i[t][h]>      for t = 0 .. L - n_i + j
 *     out[row][hq] = sum_t softmax(s)_t * V_i[t][h]
 * -- its own position and earlier ones, never a later one ([KG] "A Tiny
 * Block-Table Example", closing paragraphs).  A token whose position is
 * negative (n_i > L) sees nothing and gives zeros.  With n_i = 1 this is
 * pa_decode.
 *
 * Arguments: as pa_decode, plus
 *   q, out        [total_q][Hq][head_dim] packed rows (dtype == c->dtype)
 *   q_start       [num_seqs + 1] int32, q_start[0] = 0, non-decreasing,
 *                 q_start[num_seqs] = total_q (device)
 *   total_q       rows of q and out, 0 .. 65535 (host)
 *   max_q_len     >= every n_i (host); sizes the grid
 *   workspace     >= pa_prefill_workspace_bytes(...) bytes
 *   flags         0
 * MFMA prefill kernels: bf16, head_dim 64, 128 or 256, Hq/Hkv dividing 16,
 * block size 8, 16, 32 or 64 when max_q_len >= 2 * 16 / (Hq/Hkv), and any
 * max_q_len at head_dim 128 with blocks of 16 (partition_tokens 0 or a
 * multiple of max(16, block_size) up to 2^20).  Every other
 * shape pa_decode accepts runs each query row as a decode request: a small
 * kernel gives row r of request i a copy of i's first ceil(max_context_len /
 * block_size) table entries and its visible length L - n_i + j + 1 (clamped
 * to [0, L]; a row outside every request's range gets 0), then the decode
 * kernels run total_q requests; partition_tokens then follows pa_decode's
 * rule with num_seqs = total_q, and the workspace holds the copies too.
 * Indices and row offsets read on the device are clamped into range (no
 * fault); PA_VALIDATE=1 rejects them.
 */
size_t pa_prefill_workspace_bytes(const pa_cache_desc_t* c, int32_t num_seqs, int32_t total_q,
                                  int32_t max_q_len, int32_t num_q_heads,
                                  int32_t max_context_len, int32_t partition_tokens);

int pa_prefill(const pa_cache_desc_t* c, const void* k_cache, const void* v_cache,
               const void* q, const int32_t* q_start, const int32_t* block_tables,
               const int32_t* context_lens, int32_t num_seqs, int32_t total_q,
               int32_t max_q_len, int32_t num_q_heads, int32_t max_blocks_per_seq,
               int32_t max_context_len, float scale, void* out, void* workspace,
               size_t workspace_bytes, int32_t partition_tokens, uint32_t flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_PA_H */
