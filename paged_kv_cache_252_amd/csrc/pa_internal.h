// Internal declarations shared by the libpagedkv translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "pa.h"

namespace pa {

// ---- error reporting ------------------------------------------------------

// Records a printf-style message for pa_last_error() and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the thread's last error and returns PA_OK.
int ok();

// Maps the runtime's last launch error (if any) to PA_ERR_HIP.
int check_launch(const char* what);

// True when PA_VALIDATE=1 is set: index arrays are checked on the host.
bool validate_enabled();

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int elem_bytes(int dtype) { return dtype == PA_BF16 ? 2 : 4; }

// Checks the descriptor itself: dtype, sizes, supported head_dim.
int check_desc(const pa_cache_desc_t* c);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Elements of one block's K (or V) data: Hkv * block_size * head_dim.
inline int64_t block_elems(const pa_cache_desc_t* c) {
    return static_cast<int64_t>(c->num_kv_heads) * c->block_size * c->head_dim;
}

// Elements from one block to the next (the descriptor's stride, or dense).
inline int64_t block_stride(const pa_cache_desc_t* c) {
    return c->block_stride ? c->block_stride : block_elems(c);
}

// ---- in-block layout ----------------------------------------------------------
//
// One (block, head) region holds block_size * head_dim elements.  Positions
// are grouped in tiles of T = 16 when the block size is a multiple of 16
// (else T = the block size): K is [tile][D/X][T][X] with X elements = 16
// bytes, V is [tile][D][T].  A 16-position tile is thus the same 4 KiB K and
// 4 KiB V (bf16, D 128) whatever the block size.

__host__ __device__ inline int tile_tokens(int block_size) {
    return block_size % 16 == 0 ? 16 : block_size;
}

// Offset of K element (position pos, dim d) inside its (block, head) region.
__host__ __device__ inline int64_t k_elem(int pos, int d, int block_size, int head_dim, int x) {
    const int t = tile_tokens(block_size);
    const int tile = pos / t, p = pos - tile * t;
    return static_cast<int64_t>(tile) * t * head_dim + (static_cast<int64_t>(d / x) * t + p) * x + d % x;
}

// Offset of V element (position pos, dim d) inside its (block, head) region.
__host__ __device__ inline int64_t v_elem(int pos, int d, int block_size, int head_dim) {
    const int t = tile_tokens(block_size);
    const int tile = pos / t, p = pos - tile * t;
    return static_cast<int64_t>(tile) * t * head_dim + static_cast<int64_t>(d) * t + p;
}

// ---- decode planning --------------------------------------------------------

// Compute units of the current device (cached per device).
int device_cu_count();

// The MFMA kernels for block size 16 (decode, grouped decode, prefill) handle this shape.
inline bool fast_path_ok(const pa_cache_desc_t* c, int group) {
    return c->dtype == PA_BF16 && c->head_dim == 128 && c->block_size == 16 && group >= 1 &&
           group <= 16;
}

// The MFMA decode kernel handles this shape: bf16 at head_dim 64, 128 or 256,
// fp32 (the fp32 MFMA) at 64 or 128; blocks of 8 pair up into its 16-token
// tiles, blocks of 32 or 64 split into them.
inline bool fast_decode_ok(const pa_cache_desc_t* c, int group) {
    const int bs = c->block_size, d = c->head_dim;
    const bool dims = c->dtype == PA_BF16 ? (d == 64 || d == 128 || d == 256)
                                          : (c->dtype == PA_F32 && (d == 64 || d == 128));
    return dims && (bs == 8 || bs == 16 || bs == 32 || bs == 64) && group >= 1 && group <= 16;
}

// Partitions of the MFMA decode kernel are whole tiles and whole blocks.
inline int fast_granule(int block_size) { return block_size > 16 ? block_size : 16; }

// ... and hold at most one block-table entry per lane of a wave.
inline int fast_max_partition(int block_size) { return 64 * block_size < 1024 ? 64 * block_size : 1024; }

// ---- kernel launchers (defined in the .hip files) --------------------------

struct DecodeArgs {
    const void* k_cache;
    const void* v_cache;
    const void* q;
    const int32_t* block_tables;
    const int32_t* context_lens;
    int64_t num_blocks;
    int64_t block_stride;    // elements between consecutive blocks of k_cache / v_cache
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t group;
    int32_t max_blocks_per_seq;
    int32_t len_clamp;       // min(max_context_len, max_blocks_per_seq * block_size)
    int32_t part_tokens;
    int32_t max_parts;
    float scale;
    uint32_t flags;
    void* out;
    float* ws_acc;           // [S][Hq][max_parts][D]
    float* ws_m;             // [S][Hq][max_parts]  (log2 domain running max)
    float* ws_l;             // [S][Hq][max_parts]
    const void* k_new;       // non-null: append each request's token at position L-1
    const void* v_new;
    const int32_t* cow_src;  // non-null (with k_new): request i's block holding L-1 first
                             // receives a copy of block cow_src[i] (negative: none)
    hipStream_t stream;
};

int launch_decode(const DecodeArgs& a);

// Several query tokens per request: the DecodeArgs fields above plus these.
struct PrefillArgs {
    DecodeArgs d;            // num_seqs, q (packed rows), out (packed rows), ws_* per query row
    const int32_t* q_start;  // [num_seqs + 1] row offsets of each request's query tokens
    int32_t total_q;         // rows of q and out
    int32_t max_q_len;       // longest chunk; sizes the grid
    int32_t* ws_len;         // [total_q] visible positions per query row, for the merge
};

int launch_prefill(const PrefillArgs& a);

// Shapes without an MFMA prefill kernel: row r of the packed query rows gets
// row_tables[r][0 .. row_blocks) = its request's first row_blocks table
// entries (row_blocks <= max_blocks_per_seq) and row_lens[r] = the positions
// it sees, so that launch_decode runs the rows as total_q requests.
int launch_prefill_rows(const int32_t* q_start, const int32_t* block_tables,
                        const int32_t* context_lens, int32_t num_seqs, int32_t total_q,
                        int32_t max_blocks_per_seq, int32_t row_blocks, int32_t len_clamp,
                        int32_t* row_tables, int32_t* row_lens, hipStream_t stream);

// The split-K merge of bf16 partials at head_dim 64, 128 or 256: row r (of
// `rows`) and query head hq combine the ceil(lens[r] / part_tokens)
// partitions of ws_* [rows][Hq][max_parts] into out[r][hq] (rows with one
// partition are left alone: their kernel wrote them).
int launch_merge(const int32_t* lens, int32_t rows, int32_t num_q_heads, int32_t head_dim,
                 int32_t len_clamp, int32_t part_tokens, int32_t max_parts, const float* ws_acc,
                 const float* ws_m, const float* ws_l, void* out, hipStream_t stream);

int launch_write_kv(const pa_cache_desc_t* c, void* k_cache, void* v_cache, const void* k_new,
                    const void* v_new, const int64_t* slots, int32_t num_tokens,
                    hipStream_t stream);

int launch_copy_blocks(const pa_cache_desc_t* c, void* k_cache, void* v_cache,
                       const int64_t* pairs, int32_t num_pairs, hipStream_t stream);

int launch_cow_last_block(const pa_cache_desc_t* c, void* k_cache, void* v_cache,
                          const int32_t* cow_src, const int32_t* block_tables,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t max_blocks_per_seq, int32_t len_clamp, hipStream_t stream);

int launch_slot_mapping(int32_t block_size, const int32_t* block_tables, int32_t num_seqs,
                        int32_t max_blocks_per_seq, const int32_t* seq_ids,
                        const int32_t* positions, int32_t num_tokens, int64_t* slots,
                        hipStream_t stream);

int launch_append_kv(const pa_cache_desc_t* c, void* k_cache, void* v_cache, const void* k_new,
                     const void* v_new, const int32_t* block_tables, const int32_t* context_lens,
                     int32_t num_seqs, int32_t max_blocks_per_seq, int32_t len_clamp,
                     hipStream_t stream);

int launch_gather_kv(const pa_cache_desc_t* c, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, int32_t context_len, void* k_out, void* v_out,
                     hipStream_t stream);

}  // namespace pa
