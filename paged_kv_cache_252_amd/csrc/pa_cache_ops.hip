// Cache-side kernels: KV-write scatter, copy-on-write block copy, address
// translation (slot mapping) and the history gather used to test it.
//
// All of them move bits unchanged (no floating-point conversion), so a NaN
// payload or a signed zero arrives exactly as it left.  Every index read
// from device memory is range-checked before use; an out-of-range index
// skips the element (or yields slot -1), so a contract violation cannot
// reach outside the buffers.

#include "pa_internal.h"

namespace pa {
namespace {

// ---- write: [KG] "Follow One Token Address" read backwards -----------------
// One workgroup per (16 consecutive new tokens, KV head, 256-byte slab of the
// head's dims).  Tokens whose slots follow one another inside one aligned
// window of 16 positions of a tile (a prompt or a chunk written in order) form
// a segment, written by the workgroup that holds its first token, so a
// workgroup covers at most 31 tokens.  Their rows are staged in LDS with every
// load in flight at once (the slot loads and these are the only waits); then K
// goes out as 16-byte chunks of x consecutive dims, position-fastest (a
// segment's chunk is one contiguous run), and V as 16-byte runs of x
// consecutive positions of one dim row; a run only partly inside the segment
// is stored element by element.  A lone token (a decode step) is a segment of
// one.
template <typename E>
__global__ __launch_bounds__(256) void write_kv_kernel(E* __restrict__ k_cache,
                                                       E* __restrict__ v_cache,
                                                       const E* __restrict__ k_new,
                                                       const E* __restrict__ v_new,
                                                       const int64_t* __restrict__ slots,
                                                       int num_tokens, int64_t num_slots,
                                                       int64_t blk_stride, int block_size,
                                                       int head_dim) {
    constexpr int X = 16 / sizeof(E);
    constexpr int Q = 16 / X;                  // runs of X positions per 16-position window
    constexpr int SLAB = 256 / sizeof(E);      // most dims per workgroup
    constexpr int LD = SLAB + X;               // LDS row, padded by 16 bytes
    constexpr int ROWS = 32;
    __shared__ int64_t sl[33];                 // tokens t0 - 1 .. t0 + 31: slot (-1: none),
    __shared__ int64_t sb[33];                 // block,
    __shared__ int so[33];                     // offset in the block
    __shared__ int seg[16];                    // length of the segment starting at t0 + i, or 0
    __shared__ __align__(16) E ks[ROWS * LD];
    __shared__ __align__(16) E vs[ROWS * LD];
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int h = blockIdx.y;
    const int num_kv_heads = gridDim.y;
    const int se = head_dim < SLAB ? head_dim : SLAB;    // dims of this slab
    const int dof = blockIdx.z * se;                      // its first dim
    const int cs = se / X;                                // its 16-byte chunks per row
    const int tt = tile_tokens(block_size);
    const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * head_dim;
    const int64_t col0 = static_cast<int64_t>(h) * head_dim + dof;
    // The window's own rows t0 .. t0 + 15 go out now, beside the slot loads:
    // a chunk's slots are almost always its rows' (only rows of segments
    // that run past the window, t0 + 16 .. t0 + 30, wait for the slots).
    uint4 kp = {0u, 0u, 0u, 0u}, vp = {0u, 0u, 0u, 0u};
    const int pr = threadIdx.x / cs, pc = threadIdx.x - (threadIdx.x / cs) * cs;
    const bool pre = threadIdx.x < 16 * cs && t0 + pr < num_tokens;
    if (pre) {
        const int64_t src = (t0 + pr) * row_stride + col0 + pc * X;
        kp = *reinterpret_cast<const uint4*>(k_new + src);
        vp = *reinterpret_cast<const uint4*>(v_new + src);
    }
    for (int i = threadIdx.x; i < 33; i += blockDim.x) {
        const int64_t t = t0 - 1 + i;
        int64_t v = (t >= 0 && t < num_tokens) ? slots[t] : -1;
        v = (v >= 0 && v < num_slots) ? v : -1;
        const int64_t b = v >= 0 ? v / block_size : 0;
        sl[i] = v;
        sb[i] = b;
        so[i] = static_cast<int>(v - b * block_size);
    }
    __syncthreads();
    if (threadIdx.x < 16) {
        const int i = threadIdx.x;
        const int64_t s = sl[i + 1];
        const int p = so[i + 1] % tt;          // position inside the tile
        int k = 0;
        if (s >= 0 && !(p % 16 != 0 && sl[i] == s - 1)) {   // else: none, or a continuation
            k = 1;                             // up to the next window start: i + k <= 31
            while (p + k < tt && (p + k) % 16 != 0 && sl[i + 1 + k] == s + k) ++k;
        }
        seg[i] = k;
    }
    __syncthreads();
    int jmin = 16, jmax = 0;                   // rows t0 + jmin .. t0 + jmax - 1 are needed
    for (int i = 0; i < 16; ++i) {
        if (seg[i] == 0) continue;
        jmin = i < jmin ? i : jmin;
        jmax = i + seg[i] > jmax ? i + seg[i] : jmax;
    }
    if (jmin >= jmax) return;                  // uniform: nothing starts here
    // LDS row r holds token t0 + r: the prefetched rows, then rows 16 ..
    // jmax - 1 of segments that run past the window
    if (pre) {
        *reinterpret_cast<uint4*>(ks + pr * LD + pc * X) = kp;
        *reinterpret_cast<uint4*>(vs + pr * LD + pc * X) = vp;
    }
    const int extra = jmax > 16 ? (jmax - 16) * cs : 0;   // <= 15 * 16 < 256
    if (static_cast<int>(threadIdx.x) < extra) {
        const int r = 16 + static_cast<int>(threadIdx.x) / cs;
        const int c = static_cast<int>(threadIdx.x) - (static_cast<int>(threadIdx.x) / cs) * cs;
        const int64_t src = (t0 + r) * row_stride + col0 + c * X;
        *reinterpret_cast<uint4*>(ks + r * LD + c * X) = *reinterpret_cast<const uint4*>(k_new + src);
        *reinterpret_cast<uint4*>(vs + r * LD + c * X) = *reinterpret_cast<const uint4*>(v_new + src);
    }
    __syncthreads();
    const int64_t head_region = static_cast<int64_t>(head_dim) * block_size;
    const bool vec_ok = tt % X == 0;           // a dim row keeps 16-byte alignment
    for (int j = jmin; j < 16; ++j) {
        const int k = seg[j];
        if (k == 0) continue;
        const int o = so[j + 1];
        const int p = o % tt;
        const int i0 = p % 16;                 // the segment holds window positions [i0, i0 + k)
        const int w0 = p - i0;                 // the window's first position in the tile
        const int64_t base = sb[j + 1] * blk_stride + h * head_region +
                             static_cast<int64_t>(o - p) * head_dim;   // the tile
        const int r0 = j - i0;                 // LDS row of window position 0
        for (int idx = threadIdx.x; idx < 16 * cs; idx += blockDim.x) {
            const int i = idx & 15;
            const int c = idx >> 4;
            if (i < i0 || i >= i0 + k) continue;
            *reinterpret_cast<uint4*>(k_cache + base +
                                      (static_cast<int64_t>(dof / X + c) * tt + w0 + i) * X) =
                *reinterpret_cast<const uint4*>(ks + (r0 + i) * LD + c * X);
        }
        for (int idx = threadIdx.x; idx < Q * se; idx += blockDim.x) {
            const int q = idx % Q;
            const int dd = idx / Q;
            const int first = q * X;           // window positions first .. first + X - 1
            if (first + X <= i0 || first >= i0 + k) continue;
            E* dst = v_cache + base + static_cast<int64_t>(dof + dd) * tt + w0 + first;
            if (vec_ok && first >= i0 && first + X <= i0 + k) {
                E e[X];
#pragma unroll
                for (int x = 0; x < X; ++x) e[x] = vs[(r0 + first + x) * LD + dd];
                *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(e);
            } else {
                for (int x = 0; x < X; ++x) {
                    const int i = first + x;
                    if (i >= i0 && i < i0 + k) dst[x] = vs[(r0 + i) * LD + dd];
                }
            }
        }
    }
}

// ---- append: the same scatter for one token per request at position L-1, with
// the slot translated here from the request's table -----------------------------
template <typename E>
__global__ __launch_bounds__(256) void append_kv_kernel(E* __restrict__ k_cache,
                                                        E* __restrict__ v_cache,
                                                        const E* __restrict__ k_new,
                                                        const E* __restrict__ v_new,
                                                        const int32_t* __restrict__ block_tables,
                                                        const int32_t* __restrict__ context_lens,
                                                        int max_blocks_per_seq, int len_clamp,
                                                        int64_t num_blocks, int64_t blk_stride,
                                                        int block_size, int num_kv_heads,
                                                        int head_dim) {
    constexpr int X = 16 / sizeof(E);
    const int t = blockIdx.x;
    int L = context_lens[t];
    L = L > len_clamp ? len_clamp : L;
    if (L <= 0) return;
    const int lb = (L - 1) / block_size;
    const int o = (L - 1) - lb * block_size;
    const int phys = block_tables[static_cast<int64_t>(t) * max_blocks_per_seq + lb];
    if (phys < 0 || phys >= num_blocks) return;
    const int64_t b = phys;
    const int chunks = head_dim / X;
    const int64_t tile = static_cast<int64_t>(head_dim) * block_size;
    const int64_t row = static_cast<int64_t>(t) * num_kv_heads * head_dim;
    for (int i = threadIdx.x; i < num_kv_heads * chunks; i += blockDim.x) {
        const int h = i / chunks;
        const int c = i - h * chunks;
        const uint4 v = *reinterpret_cast<const uint4*>(k_new + row + h * head_dim + c * X);
        E* dst = k_cache + b * blk_stride + h * tile + k_elem(o, c * X, block_size, head_dim, X);
        *reinterpret_cast<uint4*>(dst) = v;
    }
    for (int i = threadIdx.x; i < num_kv_heads * head_dim; i += blockDim.x) {
        const int h = i / head_dim;
        const int d = i - h * head_dim;
        v_cache[b * blk_stride + h * tile + v_elem(o, d, block_size, head_dim)] = v_new[row + i];
    }
}

// ---- copy: [ZQ] answer, [KG] "Shared Blocks Must Not Be Changed in Place" --
// grid.x is the pair, grid.y covers one block's bytes in 4 KiB pieces (256
// lanes x 16 bytes); K and V are copied by the same lanes.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          const int64_t* __restrict__ pairs,
                                                          int64_t num_blocks,
                                                          int64_t vecs_per_block,
                                                          int64_t vecs_stride) {
    const int64_t src = pairs[2 * static_cast<int64_t>(blockIdx.x)];
    const int64_t dst = pairs[2 * static_cast<int64_t>(blockIdx.x) + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    const int64_t i = static_cast<int64_t>(blockIdx.y) * blockDim.x + threadIdx.x;
    if (i >= vecs_per_block) return;
    const uint4 kv = k_cache[src * vecs_stride + i];
    const uint4 vv = v_cache[src * vecs_stride + i];
    k_cache[dst * vecs_stride + i] = kv;
    v_cache[dst * vecs_stride + i] = vv;
}

// ---- copy-on-write of each request's last block from cow_src[i] ---------------
// The decode step's copies given per request: request i's block holding
// position L-1 (its table entry) receives a copy of block cow_src[i]
// (skipped when negative).  grid.x is the request, grid.y as copy_blocks.
__global__ __launch_bounds__(256) void cow_last_block_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, const int32_t* __restrict__ cow_src,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int max_blocks_per_seq, int len_clamp, int block_size, int64_t num_blocks,
    int64_t vecs_per_block, int64_t vecs_stride) {
    const int seq = blockIdx.x;
    const int64_t src = cow_src[seq];
    int L = context_lens[seq];
    L = L > len_clamp ? len_clamp : L;
    if (src < 0 || src >= num_blocks || L <= 0) return;
    const int64_t dst = block_tables[static_cast<int64_t>(seq) * max_blocks_per_seq + (L - 1) / block_size];
    if (dst < 0 || dst >= num_blocks) return;
    const int64_t i = static_cast<int64_t>(blockIdx.y) * blockDim.x + threadIdx.x;
    if (i >= vecs_per_block) return;
    const uint4 kv = k_cache[src * vecs_stride + i];
    const uint4 vv = v_cache[src * vecs_stride + i];
    k_cache[dst * vecs_stride + i] = kv;
    v_cache[dst * vecs_stride + i] = vv;
}

// ---- translate: [KG] "Follow One Token Address" ----------------------------
__global__ __launch_bounds__(256) void slot_mapping_kernel(
    int block_size, const int32_t* __restrict__ block_tables, int num_seqs,
    int max_blocks_per_seq, const int32_t* __restrict__ seq_ids,
    const int32_t* __restrict__ positions, int num_tokens, int64_t* __restrict__ slots) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= num_tokens) return;
    const int s = seq_ids ? seq_ids[t] : t;
    const int p = positions[t];
    int64_t slot = -1;
    if (p >= 0 && s >= 0 && s < num_seqs) {
        const int logical = p / block_size;
        if (logical < max_blocks_per_seq) {
            const int phys = block_tables[static_cast<int64_t>(s) * max_blocks_per_seq + logical];
            if (phys >= 0) slot = static_cast<int64_t>(phys) * block_size + (p - logical * block_size);
        }
    }
    slots[t] = slot;
}

// ---- gather: [KG] "Batching Becomes More Flexible" -------------------------
// One thread per (token, head, dim) element of the contiguous output.
template <typename E>
__global__ __launch_bounds__(256) void gather_kv_kernel(const E* __restrict__ k_cache,
                                                        const E* __restrict__ v_cache,
                                                        const int32_t* __restrict__ table,
                                                        int64_t num_blocks, int64_t blk_stride,
                                                        int block_size, int num_kv_heads,
                                                        int head_dim,
                                                        int64_t total, E* __restrict__ k_out,
                                                        E* __restrict__ v_out) {
    constexpr int X = 16 / sizeof(E);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int d = static_cast<int>(i % head_dim);
    const int64_t th = i / head_dim;
    const int h = static_cast<int>(th % num_kv_heads);
    const int t = static_cast<int>(th / num_kv_heads);
    const int lb = t / block_size;
    const int o = t - lb * block_size;
    int phys = table[lb];
    if (phys < 0 || phys >= num_blocks) phys = 0;
    const int64_t tile = static_cast<int64_t>(phys) * blk_stride + static_cast<int64_t>(h) * head_dim * block_size;
    k_out[i] = k_cache[tile + k_elem(o, d, block_size, head_dim, X)];
    v_out[i] = v_cache[tile + v_elem(o, d, block_size, head_dim)];
}

}  // namespace

int launch_write_kv(const pa_cache_desc_t* c, void* k_cache, void* v_cache, const void* k_new,
                    const void* v_new, const int64_t* slots, int32_t num_tokens,
                    hipStream_t stream) {
    if (num_tokens == 0) return PA_OK;
    const int64_t num_slots = c->num_blocks * c->block_size;
    const int slab = 256 / elem_bytes(c->dtype);
    const dim3 grid((num_tokens + 15) / 16, c->num_kv_heads,
                    c->head_dim > slab ? c->head_dim / slab : 1);
    if (c->dtype == PA_BF16) {
        hipLaunchKernelGGL(write_kv_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                           static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                           slots, num_tokens, num_slots, block_stride(c), c->block_size,
                           c->head_dim);
    } else {
        hipLaunchKernelGGL(write_kv_kernel<uint32_t>, grid, dim3(256), 0, stream,
                           static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache),
                           static_cast<const uint32_t*>(k_new), static_cast<const uint32_t*>(v_new),
                           slots, num_tokens, num_slots, block_stride(c), c->block_size,
                           c->head_dim);
    }
    return check_launch("write_kv");
}

int launch_append_kv(const pa_cache_desc_t* c, void* k_cache, void* v_cache, const void* k_new,
                     const void* v_new, const int32_t* block_tables, const int32_t* context_lens,
                     int32_t num_seqs, int32_t max_blocks_per_seq, int32_t len_clamp,
                     hipStream_t stream) {
    if (num_seqs == 0) return PA_OK;
    if (c->dtype == PA_BF16) {
        hipLaunchKernelGGL(append_kv_kernel<uint16_t>, dim3(num_seqs), dim3(256), 0, stream,
                           static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                           static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                           block_tables, context_lens, max_blocks_per_seq, len_clamp, c->num_blocks,
                           block_stride(c), c->block_size, c->num_kv_heads, c->head_dim);
    } else {
        hipLaunchKernelGGL(append_kv_kernel<uint32_t>, dim3(num_seqs), dim3(256), 0, stream,
                           static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache),
                           static_cast<const uint32_t*>(k_new), static_cast<const uint32_t*>(v_new),
                           block_tables, context_lens, max_blocks_per_seq, len_clamp, c->num_blocks,
                           block_stride(c), c->block_size, c->num_kv_heads, c->head_dim);
    }
    return check_launch("append_kv");
}

int launch_copy_blocks(const pa_cache_desc_t* c, void* k_cache, void* v_cache,
                       const int64_t* pairs, int32_t num_pairs, hipStream_t stream) {
    if (num_pairs == 0) return PA_OK;
    const int64_t vecs = block_elems(c) * elem_bytes(c->dtype) / 16;
    const int64_t vstride = block_stride(c) * elem_bytes(c->dtype) / 16;
    const int64_t gy = (vecs + 255) / 256;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, static_cast<unsigned>(gy)), dim3(256),
                       0, stream, static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache),
                       pairs, c->num_blocks, vecs, vstride);
    return check_launch("copy_blocks");
}

int launch_cow_last_block(const pa_cache_desc_t* c, void* k_cache, void* v_cache,
                          const int32_t* cow_src, const int32_t* block_tables,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t max_blocks_per_seq, int32_t len_clamp, hipStream_t stream) {
    if (num_seqs == 0) return PA_OK;
    const int64_t vecs = block_elems(c) * elem_bytes(c->dtype) / 16;
    const int64_t vstride = block_stride(c) * elem_bytes(c->dtype) / 16;
    const int64_t gy = (vecs + 255) / 256;
    hipLaunchKernelGGL(cow_last_block_kernel, dim3(num_seqs, static_cast<unsigned>(gy)), dim3(256),
                       0, stream, static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache),
                       cow_src, block_tables, context_lens, max_blocks_per_seq, len_clamp,
                       c->block_size, c->num_blocks, vecs, vstride);
    return check_launch("copy-on-write of last blocks");
}

int launch_slot_mapping(int32_t block_size, const int32_t* block_tables, int32_t num_seqs,
                        int32_t max_blocks_per_seq, const int32_t* seq_ids,
                        const int32_t* positions, int32_t num_tokens, int64_t* slots,
                        hipStream_t stream) {
    if (num_tokens == 0) return PA_OK;
    hipLaunchKernelGGL(slot_mapping_kernel, dim3((num_tokens + 255) / 256), dim3(256), 0, stream,
                       block_size, block_tables, num_seqs, max_blocks_per_seq, seq_ids, positions,
                       num_tokens, slots);
    return check_launch("slot_mapping");
}

int launch_gather_kv(const pa_cache_desc_t* c, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, int32_t context_len, void* k_out, void* v_out,
                     hipStream_t stream) {
    if (context_len == 0) return PA_OK;
    const int64_t total = static_cast<int64_t>(context_len) * c->num_kv_heads * c->head_dim;
    const unsigned grid = static_cast<unsigned>((total + 255) / 256);
    if (c->dtype == PA_BF16) {
        hipLaunchKernelGGL(gather_kv_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
                           block_table, c->num_blocks, block_stride(c), c->block_size,
                           c->num_kv_heads, c->head_dim,
                           total, static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
    } else {
        hipLaunchKernelGGL(gather_kv_kernel<uint32_t>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const uint32_t*>(k_cache), static_cast<const uint32_t*>(v_cache),
                           block_table, c->num_blocks, block_stride(c), c->block_size,
                           c->num_kv_heads, c->head_dim,
                           total, static_cast<uint32_t*>(k_out), static_cast<uint32_t*>(v_out));
    }
    return check_launch("gather_kv");
}

}  // namespace pa
