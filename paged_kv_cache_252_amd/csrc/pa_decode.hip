// Decode attention over a paged KV cache, gfx950.
//
// Attention of one query per request over its history, found through the
// request's block table: logical block = position / block_size, offset =
// position % block_size, physical block = table[logical block]
// ([KG] kgptalkie "Day 28: PagedAttention", "Follow One Token Address";
// "The Block Table Is the Map").  The arithmetic is organised the way
// FlashAttention-style kernels do it (running max and sum, one pass over
// the keys), which the same page's closing section says combines with
// paged storage; long histories are split into partitions whose partial
// states are merged by a second, fixed-order reduction.
//
// Fast path (bf16, head_dim D = 64, 128 or 256, block_size 8, 16, 32 or 64,
// up to 16 query heads per KV head): one 64-lane wave per (request, KV head,
// partition).  Per tile of 16 tokens (written for D 128; the counts scale
// with D):
//   * K tile (4 KiB) -> 4 x 16-byte loads per lane, each wave-wide load a
//     contiguous 1 KiB, straight into the A operand of
//     v_mfma_f32_16x16x32_bf16 (16 tokens x 32 dims) against the query
//     group as B operand (dims x 16 query rows, rows >= group are zero).
//     Output lane l holds scores of tokens 4*(l/16)+i for query row l%16.
//   * Online softmax on those scores in the log2 domain; the row maximum
//     is shared by the four lanes of a query row with two lane exchanges.
//   * V tile (4 KiB, stored dim-major) -> 8 x 8-byte loads per lane into
//     the A operand of v_mfma_f32_16x16x16_bf16 (16 dims x 16 tokens);
//     the probabilities, rounded to bf16, are the B operand exactly where
//     the score MFMA left them, so no lane shuffles are needed.
//   * The output accumulator (128 dims x 16 rows, fp32) stays in 32 VGPRs;
//     lane l holds dims 16*j + 4*(l/16) + i of query row l%16.
// Tokens at or past the context length are removed by selecting -inf for
// their scores and zero for their values (never by multiplying by zero, so
// stale NaN bytes in a block's tail cannot leak).
//
// Shared blocks (same tile consumer, same bits): the grouped path serves up
// to 16/g consecutive requests per wave and loads a block they all name once;
// the prefix-runs path decodes a partition that a whole chunk of requests
// shares once for the chunk, four waves reading each tile through LDS.
//
// Generic path (fp32 or bf16, other head_dim / block_size): one wave per
// (request, query head, partition), one token per step, lanes over dims.
#include "pa_tile.h"

namespace pa {
namespace {

#ifndef PA_FAST_NBUF
#define PA_FAST_NBUF 2           // tiles in the load ring of the fast path
#endif
#ifndef PA_FAST_NBUF_D64
#define PA_FAST_NBUF_D64 3       // ... at head_dim 64, whose tiles are half as large
#endif

constexpr int kMaxWgParts = 8;   // partitions merged inside one workgroup
constexpr size_t kMaxWgLds = 32768;

// Load-ring depth of the fast path at head_dim d.
constexpr int fast_nbuf(int d) { return d <= 64 ? PA_FAST_NBUF_D64 : PA_FAST_NBUF; }

// Waves of a workgroup-merge workgroup of the fast path at head_dim d with
// elements of esize bytes: with tiles twice those of bf16 at 128 (bf16 at 256,
// fp32 at 128) a wave needs more than the 256 registers each of eight waves
// may have, so those workgroups take at most four.
constexpr int fast_wg_parts(int d, int esize = 2) { return d * esize > FD * 2 ? 4 : kMaxWgParts; }

// ============================================================================
// Fast path
// ============================================================================

// The arguments of one decode launch on the fast path (element type E).
template <typename E>
struct FastArgsT {
    const E* __restrict__ k_cache;
    const E* __restrict__ v_cache;
    const E* __restrict__ q;
    const int32_t* __restrict__ block_tables;
    const int32_t* __restrict__ context_lens;
    int64_t num_blocks, blk_stride;
    int num_q_heads, group, max_blocks_per_seq, len_clamp, part_tokens, max_parts;
    float scale_log2;
    E* __restrict__ out;
    float* __restrict__ ws_acc;
    float* __restrict__ ws_m;
    float* __restrict__ ws_l;
    const E* __restrict__ k_new;
    const E* __restrict__ v_new;
    int num_kv_heads;
    const int32_t* __restrict__ cow_src;
    int append_tiles;   // the appended token's tile is written back whole (blocks of 16 or more)
};
using FastArgs = FastArgsT<__bf16>;

// Four consecutive output elements: bf16 (rounded to nearest even) or fp32.
template <typename E> struct Out4T;
template <> struct Out4T<__bf16> { using T = uint2; };
template <> struct Out4T<float> { using T = f32x4; };
template <typename E>
__device__ __forceinline__ typename Out4T<E>::T out4(const f32x4 v, const float inv) {
    if constexpr (std::is_same<E, float>::value) {
        return f32x4{v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
    } else {
        return make_uint2(pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv));
    }
}
template <typename E>
__device__ __forceinline__ typename Out4T<E>::T out4_zero() {
    if constexpr (std::is_same<E, float>::value) return f32x4{0.f, 0.f, 0.f, 0.f};
    else return make_uint2(0u, 0u);
}

// Merge of the partitions 0..nparts-1 of one query row whose partial states
// sit in LDS at base + p * pstride (acc[D], then m and l), with the merge
// kernel's formula: global maximum first, then fused multiply-adds in
// partition order, one division.  Lane quad writes dims D/4*quad..+D/4-1 of
// the output row o.
template <int D, typename E = __bf16>
__device__ __forceinline__ void merge_lds_row(const float* base, int pstride, int nparts, int quad,
                                              typename Out4T<E>::T* o) {
    constexpr int K = D / 16;                    // float4 chunks per lane
    float M = base[D];
    for (int p = 1; p < nparts; ++p) M = fmaxf(M, base[p * pstride + D]);
    float den = 0.f;
    f32x4 num[K];
#pragma unroll
    for (int k = 0; k < K; ++k) num[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < nparts; ++p) {
        const float* src = base + p * pstride;
        const float w = fast_exp2(src[D] - M);
#pragma unroll
        for (int k = 0; k < K; ++k)
            num[k] = fma4(*reinterpret_cast<const f32x4*>(src + (D / 4) * quad + 4 * k), w, num[k]);
        den = __builtin_fmaf(src[D + 1], w, den);
    }
    const float inv = 1.f / den;
    typename Out4T<E>::T* ob = o + K * quad;
#pragma unroll
    for (int k = 0; k < K; ++k) ob[k] = out4<E>(num[k], inv);
}

// One wave's item of the fast path: partition `part` of request `seq` for KV
// head h (the grid and the flags are described at decode_fast_kernel); head_dim
// D, element type E (bf16, or fp32 through the fp32 MFMAs).
template <int NBUF, bool NT, bool APPEND, bool WGM, int BS, int D, typename E = __bf16>
__device__ __forceinline__ void fast_item(const FastArgsT<E>& a, const int h, const int seq, const int part) {
    using KChunk = typename ElemT<E>::KChunk;         // 16 bytes of a K row (and of q)
    using VElem = std::conditional_t<std::is_same<E, float>::value, float, short>;
    using O4 = typename Out4T<E>::T;
    constexpr int KC = TileT<D, E>::KC;               // K chunks (and q chunks) per lane
    constexpr int VJ = D / 16;                        // V operands / accumulator chunks per lane
    const E* __restrict__ k_cache = a.k_cache;
    const E* __restrict__ v_cache = a.v_cache;
    const E* __restrict__ q = a.q;
    const int32_t* __restrict__ block_tables = a.block_tables;
    const int32_t* __restrict__ context_lens = a.context_lens;
    const int64_t num_blocks = a.num_blocks, blk_stride = a.blk_stride;
    const int num_q_heads = a.num_q_heads, group = a.group, max_blocks_per_seq = a.max_blocks_per_seq;
    const int len_clamp = a.len_clamp, part_tokens = a.part_tokens, max_parts = a.max_parts;
    const float scale_log2 = a.scale_log2;
    E* __restrict__ out = a.out;
    float* __restrict__ ws_acc = a.ws_acc;
    float* __restrict__ ws_m = a.ws_m;
    float* __restrict__ ws_l = a.ws_l;
    const E* __restrict__ k_new = a.k_new;
    const E* __restrict__ v_new = a.v_new;
    const int num_kv_heads = a.num_kv_heads;
    const int32_t* __restrict__ cow_src = a.cow_src;
    const int lane = threadIdx.x & 63;
    const int row = lane & 15;
    const int quad = lane >> 4;

    int L = context_lens[seq];
    L = L < 0 ? 0 : (L > len_clamp ? len_clamp : L);
    const int tok0 = part * part_tokens;
    const int hq = h * group + row;
    const bool row_ok = row < group;
    auto out_row = [&]() {
        return reinterpret_cast<O4*>(out + (static_cast<int64_t>(seq) * num_q_heads + hq) * D);
    };

    if (!WGM && tok0 >= L) {
        if (L == 0 && part == 0 && row_ok) {   // empty history: zero output
            O4* o = out_row();
#pragma unroll
            for (int j = 0; j < VJ; ++j) o[4 * j + quad] = out4_zero<E>();
        }
        return;
    }
    const bool active = tok0 < L;
    const int tok1 = min(L, tok0 + part_tokens);
    const int nparts = (L + part_tokens - 1) / part_tokens;
    // tiles of 16 tokens; table entries (blocks of BS tokens), one per lane
    const int nblk = (tok1 - tok0 + FBS - 1) / FBS;
    const int last_valid = tok1 - (tok0 + (nblk - 1) * FBS);
    const int blk0 = tok0 / BS;
    const int nent = (tok1 - tok0 + BS - 1) / BS;     // 1..64
    constexpr int HT = BS * D;                        // elements of one (block, head) region

    SoftmaxStateT<D> st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int j = 0; j < VJ; ++j) st.acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;

    if (active) {
    // Block-table entries of this partition: one per lane, read back with readlane.
    int my_phys = 0;
    if (lane < nent)
        my_phys = clamp_block(block_tables[static_cast<int64_t>(seq) * max_blocks_per_seq + blk0 + lane],
                              num_blocks);

    // Appending: the last partition holds position L-1 at offset o of its
    // last block.  The four lanes of row o hold that token's D/8 key chunks
    // (the same chunk order as the K tile); the 16 lanes of quad o/4 hold its
    // D value dims (dim 16*j + row).  They also store them to the cache.
    const bool append_here = APPEND && part == nparts - 1;
    const int o_new = (L - 1) % FBS;                  // slot within the last tile
    const int ob_new = (L - 1) % BS;                  // slot within the last block
    KChunk fk[KC];
    VElem fv[VJ];
    // append_tiles (blocks of 16 or more): the tile that receives the token
    // is written back whole from registers once it is loaded (full lines),
    // instead of the token's 16-byte K chunks and 2-byte V elements being
    // stored at once, which land in partial sectors.  (wave-uniform)
    const bool whole_tile = BS >= 16 && a.append_tiles != 0;
    // Copy-on-write folded in (blocks of 16): the last block is read from
    // cow_src[seq] and written back whole, new token included, to the
    // request's own block, so the token needs no store of its own.
    int cow_phys = -1;
    if constexpr (APPEND && BS == 16) {
        if (append_here && cow_src != nullptr) {
            const int cs = cow_src[seq];
            if (cs >= 0 && static_cast<int64_t>(cs) < num_blocks) cow_phys = cs;
        }
    }
    if constexpr (APPEND) {
        if (append_here) {
            const int64_t nrow = (static_cast<int64_t>(seq) * num_kv_heads + h) * D;
            const KChunk* kn = reinterpret_cast<const KChunk*>(k_new + nrow);
            const VElem* vn = reinterpret_cast<const VElem*>(v_new + nrow);
#pragma unroll
            for (int s4 = 0; s4 < KC; ++s4) fk[s4] = kn[4 * s4 + quad];
#pragma unroll
            for (int j = 0; j < VJ; ++j) fv[j] = vn[16 * j + row];
            const int64_t toff = static_cast<int64_t>(__builtin_amdgcn_readlane(my_phys, nent - 1)) *
                                     blk_stride + static_cast<int64_t>(h) * HT;
            // the slot's tile inside the block, and its position in that tile
            constexpr int TT = BS >= 16 ? 16 : BS;
            const int64_t tile_base = toff + static_cast<int64_t>(ob_new / TT) * TT * D;
            const int pt = ob_new % TT;
            if (!whole_tile && cow_phys < 0 && row == o_new) {
                KChunk* kd = reinterpret_cast<KChunk*>(const_cast<E*>(k_cache) + tile_base);
#pragma unroll
                for (int s4 = 0; s4 < KC; ++s4) kd[(4 * s4 + quad) * TT + pt] = fk[s4];
            }
            if (!whole_tile && cow_phys < 0 && quad == o_new / 4) {
                VElem* vd = reinterpret_cast<VElem*>(const_cast<E*>(v_cache) + tile_base);
#pragma unroll
                for (int j = 0; j < VJ; ++j) vd[(16 * j + row) * TT + pt] = fv[j];
            }
        }
    }

    // Query rows of this KV head as the B operand (rows >= group are zero).
    KChunk qv[KC];
    {
        const KChunk* qp = reinterpret_cast<const KChunk*>(
            q + (static_cast<int64_t>(seq) * num_q_heads + (row_ok ? hq : 0)) * D);
#pragma unroll
        for (int s = 0; s < KC; ++s) {
            KChunk v = qp[4 * s + quad];
            qv[s] = row_ok ? v : KChunk{};
        }
    }

    const E* k_head = k_cache + static_cast<int64_t>(h) * HT;
    const E* v_head = v_cache + static_cast<int64_t>(h) * HT;

    // A ring of NBUF tiles: while block j is consumed, blocks j+1 .. j+NBUF-1
    // are in flight.  Loads are unconditional (past the end they repeat the
    // last block, which is then still in cache), so every path through the
    // loop has the same loads outstanding and the waits stay exact.  The
    // scheduling barriers keep each tile's loads issued ahead of the previous
    // tile's arithmetic; without them the compiler sinks loads next to their
    // first use and every block waits a full memory latency.
    TileT<D, E> buf[NBUF];
    auto entry_off = [&](int e) {
        return static_cast<int64_t>(__builtin_amdgcn_readlane(my_phys, e < nent ? e : nent - 1)) * blk_stride;
    };
    auto load_t = [&](TileT<D, E>& t, int jj) {   // tile jj (clamped to the last)
        const int jc = jj < nblk ? jj : nblk - 1;
        if constexpr (BS >= 16) {
            const int64_t o = (BS == 16 && cow_phys >= 0 && jc == nblk - 1)
                                  ? static_cast<int64_t>(cow_phys) * blk_stride
                                  : entry_off(jc / (BS / 16));
            load_tile_bs<NT, BS, D, E>(t, k_head + o, v_head + o, nullptr, nullptr, jc % (BS / 16), lane);
        } else {
            const int64_t oa = entry_off(2 * jc), ob = entry_off(2 * jc + 1);
            load_tile_bs<NT, BS, D, E>(t, k_head + oa, v_head + oa, k_head + ob, v_head + ob, 0, lane);
        }
    };
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u) load_t(buf[u], u);
    for (int j0 = 0; j0 < nblk; j0 += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
            const int j = j0 + u;
            load_t(buf[(u + NBUF - 1) % NBUF], j + NBUF - 1);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (APPEND) {
                if (append_here && j == nblk - 1) {
#pragma unroll
                    for (int s4 = 0; s4 < KC; ++s4)
                        if (row == o_new) buf[u].k[s4] = fk[s4];
#pragma unroll
                    for (int jj = 0; jj < VJ; ++jj)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (quad * 4 + e == o_new) buf[u].v[jj][e] = fv[jj];
                    if (cow_phys >= 0) {                  // the copy, with the token in it
                        const int64_t o = entry_off(nent - 1);
                        store_tile(buf[u], const_cast<E*>(k_head) + o, const_cast<E*>(v_head) + o, lane);
                    } else if (BS >= 16 && whole_tile) {   // the tile back, with the token in it
                        constexpr int SUB = BS >= 16 ? BS / 16 : 1;   // tiles per block
                        const int64_t o = entry_off(j / SUB) + static_cast<int64_t>(j % SUB) * (D * FBS);
                        store_tile(buf[u], const_cast<E*>(k_head) + o, const_cast<E*>(v_head) + o, lane);
                    }
                }
            }
            if (j < nblk)
                consume_tile(st, buf[u], qv, scale_log2, lane, j == nblk - 1 ? last_valid : FBS);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // The four lanes of a query row each summed a quarter of the tokens.
    lsum = sum_across_rows(st.l);
    }   // active

    if constexpr (WGM) {
        // LDS: [partition][row < group][acc D | m | l | pad 2]
        extern __shared__ float wg_part[];
        constexpr int RS = D + 4;
        if (active && nparts > 1 && row_ok) {
            float* dst = wg_part + (part * group + row) * RS;
#pragma unroll
            for (int jj = 0; jj < VJ; ++jj) *reinterpret_cast<f32x4*>(dst + 16 * jj + 4 * quad) = st.acc[jj];
            if (quad == 0) {
                dst[D] = st.m;
                dst[D + 1] = lsum;
            }
        }
        __syncthreads();
        if (part != 0 || !row_ok) return;
        O4* o = out_row();
        if (L == 0) {                          // empty history: zero output
#pragma unroll
            for (int j = 0; j < VJ; ++j) o[4 * j + quad] = out4_zero<E>();
            return;
        }
        if (nparts > 1) {
            // merge partitions 0..nparts-1 in order (the merge kernel's formula:
            // global max first, then fused multiply-adds in partition order);
            // lane: row, dims 32*quad..+31
            merge_lds_row<D, E>(wg_part + row * RS, group * RS, nparts, quad, o);
            return;
        }
        // a single partition: wave 0 holds the whole result (falls through)
    }

    if (nparts == 1) {
        if (!row_ok) return;
        const float inv = 1.f / lsum;
        O4* o = out_row();
#pragma unroll
        for (int jj = 0; jj < VJ; ++jj) o[4 * jj + quad] = out4<E>(st.acc[jj], inv);
        return;
    }

    if (!row_ok) return;
    const int64_t pidx = (static_cast<int64_t>(seq) * num_q_heads + hq) * max_parts + part;
    f32x4* acc_out = reinterpret_cast<f32x4*>(ws_acc + pidx * D);
#pragma unroll
    for (int jj = 0; jj < VJ; ++jj) acc_out[4 * jj + quad] = st.acc[jj];
    if (quad == 0) {
        ws_m[pidx] = st.m;
        ws_l[pidx] = lsum;
    }
}

// APPEND: the call also appends each request's newest token (position L-1):
// the wave of the request's last partition stores k_new/v_new into the cache
// and uses them in place of whatever its load of that slot returned.
// WGM: the partitions of one (request, KV head) are the waves of one
// workgroup (wave w = partition w, at most fast_wg_parts(D, sizeof(E)) of them) and are
// merged through LDS after a workgroup barrier, instead of by the merge
// kernel.  Waves without a partition wait at the barrier.
//
// PERSIST (with at most 64 requests): the grid is (KV head, Z) and wave z of
// a head takes items z, z + Z, z + 2Z, ... of the list of (request,
// partition) pairs of all requests, request-major, built from the lengths in
// the wave.  The host sizes Z so that every wave of the grid is resident at
// once: with more items than that, a one-wave-per-item grid would leave its
// last items running as a tail on a mostly idle device.  Each item is
// computed exactly as in the plain grid, so the bits are the same.
//
// The bf16 block-16 workgroup-merge kernels at head_dim 64 and 128 are held
// to three waves per SIMD (at most 168 VGPRs), which the append variant with
// its tile write-back would otherwise exceed by two registers.
//
// E = float: the same kernel on fp32 caches, with the fp32 MFMA (K 4) for
// scores and values; the probabilities stay fp32.
template <int NBUF, bool NT, bool APPEND, bool WGM, int BS, bool PERSIST, int D, typename E>
__global__ __launch_bounds__(WGM ? 64 * fast_wg_parts(D, sizeof(E)) : 64)
__attribute__((amdgpu_waves_per_eu((std::is_same<E, __bf16>::value && WGM && BS == 16 && D <= 128) ? 3 : 1)))
void decode_fast_kernel(
    const E* __restrict__ k_cache, const E* __restrict__ v_cache,
    const E* __restrict__ q, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int64_t num_blocks, int64_t blk_stride,
    int num_q_heads, int group, int max_blocks_per_seq, int len_clamp, int part_tokens,
    int max_parts, float scale_log2, E* __restrict__ out, float* __restrict__ ws_acc,
    float* __restrict__ ws_m, float* __restrict__ ws_l, const E* __restrict__ k_new,
    const E* __restrict__ v_new, int num_kv_heads, const int32_t* __restrict__ cow_src,
    int num_seqs, int append_tiles) {
    // Grid (Hkv, S, partitions) with the KV head fastest: workgroups are
    // dealt to the XCDs round-robin, so each XCD sees every partition index
    // and the same heads for all requests (a shared prefix's head slice then
    // stays in one XCD's L2).
    const int h = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int row = lane & 15;
    const int quad = lane >> 4;

  // one (request, partition) item
  const FastArgsT<E> fa{k_cache, v_cache, q, block_tables, context_lens, num_blocks, blk_stride,
                        num_q_heads, group, max_blocks_per_seq, len_clamp, part_tokens, max_parts,
                        scale_log2, out, ws_acc, ws_m, ws_l, k_new, v_new, num_kv_heads, cow_src,
                        append_tiles};
  auto body = [&](const int seq, const int part) {
      fast_item<NBUF, NT, APPEND, WGM, BS, D, E>(fa, h, seq, part);
  };

    if constexpr (PERSIST) {
        static_assert(!WGM, "persistent waves merge through the merge kernel");
        int np = 0;                                  // lane i: request i's partitions
        if (lane < num_seqs) {
            int Li = context_lens[lane];
            Li = Li < 0 ? 0 : (Li > len_clamp ? len_clamp : Li);
            np = (Li + part_tokens - 1) / part_tokens;
        }
        int incl = np;                               // inclusive prefix sum over lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off);
            if (lane >= off) incl += v;
        }
        const int total = __builtin_amdgcn_readlane(incl, 63);
        for (int it = static_cast<int>(blockIdx.y); it < total; it += static_cast<int>(gridDim.y)) {
            const int seq = static_cast<int>(__builtin_ctzll(__ballot(lane < num_seqs && incl > it)));
            body(seq, it - (__builtin_amdgcn_readlane(incl, seq) - __builtin_amdgcn_readlane(np, seq)));
        }
        if (blockIdx.y == 0) {                       // empty histories: zero output
            uint64_t zm = __ballot(lane < num_seqs && np == 0);
            while (zm != 0) {
                const int seq = static_cast<int>(__builtin_ctzll(zm));
                zm &= zm - 1;
                if (row < group) {
                    auto* o = reinterpret_cast<typename Out4T<E>::T*>(
                        out + (static_cast<int64_t>(seq) * num_q_heads + h * group + row) * D);
#pragma unroll
                    for (int j = 0; j < D / 16; ++j) o[4 * j + quad] = out4_zero<E>();
                }
            }
        }
    } else {
        body(static_cast<int>(blockIdx.y), WGM ? static_cast<int>(threadIdx.x >> 6) : static_cast<int>(blockIdx.z));
    }
}

// ============================================================================
// Grouped path: several requests per wave, shared blocks read once
// ============================================================================
//
// The score MFMA has 16 query rows but a KV head has only g query heads, so
// the fast path leaves 16 - g rows empty.  Here the rows hold up to
// R = 16 / g consecutive requests (row = member * g + head in group).  For
// each block position of the partition, if every member that has tokens in
// that block names the same physical block with the same number of visible
// tokens (a shared prefix, [ZQ] answer; [KG] "Prefix Sharing Is a Natural
// Extension"), the tile is loaded once and scored against all members'
// queries together.  Otherwise each member's tile is processed on its own
// with the other members' rows masked out.  Rows keep separate online-softmax
// states, so the arithmetic per row is the same as one request per wave; only
// the partition's tile sequence differs.

// A task is one tile to consume: block position j of the partition, for all
// members (r = kShared) or for member r alone.
constexpr int kShared = -1;

// APPEND: as on the fast path, each member's newest token (position L-1) is
// stored by the wave that handles the member's last block and substituted
// into that tile; the token is staged in LDS because one wave may append for
// several members.
// WGM (at most three partitions): the partitions of a group are the waves of
// one workgroup per member slot (z = r_wave).  After each wave has decided
// its partition's mode, the waves compare: if every partition with tokens took
// the same mode, the workgroup that serves a row holds all of that row's
// partitions, merges them in LDS with the merge kernel's formula and stores
// -1 as the row's partition-0 l in the workspace; the merge kernel launched
// after it skips rows marked so.  Otherwise every wave writes its partials
// and the merge kernel merges them, as without WGM.  Same bits either way.
template <int MAXR, bool NT, bool APPEND, bool WGM>
__global__ __launch_bounds__(WGM ? 64 * kMaxWgParts : 64) void decode_grouped_kernel(
    const __bf16* __restrict__ k_cache, const __bf16* __restrict__ v_cache,
    const __bf16* __restrict__ q, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int64_t num_blocks, int64_t blk_stride,
    int num_seqs, int num_q_heads, int group, int members, int max_blocks_per_seq,
    int len_clamp, int part_tokens, int max_parts, float scale_log2, __bf16* __restrict__ out,
    float* __restrict__ ws_acc, float* __restrict__ ws_m, float* __restrict__ ws_l,
    const __bf16* __restrict__ k_new, const __bf16* __restrict__ v_new, int num_kv_heads,
    const int32_t* __restrict__ cow_src) {
    const int h = blockIdx.x;
    const int grp = blockIdx.y;
    // z = r_wave * max_parts + part: the waves that do the work of grouped
    // partitions (r_wave 0) are dispatched before the ones that only work in
    // per-member partitions and otherwise exit at once.  WGM: z = r_wave and
    // the partitions are the waves of the workgroup.
    const int r_wave = WGM ? static_cast<int>(blockIdx.z)
                           : static_cast<int>(blockIdx.z) / max_parts;   // member in per-member mode
    const int part = WGM ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6))
                         : static_cast<int>(blockIdx.z) - r_wave * max_parts;
    const int lane = WGM ? static_cast<int>(threadIdx.x & 63) : static_cast<int>(threadIdx.x);
    const int row = lane & 15;
    const int quad = lane >> 4;

    const int seq0 = grp * members;
    const int nmem = min(members, num_seqs - seq0);
    const int my_mem = row / group;
    const bool row_ok = my_mem < nmem;
    const int my_seq = seq0 + (row_ok ? my_mem : 0);
    const int hq = h * group + row % group;
    auto clampL = [&](int L) { return L < 0 ? 0 : (L > len_clamp ? len_clamp : L); };

    // Lane r < nmem holds member r's length; each lane also holds its row's.
    const int Lr = lane < nmem ? clampL(context_lens[seq0 + lane]) : 0;
    const int my_L = row_ok ? clampL(context_lens[my_seq]) : 0;
    int Lmax = 0;
#pragma unroll
    for (int r = 0; r < MAXR; ++r)
        if (r < nmem) Lmax = max(Lmax, __builtin_amdgcn_readlane(Lr, r));

    const int tok0 = part * part_tokens;
    auto write_zero_row = [&]() {
        uint2* o = reinterpret_cast<uint2*>(out + (static_cast<int64_t>(my_seq) * num_q_heads + hq) * FD);
#pragma unroll
        for (int j = 0; j < 8; ++j) o[4 * j + quad] = make_uint2(0u, 0u);
    };
    // (WGM: a wave past the longest member's history keeps going with no
    // tiles, to meet the workgroup's barriers; it has no tasks and no rows.)
    if (!WGM && tok0 >= Lmax) {
        if (part == 0 && r_wave == 0 && row_ok && my_L == 0) write_zero_row();
        return;
    }
    const int tok1 = max(tok0, min(Lmax, tok0 + part_tokens));
    const int blk0 = tok0 / FBS;
    const int nblk = (tok1 - tok0 + FBS - 1) / FBS;   // 1..64 (WGM: 0..64)

    // Appending: the token of each member this wave handles whose newest
    // position lies in this partition goes to the cache and to LDS, from
    // which it replaces that slot of the loaded tile.  A token is 256 B of K
    // and 256 B of V; a quarter-wave moves one member (16 B of K and 8 dims
    // of V per lane), four members a round.  The token loads go out here,
    // ahead of the block-table reads, so that they have landed when the
    // stores need them.
    constexpr int kRounds = APPEND ? (MAXR + 3) / 4 : 1;
    bf16x8 nk[kRounds], nv[kRounds];
    bool nload[kRounds];
    if constexpr (APPEND) {
#pragma unroll
        for (int it = 0; it < kRounds; ++it) {
            const int r = 4 * it + quad;
            const int Lm = __shfl(Lr, r);
            nload[it] = r < nmem && Lm > 0 && Lm - 1 >= tok0 && Lm - 1 < tok1;
            if (nload[it]) {
                const int64_t nrow = (static_cast<int64_t>(seq0 + r) * num_kv_heads + h) * FD;
                nk[it] = reinterpret_cast<const bf16x8*>(k_new + nrow)[row];
                nv[it] = reinterpret_cast<const bf16x8*>(v_new + nrow)[row];
            }
        }
    }

    // Lane j: each member's physical block at position j (-1 where the member
    // has no tokens), then whether position j is shared.
    int phys[MAXR];
    int p_sh = 0, v_sh = 0;
    int mem_at = 0;          // lane j: the members with tokens at position j (a bit each)
    bool sh = true, full = true;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
        phys[r] = -1;
        if (r < nmem) {
            const int Lm = __builtin_amdgcn_readlane(Lr, r);
            const int valid = min(max(Lm - (tok0 + FBS * lane), 0), FBS);
            if (lane < nblk && valid > 0) {
                mem_at |= 1 << r;
                phys[r] = clamp_block(
                    block_tables[static_cast<int64_t>(seq0 + r) * max_blocks_per_seq + blk0 + lane],
                    num_blocks);
                if (v_sh == 0) {
                    p_sh = phys[r];
                    v_sh = valid;
                } else if (phys[r] != p_sh || valid != v_sh) {
                    sh = false;
                }
            }
            if (valid < FBS) full = false;
        }
    }
    const uint64_t shared_mask = __ballot(sh && lane < nblk);
    const uint64_t full_mask = __ballot(full && sh && lane < nblk);

    // Grouped if walking all members' tiles in one wave costs at most 1.5x the
    // longest member's own tile count; otherwise each member gets its own wave
    // (all R waves of the group reach the same decision).
    int tasks_here = 0, longest = 0;
    if (lane < nblk) {
        if (sh) {
            tasks_here = 1;
        } else {
#pragma unroll
            for (int r = 0; r < MAXR; ++r) tasks_here += phys[r] >= 0 ? 1 : 0;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tasks_here += __shfl_xor(tasks_here, off);
#pragma unroll
    for (int r = 0; r < MAXR; ++r)
        if (r < nmem) longest = max(longest, static_cast<int>(__popcll(__ballot(phys[r] >= 0))));
    bool grouped = 2 * tasks_here <= 3 * longest;
    // WGM: if every partition of the group that has tokens takes the same mode,
    // one workgroup holds all partitions of each row it serves and merges them
    // in LDS (uniform); otherwise each wave goes its own way and writes its
    // partials for the merge kernel, as without WGM.
    bool uniform = false;
    if constexpr (WGM) {
        __shared__ int wg_mode[kMaxWgParts];   // 0: no tokens, 1: grouped, 2: per member
        if (lane == 0) wg_mode[part] = nblk == 0 ? 0 : (grouped ? 1 : 2);
        __syncthreads();
        int seen = 0;
        for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) seen |= 1 << wg_mode[w];
        uniform = (seen & 6) != 6;
        if (uniform) grouped = (seen & 4) == 0;
    }
    if (grouped ? r_wave != 0 : r_wave >= nmem) return;   // (uniform: the whole workgroup)
    const bool mine = row_ok && (grouped || my_mem == r_wave);

    auto is_shared = [&](int j) { return ((shared_mask >> j) & 1ull) != 0; };
    auto valid_of = [&](int r, int j) {
        return min(max(__builtin_amdgcn_readlane(Lr, r) - (tok0 + FBS * j), 0), FBS);
    };
    // first task at position j (j < nblk): shared, or the first member with tokens
    // there; in per-member mode this wave's member (MAXR: it has no tokens at j)
    auto first_task = [&](int j) {
        if (!grouped) return valid_of(r_wave, j) > 0 ? r_wave : MAXR;
        if (is_shared(j)) return kShared;
        const unsigned m = static_cast<unsigned>(__builtin_amdgcn_readlane(mem_at, j));
        return m != 0 ? static_cast<int>(__builtin_ctz(m)) : MAXR;
    };
    struct Cursor { int j, r; };
    auto advance = [&](Cursor c) {
        if (!grouped) {
            const int j = c.j + 1;
            return (j < nblk && valid_of(r_wave, j) > 0) ? Cursor{j, r_wave} : Cursor{nblk, 0};
        }
        if (c.r != kShared) {   // the next member with tokens at this position
            const unsigned m = static_cast<unsigned>(__builtin_amdgcn_readlane(mem_at, c.j)) &
                               ~((2u << c.r) - 1u);
            if (m != 0) return Cursor{c.j, static_cast<int>(__builtin_ctz(m))};
        }
        const int j = c.j + 1;
        return Cursor{j, j < nblk ? first_task(j) : 0};
    };
    auto task_phys = [&](Cursor c) {
        if (c.r == kShared) return __builtin_amdgcn_readlane(p_sh, c.j);
        int ph = 0;
#pragma unroll
        for (int r = 0; r < MAXR; ++r)
            if (r == c.r) ph = __builtin_amdgcn_readlane(phys[r], c.j);
        return ph;
    };

    __shared__ bf16x8 fresh_k[APPEND ? MAXR : 1][FD / 8];   // K chunk c at [r][c]
    __shared__ bf16x8 fresh_v[APPEND ? MAXR : 1][FD / 8];   // dims 8c..8c+7 at [r][c]
    auto substitute = [&](Tile& t, int r) {   // the newest slot of member r's tile
        const int om = (__builtin_amdgcn_readlane(Lr, r) - 1) % FBS;
        if (row == om) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) t.k[s4] = fresh_k[r][4 * s4 + quad];
        }
        const short* fv = reinterpret_cast<const short*>(&fresh_v[r][0]);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (quad * 4 + e == om) t.v[jj][e] = fv[16 * jj + row];
    };
    // Lane j: the members whose newest token lies at position j (a bit each);
    // the tokens go to LDS now and to the cache once the tiles are consumed
    // (stores issued ahead of the tile loads would hold up the loop's waits).
    auto appends_here = [&](int r, int& Lm) {
        if (r >= nmem || (!grouped && r != r_wave)) return false;
        Lm = __builtin_amdgcn_readlane(Lr, r);
        return Lm > 0 && Lm - 1 >= tok0 && Lm - 1 < tok1;
    };
    // Copy-on-write folded in: lane r holds member r's source block (or -1);
    // a member with one has its newest tile read from there and written back
    // whole, token included, to its own block.
    int cow_r = -1;
    if constexpr (APPEND) {
        if (cow_src != nullptr && lane < nmem) {
            const int cs = cow_src[seq0 + lane];
            if (cs >= 0 && static_cast<int64_t>(cs) < num_blocks) cow_r = cs;
        }
    }
    const uint64_t cow_members = APPEND ? __ballot(cow_r >= 0) : 0ull;
    int newest_mask = 0;
    if constexpr (APPEND) {
#pragma unroll
        for (int r = 0; r < MAXR; ++r) {
            int Lm;
            if (!appends_here(r, Lm)) continue;
            if (lane == (Lm - 1) / FBS - blk0) newest_mask |= 1 << r;
            if (quad == r % 4) {   // the quarter-wave that loaded member r's token
                fresh_k[r][row] = nk[r / 4];
                fresh_v[r][row] = nv[r / 4];
            }
        }
    }
    auto store_new_tokens = [&]() {   // quarter-wave q stores member 4*it + q
#pragma unroll
        for (int it = 0; it < kRounds; ++it) {
            bool act = false;
            int om = 0;
            int64_t toff = 0;
#pragma unroll
            for (int q4 = 0; q4 < 4 && 4 * it + q4 < MAXR; ++q4) {
                int Lm;
                if (!appends_here(4 * it + q4, Lm) || quad != q4) continue;
                if ((cow_members >> (4 * it + q4)) & 1ull) continue;   // written with its tile
                const int jl = (Lm - 1) / FBS - blk0;
                act = true;
                om = (Lm - 1) % FBS;
                toff = static_cast<int64_t>(__builtin_amdgcn_readlane(phys[4 * it + q4], jl)) * blk_stride +
                       static_cast<int64_t>(h) * FTILE;
            }
            if (!act) continue;
            const int r = 4 * it + quad;
            reinterpret_cast<bf16x8*>(const_cast<__bf16*>(k_cache) + toff)[row * FBS + om] = fresh_k[r][row];
            // V: sixteen consecutive dims per store, 512 B of the tile apart
            const short* fv = reinterpret_cast<const short*>(&fresh_v[r][0]);
            short* vd = reinterpret_cast<short*>(const_cast<__bf16*>(v_cache) + toff);
#pragma unroll
            for (int e = 0; e < 8; ++e) vd[(16 * e + row) * FBS + om] = fv[16 * e + row];
        }
    };

    // Query rows: member my_mem's query head hq (rows of absent members are zero).
    bf16x8 qv[4];
    {
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(
            q + (static_cast<int64_t>(my_seq) * num_q_heads + hq) * FD);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            bf16x8 v = qp[4 * s4 + quad];
            qv[s4] = row_ok ? v : bf16x8{};
        }
    }

    SoftmaxState st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const __bf16* k_head = k_cache + static_cast<int64_t>(h) * FTILE;
    const __bf16* v_head = v_cache + static_cast<int64_t>(h) * FTILE;
    // the member whose newest token this task's tile holds, or -1
    auto newest_member = [&](Cursor c) {
        if constexpr (!APPEND) return -1;
        const int nm = __builtin_amdgcn_readlane(newest_mask, c.j);
        if (c.r == kShared) return nm != 0 ? static_cast<int>(__builtin_ctz(nm)) : -1;
        return ((nm >> c.r) & 1) ? c.r : -1;
    };
    auto load_task = [&](Tile& t, Cursor c) {
        int ph = task_phys(c);
        if constexpr (APPEND) {
            const int r = newest_member(c);
            if (r >= 0 && ((cow_members >> r) & 1ull)) ph = __builtin_amdgcn_readlane(cow_r, r);
        }
        const int64_t o = static_cast<int64_t>(ph) * blk_stride;
        load_tile<NT>(t, k_head + o, v_head + o, lane);
    };
    auto consume_task = [&](Tile& t, Cursor c) {
        const int my_valid = min(max(my_L - (tok0 + FBS * c.j), 0), FBS);
        int row_valid, v_valid;
        bool masked;
        if (c.r == kShared) {
            row_valid = my_valid;
            v_valid = __builtin_amdgcn_readlane(v_sh, c.j);
            masked = ((full_mask >> c.j) & 1ull) == 0;
        } else {
            row_valid = (row_ok && my_mem == c.r) ? my_valid : 0;
            v_valid = valid_of(c.r, c.j);
            masked = true;
        }
        if constexpr (APPEND) {   // (a position held by one member only counts as shared)
            const int r = newest_member(c);
            if (r >= 0) {
                substitute(t, r);
            }
        }
        consume_tile_rows(st, t, qv, scale_log2, lane, row_valid, v_valid, masked);
    };

    // The copies first: each member whose newest token this partition holds
    // has that tile read from its source block, the token put in, and the
    // tile written to its own block before the walk starts (the walk reads it
    // from the source again; 139 against 142 us on the fan-out step, where the
    // copies, written at the end of each walk, met the read stream of the
    // waves still walking)
    if constexpr (APPEND) {
        if (cow_members != 0) {
            Tile t;
            int loaded = -1, loaded_om = -1;   // source and newest slot of the tile held
#pragma unroll
            for (int r = 0; r < MAXR; ++r) {
                int Lm;
                if (!((cow_members >> r) & 1ull) || !appends_here(r, Lm)) continue;
                const int jl = (Lm - 1) / FBS - blk0;
                const int src = __builtin_amdgcn_readlane(cow_r, r);
                const int om = (Lm - 1) % FBS;
                // (wave-uniform) the branches of one prompt copy the same tile
                // and put their token in the same slot, which substitute
                // overwrites whole: one load serves them all (136.6 against
                // 139.0 us on the fan-out step)
                if (src != loaded || om != loaded_om) {
                    const int64_t so = static_cast<int64_t>(src) * blk_stride;
                    load_tile<NT>(t, k_head + so, v_head + so, lane);
                    loaded = src;
                    loaded_om = om;
                }
                substitute(t, r);
                const int64_t dst = static_cast<int64_t>(__builtin_amdgcn_readlane(phys[r], jl)) * blk_stride;
                store_tile(t, const_cast<__bf16*>(k_head) + dst, const_cast<__bf16*>(v_head) + dst, lane);
            }
        }
    }
    // Two tiles in flight, as on the fast path; past the last task the
    // prefetch repeats the current tile (still in cache).
    Tile ta, tb;
    Cursor cu{0, first_task(0)};
    if (cu.r == MAXR) cu.j = nblk;   // per-member mode, member without tokens here
    Cursor cl = cu;
    if (cu.j < nblk) {
        load_task(ta, cl);
        cl = advance(cl);
    }
    while (cu.j < nblk) {
        load_task(tb, cl.j < nblk ? cl : cu);
        if (cl.j < nblk) cl = advance(cl);
        __builtin_amdgcn_sched_barrier(0);
        consume_task(ta, cu);
        cu = advance(cu);
        __builtin_amdgcn_sched_barrier(0);
        if (cu.j >= nblk) break;
        load_task(ta, cl.j < nblk ? cl : cu);
        if (cl.j < nblk) cl = advance(cl);
        __builtin_amdgcn_sched_barrier(0);
        consume_task(tb, cu);
        cu = advance(cu);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (APPEND) store_new_tokens();

    const float lsum = sum_across_rows(st.l);
    const int my_nparts = (my_L + part_tokens - 1) / part_tokens;
    if (WGM && uniform) {
        // LDS: [partition][row][acc FD | m | l | pad 2]; wave 0 merges and
        // marks the row as done for the merge kernel (l of partition 0 < 0)
        extern __shared__ float wg_part[];
        constexpr int RS = FD + 4;
        if (mine && tok0 < my_L && my_nparts > 1) {
            float* dst = wg_part + (part * FG + row) * RS;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) *reinterpret_cast<f32x4*>(dst + 16 * jj + 4 * quad) = st.acc[jj];
            if (quad == 0) {
                dst[FD] = st.m;
                dst[FD + 1] = lsum;
            }
        }
        __syncthreads();
        if (part != 0 || !mine) return;
        if (my_L > 0 && my_nparts > 1) {
            merge_lds_row<FD>(wg_part + row * RS, FG * RS, my_nparts, quad,
                          reinterpret_cast<uint2*>(out + (static_cast<int64_t>(my_seq) * num_q_heads + hq) * FD));
            if (quad == 0) ws_l[(static_cast<int64_t>(my_seq) * num_q_heads + hq) * max_parts] = -1.f;
            return;
        }
        // an empty history or a single partition: wave 0 writes it below
    }
    if (!mine) return;
    if (tok0 >= my_L) {                       // this row has no tokens in this partition
        if (part == 0 && my_L == 0) write_zero_row();
        return;
    }
    if (my_nparts == 1) {
        const float inv = 1.f / lsum;
        uint2* o = reinterpret_cast<uint2*>(out + (static_cast<int64_t>(my_seq) * num_q_heads + hq) * FD);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            o[4 * jj + quad] = make_uint2(pack_bf16x2(st.acc[jj][0] * inv, st.acc[jj][1] * inv),
                                          pack_bf16x2(st.acc[jj][2] * inv, st.acc[jj][3] * inv));
        return;
    }
    const int64_t pidx = (static_cast<int64_t>(my_seq) * num_q_heads + hq) * max_parts + part;
    f32x4* acc_out = reinterpret_cast<f32x4*>(ws_acc + pidx * FD);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc_out[4 * jj + quad] = st.acc[jj];
    if (quad == 0) {
        ws_m[pidx] = st.m;
        ws_l[pidx] = lsum;
    }
}

// ============================================================================
// Runs of requests with a common prefix: cooperative shared partitions
// ============================================================================
//
// For a batch in which long runs of consecutive requests share their leading
// blocks ([ZQ] answer and TL;DR: one prefix, many requests).  A workgroup of
// four waves is (KV head, chunk of M = 4 * 16/g consecutive requests,
// partition, slot).  It first checks whether the partition is shared by the
// whole chunk: every member's history extends past the partition's end and
// names the same physical blocks there.
//   * Shared: slot 0 decodes the partition for all M members at once.  Each
//     tile is copied from memory to LDS once (2 KiB per wave, global_load_lds,
//     S - 1 tiles ahead) and every wave consumes it for its 16 rows (16/g
//     members x g heads).  The other slots exit.
//   * Otherwise: wave w of slot s decodes alone the member whose history is
//     the (4 s + w)-th longest of the chunk, as the fast path does (one wave
//     per request, KV head and partition).
// Both kinds of workgroup run in the same launch, so the shared partitions'
// matrix work proceeds while the private suffixes stream from HBM.  The
// arithmetic per row is the fast path's (same tiles in the same order, same
// tile consumer), so the bits equal one request per wave; the partials go to
// the usual merge.  A shared partition never holds a member's newest
// position (the member's history extends past it), so the append, when
// asked for, is always done by the per-member waves.
constexpr int kCascadeStages = 4;
// At least two waves per SIMD: the decode-only variant takes 139 VGPRs
// (three waves), the append variant 176 (two; held to 168 for three, it
// spilled 24 to 32 bytes per lane: with the members dealt longest first the
// shared-prefix step measured 81.3-81.4 us that way against 79.1-79.3).

template <bool NT, bool APPEND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_cascade_kernel(
    const __bf16* __restrict__ k_cache, const __bf16* __restrict__ v_cache,
    const __bf16* __restrict__ q, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int64_t num_blocks, int64_t blk_stride,
    int num_seqs, int num_q_heads, int group, int max_blocks_per_seq, int len_clamp,
    int part_tokens, int max_parts, float scale_log2, __bf16* __restrict__ out,
    float* __restrict__ ws_acc, float* __restrict__ ws_m, float* __restrict__ ws_l,
    const __bf16* __restrict__ k_new, const __bf16* __restrict__ v_new, int num_kv_heads,
    int append_tiles) {
    constexpr int S = kCascadeStages;
    constexpr int kCopies = 2;                       // KiB of each 8 KiB tile per wave
    __shared__ __align__(16) __bf16 ring[S][2 * FTILE];
    __shared__ int tbl[64];
    __shared__ int not_shared;
    const int h = blockIdx.x;
    const int chunk = blockIdx.y;
    const int per = FG / group;                      // members per wave in a shared partition
    // Dispatch order (z is the slowest grid index): first slot 0 of every
    // partition (the shared work, and the four longest members of unshared
    // partitions),
    // then the other slots from the last partition down.  A chunk's prefix
    // is shared at its start, so the later partitions are the ones whose
    // other slots have members to decode; the slots of shared partitions
    // (which exit after the check) come last and no longer hold back the
    // private waves from the resident set.
    // (With the append, slot 0 of the partitions goes last partition first:
    // the requests' private partitions, which store the new tokens, start
    // ahead of the shared ones; the step measured 76.6-77.5 us that way
    // against 79.0-79.1, while the decode alone is faster in the order
    // above, 68.2 against 72.5 us.)
    int slot = 0, part = static_cast<int>(blockIdx.z);
    if (APPEND && part < max_parts) part = max_parts - 1 - part;
    if (static_cast<int>(blockIdx.z) >= max_parts) {
        const int k = part - max_parts;
        part = max_parts - 1 - k / (per - 1);
        slot = 1 + k % (per - 1);
    }
    const int wave = static_cast<int>(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int row = lane & 15;
    const int quad = lane >> 4;
    const int M = 4 * per;
    const int seq0 = chunk * M;
    const int nmem = min(M, num_seqs - seq0);
    const int tok0 = part * part_tokens;
    const int tok1 = tok0 + part_tokens;
    const int blk0 = tok0 / FBS;
    const int nblk = part_tokens / FBS;              // tiles of a whole partition, <= 64
    auto clampL = [&](int L) { return L < 0 ? 0 : (L > len_clamp ? len_clamp : L); };

    // Is the partition shared by the whole chunk?
    if (threadIdx.x == 0) not_shared = nmem < 2 || blk0 + nblk > max_blocks_per_seq;
    __syncthreads();
    if (!not_shared) {
        const int32_t* tab0 = block_tables + static_cast<int64_t>(seq0) * max_blocks_per_seq + blk0;
        bool bad = false;
        for (int i = threadIdx.x; i < nmem * nblk; i += 256) {
            const int m = i / nblk;
            const int j = i - m * nblk;
            bad = bad || tab0[static_cast<int64_t>(m) * max_blocks_per_seq + j] != tab0[j];
            if (j == 0) bad = bad || clampL(context_lens[seq0 + m]) <= tok1;
        }
        // one LDS write per wave (many lanes storing to one word would serialise)
        if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) not_shared = 1;
    }
    __syncthreads();
    const bool shared = not_shared == 0;

    if (shared) {
        if (slot != 0) return;                       // (whole workgroup)
        const int mem = wave * per + row / group;
        const bool row_ok = mem < nmem;
        const int seq = seq0 + (row_ok ? mem : 0);
        const int hq = h * group + row % group;
        bf16x8 qv[4];
        {
            const bf16x8* qp = reinterpret_cast<const bf16x8*>(
                q + (static_cast<int64_t>(seq) * num_q_heads + hq) * FD);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                bf16x8 v = qp[4 * s4 + quad];
                qv[s4] = row_ok ? v : bf16x8{};
            }
        }
        SoftmaxState st;
        st.m = -INFINITY;
        st.l = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) st.acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (threadIdx.x < nblk)
            tbl[threadIdx.x] = clamp_block(
                block_tables[static_cast<int64_t>(seq0) * max_blocks_per_seq + blk0 + threadIdx.x],
                num_blocks);
        __syncthreads();
        const unsigned ring0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(
            (__attribute__((address_space(3))) __bf16*)(&ring[0][0])));
        // tile t (past the end: the last one again, so every thread issues the
        // same number of copies per tile) into stage t % S: K then V, wave w
        // copying KiB 2w and 2w + 1
        // V stage layout: 16-byte chunk c of the tile sits at chunk c ^ ((c >> 4) & 1)
        // (the two chunks of a dim swap for dims 8..15 of every 16), so the 8-byte
        // reads of rows r and r + 8, 256 bytes apart, fall in different LDS banks.
        const int v_swz_lane = lane ^ ((lane >> 4) & 1);
        auto issue = [&](int t) {
            const int tc = t < nblk ? t : nblk - 1;
            const int64_t o = static_cast<int64_t>(tbl[tc]) * blk_stride +
                              static_cast<int64_t>(h) * FTILE;
            const unsigned sb = ring0 + static_cast<unsigned>((t % S) * 2 * FTILE * 2);
#pragma unroll
            for (int c = 0; c < kCopies; ++c) {
                const int kib = wave * kCopies + c;  // 0..3 K, 4..7 V
                const __bf16* src = kib < 4 ? k_cache + o + (kib & 3) * 512 + lane * 8
                                          : v_cache + o + (kib & 3) * 512 + v_swz_lane * 8;
                lds_copy16(src, __builtin_amdgcn_readfirstlane(sb + kib * 1024));
            }
        };
#pragma unroll
        for (int t = 0; t < S - 1; ++t) issue(t);
        for (int b = 0; b < nblk; ++b) {
            wait_vmcnt<kCopies * (S - 2)>();         // this thread's copies of tile b have landed
            __builtin_amdgcn_s_barrier();            // everyone's; and tile b - 1 is consumed
            issue(b + S - 1);                        // into tile b - 1's stage
            const __bf16* stage = &ring[b % S][0];
            Tile t;
            const bf16x8* kp = reinterpret_cast<const bf16x8*>(stage) + lane;
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) t.k[s4] = kp[64 * s4];
            const s16x4* vp = reinterpret_cast<const s16x4*>(stage + FTILE) +
                              2 * ((2 * row + (quad >> 1)) ^ (row >> 3)) + (quad & 1);
#pragma unroll
            for (int j = 0; j < 8; ++j) t.v[j] = vp[64 * j];
            consume_tile(st, t, qv, scale_log2, lane, FBS);
        }
        wait_vmcnt<0>();                             // no copy may land after the workgroup ends
        const float lsum = sum_across_rows(st.l);
        if (!row_ok) return;
        // every member's history extends past this partition: a partial
        const int64_t pidx = (static_cast<int64_t>(seq) * num_q_heads + hq) * max_parts + part;
        f32x4* acc_out = reinterpret_cast<f32x4*>(ws_acc + pidx * FD);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc_out[4 * jj + quad] = st.acc[jj];
        if (quad == 0) {
            ws_m[pidx] = st.m;
            ws_l[pidx] = lsum;
        }
        return;
    }

    // One member per wave, as the fast path does (one wave per request, KV
    // head and partition, block size 16; no copy-on-write here).  Members go
    // to waves longest history first (slot 0 is dispatched first): the
    // private suffixes differ in length, and the call ends with its longest
    // walks, so those start first.  (Ties by position in the chunk; the
    // order depends on the lengths only, and each member's arithmetic is
    // the same in any wave.)
    const int m_slot = slot * 4 + wave;
    if (m_slot >= nmem) return;
    int m = m_slot;
    {
        const int key = lane < nmem ? clampL(context_lens[seq0 + lane]) : -1;   // nmem <= 64
        int r = 0;
        for (int t = 0; t < nmem; ++t) {
            const int kt = __shfl(key, t);
            r += (kt > key || (kt == key && t < lane)) ? 1 : 0;
        }
        const unsigned long long b = __ballot(lane < nmem && r == m_slot);
        m = b ? __ffsll(b) - 1 : m_slot;
    }
    const FastArgs fa{k_cache, v_cache, q, block_tables, context_lens, num_blocks, blk_stride,
                      num_q_heads, group, max_blocks_per_seq, len_clamp, part_tokens, max_parts,
                      scale_log2, out, ws_acc, ws_m, ws_l, k_new, v_new, num_kv_heads, nullptr,
                      append_tiles};
    fast_item<PA_FAST_NBUF, NT, APPEND, false, FBS, FD>(fa, h, seq0 + m, part);
}

// ============================================================================
// Generic path
// ============================================================================

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_generic_kernel(
    const T* __restrict__ k_cache, const T* __restrict__ v_cache, const T* __restrict__ q,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int64_t num_blocks, int64_t blk_stride, int block_size, int num_q_heads, int group,
    int max_blocks_per_seq, int len_clamp, int part_tokens, int max_parts, float scale_log2,
    T* __restrict__ out, float* __restrict__ ws_acc, float* __restrict__ ws_m,
    float* __restrict__ ws_l) {
    constexpr int X = 16 / sizeof(T);
    constexpr int DPL = (D + 63) / 64;   // dims per lane
    const int hq = blockIdx.x;      // grid (Hq, S, partitions), head fastest
    const int seq = blockIdx.y;
    const int part = blockIdx.z;
    const int lane = threadIdx.x;
    const int h = hq / group;

    int L = context_lens[seq];
    L = L < 0 ? 0 : (L > len_clamp ? len_clamp : L);
    const int tok0 = part * part_tokens;
    T* orow = out + (static_cast<int64_t>(seq) * num_q_heads + hq) * D;
    if (tok0 >= L) {
        if (L == 0 && part == 0)
            for (int d = lane; d < D; d += 64) store_f32(orow + d, 0.f);
        return;
    }
    const int tok1 = min(L, tok0 + part_tokens);
    const int nparts = (L + part_tokens - 1) / part_tokens;

    float qv[DPL], acc[DPL];
#pragma unroll
    for (int r = 0; r < DPL; ++r) {
        const int d = lane + 64 * r;
        qv[r] = d < D ? load_f32(q + (static_cast<int64_t>(seq) * num_q_heads + hq) * D + d) : 0.f;
        acc[r] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int32_t* table = block_tables + static_cast<int64_t>(seq) * max_blocks_per_seq;
    const int64_t tile = static_cast<int64_t>(D) * block_size;

    for (int t = tok0; t < tok1; ++t) {
        const int lb = t / block_size;
        const int o = t - lb * block_size;
        const int phys = clamp_block(table[lb], num_blocks);
        const int64_t base = static_cast<int64_t>(phys) * blk_stride + h * tile;
        float kd[DPL], vd[DPL];
        float dot = 0.f;
#pragma unroll
        for (int r = 0; r < DPL; ++r) {
            const int d = lane + 64 * r;
            if (d < D) {
                kd[r] = load_f32(k_cache + base + k_elem(o, d, block_size, D, X));
                vd[r] = load_f32(v_cache + base + v_elem(o, d, block_size, D));
            } else {
                kd[r] = 0.f;
                vd[r] = 0.f;
            }
            dot += qv[r] * kd[r];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
        const float s = dot * scale_log2;
        const float m_new = fmaxf(m, s);
        const float alpha = fast_exp2(m - m_new);
        const float p = fast_exp2(s - m_new);
        l = l * alpha + p;
#pragma unroll
        for (int r = 0; r < DPL; ++r) acc[r] = acc[r] * alpha + p * vd[r];
        m = m_new;
    }

    if (nparts == 1) {
        const float inv = 1.f / l;
#pragma unroll
        for (int r = 0; r < DPL; ++r) {
            const int d = lane + 64 * r;
            if (d < D) store_f32(orow + d, acc[r] * inv);
        }
    } else {
        const int64_t pidx = (static_cast<int64_t>(seq) * num_q_heads + hq) * max_parts + part;
#pragma unroll
        for (int r = 0; r < DPL; ++r) {
            const int d = lane + 64 * r;
            if (d < D) ws_acc[pidx * D + d] = acc[r];
        }
        if (lane == 0) {
            ws_m[pidx] = m;
            ws_l[pidx] = l;
        }
    }
}

// ============================================================================
// Split-K merge: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p, with
// p visited in increasing order.
// ============================================================================

// One 256-lane workgroup per (request, query head).  Lane (c, g) owns dims
// 4c..4c+3 and the partitions p = g, g + G, g + 2G, ... (G = 256 / (D/4)).
// Each lane folds its partitions into a running (max, sum, acc) as they
// arrive -- one round trip to memory when there are at most G partitions --
// and the G group states are then combined in increasing g.  Every sum has a
// fixed shape, so the result is deterministic and independent of placement.
constexpr int kMergeThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void reduce_kernel(
    const int32_t* __restrict__ context_lens, int num_q_heads, int len_clamp, int part_tokens,
    int max_parts, const float* __restrict__ ws_acc, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, T* __restrict__ out) {
    constexpr int C = D / 4;                   // float4 chunks per row
    constexpr int G = kMergeThreads / C;       // partition groups
    __shared__ f32x4 s_num[G][C];
    __shared__ float s_m[G];
    __shared__ float s_den[G];

    const int hq = blockIdx.x;
    const int seq = blockIdx.y;
    const int tid = threadIdx.x;
    int L = context_lens[seq];
    L = L < 0 ? 0 : (L > len_clamp ? len_clamp : L);
    const int nparts = (L + part_tokens - 1) / part_tokens;
    if (nparts <= 1) return;   // written directly by the partition kernel
    const int64_t base = (static_cast<int64_t>(seq) * num_q_heads + hq) * max_parts;

    const int c = tid % C;
    const int g = tid / C;
    // group g's first partition is taken as is; later ones are folded in with
    // a running max (only when there are more than G partitions)
    float M = -INFINITY, den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    if (g < nparts) {
        M = ws_m[base + g];
        den = ws_l[base + g];
        num = reinterpret_cast<const f32x4*>(ws_acc + (base + g) * D)[c];
    }
#pragma unroll 4
    for (int p = g + G; p < nparts; p += G) {
        const float mp = ws_m[base + p];
        const float lp = ws_l[base + p];
        const f32x4 ap = reinterpret_cast<const f32x4*>(ws_acc + (base + p) * D)[c];
        const float Mn = fmaxf(M, mp);
        const float a = fast_exp2(M - Mn);
        const float w = fast_exp2(mp - Mn);
        num = fma4(ap, w, num * a);
        den = __builtin_fmaf(lp, w, den * a);
        M = Mn;
    }
    s_num[g][c] = num;
    if (c == 0) {
        s_m[g] = M;
        s_den[g] = den;
    }
    __syncthreads();
    if (g != 0) return;
    // global max first, then fused multiply-adds in group order (with at most
    // G partitions: in partition order -- the same formula as the in-workgroup
    // merge of the decode kernel)
    const int ng = nparts < G ? nparts : G;
    float Mt = s_m[0];
    for (int k = 1; k < ng; ++k) Mt = fmaxf(Mt, s_m[k]);
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    float dtot = 0.f;
    for (int k = 0; k < ng; ++k) {
        const float w = fast_exp2(s_m[k] - Mt);
        tot = fma4(s_num[k][c], w, tot);
        dtot = __builtin_fmaf(s_den[k], w, dtot);
    }
    const float inv = 1.f / dtot;
    T* o = out + (static_cast<int64_t>(seq) * num_q_heads + hq) * D + 4 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) store_f32(o + i, tot[i] * inv);
}

// The same merge for at most kMaxWgParts partitions, bf16 output, head_dim
// 128: 8 lanes per (request, query head), each with four 16-byte chunks of
// the row (lane c: chunks c, c+8, c+16, c+24), 32 rows per workgroup, and
// each lane loads all of its row's partitions at once (one memory round trip).
// The arithmetic is the formula above for that case -- global max first, then
// fused multiply-adds in partition order -- so the bits are the same as from
// reduce_kernel or the in-workgroup merge of the decode kernel.
constexpr int kMergeChunks = 4;                               // float4 chunks per lane
constexpr int kMergeLanes = FD / 4 / kMergeChunks;            // lanes per row
constexpr int kSmallMergeRows = kMergeThreads / kMergeLanes;   // rows per workgroup

// SKIP_DONE: rows whose partition-0 l is negative were merged already (by
// the grouped kernel's workgroups that held all of their partitions).
template <bool SKIP_DONE>
__global__ __launch_bounds__(kMergeThreads) void reduce_small_kernel(
    const int32_t* __restrict__ context_lens, int64_t rows, int num_q_heads, int len_clamp,
    int part_tokens, int max_parts, const float* __restrict__ ws_acc,
    const float* __restrict__ ws_m, const float* __restrict__ ws_l, uint16_t* __restrict__ out) {
    const int c = threadIdx.x % kMergeLanes;   // chunks c + kMergeLanes * i of the row
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kSmallMergeRows + threadIdx.x / kMergeLanes;
    if (row >= rows) return;
    const int64_t seq = row / num_q_heads;
    const int64_t base = row * max_parts;
    int L = context_lens[seq];
    // (the mark is loaded beside the length, not after it: one round trip)
    const float l0 = SKIP_DONE ? ws_l[base] : 0.f;
    L = L < 0 ? 0 : (L > len_clamp ? len_clamp : L);
    int nparts = (L + part_tokens - 1) / part_tokens;
    // one partition: written directly by the partition kernel; a marked row:
    // merged by the partition kernel's workgroup
    if ((nparts <= 1) | (SKIP_DONE && l0 < 0.f)) return;
    nparts = nparts < kMaxWgParts ? nparts : kMaxWgParts;
    float m[kMaxWgParts], l[kMaxWgParts];
    f32x4 acc[kMaxWgParts][kMergeChunks];
#pragma unroll
    for (int p = 0; p < kMaxWgParts; ++p) {
        if (p < nparts) {
            m[p] = ws_m[base + p];
            l[p] = ws_l[base + p];
#pragma unroll
            for (int i = 0; i < kMergeChunks; ++i)
                acc[p][i] = reinterpret_cast<const f32x4*>(ws_acc + (base + p) * FD)[c + kMergeLanes * i];
        }
    }
    float M = m[0];
#pragma unroll
    for (int p = 1; p < kMaxWgParts; ++p)
        if (p < nparts) M = fmaxf(M, m[p]);
    f32x4 tot[kMergeChunks];
#pragma unroll
    for (int i = 0; i < kMergeChunks; ++i) tot[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dtot = 0.f;
#pragma unroll
    for (int p = 0; p < kMaxWgParts; ++p) {
        if (p < nparts) {
            const float w = fast_exp2(m[p] - M);
#pragma unroll
            for (int i = 0; i < kMergeChunks; ++i) tot[i] = fma4(acc[p][i], w, tot[i]);
            dtot = __builtin_fmaf(l[p], w, dtot);
        }
    }
    const float inv = 1.f / dtot;
    uint2* o = reinterpret_cast<uint2*>(out + row * FD) + c;
#pragma unroll
    for (int i = 0; i < kMergeChunks; ++i)
        o[kMergeLanes * i] = make_uint2(pack_bf16x2(tot[i][0] * inv, tot[i][1] * inv),
                                        pack_bf16x2(tot[i][2] * inv, tot[i][3] * inv));
}

// The split-K merge of bf16, head_dim-128 partials of `rows` rows
// (request-major, num_q_heads per request).
// (skip_done: rows marked as merged are left alone; at most kMaxWgParts
// partitions.)
int merge_bf16(const int32_t* lens, int64_t rows, int num_q_heads, int len_clamp, int part_tokens,
               int max_parts, const float* ws_acc, const float* ws_m, const float* ws_l, void* out,
               hipStream_t stream, bool skip_done = false) {
    if (rows == 0) return PA_OK;
    if (max_parts <= kMaxWgParts) {
        const int64_t wgs = (rows + kSmallMergeRows - 1) / kSmallMergeRows;
        hipLaunchKernelGGL(skip_done ? reduce_small_kernel<true> : reduce_small_kernel<false>,
                           dim3(static_cast<unsigned>(wgs)), dim3(kMergeThreads), 0,
                           stream, lens, rows, num_q_heads, len_clamp, part_tokens, max_parts, ws_acc,
                           ws_m, ws_l, static_cast<uint16_t*>(out));
        return check_launch("decode merge");
    }
    hipLaunchKernelGGL((reduce_kernel<uint16_t, 128>), dim3(num_q_heads, static_cast<unsigned>(rows / num_q_heads)),
                       dim3(kMergeThreads), 0, stream, lens, num_q_heads, len_clamp, part_tokens,
                       max_parts, ws_acc, ws_m, ws_l, static_cast<uint16_t*>(out));
    return check_launch("decode merge");
}

template <typename T, int D>
int launch_generic(const DecodeArgs& a) {
    dim3 grid(a.num_q_heads, a.num_seqs, a.max_parts);
    const float sl2 = a.scale * kLog2e;
    hipLaunchKernelGGL((decode_generic_kernel<T, D>), grid, dim3(64), 0, a.stream,
                       static_cast<const T*>(a.k_cache), static_cast<const T*>(a.v_cache),
                       static_cast<const T*>(a.q), a.block_tables, a.context_lens, a.num_blocks,
                       a.block_stride, a.block_size, a.num_q_heads, a.group,
                       a.max_blocks_per_seq, a.len_clamp, a.part_tokens, a.max_parts, sl2,
                       static_cast<T*>(a.out), a.ws_acc, a.ws_m, a.ws_l);
    int st = check_launch("decode (generic)");
    if (st != PA_OK || a.max_parts <= 1) return st;
    hipLaunchKernelGGL((reduce_kernel<T, D>), dim3(a.num_q_heads, a.num_seqs), dim3(kMergeThreads), 0,
                       a.stream, a.context_lens, a.num_q_heads, a.len_clamp, a.part_tokens,
                       a.max_parts, a.ws_acc, a.ws_m, a.ws_l, static_cast<T*>(a.out));
    return check_launch("decode reduce");
}

template <typename T>
int launch_generic_d(const DecodeArgs& a) {
    switch (a.head_dim) {
        case 16: return launch_generic<T, 16>(a);
        case 32: return launch_generic<T, 32>(a);
        case 64: return launch_generic<T, 64>(a);
        case 128: return launch_generic<T, 128>(a);
        case 256: return launch_generic<T, 256>(a);
        default: return fail(PA_ERR_UNSUPPORTED, "head_dim %d not compiled", a.head_dim);
    }
}

// One-wave workgroups of `kernel` that one CU keeps resident at once (from the
// kernel's registers), or 0 if the runtime cannot say.
int workgroups_per_cu(const void* kernel) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64, 0) != hipSuccess || per_cu <= 0)
        return 0;
    return per_cu;
}

// Whether the append writes each token's tile back whole: asked for, or a
// batch of at least kAppendTilesMin (request, KV head) appends.  Measured
// (blocks of 16, D 128): 2,048 appends (the shared-prefix step) 87.6 -> 84.4
// us; 256 (the GQA step) 53.1 -> 54.3 us, where the whole-tile stores come at
// the end of the longest walks.
constexpr int64_t kAppendTilesMin = 1024;
int append_tiles(const DecodeArgs& a) {
    return (a.flags & PA_DECODE_APPEND_TILES) != 0 ||
           static_cast<int64_t>(a.num_seqs) * a.num_kv_heads >= kAppendTilesMin;
}

template <bool NT, bool APPEND, int BS, int D, typename E>
int launch_fast(const DecodeArgs& a) {
    const float sl2 = a.scale * kLog2e;
    const size_t wg_lds = static_cast<size_t>(a.max_parts) * a.group * (D + 4) * sizeof(float);
    constexpr int NB = fast_nbuf(D);
    const E* kc = static_cast<const E*>(a.k_cache);
    const E* vc = static_cast<const E*>(a.v_cache);
    const E* qq = static_cast<const E*>(a.q);
    const E* kn = static_cast<const E*>(a.k_new);
    const E* vn = static_cast<const E*>(a.v_new);
    E* out = static_cast<E*>(a.out);
    if (a.max_parts >= 2 && a.max_parts <= fast_wg_parts(D, sizeof(E)) && wg_lds <= kMaxWgLds) {
        // partitions of a request are the waves of one workgroup, merged in LDS
        hipLaunchKernelGGL((decode_fast_kernel<NB, NT, APPEND, true, BS, false, D, E>),
                           dim3(a.num_kv_heads, a.num_seqs, 1), dim3(64 * a.max_parts), wg_lds,
                           a.stream, kc, vc, qq, a.block_tables, a.context_lens, a.num_blocks,
                           a.block_stride, a.num_q_heads, a.group, a.max_blocks_per_seq, a.len_clamp,
                           a.part_tokens, a.max_parts, sl2, out, a.ws_acc, a.ws_m, a.ws_l, kn, vn,
                           a.num_kv_heads, a.cow_src, a.num_seqs, append_tiles(a));
        return check_launch("decode (fast, workgroup merge)");
    }
    // One wave per (KV head, request, partition), unless that grid holds more
    // waves than the device keeps resident: then as many persistent waves per
    // head as fit, each taking every Z-th item (at most 64 requests).
    const int64_t upper = static_cast<int64_t>(a.num_kv_heads) * a.num_seqs * a.max_parts;
    static const int per_cu = workgroups_per_cu(reinterpret_cast<const void*>(
        &decode_fast_kernel<NB, NT, APPEND, false, BS, true, D, E>));
    const int64_t resident = static_cast<int64_t>(per_cu) * device_cu_count();
    const bool persist = a.num_seqs <= 64 && resident >= a.num_kv_heads && upper > resident;
    const dim3 grid = persist ? dim3(a.num_kv_heads, static_cast<unsigned>(std::min<int64_t>(resident / a.num_kv_heads, 65535)), 1)
                              : dim3(a.num_kv_heads, a.num_seqs, a.max_parts);
    auto kernel = persist ? &decode_fast_kernel<NB, NT, APPEND, false, BS, true, D, E>
                          : &decode_fast_kernel<NB, NT, APPEND, false, BS, false, D, E>;
    hipLaunchKernelGGL(kernel, grid, dim3(64), 0, a.stream, kc, vc, qq, a.block_tables,
                       a.context_lens, a.num_blocks, a.block_stride, a.num_q_heads, a.group,
                       a.max_blocks_per_seq, a.len_clamp, a.part_tokens, a.max_parts, sl2, out,
                       a.ws_acc, a.ws_m, a.ws_l, kn, vn, a.num_kv_heads, a.cow_src, a.num_seqs,
                       append_tiles(a));
    int st = check_launch("decode (fast)");
    if (st != PA_OK || a.max_parts <= 1) return st;
    if constexpr (std::is_same<E, float>::value) {
        hipLaunchKernelGGL((reduce_kernel<float, D>), dim3(a.num_q_heads, a.num_seqs), dim3(kMergeThreads), 0,
                           a.stream, a.context_lens, a.num_q_heads, a.len_clamp, a.part_tokens,
                           a.max_parts, a.ws_acc, a.ws_m, a.ws_l, out);
        return check_launch("decode merge");
    } else {
        if constexpr (D == FD)
            return merge_bf16(a.context_lens, static_cast<int64_t>(a.num_seqs) * a.num_q_heads, a.num_q_heads,
                              a.len_clamp, a.part_tokens, a.max_parts, a.ws_acc, a.ws_m, a.ws_l, a.out, a.stream);
        hipLaunchKernelGGL((reduce_kernel<uint16_t, D>), dim3(a.num_q_heads, a.num_seqs), dim3(kMergeThreads), 0,
                           a.stream, a.context_lens, a.num_q_heads, a.len_clamp, a.part_tokens,
                           a.max_parts, a.ws_acc, a.ws_m, a.ws_l, static_cast<uint16_t*>(a.out));
        return check_launch("decode merge");
    }
}

template <int MAXR, bool NT, bool APPEND>
int launch_grouped(const DecodeArgs& a, int members) {
    const int groups = (a.num_seqs + members - 1) / members;
    const float sl2 = a.scale * kLog2e;
    const size_t wg_lds = static_cast<size_t>(a.max_parts) * FG * (FD + 4) * sizeof(float);
    if (a.max_parts >= 2 && a.max_parts <= kMaxWgParts && wg_lds <= kMaxWgLds) {
        // the partitions of a group are the waves of one workgroup, merged in LDS
        hipLaunchKernelGGL((decode_grouped_kernel<MAXR, NT, APPEND, true>),
                           dim3(a.num_kv_heads, groups, members), dim3(64 * a.max_parts), wg_lds, a.stream,
                           static_cast<const __bf16*>(a.k_cache), static_cast<const __bf16*>(a.v_cache),
                           static_cast<const __bf16*>(a.q), a.block_tables, a.context_lens,
                           a.num_blocks, a.block_stride, a.num_seqs, a.num_q_heads, a.group, members,
                           a.max_blocks_per_seq, a.len_clamp, a.part_tokens, a.max_parts, sl2,
                           static_cast<__bf16*>(a.out), a.ws_acc, a.ws_m, a.ws_l,
                           static_cast<const __bf16*>(a.k_new), static_cast<const __bf16*>(a.v_new),
                           a.num_kv_heads, a.cow_src);
        const int st = check_launch("decode (grouped, workgroup merge)");
        if (st != PA_OK) return st;
        // groups whose partitions took different modes are merged here
        return merge_bf16(a.context_lens, static_cast<int64_t>(a.num_seqs) * a.num_q_heads, a.num_q_heads,
                          a.len_clamp, a.part_tokens, a.max_parts, a.ws_acc, a.ws_m, a.ws_l, a.out, a.stream,
                          true);
    }
    dim3 grid(a.num_kv_heads, groups, a.max_parts * members);
    hipLaunchKernelGGL((decode_grouped_kernel<MAXR, NT, APPEND, false>), grid, dim3(64), 0, a.stream,
                       static_cast<const __bf16*>(a.k_cache), static_cast<const __bf16*>(a.v_cache),
                       static_cast<const __bf16*>(a.q), a.block_tables, a.context_lens,
                       a.num_blocks, a.block_stride, a.num_seqs, a.num_q_heads, a.group, members,
                       a.max_blocks_per_seq, a.len_clamp, a.part_tokens, a.max_parts, sl2,
                       static_cast<__bf16*>(a.out), a.ws_acc, a.ws_m, a.ws_l,
                       static_cast<const __bf16*>(a.k_new), static_cast<const __bf16*>(a.v_new),
                       a.num_kv_heads, a.cow_src);
    int st = check_launch("decode (grouped)");
    if (st != PA_OK || a.max_parts <= 1) return st;
    return merge_bf16(a.context_lens, static_cast<int64_t>(a.num_seqs) * a.num_q_heads, a.num_q_heads,
                      a.len_clamp, a.part_tokens, a.max_parts, a.ws_acc, a.ws_m, a.ws_l, a.out, a.stream);
}

template <bool NT, bool APPEND>
int launch_cascade(const DecodeArgs& a) {
    const int per = FG / a.group;
    const int chunks = (a.num_seqs + 4 * per - 1) / (4 * per);
    dim3 grid(a.num_kv_heads, chunks, a.max_parts * per);
    const float sl2 = a.scale * kLog2e;
    hipLaunchKernelGGL((decode_cascade_kernel<NT, APPEND>), grid, dim3(256), 0, a.stream,
                       static_cast<const __bf16*>(a.k_cache), static_cast<const __bf16*>(a.v_cache),
                       static_cast<const __bf16*>(a.q), a.block_tables, a.context_lens,
                       a.num_blocks, a.block_stride, a.num_seqs, a.num_q_heads, a.group,
                       a.max_blocks_per_seq, a.len_clamp, a.part_tokens, a.max_parts, sl2,
                       static_cast<__bf16*>(a.out), a.ws_acc, a.ws_m, a.ws_l,
                       static_cast<const __bf16*>(a.k_new), static_cast<const __bf16*>(a.v_new),
                       a.num_kv_heads, append_tiles(a));
    int st = check_launch("decode (prefix runs)");
    if (st != PA_OK) return st;
    return merge_bf16(a.context_lens, static_cast<int64_t>(a.num_seqs) * a.num_q_heads, a.num_q_heads,
                      a.len_clamp, a.part_tokens, a.max_parts, a.ws_acc, a.ws_m, a.ws_l, a.out, a.stream);
}

template <int BS, int D, typename E>
int launch_fast_bsd(const DecodeArgs& a, bool nt) {
    if (a.k_new) return nt ? launch_fast<true, true, BS, D, E>(a) : launch_fast<false, true, BS, D, E>(a);
    return nt ? launch_fast<true, false, BS, D, E>(a) : launch_fast<false, false, BS, D, E>(a);
}

template <int BS>
int launch_fast_bs(const DecodeArgs& a, bool nt) {
    if (a.dtype == PA_F32)   // fp32: head_dim 64 or 128 (fast_decode_ok)
        return a.head_dim == 64 ? launch_fast_bsd<BS, 64, float>(a, nt) : launch_fast_bsd<BS, FD, float>(a, nt);
    switch (a.head_dim) {
        case 64: return launch_fast_bsd<BS, 64, __bf16>(a, nt);
        case 256: return launch_fast_bsd<BS, 256, __bf16>(a, nt);
        default: return launch_fast_bsd<BS, FD, __bf16>(a, nt);
    }
}

template <bool NT, bool APPEND>
int launch_grouped_r(const DecodeArgs& a) {
    const int members = FG / a.group;   // requests per wave
    if (members <= 2) return launch_grouped<2, NT, APPEND>(a, members);
    if (members <= 4) return launch_grouped<4, NT, APPEND>(a, members);
    if (members <= 8) return launch_grouped<8, NT, APPEND>(a, members);
    return launch_grouped<16, NT, APPEND>(a, members);
}

}  // namespace

int launch_merge(const int32_t* lens, int32_t rows, int32_t num_q_heads, int32_t head_dim,
                 int32_t len_clamp, int32_t part_tokens, int32_t max_parts, const float* ws_acc,
                 const float* ws_m, const float* ws_l, void* out, hipStream_t stream) {
    // rows here are query rows, each with its own visible length in lens
    if (head_dim == 128)
        return merge_bf16(lens, static_cast<int64_t>(rows) * num_q_heads, num_q_heads, len_clamp,
                          part_tokens, max_parts, ws_acc, ws_m, ws_l, out, stream);
    if (rows == 0) return PA_OK;
    auto kernel = head_dim == 64 ? reduce_kernel<uint16_t, 64> : reduce_kernel<uint16_t, 256>;
    if (head_dim != 64 && head_dim != 256) return fail(PA_ERR_UNSUPPORTED, "merge: head_dim %d", head_dim);
    hipLaunchKernelGGL(kernel, dim3(num_q_heads, static_cast<unsigned>(rows)), dim3(kMergeThreads), 0, stream,
                       lens, num_q_heads, len_clamp, part_tokens, max_parts, ws_acc, ws_m, ws_l,
                       static_cast<uint16_t*>(out));
    return check_launch("merge");
}

int launch_decode(const DecodeArgs& a_in) {
    pa_cache_desc_t c{a_in.num_blocks, a_in.block_size, a_in.num_kv_heads, a_in.head_dim, a_in.dtype,
                      a_in.block_stride};
    DecodeArgs a = a_in;
    if (a.cow_src != nullptr && a.k_new != nullptr &&
        !(fast_decode_ok(&c, a.group) && a.block_size == FBS && a.part_tokens % FBS == 0)) {
        // only the block-size-16 MFMA kernels fold the copy in: copy first
        int st = launch_cow_last_block(&c, const_cast<void*>(a.k_cache), const_cast<void*>(a.v_cache),
                                       a.cow_src, a.block_tables, a.context_lens, a.num_seqs,
                                       a.max_blocks_per_seq, a.len_clamp, a.stream);
        if (st != PA_OK) return st;
        a.cow_src = nullptr;
    }
    const bool nt = (a.flags & PA_DECODE_STREAM_KV) != 0;
    if ((a.flags & PA_DECODE_PREFIX_RUNS) && a.cow_src == nullptr && fast_path_ok(&c, a.group) &&
        FG % a.group == 0 && a.part_tokens % FBS == 0 && a.part_tokens <= 64 * FBS && a.max_parts >= 2 &&
        static_cast<int64_t>(a.max_parts) * (FG / a.group) <= 65535) {
        if (a.k_new) return nt ? launch_cascade<true, true>(a) : launch_cascade<false, true>(a);
        return nt ? launch_cascade<true, false>(a) : launch_cascade<false, false>(a);
    }
    const int64_t grouped_z = static_cast<int64_t>(a.max_parts) * (FG / a.group);
    if (fast_path_ok(&c, a.group) && a.part_tokens % FBS == 0 && (a.flags & PA_DECODE_GROUP_SHARED) &&
        a.group <= FG / 2 && grouped_z <= 65535) {
        if (a.k_new) return nt ? launch_grouped_r<true, true>(a) : launch_grouped_r<false, true>(a);
        return nt ? launch_grouped_r<true, false>(a) : launch_grouped_r<false, false>(a);
    }
    if (fast_decode_ok(&c, a.group) && a.part_tokens % fast_granule(a.block_size) == 0) {
        switch (a.block_size) {
            case 8: return launch_fast_bs<8>(a, nt);
            case 32: return launch_fast_bs<32>(a, nt);
            case 64: return launch_fast_bs<64>(a, nt);
            default: return launch_fast_bs<16>(a, nt);
        }
    }
    if (a.k_new) {   // generic path: append with its own kernel, then decode
        int st = launch_append_kv(&c, const_cast<void*>(a.k_cache), const_cast<void*>(a.v_cache),
                                  a.k_new, a.v_new, a.block_tables, a.context_lens, a.num_seqs,
                                  a.max_blocks_per_seq, a.len_clamp, a.stream);
        if (st != PA_OK) return st;
    }
    if (a.dtype == PA_BF16) return launch_generic_d<uint16_t>(a);
    return launch_generic_d<float>(a);
}

}  // namespace pa
