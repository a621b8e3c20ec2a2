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
// Fast path (bf16, head_dim 128, block_size 16, up to 16 query heads per
// KV head): one 64-lane wave per (request, KV head, partition).  Per block
// of 16 tokens:
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
// Generic path (fp32 or bf16, other head_dim / block_size): one wave per
// (request, query head, partition), one token per step, lanes over dims.

#include <math.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    __bf16 h = static_cast<__bf16>(f);   // round to nearest even (v_cvt_pk_bf16_f32)
    return __builtin_bit_cast(uint16_t, h);
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p) {
    return bf16_bits_to_float(*p);
}

template <typename T> __device__ __forceinline__ void store_f32(T* p, float v);
template <> __device__ __forceinline__ void store_f32<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_f32<uint16_t>(uint16_t* p, float v) {
    *p = float_to_bf16_bits(v);
}

__device__ __forceinline__ int clamp_block(int e, int64_t num_blocks) {
    return (e >= 0 && static_cast<int64_t>(e) < num_blocks) ? e : 0;
}

// ============================================================================
// Fast path
// ============================================================================

#ifndef PA_FAST_NBUF
#define PA_FAST_NBUF 2           // tiles in the load ring of the fast path
#endif


constexpr int FD = 128;          // head_dim
constexpr int FBS = 16;          // block_size
constexpr int FTILE = FD * FBS;  // elements of one (block, head) tile

struct Tile {
    bf16x8 k[4];   // K: chunk (4*s + l/16), token l%16 -> A operand of step s
    s16x4 v[8];    // V: dim 16*j + l%16, tokens 4*(l/16)..+3 -> A operand of PV j
};

// NT: non-temporal loads (streaming hint), for batches without shared blocks.
template <bool NT, typename V>
__device__ __forceinline__ V load16(const V* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ __forceinline__ void load_tile(Tile& t, const __bf16* __restrict__ k_tile,
                                          const __bf16* __restrict__ v_tile, int lane) {
    const bf16x8* kp = reinterpret_cast<const bf16x8*>(k_tile) + lane;
#pragma unroll
    for (int s = 0; s < 4; ++s) t.k[s] = load16<NT>(kp + 64 * s);
    const s16x4* vp = reinterpret_cast<const s16x4*>(v_tile) + (lane & 15) * 4 + (lane >> 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) t.v[j] = load16<NT>(vp + 64 * j);
}

struct SoftmaxState {
    float m;        // running max of log2-domain scores for query row lane%16
    float l;        // this lane's share of the running sum
    f32x4 acc[8];   // output accumulator
};

// Reductions across the four 16-lane rows of the wave with the gfx950 row
// swaps: permlane16_swap exchanges rows (0,1) and (2,3), permlane32_swap
// exchanges rows (0,2) and (1,3); each lane keeps its position in the row.
__device__ __forceinline__ float max_across_rows(float x) {
    const unsigned u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned w = __float_as_uint(y);
    auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_across_rows(float x) {
    const unsigned u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned w = __float_as_uint(y);
    auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    return static_cast<unsigned>(float_to_bf16_bits(lo)) |
           (static_cast<unsigned>(float_to_bf16_bits(hi)) << 16);
}

// One block of 16 tokens.  `valid` = number of this block's tokens that are
// visible (16 except in the last block of a request).
__device__ __forceinline__ void consume_tile(SoftmaxState& st, Tile& t, const bf16x8 (&qv)[4],
                                             float scale_log2, int lane, int valid) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[k], qv[k], s, 0, 0, 0);

    const int tok_base = 4 * (lane >> 4);
    const bool masked = valid < FBS;   // uniform
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = s[i] * scale_log2;
    if (masked) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (tok_base + i >= valid) sc[i] = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tok_base + i >= valid) t.v[j][i] = 0;
    }
    const float mx = max_across_rows(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const float m_new = fmaxf(st.m, mx);
    const float alpha = fast_exp2(st.m - m_new);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[i] - m_new);
    st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    st.m = m_new;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[j] *= alpha;

    const unsigned p01 = pack_bf16x2(p[0], p[1]);
    const unsigned p23 = pack_bf16x2(p[2], p[3]);
    s16x4 pb;
    pb[0] = static_cast<short>(p01 & 0xffff);
    pb[1] = static_cast<short>(p01 >> 16);
    pb[2] = static_cast<short>(p23 & 0xffff);
    pb[3] = static_cast<short>(p23 >> 16);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        st.acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[j], pb, st.acc[j], 0, 0, 0);
}

// APPEND: the call also appends each request's newest token (position L-1):
// the wave of the request's last partition stores k_new/v_new into the cache
// and uses them in place of whatever its load of that slot returned.
template <int NBUF, bool NT, bool APPEND>
__global__ __launch_bounds__(64) void decode_fast_kernel(
    const __bf16* __restrict__ k_cache, const __bf16* __restrict__ v_cache,
    const __bf16* __restrict__ q, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int64_t num_blocks, int64_t blk_stride,
    int num_q_heads, int group, int max_blocks_per_seq, int len_clamp, int part_tokens,
    int max_parts, float scale_log2, __bf16* __restrict__ out, float* __restrict__ ws_acc,
    float* __restrict__ ws_m, float* __restrict__ ws_l, const __bf16* __restrict__ k_new,
    const __bf16* __restrict__ v_new, int num_kv_heads) {
    // Grid (Hkv, S, partitions) with the KV head fastest: workgroups are
    // dealt to the XCDs round-robin, so each XCD sees every partition index
    // and the same heads for all requests (a shared prefix's head slice then
    // stays in one XCD's L2).
    const int h = blockIdx.x;
    const int seq = blockIdx.y;
    const int part = blockIdx.z;
    const int lane = threadIdx.x;
    const int row = lane & 15;
    const int quad = lane >> 4;

    int L = context_lens[seq];
    L = L < 0 ? 0 : (L > len_clamp ? len_clamp : L);
    const int tok0 = part * part_tokens;
    const int hq = h * group + row;
    const bool row_ok = row < group;

    if (tok0 >= L) {
        if (L == 0 && part == 0 && row_ok) {   // empty history: zero output
            uint2* o = reinterpret_cast<uint2*>(out + (static_cast<int64_t>(seq) * num_q_heads + hq) * FD);
#pragma unroll
            for (int j = 0; j < 8; ++j) o[4 * j + quad] = make_uint2(0u, 0u);
        }
        return;
    }
    const int tok1 = min(L, tok0 + part_tokens);
    const int nparts = (L + part_tokens - 1) / part_tokens;
    const int blk0 = tok0 / FBS;
    const int nblk = (tok1 - tok0 + FBS - 1) / FBS;   // 1..64
    const int last_valid = tok1 - (tok0 + (nblk - 1) * FBS);

    // Block-table entries of this partition: one per lane, read back with readlane.
    int my_phys = 0;
    if (lane < nblk)
        my_phys = clamp_block(block_tables[static_cast<int64_t>(seq) * max_blocks_per_seq + blk0 + lane],
                              num_blocks);

    // Appending: the last partition holds position L-1 at offset o of its
    // last block.  The four lanes of row o hold that token's 16 key chunks
    // (the same chunk order as the K tile); the 16 lanes of quad o/4 hold its
    // 128 value dims (dim 16*j + row).  They also store them to the cache.
    const bool append_here = APPEND && part == nparts - 1;
    const int o_new = (L - 1) % FBS;
    bf16x8 fk[4];
    short fv[8];
    if constexpr (APPEND) {
        if (append_here) {
            const int64_t nrow = (static_cast<int64_t>(seq) * num_kv_heads + h) * FD;
            const bf16x8* kn = reinterpret_cast<const bf16x8*>(k_new + nrow);
            const short* vn = reinterpret_cast<const short*>(v_new + nrow);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) fk[s4] = kn[4 * s4 + quad];
#pragma unroll
            for (int j = 0; j < 8; ++j) fv[j] = vn[16 * j + row];
            const int64_t toff = static_cast<int64_t>(__builtin_amdgcn_readlane(my_phys, nblk - 1)) *
                                     blk_stride + static_cast<int64_t>(h) * FTILE;
            if (row == o_new) {
                bf16x8* kd = reinterpret_cast<bf16x8*>(const_cast<__bf16*>(k_cache) + toff);
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) kd[(4 * s4 + quad) * FBS + o_new] = fk[s4];
            }
            if (quad == o_new / 4) {
                short* vd = reinterpret_cast<short*>(const_cast<__bf16*>(v_cache) + toff);
#pragma unroll
                for (int j = 0; j < 8; ++j) vd[(16 * j + row) * FBS + o_new] = fv[j];
            }
        }
    }

    // Query rows of this KV head as the B operand (rows >= group are zero).
    bf16x8 qv[4];
    {
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(
            q + (static_cast<int64_t>(seq) * num_q_heads + (row_ok ? hq : 0)) * FD);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 v = qp[4 * s + quad];
            qv[s] = row_ok ? v : bf16x8{};
        }
    }

    const __bf16* k_head = k_cache + static_cast<int64_t>(h) * FTILE;
    const __bf16* v_head = v_cache + static_cast<int64_t>(h) * FTILE;

    SoftmaxState st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // A ring of NBUF tiles: while block j is consumed, blocks j+1 .. j+NBUF-1
    // are in flight.  Loads are unconditional (past the end they repeat the
    // last block, which is then still in cache), so every path through the
    // loop has the same loads outstanding and the waits stay exact.  The
    // scheduling barriers keep each tile's loads issued ahead of the previous
    // tile's arithmetic; without them the compiler sinks loads next to their
    // first use and every block waits a full memory latency.
    Tile buf[NBUF];
    auto tile_off = [&](int jj) {
        const int jc = jj < nblk ? jj : nblk - 1;
        return static_cast<int64_t>(__builtin_amdgcn_readlane(my_phys, jc)) * blk_stride;
    };
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u) {
        const int64_t o = tile_off(u);
        load_tile<NT>(buf[u], k_head + o, v_head + o, lane);
    }
    for (int j0 = 0; j0 < nblk; j0 += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
            const int j = j0 + u;
            {
                const int64_t o = tile_off(j + NBUF - 1);
                load_tile<NT>(buf[(u + NBUF - 1) % NBUF], k_head + o, v_head + o, lane);
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (APPEND) {
                if (append_here && j == nblk - 1) {
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
                        if (row == o_new) buf[u].k[s4] = fk[s4];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (quad * 4 + e == o_new) buf[u].v[jj][e] = fv[jj];
                }
            }
            if (j < nblk)
                consume_tile(st, buf[u], qv, scale_log2, lane, j == nblk - 1 ? last_valid : FBS);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // The four lanes of a query row each summed a quarter of the tokens.
    const float lsum = sum_across_rows(st.l);

    if (nparts == 1) {
        if (!row_ok) return;
        const float inv = 1.f / lsum;
        uint2* o = reinterpret_cast<uint2*>(out + (static_cast<int64_t>(seq) * num_q_heads + hq) * FD);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            o[4 * jj + quad] = make_uint2(pack_bf16x2(st.acc[jj][0] * inv, st.acc[jj][1] * inv),
                                          pack_bf16x2(st.acc[jj][2] * inv, st.acc[jj][3] * inv));
        return;
    }

    if (!row_ok) return;
    const int64_t pidx = (static_cast<int64_t>(seq) * num_q_heads + hq) * max_parts + part;
    f32x4* acc_out = reinterpret_cast<f32x4*>(ws_acc + pidx * FD);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc_out[4 * jj + quad] = st.acc[jj];
    if (quad == 0) {
        ws_m[pidx] = st.m;
        ws_l[pidx] = lsum;
    }
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
                kd[r] = load_f32(k_cache + base + (static_cast<int64_t>(d / X) * block_size + o) * X + d % X);
                vd[r] = load_f32(v_cache + base + static_cast<int64_t>(d) * block_size + o);
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
    float M = -INFINITY, den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int p = g; p < nparts; p += G) {
        const float mp = ws_m[base + p];
        const float lp = ws_l[base + p];
        const f32x4 ap = reinterpret_cast<const f32x4*>(ws_acc + (base + p) * D)[c];
        const float Mn = fmaxf(M, mp);
        const float a = fast_exp2(M - Mn);     // 0 on the first partition (M = -inf)
        const float w = fast_exp2(mp - Mn);
        num = num * a + ap * w;
        den = den * a + lp * w;
        M = Mn;
    }
    s_num[g][c] = num;
    if (c == 0) {
        s_m[g] = M;
        s_den[g] = den;
    }
    __syncthreads();
    if (g != 0) return;
    float Mt = s_m[0];
#pragma unroll
    for (int k = 1; k < G; ++k) Mt = fmaxf(Mt, s_m[k]);
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    float dtot = 0.f;
#pragma unroll
    for (int k = 0; k < G; ++k) {
        const float w = fast_exp2(s_m[k] - Mt);   // groups without partitions: 0 * 0
        tot += s_num[k][c] * w;
        dtot += s_den[k] * w;
    }
    const float inv = 1.f / dtot;
    T* o = out + (static_cast<int64_t>(seq) * num_q_heads + hq) * D + 4 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) store_f32(o + i, tot[i] * inv);
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

template <bool NT, bool APPEND>
int launch_fast(const DecodeArgs& a) {
    dim3 grid(a.num_kv_heads, a.num_seqs, a.max_parts);
    const float sl2 = a.scale * kLog2e;
    hipLaunchKernelGGL((decode_fast_kernel<PA_FAST_NBUF, NT, APPEND>), grid, dim3(64), 0, a.stream,
                       static_cast<const __bf16*>(a.k_cache), static_cast<const __bf16*>(a.v_cache),
                       static_cast<const __bf16*>(a.q), a.block_tables, a.context_lens,
                       a.num_blocks, a.block_stride, a.num_q_heads, a.group,
                       a.max_blocks_per_seq, a.len_clamp, a.part_tokens, a.max_parts, sl2,
                       static_cast<__bf16*>(a.out), a.ws_acc, a.ws_m, a.ws_l,
                       static_cast<const __bf16*>(a.k_new), static_cast<const __bf16*>(a.v_new),
                       a.num_kv_heads);
    int st = check_launch("decode (fast)");
    if (st != PA_OK || a.max_parts <= 1) return st;
    hipLaunchKernelGGL((reduce_kernel<uint16_t, 128>), dim3(a.num_q_heads, a.num_seqs), dim3(kMergeThreads),
                       0, a.stream, a.context_lens, a.num_q_heads, a.len_clamp, a.part_tokens,
                       a.max_parts, a.ws_acc, a.ws_m, a.ws_l, static_cast<uint16_t*>(a.out));
    return check_launch("decode reduce");
}

}  // namespace

int launch_decode(const DecodeArgs& a) {
    pa_cache_desc_t c{a.num_blocks, a.block_size, a.num_kv_heads, a.head_dim, a.dtype, a.block_stride};
    const bool nt = (a.flags & PA_DECODE_STREAM_KV) != 0;
    if (fast_path_ok(&c, a.group) && a.part_tokens % FBS == 0) {
        if (a.k_new) return nt ? launch_fast<true, true>(a) : launch_fast<false, true>(a);
        return nt ? launch_fast<true, false>(a) : launch_fast<false, false>(a);
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
