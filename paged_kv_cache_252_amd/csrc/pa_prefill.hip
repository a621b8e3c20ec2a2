// Several query tokens per request over a paged KV cache, gfx950: a chunk
// of a prompt after a prefix-cache hit, a chunked prefill, or several tokens
// checked at once.  Built from the MFMA tile of the decode kernels
// (pa_tile.h); the split-K merge is decode's (launch_merge).

#include <float.h>

#include "pa_tile.h"

namespace pa {
namespace {

// tile_softmax_pv for two tiles A and B at once (32 positions), for the
// several-token kernels, whose matrix work is the bound.  The bf16 MFMA of K
// 32 costs the same issue time as the one of K 16 (measured on gfx950), so
// the PV of both tiles is one 16x16x32 MFMA per 16 dims instead of two
// 16x16x16: lane l's eight K slots are A's positions 4*(l/16)..+3 then B's,
// which is how the lane already holds both V operands (va, vb) and both
// tiles' probabilities, so nothing moves between lanes.  The running maximum
// is raised at most once per pair.  The caller has masked V past the
// visible positions of each tile (a tile with nothing visible: V all zero,
// row_valid 0).
template <int RG, int D>
__device__ __forceinline__ void pair_softmax_pv(SoftmaxStateT<D> (&st)[RG], f32x4 (&sa)[RG],
                                                f32x4 (&sb)[RG], const s16x4 (&va)[D / 16],
                                                const s16x4 (&vb)[D / 16], float scale_log2, int lane,
                                                const int (&rva)[RG], const int (&rvb)[RG],
                                                bool masked) {
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const int tok_base = 4 * (lane >> 4);
    float mx[RG];
    bool raise[RG];
    bool any = false;
#pragma unroll
    for (int u = 0; u < RG; ++u) {
        if (masked) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (tok_base + i >= rva[u]) sa[u][i] = -INFINITY;
                if (tok_base + i >= rvb[u]) sb[u][i] = -INFINITY;
            }
        }
        if constexpr (RG % 2 == 0) {   // the lane's maximum; rows combined below two groups at once
            float x = vmax3(sa[u][0], sa[u][1], sa[u][2]);
            x = vmax3(sa[u][3], sb[u][0], x);
            x = vmax3(sb[u][1], sb[u][2], x);
            mx[u] = vmax(sb[u][3], x);
            continue;
        }
        const float ma = vmax3(sa[u][0], sa[u][1], vmax(sa[u][2], sa[u][3]));
        const float mb = vmax3(sb[u][0], sb[u][1], vmax(sb[u][2], sb[u][3]));
        mx[u] = vmax_across_rows(vmax(ma, mb)) * scale_log2;
        raise[u] = mx[u] > st[u].m + kLazyMaxLog2;
        any = any || raise[u];
    }
    if constexpr (RG % 2 == 0) {
        // Two groups' row maxima with three row swaps instead of four: the
        // first swaps group u's odd rows against group u + 1's even rows, so
        // the pairwise maximum holds group u in rows 0, 2 and group u + 1 in
        // rows 1, 3; the second completes each; the third hands every row both.
#pragma unroll
        for (int u = 0; u < RG; u += 2) {
            auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx[u]), __float_as_uint(mx[u + 1]),
                                                      false, false);
            const float m1 = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
            auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m1), __float_as_uint(m1), false,
                                                      false);
            const float m2 = vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
            auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(m2), __float_as_uint(m2), false,
                                                      false);
            mx[u] = __uint_as_float(c[0]) * scale_log2;
            mx[u + 1] = __uint_as_float(c[1]) * scale_log2;
        }
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            raise[u] = mx[u] > st[u].m + kLazyMaxLog2;
            any = any || raise[u];
        }
    }
    if (__builtin_amdgcn_ballot_w64(any) != 0) {   // wave-uniform
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            const float alpha = raise[u] ? fast_exp2(st[u].m - mx[u]) : 1.f;
            st[u].m = raise[u] ? mx[u] : st[u].m;
            st[u].l *= alpha;
#pragma unroll
            for (int j = 0; j < D / 16; ++j) st[u].acc[j] *= alpha;
        }
    }
#pragma unroll
    for (int u = 0; u < RG; ++u) {
        const float nm = -st[u].m;
        float p[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(__builtin_fmaf(sa[u][i], scale_log2, nm));
            p[4 + i] = fast_exp2(__builtin_fmaf(sb[u][i], scale_log2, nm));
        }
        const u32x4 pp = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        st[u].l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pp);
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
            const s16x8 v = __builtin_shufflevector(va[j], vb[j], 0, 1, 2, 3, 4, 5, 6, 7);
            st[u].acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), pb,
                                                                  st[u].acc[j], 0, 0, 0);
        }
    }
}


// ============================================================================
// Several query tokens per request (chunked prefill, several-token checks)
// ============================================================================
//
// A request's query tokens are its last n positions: token j (position
// L - n + j) sees positions [0, L - n + j] ([KG] "A Tiny Block-Table
// Example", closing paragraphs: never a later token).  One wave takes
// RG * 16/g consecutive tokens of one request and KV head as RG groups of
// 16 MFMA rows: row r of group u is token j0 + u * 16/g + r / g, query head
// h * g + r % g.  All rows read the same physical blocks, so each tile is
// loaded once and consumed by every group, masked row by row (RG groups per
// load cut the tile reads from L2 RG times); the partitions and their merge
// are those of decode, per query row.  This kernel keeps the tiles in
// registers (short chunks); prefill_lds_kernel below stages them in LDS.
template <bool NT, int RG, int W>
__global__ __launch_bounds__(64 * W) void prefill_kernel(
    const __bf16* __restrict__ k_cache, const __bf16* __restrict__ v_cache,
    const __bf16* __restrict__ q, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int64_t num_blocks, int64_t blk_stride, int total_q, int num_q_heads, int group,
    int tiles_per_seq, int max_blocks_per_seq, int len_clamp, int part_tokens, int max_parts,
    float scale_log2, unsigned q_sign, __bf16* __restrict__ out, float* __restrict__ ws_acc,
    float* __restrict__ ws_m, float* __restrict__ ws_l, int32_t* __restrict__ ws_len) {
    // W waves of a workgroup take W consecutive query tiles of one request and
    // KV head: they read the same blocks at about the same time, so most of
    // their tile loads are served by the CU's L1.
    const int h = blockIdx.x;
    const int seq = blockIdx.y / tiles_per_seq;
    const int tile = (blockIdx.y - seq * tiles_per_seq) * W + static_cast<int>(threadIdx.x >> 6);
    const int part = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int row = lane & 15;
    const int quad = lane >> 4;
    auto clampi = [](int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); };

    // rows are clamped to [0, total_q): a bad q_start cannot move an access
    const int qs = clampi(q_start[seq], 0, total_q);
    const int n = clampi(q_start[seq + 1], qs, total_q) - qs;
    const int tpg = FG / group;                 // query tokens per row group
    const int j0 = tile * RG * tpg;
    if (j0 >= n) return;
    const int L = clampi(context_lens[seq], 0, len_clamp);
    const int hq = h * group + row % group;
    int qi[RG], lim[RG];
    bool row_ok[RG];
#pragma unroll
    for (int u = 0; u < RG; ++u) {
        const int j = j0 + u * tpg + row / group;
        row_ok[u] = j < n;
        qi[u] = qs + (row_ok[u] ? j : j0);
        lim[u] = row_ok[u] ? clampi(L - n + j + 1, 0, L) : 0;   // positions this row sees
    }
    const int lim_min = clampi(L - n + j0 + 1, 0, L);
    const int lim_max = clampi(L - n + min(j0 + RG * tpg, n), 0, L);

#pragma unroll
    for (int u = 0; u < RG; ++u)
        if (max_parts > 1 && part == 0 && h == 0 && row_ok[u] && row % group == 0 && quad == 0)
            ws_len[qi[u]] = lim[u];             // the merge's per-row partition count
    auto out_row = [&](int u) {
        return reinterpret_cast<uint2*>(out + (static_cast<int64_t>(qi[u]) * num_q_heads + hq) * FD);
    };
    const int tok0 = part * part_tokens;
    if (tok0 >= lim_max) {
#pragma unroll
        for (int u = 0; u < RG; ++u)
            if (part == 0 && row_ok[u] && lim[u] == 0) {
                uint2* o = out_row(u);
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) o[4 * jj + quad] = make_uint2(0u, 0u);
            }
        return;
    }
    const int tok1 = min(lim_max, tok0 + part_tokens);

    bf16x8 qv[RG][4];
    SoftmaxState st[RG];
#pragma unroll
    for (int u = 0; u < RG; ++u) {
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(
            q + (static_cast<int64_t>(qi[u]) * num_q_heads + hq) * FD);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 v = __builtin_bit_cast(u32x4, qp[4 * s4 + quad]) ^ q_sign;   // sign of the scale
            qv[u][s4] = row_ok[u] ? __builtin_bit_cast(bf16x8, v) : bf16x8{};
        }
        st[u].m = kNoMaxLog2;
        st[u].l = 0.f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) st[u].acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const __bf16* k_head = k_cache + static_cast<int64_t>(h) * FTILE;
    const __bf16* v_head = v_cache + static_cast<int64_t>(h) * FTILE;
    // The partition is walked in chunks of 64 blocks, one table entry per lane.
    for (int c0 = tok0; c0 < tok1; c0 += 64 * FBS) {
        const int blk0 = c0 / FBS;
        const int nblk = (min(tok1, c0 + 64 * FBS) - c0 + FBS - 1) / FBS;   // 1..64
        const int my_phys = lane < nblk
            ? clamp_block(block_tables[static_cast<int64_t>(seq) * max_blocks_per_seq + blk0 + lane],
                          num_blocks)
            : 0;
        auto load_blk = [&](Tile& t, int b) {
            const int64_t o = static_cast<int64_t>(__builtin_amdgcn_readlane(my_phys, b)) * blk_stride;
            load_tile<NT>(t, k_head + o, v_head + o, lane);
        };
        auto consume_blk = [&](Tile& t, int b) {
            const int start = c0 + FBS * b;
            const int v_valid = clampi(lim_max - start, 0, FBS);
            const bool masked = start + FBS > lim_min;
            int rv[RG];
#pragma unroll
            for (int u = 0; u < RG; ++u) rv[u] = clampi(lim[u] - start, 0, FBS);
            consume_tile_groups<RG>(st, t, qv, scale_log2, lane, rv, v_valid, masked);
        };
        // two tiles in flight; past the end the prefetch repeats the last tile.
        // (No scheduling barriers here, unlike decode: the compiler's
        // interleaving of one tile's loads and score MFMAs with the other's
        // softmax measured 6% faster.  A third tile in flight, or issuing the
        // next tile's score MFMAs ahead of this tile's softmax, measured no
        // faster.)
        Tile ta, tb;
        load_blk(ta, 0);
        for (int b = 0; b < nblk; b += 2) {
            load_blk(tb, min(b + 1, nblk - 1));
            consume_blk(ta, b);
            if (b + 1 >= nblk) break;
            load_blk(ta, min(b + 2, nblk - 1));
            consume_blk(tb, b + 1);
        }
    }

#pragma unroll
    for (int u = 0; u < RG; ++u) {
        const float lsum = sum_across_rows(st[u].l);
        if (!row_ok[u]) continue;
        if (tok0 >= lim[u]) {                   // nothing of this partition is visible
            if (part == 0 && lim[u] == 0) {
                uint2* o = out_row(u);
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) o[4 * jj + quad] = make_uint2(0u, 0u);
            }
            continue;
        }
        const int my_nparts = (lim[u] + part_tokens - 1) / part_tokens;
        if (my_nparts == 1) {
            const float inv = 1.f / lsum;
            uint2* o = out_row(u);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                o[4 * jj + quad] = make_uint2(pack_bf16x2(st[u].acc[jj][0] * inv, st[u].acc[jj][1] * inv),
                                              pack_bf16x2(st[u].acc[jj][2] * inv, st[u].acc[jj][3] * inv));
            continue;
        }
        const int64_t pidx = (static_cast<int64_t>(qi[u]) * num_q_heads + hq) * max_parts + part;
        f32x4* acc_out = reinterpret_cast<f32x4*>(ws_acc + pidx * FD);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc_out[4 * jj + quad] = st[u].acc[jj];
        if (quad == 0) {
            ws_m[pidx] = st[u].m;
            ws_l[pidx] = lsum;
        }
    }
}

// ---------------------------------------------------------------------------
// The same work with the tiles staged in LDS: a workgroup of W waves takes
// W * RG * 16/g consecutive query tokens of one request and KV head; each tile
// is copied from memory to LDS once per workgroup by the waves together (a
// tile is 64 * D bytes of K and V, D / 16 / W KiB per wave, global_load_lds:
// no registers on the way), and every wave reads
// its MFMA operands from LDS.  Tiles are consumed in pairs (pair_softmax_pv:
// one PV MFMA of K 32 for both), S - 2 tiles ahead of the pair being
// consumed.  One barrier per pair: after it, the pair is in LDS and every
// wave is done with the previous pair, whose stages are then refilled.

// LDS stages (an even number), waves per workgroup sharing them, row groups
// per wave and the occupancy asked of the compiler.  Measured on the
// chunked-prefill workload (us per call, with the loop at 189 us): 4, 6 or 8
// stages 189.0-189.2 alike; 2 waves 249, 8 waves 201; one row group (134
// VGPRs, three waves per SIMD, each tile read from LDS for half as many rows)
// 223, and at four stages held to 128 VGPRs (four waves) 214; three groups
// 280 (one wave per SIMD) or 197 held to 256 VGPRs; four groups 232.  Two
// groups at 194 VGPRs leave two waves per SIMD; held to 168 (three) they
// spill.  With the loop at 159-160 us: 4, 6 or 8 stages 160, 161-162,
// 161-162; 8 waves 165 (171 with 8 stages); three groups held to 256 VGPRs
// 182.
#ifndef PA_PREFILL_STAGES
#define PA_PREFILL_STAGES 6
#endif
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 4
#endif
#ifndef PA_PREFILL_ROW_GROUPS
#define PA_PREFILL_ROW_GROUPS 2
#endif
#ifndef PA_PREFILL_WAVES_PER_SIMD
#define PA_PREFILL_WAVES_PER_SIMD 1
#endif
// The same at head_dim 64 and 256 (tiles of 4 and 16 KiB).  Measured on the
// chunked-prefill shape at those head dims (us per call): D 64 with six or
// eight stages 100 alike, three or four row groups 113-114, two waves 124;
// D 256 with one row group, four waves and four stages 348-360, six stages
// 521, two row groups 373; eight waves (one workgroup per CU) with four, six
// or eight stages 352-358, 340-347 and 355-359.
#ifndef PA_PREFILL_ROW_GROUPS_D64
#define PA_PREFILL_ROW_GROUPS_D64 2
#endif
#ifndef PA_PREFILL_STAGES_D64
#define PA_PREFILL_STAGES_D64 6
#endif
#ifndef PA_PREFILL_WAVES_D64
#define PA_PREFILL_WAVES_D64 4   // (a 4 KiB tile is four 1 KiB copies: at most four waves)
#endif
#ifndef PA_PREFILL_ROW_GROUPS_D256
#define PA_PREFILL_ROW_GROUPS_D256 1
#endif
#ifndef PA_PREFILL_STAGES_D256
#define PA_PREFILL_STAGES_D256 6
#endif
#ifndef PA_PREFILL_WAVES_D256
#define PA_PREFILL_WAVES_D256 8
#endif
constexpr int kPrefillStages = PA_PREFILL_STAGES;
constexpr int kPrefillLdsWaves = PA_PREFILL_WAVES;
constexpr int kPrefillRowGroups = PA_PREFILL_ROW_GROUPS;
template <int D>
constexpr int prefill_row_groups() {
    return D == 64 ? PA_PREFILL_ROW_GROUPS_D64 : (D == 256 ? PA_PREFILL_ROW_GROUPS_D256 : kPrefillRowGroups);
}
template <int D>
constexpr int prefill_stages() {
    return D == 64 ? PA_PREFILL_STAGES_D64 : (D == 256 ? PA_PREFILL_STAGES_D256 : kPrefillStages);
}

// Workgroups start in grid order, and a request's workgroups run about as
// long as its history: when the longest requests come last, their
// workgroups start in the second wave of the grid and set the end of the
// call.  Requests are therefore taken longest first (ties by index): rank r
// of the grid's request axis is the request with the r-th longest length.
// One lane per request ranks it against the others; more than 64 requests
// keep the grid order.
__device__ __forceinline__ int longest_first(const int32_t* __restrict__ context_lens,
                                             int num_seqs, int rank, int len_clamp) {
    if (num_seqs > 64) return rank;
    const int lane = threadIdx.x & 63;
    const int key = lane < num_seqs ? min(max(context_lens[lane], 0), len_clamp) : -1;
    int r = 0;
    for (int t = 0; t < num_seqs; ++t) {
        const int kt = __shfl(key, t);
        r += (kt > key || (kt == key && t < lane)) ? 1 : 0;
    }
    const unsigned long long b = __ballot(lane < num_seqs && r == rank);
    return b ? __ffsll(b) - 1 : rank;
}

template <int RG, int S, int W, int BS, int D>
__global__ __launch_bounds__(64 * W)
__attribute__((amdgpu_waves_per_eu(PA_PREFILL_WAVES_PER_SIMD))) void prefill_lds_kernel(
    const __bf16* __restrict__ k_cache, const __bf16* __restrict__ v_cache,
    const __bf16* __restrict__ q, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int64_t num_blocks, int64_t blk_stride, int total_q, int num_q_heads, int group,
    int tiles_per_seq, int max_blocks_per_seq, int len_clamp, int part_tokens, int max_parts,
    float scale_log2, unsigned q_sign, __bf16* __restrict__ out, float* __restrict__ ws_acc,
    float* __restrict__ ws_m, float* __restrict__ ws_l, int32_t* __restrict__ ws_len) {
    static_assert(W == 2 || W == 4 || W == 8, "waves per workgroup");
    static_assert(S % 2 == 0 && S >= 4, "stages hold whole pairs of tiles");
    static_assert(BS == 8 || BS == 16 || BS == 32 || BS == 64,
                  "blocks of half, one, two or four 16-position tiles");
    constexpr int TL = FBS * D;                   // elements of a 16-position tile
    constexpr int KC = D / 32;                    // 16-byte K chunks per lane and tile
    constexpr int VJ = D / 16;                    // V operands (and accumulators) per lane
    constexpr int KK = D / 32;                    // KiB of the K half of a tile (a power of 2)
    static_assert((2 * KK) % W == 0, "each wave copies whole KiB of every tile");
    constexpr int kCopies = 2 * KK / W;
    constexpr int SUB = BS >= FBS ? BS / FBS : 1;  // tiles per block, back to back in its head region
    // the first block entry of tile t (blocks of 8: a tile is two blocks)
    auto first_entry = [](int t) { return BS == 8 ? 2 * t : t / SUB; };
    __shared__ __align__(16) __bf16 ring[S][2 * TL];      // stage: K tile, then V tile
    const int h = blockIdx.x;
    const int rank = blockIdx.y / tiles_per_seq;
    // a request's last query tokens see the most positions: they go first
    const int wgt = tiles_per_seq - 1 - (blockIdx.y - rank * tiles_per_seq);
    const int seq = longest_first(context_lens, gridDim.y / tiles_per_seq, rank, len_clamp);
    const int part = blockIdx.z;
    const int wave = static_cast<int>(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int row = lane & 15;
    const int quad = lane >> 4;
    auto clampi = [](int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); };
    const int qs = clampi(q_start[seq], 0, total_q);
    const int n = clampi(q_start[seq + 1], qs, total_q) - qs;
    const int tpg = FG / group;
    const int j0w = wgt * W * RG * tpg;          // the workgroup's first query token
    if (j0w >= n) return;                        // (whole workgroup)
    const int j0 = j0w + wave * RG * tpg;        // this wave's
    const bool active = j0 < n;
    const int L = clampi(context_lens[seq], 0, len_clamp);
    const int hq = h * group + row % group;
    int qi[RG], lim[RG];
    bool row_ok[RG];
#pragma unroll
    for (int u = 0; u < RG; ++u) {
        const int j = j0 + u * tpg + row / group;
        row_ok[u] = j < n;
        qi[u] = qs + (row_ok[u] ? j : j0w);
        lim[u] = row_ok[u] ? clampi(L - n + j + 1, 0, L) : 0;
    }
    const int lim_min = clampi(L - n + j0 + 1, 0, L);
    const int lim_max = active ? clampi(L - n + min(j0 + RG * tpg, n), 0, L) : 0;
    const int wg_lim_max = clampi(L - n + min(j0w + W * RG * tpg, n), 0, L);

#pragma unroll
    for (int u = 0; u < RG; ++u)
        if (max_parts > 1 && part == 0 && h == 0 && row_ok[u] && row % group == 0 && quad == 0)
            ws_len[qi[u]] = lim[u];
    auto out_row = [&](int u) {
        return reinterpret_cast<uint2*>(out + (static_cast<int64_t>(qi[u]) * num_q_heads + hq) * D);
    };
    auto zero_rows = [&]() {
#pragma unroll
        for (int u = 0; u < RG; ++u)
            if (part == 0 && row_ok[u] && lim[u] == 0) {
                uint2* o = out_row(u);
#pragma unroll
                for (int jj = 0; jj < VJ; ++jj) o[4 * jj + quad] = make_uint2(0u, 0u);
            }
    };
    const int tok0 = part * part_tokens;
    if (tok0 >= wg_lim_max) {                    // (whole workgroup)
        zero_rows();
        return;
    }
    const int tok1 = min(wg_lim_max, tok0 + part_tokens);

    bf16x8 qv[RG][KC];
    SoftmaxStateT<D> st[RG];
#pragma unroll
    for (int u = 0; u < RG; ++u) {
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(
            q + (static_cast<int64_t>(qi[u]) * num_q_heads + hq) * D);
#pragma unroll
        for (int s4 = 0; s4 < KC; ++s4) {
            typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 v = __builtin_bit_cast(u32x4, qp[4 * s4 + quad]) ^ q_sign;
            qv[u][s4] = row_ok[u] ? __builtin_bit_cast(bf16x8, v) : bf16x8{};
        }
        st[u].m = kNoMaxLog2;
        st[u].l = 0.f;
#pragma unroll
        for (int jj = 0; jj < VJ; ++jj) st[u].acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int blk0 = tok0 / BS;                  // (partitions are whole blocks)
    const int nblk = (tok1 - tok0 + FBS - 1) / FBS;   // tiles of the walk
    const int nent = (tok1 - tok0 + BS - 1) / BS;     // blocks of the walk
    const int32_t* tab = block_tables + static_cast<int64_t>(seq) * max_blocks_per_seq + blk0;
    // the partition's table entries, kTbl at a time, in LDS: the copies need
    // them without a scalar-load wait in the loop
    constexpr int kTbl = 256;
    __shared__ __align__(16) int tbl[kTbl];
    // block entries e0 .. e0 + kTbl - 1; those past the walk repeat its last
    // entry, so a copy past the end reads a valid block
    auto load_tbl = [&](int e0) {
        for (int i = threadIdx.x; i < kTbl; i += 64 * W)
            tbl[i] = clamp_block(tab[min(e0 + i, nent - 1)], num_blocks);
        __syncthreads();
    };
    load_tbl(0);
    const unsigned ring0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) __bf16*)(&ring[0][0])));
    // tile t (past the end: a block of the walk, so every thread issues the
    // same number of copies per tile) into stage t % S; the stage's 2 * KK KiB
    // are K then V, and wave w copies KiB w * kCopies .. (w + 1) * kCopies - 1
    // V stage layout: 16-byte chunk c of the tile sits at chunk c ^ ((c >> 4) & 1)
    // (the two chunks of a dim swap for dims 8..15 of every 16), so the 8-byte
    // reads of rows r and r + 8, 256 bytes apart, fall in different LDS banks.
    const int v_swz_lane = lane ^ ((lane >> 4) & 1);
    // the block offset is wave-uniform: scalar arithmetic, one SGPR base per
    // copy and a fixed per-lane byte offset
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto issue_e = [&](int t, int e) {   // tile t of the walk, from block e
        const int64_t o = static_cast<int64_t>(e) * blk_stride +
                          static_cast<int64_t>(h) * (SUB * TL) + static_cast<int64_t>(t % SUB) * TL;
        const unsigned sb = ring0 + static_cast<unsigned>((t % S) * 2 * TL * 2);
#pragma unroll
        for (int c = 0; c < kCopies; ++c) {
            const int kib = wave_u * kCopies + c;          // K KiB 0..KK-1, then V
            const __bf16* base = (kib < KK ? k_cache : v_cache) + o + (kib & (KK - 1)) * 512;
            const unsigned voff = static_cast<unsigned>((kib < KK ? lane : v_swz_lane) * 16);
            lds_copy16_s(base, voff, sb + kib * 1024);
        }
    };
    // tiles t, t + 1 (t even): both entries in one 8-byte LDS read (one LDS
    // round trip per pair); past the walk the window holds its last entry
    // Blocks of 8: the tile's positions 0..7 come from block ea, 8..15 from
    // eb (per block and head, K [D/8][8][8] and V [D][8]); each lane copies
    // the 16 bytes that land at its LDS chunk, from a vector address.
    auto issue_e8 = [&](int t, int ea, int eb) {
        const unsigned sb = ring0 + static_cast<unsigned>((t % S) * 2 * TL * 2);
        const int64_t oa = static_cast<int64_t>(ea) * blk_stride + static_cast<int64_t>(h) * (8 * D);
        const int64_t ob = static_cast<int64_t>(eb) * blk_stride + static_cast<int64_t>(h) * (8 * D);
#pragma unroll
        for (int c = 0; c < kCopies; ++c) {
            const int kib = wave_u * kCopies + c;          // K KiB 0..KK-1, then V
            const __bf16* src;
            if (kib < KK) {                                // chunk (dims 8c'..8c'+7, position r)
                const int C = (kib & (KK - 1)) * 64 + lane;
                const int cc = C >> 4, r = C & 15;
                src = k_cache + (r < 8 ? oa : ob) + (cc * 8 + (r & 7)) * 8;
            } else {                                       // chunk (dim d, positions 8*half..)
                const int G = (kib & (KK - 1)) * 64 + v_swz_lane;
                src = v_cache + ((G & 1) ? ob : oa) + (G >> 1) * 8;
            }
            lds_copy16(src, __builtin_amdgcn_readfirstlane(sb + kib * 1024));
        }
    };
    // (blocks of 32 or 64: tiles t, t + 1 lie in one block, one entry;
    // blocks of 8: four entries, one 16-byte LDS read)
    auto issue2 = [&](int t) {
        if constexpr (BS == 8) {
            const int4 e = *reinterpret_cast<const int4*>(&tbl[static_cast<unsigned>(2 * t) % kTbl]);
            issue_e8(t, __builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y));
            issue_e8(t + 1, __builtin_amdgcn_readfirstlane(e.z), __builtin_amdgcn_readfirstlane(e.w));
        } else if constexpr (SUB == 1) {
            const int2 e = *reinterpret_cast<const int2*>(&tbl[static_cast<unsigned>(t) % kTbl]);
            issue_e(t, __builtin_amdgcn_readfirstlane(e.x));
            issue_e(t + 1, __builtin_amdgcn_readfirstlane(e.y));
        } else {
            const int e = __builtin_amdgcn_readfirstlane(tbl[static_cast<unsigned>(t / SUB) % kTbl]);
            issue_e(t, e);
            issue_e(t + 1, e);
        }
    };
    // K half of pair b (tiles b, b + 1) into scores: tile b + 1's stage holds
    // landed bytes even past the walk (those copies read a block of the
    // walk), so it is scored unconditionally and masked later when no row
    // sees it
    auto pair_scores = [&](int b, f32x4 (&s_a)[RG], f32x4 (&s_b)[RG]) {
        const __bf16* sa = &ring[b % S][0];
        const __bf16* sb = &ring[(b + 1) % S][0];
        // the 2 * RG accumulation chains of both tiles advance together, one
        // 32-dim step at a time: a dependent MFMA waits about three issue
        // slots for its predecessor, so 2 * RG >= 4 independent chains keep
        // the matrix pipe full where one tile's RG chains left it idle
        const bf16x8* kpa = reinterpret_cast<const bf16x8*>(sa) + lane;
        const bf16x8* kpb = reinterpret_cast<const bf16x8*>(sb) + lane;
        bf16x8 ka[KC], kb[KC];
#pragma unroll
        for (int s4 = 0; s4 < KC; ++s4) {
            ka[s4] = kpa[64 * s4];
            kb[s4] = kpb[64 * s4];
        }
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            s_a[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            s_b[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k = 0; k < KC; ++k)
#pragma unroll
            for (int u = 0; u < RG; ++u) {
                s_a[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[k], qv[u][k], s_a[u], 0, 0, 0);
                s_b[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[k], qv[u][k], s_b[u], 0, 0, 0);
            }
    };
    // V half of pair b, the masks, the softmax and the PV MFMAs
    auto pair_consume = [&](int b, f32x4 (&s_a)[RG], f32x4 (&s_b)[RG]) {
        const int start = tok0 + FBS * b;
        const __bf16* sa = &ring[b % S][0];
        const __bf16* sb = &ring[(b + 1) % S][0];
        const bool has_b = b + 1 < nblk && start + FBS < lim_max;   // (wave-uniform)
        s16x4 va[VJ], vb[VJ];
        const int vo = 2 * ((2 * row + (quad >> 1)) ^ (row >> 3)) + (quad & 1);
        const s16x4* vpa = reinterpret_cast<const s16x4*>(sa + TL) + vo;
        const s16x4* vpb = reinterpret_cast<const s16x4*>(sb + TL) + vo;
        // volatile: the reads stay one per 8 bytes, in this order, and the
        // two tiles' pieces of a dim land side by side as one MFMA
        // operand; merged by the compiler into two-address reads of one
        // tile, they cost 24 register copies per pair (184 -> 169 us)
#pragma unroll
        for (int j = 0; j < VJ; ++j) {
            typedef const volatile __attribute__((address_space(3))) s16x4* lds_v;
            va[j] = *(lds_v)(vpa + 64 * j);
            vb[j] = *(lds_v)(vpb + 64 * j);
        }
        // values past the wave's visible positions may be stale bytes
        const int tok_base = 4 * quad;
        const int va_valid = clampi(lim_max - start, 0, FBS);
        const int vb_valid = has_b ? clampi(lim_max - start - FBS, 0, FBS) : 0;
        if (va_valid < FBS || vb_valid < FBS) {   // (wave-uniform)
#pragma unroll
            for (int j = 0; j < VJ; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (tok_base + i >= va_valid) va[j][i] = 0;
                    if (tok_base + i >= vb_valid) vb[j][i] = 0;
                }
        }
        const bool masked = !has_b || start + 2 * FBS > lim_min;
        int rva[RG], rvb[RG];
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            rva[u] = clampi(lim[u] - start, 0, FBS);
            rvb[u] = has_b ? clampi(lim[u] - start - FBS, 0, FBS) : 0;
        }
        pair_softmax_pv<RG, D>(st, s_a, s_b, va, vb, scale_log2, lane, rva, rvb, masked);
    };
    auto visible = [&](int b) { return tok0 + FBS * b < lim_max; };   // (wave-uniform)
    // Tiles are consumed in pairs (b, b + 1), one barrier per pair; S - 2
    // tiles are in flight while a pair is consumed.
#pragma unroll
    for (int t = 0; t < S - 2; t += 2) issue2(t);
    for (int b = 0; b < nblk; b += 2) {
        wait_vmcnt<kCopies * (S - 4)>();         // this thread's copies of tiles b, b + 1 have landed
        __builtin_amdgcn_s_barrier();            // everyone's; and tiles b - 2, b - 1 are consumed
        const int t_next = b + S - 2;            // refilling their stages
        // (uniform, rare; t_next is even, so it meets the first tile of every block)
        if (t_next % SUB == 0 && first_entry(t_next) % kTbl == 0 && t_next < nblk)
            load_tbl(first_entry(t_next));
        issue2(t_next);
        if (visible(b)) {
            // raised wave priority while a pair is consumed, normal while the
            // wave waits at the barrier and issues copies: the SIMD's other
            // wave (another workgroup) then yields its issue slots to the one
            // doing matrix and softmax work (189 -> 185 us on the chunked-prefill
            // workload; raised only around the MFMAs it was slower)
            __builtin_amdgcn_s_setprio(1);
            __builtin_amdgcn_sched_barrier(0);
            f32x4 s_a[RG], s_b[RG];
            pair_scores(b, s_a, s_b);
            pair_consume(b, s_a, s_b);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
        }
    }
    wait_vmcnt<0>();                             // no copy may land after the workgroup ends
    if (!active) return;

#pragma unroll
    for (int u = 0; u < RG; ++u) {
        const float lsum = sum_across_rows(st[u].l);
        if (!row_ok[u]) continue;
        if (tok0 >= lim[u]) {
            if (part == 0 && lim[u] == 0) {
                uint2* o = out_row(u);
#pragma unroll
                for (int jj = 0; jj < VJ; ++jj) o[4 * jj + quad] = make_uint2(0u, 0u);
            }
            continue;
        }
        const int my_nparts = (lim[u] + part_tokens - 1) / part_tokens;
        if (my_nparts == 1) {
            const float inv = 1.f / lsum;
            uint2* o = out_row(u);
#pragma unroll
            for (int jj = 0; jj < VJ; ++jj)
                o[4 * jj + quad] = make_uint2(pack_bf16x2(st[u].acc[jj][0] * inv, st[u].acc[jj][1] * inv),
                                              pack_bf16x2(st[u].acc[jj][2] * inv, st[u].acc[jj][3] * inv));
            continue;
        }
        const int64_t pidx = (static_cast<int64_t>(qi[u]) * num_q_heads + hq) * max_parts + part;
        f32x4* acc_out = reinterpret_cast<f32x4*>(ws_acc + pidx * D);
#pragma unroll
        for (int jj = 0; jj < VJ; ++jj) acc_out[4 * jj + quad] = st[u].acc[jj];
        if (quad == 0) {
            ws_m[pidx] = st[u].m;
            ws_l[pidx] = lsum;
        }
    }
}

}  // namespace


namespace {

// Short chunks (fewer than 2 * 16/g query tokens): one row group per wave,
// tiles in registers, two waves per workgroup.
int launch_prefill_short(const PrefillArgs& p, float sl2, unsigned q_sign) {
    const DecodeArgs& a = p.d;
    constexpr int W = 2;
    const int per = W * (FG / a.group);
    const int tiles = (p.max_q_len + per - 1) / per;
    dim3 grid(a.num_kv_heads, a.num_seqs * tiles, a.max_parts);
    hipLaunchKernelGGL((prefill_kernel<false, 1, W>), grid, dim3(64 * W), 0, a.stream,
                       static_cast<const __bf16*>(a.k_cache), static_cast<const __bf16*>(a.v_cache),
                       static_cast<const __bf16*>(a.q), p.q_start, a.block_tables, a.context_lens,
                       a.num_blocks, a.block_stride, p.total_q, a.num_q_heads, a.group, tiles,
                       a.max_blocks_per_seq, a.len_clamp, a.part_tokens, a.max_parts,
                       sl2, q_sign, static_cast<__bf16*>(a.out), a.ws_acc, a.ws_m, a.ws_l,
                       p.ws_len);
    return check_launch("prefill");
}

// Longer chunks: waves of a workgroup sharing each tile through LDS; four
// waves with two row groups each at head_dim 64 and 128; at 256 (where a row
// group alone holds 64 accumulator registers) eight waves of one row group
// and a ring of six 16 KiB stages.
template <int BS, int D>
int launch_prefill_lds_bsd(const PrefillArgs& p, float sl2, unsigned q_sign) {
    const DecodeArgs& a = p.d;
    constexpr int RG = prefill_row_groups<D>();
    constexpr int S = prefill_stages<D>();
    constexpr int W = D == 256 ? PA_PREFILL_WAVES_D256 : (D == 64 ? PA_PREFILL_WAVES_D64 : kPrefillLdsWaves);
    const int per = W * RG * (FG / a.group);
    const int tiles = (p.max_q_len + per - 1) / per;
    dim3 grid(a.num_kv_heads, a.num_seqs * tiles, a.max_parts);
    hipLaunchKernelGGL((prefill_lds_kernel<RG, S, W, BS, D>), grid, dim3(64 * W), 0, a.stream,
                       static_cast<const __bf16*>(a.k_cache), static_cast<const __bf16*>(a.v_cache),
                       static_cast<const __bf16*>(a.q), p.q_start, a.block_tables, a.context_lens,
                       a.num_blocks, a.block_stride, p.total_q, a.num_q_heads, a.group, tiles,
                       a.max_blocks_per_seq, a.len_clamp, a.part_tokens, a.max_parts,
                       sl2, q_sign, static_cast<__bf16*>(a.out), a.ws_acc, a.ws_m, a.ws_l,
                       p.ws_len);
    return check_launch("prefill");
}

template <int D>
int launch_prefill_lds_d(const PrefillArgs& p, float sl2, unsigned q_sign) {
    switch (p.d.block_size) {
        case 8: return launch_prefill_lds_bsd<8, D>(p, sl2, q_sign);
        case 16: return launch_prefill_lds_bsd<16, D>(p, sl2, q_sign);
        case 32: return launch_prefill_lds_bsd<32, D>(p, sl2, q_sign);
        case 64: return launch_prefill_lds_bsd<64, D>(p, sl2, q_sign);
        default: return fail(PA_ERR_UNSUPPORTED, "prefill: block size %d", p.d.block_size);
    }
}

int launch_prefill_lds(const PrefillArgs& p, float sl2, unsigned q_sign) {
    switch (p.d.head_dim) {
        case 64: return launch_prefill_lds_d<64>(p, sl2, q_sign);
        case 128: return launch_prefill_lds_d<128>(p, sl2, q_sign);
        case 256: return launch_prefill_lds_d<256>(p, sl2, q_sign);
        default: return fail(PA_ERR_UNSUPPORTED, "prefill: head_dim %d", p.d.head_dim);
    }
}

}  // namespace

int launch_prefill(const PrefillArgs& p) {
    const DecodeArgs& a = p.d;
    if (a.num_seqs == 0 || p.max_q_len == 0) return PA_OK;
    // the tile consumer takes a positive scale: a negative one flips the sign
    // of q instead (exact in bf16), zero becomes the least normal float
    // (every score then rounds to 0 in the exponent, as with scale 0)
    const float sl2 = fmaxf(fabsf(a.scale) * kLog2e, FLT_MIN);
    const unsigned q_sign = a.scale < 0.f ? 0x80008000u : 0u;
    // two row groups per wave once a chunk fills them: half the tile reads
    // (measured on the chunked-prefill workload with tiles in registers: 1
    // group 431 us, 2 groups 273 us, 4 groups 368 us -- 332 VGPRs leave one
    // wave per SIMD; staging the tiles in LDS then took it to 217 us)
    const bool lds = p.max_q_len >= 2 * (FG / a.group);
    if (!lds && (a.block_size != FBS || a.head_dim != FD))   // (the host runs such calls as decodes)
        return fail(PA_ERR_UNSUPPORTED, "prefill: short chunks need blocks of 16 and head_dim 128");
    const int st = lds ? launch_prefill_lds(p, sl2, q_sign) : launch_prefill_short(p, sl2, q_sign);
    if (st != PA_OK || a.max_parts <= 1 || p.total_q == 0) return st;
    return launch_merge(p.ws_len, p.total_q, a.num_q_heads, a.head_dim, a.len_clamp, a.part_tokens,
                        a.max_parts, a.ws_acc, a.ws_m, a.ws_l, a.out, a.stream);
}

// ----------------------------------------------------------------------------
// Shapes outside the MFMA prefill kernels: each query row as a decode request
// ----------------------------------------------------------------------------
//
// Row r of request i sees the first L_i - n_i + j + 1 positions of i's
// history (j = r - q_start[i]); that is a decode over i's block table cut at
// that length.  This kernel gives every row its own copy of the first
// row_blocks entries of i's table row and its visible length, so the decode
// kernels run the chunk unchanged with one request per row.  Workgroup r
// finds its request by binary search over q_start: the largest i with
// q_start[i] <= r (empty requests in between are skipped that way).  A row
// that falls in no request's range (a q_start that is not a partition of
// [0, total_q)) gets length 0 and decodes to zeros.
__global__ __launch_bounds__(64) void prefill_rows_kernel(
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int num_seqs, int max_blocks_per_seq,
    int row_blocks, int len_clamp, int32_t* __restrict__ row_tables,
    int32_t* __restrict__ row_lens) {
    const int r = blockIdx.x;
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (q_start[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    const int qs = q_start[lo];
    const int n = q_start[lo + 1] - qs;
    const int j = r - qs;
    const int L = min(max(context_lens[lo], 0), len_clamp);
    const int vis = (j >= 0 && j < n) ? min(max(L - n + j + 1, 0), L) : 0;
    if (threadIdx.x == 0) row_lens[r] = vis;
    const int32_t* src = block_tables + static_cast<int64_t>(lo) * max_blocks_per_seq;
    int32_t* dst = row_tables + static_cast<int64_t>(r) * row_blocks;
    for (int b = threadIdx.x; b < row_blocks; b += 64) dst[b] = src[b];
}

int launch_prefill_rows(const int32_t* q_start, const int32_t* block_tables,
                        const int32_t* context_lens, int32_t num_seqs, int32_t total_q,
                        int32_t max_blocks_per_seq, int32_t row_blocks, int32_t len_clamp,
                        int32_t* row_tables, int32_t* row_lens, hipStream_t stream) {
    if (num_seqs == 0 || total_q == 0) return PA_OK;
    hipLaunchKernelGGL(prefill_rows_kernel, dim3(total_q), dim3(64), 0, stream, q_start,
                       block_tables, context_lens, num_seqs, max_blocks_per_seq, row_blocks,
                       len_clamp, row_tables, row_lens);
    return check_launch("prefill rows");
}

}  // namespace pa
