// Several query tokens per request over a paged KV cache, gfx950: a chunk
// of a prompt after a prefix-cache hit, a chunked prefill, or several tokens
// checked at once.  Built from the MFMA tile of the decode kernels
// (pa_tile.h); the split-K merge is decode's (launch_merge).

#include <float.h>

#include "pa_tile.h"


namespace pa {
namespace {

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
// are those of decode, per query row.
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

}  // namespace

#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 2
#endif

template <int RG>
int launch_prefill_rg(const PrefillArgs& p) {
    const DecodeArgs& a = p.d;
    constexpr int W = PA_PREFILL_WAVES;
    // the tile consumer takes a positive scale: a negative one flips the sign
    // of q instead (exact in bf16), zero becomes the least normal float
    // (every score then rounds to 0 in the exponent, as with scale 0)
    const float sl2 = fmaxf(fabsf(a.scale) * kLog2e, FLT_MIN);
    const unsigned q_sign = a.scale < 0.f ? 0x80008000u : 0u;
    const int per = W * RG * (FG / a.group);
    const int tiles = (p.max_q_len + per - 1) / per;
    dim3 grid(a.num_kv_heads, a.num_seqs * tiles, a.max_parts);
    hipLaunchKernelGGL((prefill_kernel<false, RG, W>), grid, dim3(64 * W), 0, a.stream,
                       static_cast<const __bf16*>(a.k_cache), static_cast<const __bf16*>(a.v_cache),
                       static_cast<const __bf16*>(a.q), p.q_start, a.block_tables, a.context_lens,
                       a.num_blocks, a.block_stride, p.total_q, a.num_q_heads, a.group, tiles,
                       a.max_blocks_per_seq, a.len_clamp, a.part_tokens, a.max_parts,
                       sl2, q_sign, static_cast<__bf16*>(a.out), a.ws_acc, a.ws_m, a.ws_l,
                       p.ws_len);
    return check_launch("prefill");
}

int launch_prefill(const PrefillArgs& p) {
    const DecodeArgs& a = p.d;
    if (a.num_seqs == 0 || p.max_q_len == 0) return PA_OK;
    // two row groups per wave once a chunk fills them: half the tile reads
    // (measured on the chunked-prefill workload: 1 group 431 us, 2 groups
    // 273 us, 4 groups 368 us -- 332 VGPRs leave one wave per SIMD)
    const int st = p.max_q_len >= 2 * (FG / a.group) ? launch_prefill_rg<2>(p) : launch_prefill_rg<1>(p);
    if (st != PA_OK || a.max_parts <= 1 || p.total_q == 0) return st;
    return launch_merge(p.ws_len, p.total_q, a.num_q_heads, a.len_clamp, a.part_tokens, a.max_parts,
                        a.ws_acc, a.ws_m, a.ws_l, a.out, a.stream);
}

}  // namespace pa
