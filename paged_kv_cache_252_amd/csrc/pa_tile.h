// Device-side building blocks shared by the MFMA attention kernels (decode,
// grouped decode, several-token prefill): bf16 vector types, the 16-token
// K/V tile in MFMA operand layout and its loads and stores, the online-softmax
// state and the tile consumer.  Layout of a tile: see pa_internal.h.
#pragma once

#include <math.h>

#include <type_traits>

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


constexpr int FD = 128;          // head_dim of the grouped, prefix-run and prefill kernels
constexpr int FBS = 16;          // positions per tile (block_size 16)
constexpr int FTILE = FD * FBS;  // elements of one (block, head) tile at head_dim 128
constexpr int FG = 16;           // query rows of the score MFMA

// Element types of the MFMA tiles: a K chunk is 16 bytes (X elements), a V
// group the four positions 4*(l/16)..+3 of one dim.
template <typename E> struct ElemT;
template <> struct ElemT<__bf16> {
    using KChunk = bf16x8;
    using VGroup = s16x4;
    static constexpr int X = 8;
};
template <> struct ElemT<float> {
    using KChunk = f32x4;
    using VGroup = f32x4;
    static constexpr int X = 4;
};

// One 16-position tile of head_dim D (a multiple of 32, at most 256) in MFMA
// operand layout; element type E (bf16, or fp32 for the fp32 MFMAs).
template <int D, typename E = __bf16>
struct TileT {
    static_assert(D % 32 == 0 && D >= 32 && D <= 256, "head_dim a multiple of 32, at most 256");
    static constexpr int KC = D / (4 * ElemT<E>::X);   // K chunks per lane
    typename ElemT<E>::KChunk k[KC];   // K: chunk (4*s + l/16), token l%16
    typename ElemT<E>::VGroup v[D / 16];   // V: dim 16*j + l%16, tokens 4*(l/16)..+3
};
using Tile = TileT<FD>;

// NT: non-temporal loads (streaming hint), for batches without shared blocks.
template <bool NT, typename V>
__device__ __forceinline__ V load16(const V* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT, int D, typename E>
__device__ __forceinline__ void load_tile(TileT<D, E>& t, const E* __restrict__ k_tile,
                                          const E* __restrict__ v_tile, int lane) {
    using KC = typename ElemT<E>::KChunk;
    using VG = typename ElemT<E>::VGroup;
    const KC* kp = reinterpret_cast<const KC*>(k_tile) + lane;
#pragma unroll
    for (int s = 0; s < TileT<D, E>::KC; ++s) t.k[s] = load16<NT>(kp + 64 * s);
    const VG* vp = reinterpret_cast<const VG*>(v_tile) + (lane & 15) * 4 + (lane >> 4);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) t.v[j] = load16<NT>(vp + 64 * j);
}

// The inverse of load_tile: the tile's bytes back to a block (whole lines),
// with the non-temporal hint (measured: 2.4 us less on the fan-out step).
template <int D, typename E>
__device__ __forceinline__ void store_tile(const TileT<D, E>& t, E* __restrict__ k_tile,
                                           E* __restrict__ v_tile, int lane) {
    using KC = typename ElemT<E>::KChunk;
    using VG = typename ElemT<E>::VGroup;
    KC* kp = reinterpret_cast<KC*>(k_tile) + lane;
#pragma unroll
    for (int s = 0; s < TileT<D, E>::KC; ++s) __builtin_nontemporal_store(t.k[s], kp + 64 * s);
    VG* vp = reinterpret_cast<VG*>(v_tile) + (lane & 15) * 4 + (lane >> 4);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) __builtin_nontemporal_store(t.v[j], vp + 64 * j);
}

// The same tile out of blocks of BS tokens: tile `sub` of one block when BS
// is a multiple of 16 (the block holds BS/16 such tiles back to back); for
// BS = 8 (K [D/8][8][8], V [D][8] per head) the tile's first 8 tokens come
// from block `a`, the next 8 from block `b` (K rows 8..15 and V token groups
// 2..3).  k_a/v_a, k_b/v_b point at the head's region in blocks a and b.
template <bool NT, int BS, int D, typename E>
__device__ __forceinline__ void load_tile_bs(TileT<D, E>& t, const E* __restrict__ k_a,
                                             const E* __restrict__ v_a,
                                             const E* __restrict__ k_b,
                                             const E* __restrict__ v_b, int sub, int lane) {
    using KC = typename ElemT<E>::KChunk;
    using VG = typename ElemT<E>::VGroup;
    const int row = lane & 15, quad = lane >> 4;
    if constexpr (BS >= 16) {                 // tile `sub` of the block: a 16-position tile
        load_tile<NT>(t, k_a + sub * (D * FBS), v_a + sub * (D * FBS), lane);
    } else {
        static_assert(BS == 8, "blocks of 8, 16, 32 or 64 tokens");
        const KC* kp = reinterpret_cast<const KC*>(row < 8 ? k_a : k_b) + (row & 7);
#pragma unroll
        for (int s = 0; s < TileT<D, E>::KC; ++s) t.k[s] = load16<NT>(kp + (4 * s + quad) * 8);
        const VG* vp = reinterpret_cast<const VG*>(quad < 2 ? v_a : v_b) + row * 2 + (quad & 1);
#pragma unroll
        for (int j = 0; j < D / 16; ++j) t.v[j] = load16<NT>(vp + 32 * j);
    }
}

template <int D>
struct SoftmaxStateT {
    float m;            // running max of log2-domain scores for query row lane%16
    float l;            // this lane's share of the running sum
    f32x4 acc[D / 16];  // output accumulator: dims 16*j + 4*(lane/16) + i of row lane%16
};
using SoftmaxState = SoftmaxStateT<FD>;

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

__device__ __forceinline__ f32x4 fma4(f32x4 a, float w, f32x4 c) {
    return f32x4{__builtin_fmaf(a[0], w, c[0]), __builtin_fmaf(a[1], w, c[1]),
                 __builtin_fmaf(a[2], w, c[2]), __builtin_fmaf(a[3], w, c[3])};
}

// Two floats to bf16 (round to nearest even), lo in the low half: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// One block of 16 tokens for rows with their own visibility.  row_valid:
// tokens of this tile visible to this lane's row (applied when `masked`);
// v_valid: tokens whose V may be read (the rest are zeroed); rows that have
// seen nothing yet stay at m = -inf.  The running maximum is moved lazily: a row's reference maximum is
// raised only when a new score exceeds it by more than kLazyMaxLog2
// (probabilities then stay below 2^kLazyMaxLog2, safe in bf16 and fp32), and
// the rescale of the 32 accumulator registers runs only when some row of the
// wave raised it.  The result is the same softmax up to rounding (any
// reference value cancels between numerator and denominator, and the merge
// rescales partitions by their own reference values); it saves VALU work
// where the VALU, not memory, bounds the loop.
constexpr float kLazyMaxLog2 = 8.f;

template <int D, typename E>
__device__ __forceinline__ void consume_tile_rows(SoftmaxStateT<D>& st, TileT<D, E>& t,
                                                  const typename ElemT<E>::KChunk (&qv)[TileT<D, E>::KC],
                                                  float scale_log2, int lane, int row_valid,
                                                  int v_valid, bool masked) {
    constexpr bool F32 = std::is_same<E, float>::value;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (F32) {
        // fp32: K 4 per MFMA; at step (k, e) the lanes of quad q hold dim 16k + 4q + e
        // of their token (A) and of their query row (B)
#pragma unroll
        for (int k = 0; k < TileT<D, E>::KC; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s = __builtin_amdgcn_mfma_f32_16x16x4f32(t.k[k][e], qv[k][e], s, 0, 0, 0);
    } else {
#pragma unroll
        for (int k = 0; k < TileT<D, E>::KC; ++k)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[k], qv[k], s, 0, 0, 0);
    }
    const int tok_base = 4 * (lane >> 4);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = s[i] * scale_log2;
    if (masked) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (tok_base + i >= row_valid) sc[i] = -INFINITY;
    }
    if (v_valid < FBS) {   // (wave-uniform) values past the history may be stale bytes
#pragma unroll
        for (int j = 0; j < D / 16; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tok_base + i >= v_valid) t.v[j][i] = 0;
    }
    const float mx = max_across_rows(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const bool raise = mx > st.m + kLazyMaxLog2;   // false for rows that see nothing
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform
        const float alpha = raise ? fast_exp2(st.m - mx) : 1.f;
        st.m = raise ? mx : st.m;
        st.l *= alpha;
#pragma unroll
        for (int j = 0; j < D / 16; ++j) st.acc[j] *= alpha;
    }
    const bool dead = st.m == -INFINITY;           // nothing visible to this row yet
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = dead ? 0.f : fast_exp2(sc[i] - st.m);
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
    if constexpr (F32) {
        // fp32: step e takes positions 4q + e of every quad q; the lane holds
        // those probabilities (p[e]) and values (v[j][e]) already
#pragma unroll
        for (int j = 0; j < D / 16; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                st.acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.v[j][e], p[e], st.acc[j], 0, 0, 0);
    } else {
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 pp = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
        const s16x4 pb = __builtin_bit_cast(s16x4, pp);
#pragma unroll
        for (int j = 0; j < D / 16; ++j)
            st.acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[j], pb, st.acc[j], 0, 0, 0);
    }
}

// Maximum of floats on the VALU without the quieting of signalling NaNs that
// fmaxf needs in IEEE mode (inputs here are MFMA sums or -inf, never NaN).
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float vmax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmax_across_rows(float x) {
    const unsigned u = __float_as_uint(x);
    auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned w = __float_as_uint(y);
    auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Reference maximum of a row that has seen no score yet: finite, so that
// exp2(score * scale - m) needs no special case (a masked score is -inf and
// gives 0; any visible score raises the maximum past it).
constexpr float kNoMaxLog2 = -1e30f;

// consume_tile_rows for RG groups of 16 rows that read the same tile (same
// arithmetic per row): every group's score MFMAs are issued first, the V
// masking is done once, and one branch covers the rescale of all groups, so
// the matrix work of one group overlaps the softmax of another (a score
// step, tile_scores, and the rest, tile_softmax_pv).  The scale is folded
// into the exponent: `scale_log2` must be positive (a
// negative scale is applied by negating q, a zero one replaced by the least
// normal float), the row maximum is taken over raw scores and scaled once,
// and p = exp2(fma(s, scale_log2, -m)); rows start at m = kNoMaxLog2.
template <int RG>
__device__ __forceinline__ void tile_scores(f32x4 (&s)[RG], const Tile& t,
                                            const bf16x8 (&qv)[RG][4]) {
#pragma unroll
    for (int u = 0; u < RG; ++u) s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int u = 0; u < RG; ++u)
            s[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[k], qv[u][k], s[u], 0, 0, 0);
}

template <int RG>
__device__ __forceinline__ void tile_softmax_pv(SoftmaxState (&st)[RG], f32x4 (&s)[RG], Tile& t,
                                                float scale_log2, int lane,
                                                const int (&row_valid)[RG], int v_valid,
                                                bool masked) {
    const int tok_base = 4 * (lane >> 4);
    if (v_valid < FBS) {   // (wave-uniform) values past the history may be stale bytes
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tok_base + i >= v_valid) t.v[j][i] = 0;
    }
    float mx[RG];
    bool raise[RG];
    bool any = false;
#pragma unroll
    for (int u = 0; u < RG; ++u) {
        if (masked) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tok_base + i >= row_valid[u]) s[u][i] = -INFINITY;
        }
        mx[u] = vmax_across_rows(vmax3(s[u][0], s[u][1], vmax(s[u][2], s[u][3]))) * scale_log2;
        raise[u] = mx[u] > st[u].m + kLazyMaxLog2;
        any = any || raise[u];
    }
    if (__builtin_amdgcn_ballot_w64(any) != 0) {   // wave-uniform
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            const float alpha = raise[u] ? fast_exp2(st[u].m - mx[u]) : 1.f;
            st[u].m = raise[u] ? mx[u] : st[u].m;
            st[u].l *= alpha;
#pragma unroll
            for (int j = 0; j < 8; ++j) st[u].acc[j] *= alpha;
        }
    }
#pragma unroll
    for (int u = 0; u < RG; ++u) {
        const float nm = -st[u].m;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(__builtin_fmaf(s[u][i], scale_log2, nm));
        st[u].l += (p[0] + p[1]) + (p[2] + p[3]);
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 pp = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
        const s16x4 pb = __builtin_bit_cast(s16x4, pp);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            st[u].acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[j], pb, st[u].acc[j], 0, 0, 0);
    }
}

template <int RG>
__device__ __forceinline__ void consume_tile_groups(SoftmaxState (&st)[RG], Tile& t,
                                                    const bf16x8 (&qv)[RG][4], float scale_log2,
                                                    int lane, const int (&row_valid)[RG],
                                                    int v_valid, bool masked) {
    f32x4 s[RG];
    tile_scores<RG>(s, t, qv);
    tile_softmax_pv<RG>(st, s, t, scale_log2, lane, row_valid, v_valid, masked);
}

// One block of 16 tokens seen alike by every row: `valid` of its tokens are
// visible (16 except in the last block of a request).
template <int D, typename E>
__device__ __forceinline__ void consume_tile(SoftmaxStateT<D>& st, TileT<D, E>& t,
                                             const typename ElemT<E>::KChunk (&qv)[TileT<D, E>::KC],
                                             float scale_log2, int lane, int valid) {
    consume_tile_rows<D, E>(st, t, qv, scale_log2, lane, valid, valid, valid < FBS);
}

// 16 bytes per lane from gptr to LDS at lds_base + lane * 16 (lds_base
// wave-uniform; that lane layout was checked on the device).  In asm so that
// the compiler does not wait for every LDS copy before each LDS read; the
// loop waits itself, by count.  M0 is set here and used by nothing else in
// these kernels.
__device__ __forceinline__ void lds_copy16(const void* gptr, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gptr), "s"(lds_base) : "memory");
}

// The same copy addressed as a wave-uniform base (SGPR pair) plus a 32-bit
// per-lane byte offset: no 64-bit vector address arithmetic per copy.
__device__ __forceinline__ void lds_copy16_s(const void* sbase, unsigned voff, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(lds_base) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {   // at most N vector memory ops outstanding
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace
}  // namespace pa
