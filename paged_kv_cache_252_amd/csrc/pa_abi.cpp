// C ABI of libpagedkv: argument checks, split-K planning, optional host-side
// validation of device index arrays, and dispatch to the kernels.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "pa_internal.h"

namespace pa {

namespace {
thread_local std::string g_last_error;

constexpr int kMaxPartitionTokens = 1024;   // fast path: one table entry per lane of a wave
constexpr int kMinAutoPartitionTokens = 64;
// Partition plan: the longest partitions (fewest partials to merge, least
// per-wave set-up) that still give about this many waves per CU when every
// request is as long as the longest.  Measured on MI355X: 1024-token
// partitions beat 256-512 on the GQA, long-context and shared-prefix
// workloads, where even at 1024 there are >= 2 waves per CU.
constexpr int kWavesPerCu = 2;
constexpr int kMaxGridYZ = 65535;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return PA_OK;
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return PA_OK;
}

bool validate_enabled() {
    const char* v = std::getenv("PA_VALIDATE");
    return v != nullptr && v[0] == '1';
}

int check_desc(const pa_cache_desc_t* c) {
    if (c == nullptr) return fail(PA_ERR_NULL, "cache descriptor is NULL");
    if (c->dtype != PA_F32 && c->dtype != PA_BF16) return fail(PA_ERR_DTYPE, "unknown dtype %d", c->dtype);
    if (c->num_blocks < 1) return fail(PA_ERR_SHAPE, "num_blocks must be >= 1 (got %lld)", (long long)c->num_blocks);
    if (c->block_size < 1 || c->block_size > 256)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d outside [1, 256]", c->block_size);
    if (c->num_kv_heads < 1 || c->num_kv_heads > kMaxGridYZ)
        return fail(PA_ERR_SHAPE, "num_kv_heads %d outside [1, %d]", c->num_kv_heads, kMaxGridYZ);
    switch (c->head_dim) {
        case 16: case 32: case 64: case 128: case 256: break;
        default: return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {16, 32, 64, 128, 256}", c->head_dim);
    }
    if (c->block_stride != 0) {
        if (c->block_stride < block_elems(c))
            return fail(PA_ERR_SHAPE, "block_stride %lld is smaller than one block (%lld elements)",
                        (long long)c->block_stride, (long long)block_elems(c));
        if ((c->block_stride * elem_bytes(c->dtype)) % 16 != 0)
            return fail(PA_ERR_ALIGN, "block_stride %lld elements is not a multiple of 16 bytes",
                        (long long)c->block_stride);
    }
    return PA_OK;
}

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

namespace {

int granule(const pa_cache_desc_t* c, int group) {
    return fast_decode_ok(c, group) ? fast_granule(c->block_size) : c->block_size;
}

int max_partition(const pa_cache_desc_t* c, int group) {
    return fast_decode_ok(c, group) ? fast_max_partition(c->block_size) : kMaxPartitionTokens;
}

int32_t plan_partition(const pa_cache_desc_t* c, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_context_len) {
    const int group = num_q_heads / c->num_kv_heads;
    const int g = granule(c, group);
    const int cap = (max_partition(c, group) / g) * g;
    if (max_context_len <= 0) return g;
    const int64_t units = static_cast<int64_t>(num_seqs) * (fast_decode_ok(c, group) ? c->num_kv_heads : num_q_heads);
    const int64_t target = static_cast<int64_t>(device_cu_count()) * kWavesPerCu;
    int64_t p = ceil_div(static_cast<int64_t>(max_context_len) * std::max<int64_t>(units, 1), target);
    p = std::max<int64_t>(p, kMinAutoPartitionTokens);
    p = ceil_div(p, g) * g;
    p = std::min<int64_t>(p, cap);
    if (p >= max_context_len) p = std::min<int64_t>(ceil_div(max_context_len, g) * g, cap);
    return static_cast<int32_t>(std::max<int64_t>(p, g));
}

// Workspace layout: the partials acc [S][Hq][parts][D], then m and l
// [S][Hq][parts], all fp32.
size_t workspace_bytes(const pa_cache_desc_t* c, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_context_len, int32_t part) {
    const int64_t max_parts = ceil_div(std::max(max_context_len, 0), part);
    if (max_parts <= 1) return 0;
    return static_cast<size_t>(num_seqs) * num_q_heads * max_parts * (c->head_dim + 2) * sizeof(float);
}

// Host copies of small device arrays, for PA_VALIDATE=1.
template <typename T>
int fetch(std::vector<T>& host, const T* dev, size_t n, hipStream_t stream) {
    host.resize(n);
    if (n == 0) return PA_OK;
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipMemcpy(host.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "PA_VALIDATE copy failed: %s", hipGetErrorString(e));
    return PA_OK;
}

int resolve_partition(const pa_cache_desc_t* c, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_context_len, int32_t requested, int32_t* out) {
    if (requested == 0) {
        *out = plan_partition(c, num_seqs, num_q_heads, max_context_len);
        return PA_OK;
    }
    const int group = num_q_heads / c->num_kv_heads;
    const int g = granule(c, group);
    const int cap = max_partition(c, group);
    if (requested < c->block_size || requested > cap || requested % g != 0)
        return fail(PA_ERR_SHAPE,
                    "partition_tokens %d must be a multiple of %d in [%d, %d]", requested, g,
                    c->block_size, cap);
    *out = requested;
    return PA_OK;
}

int check_heads(const pa_cache_desc_t* c, int32_t num_seqs, int32_t num_q_heads) {
    if (num_seqs < 0 || num_seqs > kMaxGridYZ)
        return fail(PA_ERR_SHAPE, "num_seqs %d outside [0, %d]", num_seqs, kMaxGridYZ);
    if (num_q_heads < 1 || num_q_heads > kMaxGridYZ || num_q_heads % c->num_kv_heads != 0)
        return fail(PA_ERR_SHAPE, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                    num_q_heads, c->num_kv_heads);
    return PA_OK;
}

// Several query tokens per request: 16 / g tokens per wave.  The LDS kernel
// takes blocks of 8, 16, 32 or 64; the kernel for short chunks (fewer than
// two row groups of tokens) blocks of 16 only.
bool prefill_mfma_ok(const pa_cache_desc_t* c, int group, int32_t max_q_len) {
    const int bs = c->block_size, d = c->head_dim;
    if (c->dtype != PA_BF16 || (d != 64 && d != 128 && d != 256) || group < 1 || group > 16 ||
        16 % group != 0 || (bs != 8 && bs != 16 && bs != 32 && bs != 64))
        return false;
    // chunks shorter than two query tiles per wave: the register-tile
    // kernel, which takes blocks of 16 at head_dim 128 only
    return max_q_len >= 2 * (16 / group) || (bs == 16 && d == 128);
}

int prefill_granule(const pa_cache_desc_t* c) { return c->block_size > 16 ? c->block_size : 16; }

int64_t prefill_waves_rows(int32_t num_seqs, int32_t max_q_len, int group) {
    const int per = 16 / group;
    return static_cast<int64_t>(num_seqs) * ceil_div(std::max(max_q_len, 0), per);
}

// The partials of decode's layout for total_q rows, then the rows' visible
// lengths [total_q] int32 (for the merge).
size_t prefill_workspace(const pa_cache_desc_t* c, int32_t total_q, int32_t num_q_heads,
                         int32_t max_context_len, int32_t part) {
    const size_t partials = workspace_bytes(c, total_q, num_q_heads, max_context_len, part);
    if (partials == 0) return 0;
    return partials + static_cast<size_t>(ceil_div(static_cast<int64_t>(total_q) * 4, 16) * 16);
}

// Shapes without an MFMA prefill kernel run each query row as a decode
// request.  Workspace: the rows' table copies [total_q][row_blocks] int32,
// their visible lengths [total_q] int32, then decode's partials for total_q
// rows, each part starting on a 16-byte boundary.
int32_t prefill_row_blocks(const pa_cache_desc_t* c, int32_t max_context_len) {
    return static_cast<int32_t>(std::max<int64_t>(1, ceil_div(std::max(max_context_len, 0), c->block_size)));
}

size_t round16(size_t n) { return (n + 15) / 16 * 16; }

size_t prefill_rows_workspace(const pa_cache_desc_t* c, int32_t total_q, int32_t num_q_heads,
                              int32_t max_context_len, int32_t part) {
    if (total_q <= 0) return 0;
    const size_t rows = static_cast<size_t>(total_q);
    return round16(rows * prefill_row_blocks(c, max_context_len) * sizeof(int32_t)) +
           round16(rows * sizeof(int32_t)) +
           workspace_bytes(c, total_q, num_q_heads, max_context_len, part);
}

// A prefill wave walks any number of 64-block chunks, so its partition is not
// capped at 1024 tokens: the history is split only when there are too few
// (request, query tile, KV head) waves to fill the device.
constexpr int32_t kMaxPrefillPartitionTokens = 1 << 20;

int prefill_partition(const pa_cache_desc_t* c, int32_t num_seqs, int32_t max_q_len,
                      int32_t num_q_heads, int32_t max_context_len, int32_t requested,
                      int32_t* out) {
    const int g = prefill_granule(c);
    if (requested != 0) {
        if (requested < g || requested > kMaxPrefillPartitionTokens || requested % g != 0)
            return fail(PA_ERR_SHAPE, "partition_tokens %d must be a multiple of %d in [%d, %d]",
                        requested, g, g, kMaxPrefillPartitionTokens);
        *out = requested;
        return PA_OK;
    }
    const int64_t waves = prefill_waves_rows(num_seqs, max_q_len, num_q_heads / c->num_kv_heads) *
                          c->num_kv_heads;
    const int64_t target = static_cast<int64_t>(device_cu_count()) * kWavesPerCu;
    const int64_t whole = std::max<int64_t>(ceil_div(std::max(max_context_len, 1), g) * g, g);
    const int64_t splits = std::max<int64_t>(1, ceil_div(target, std::max<int64_t>(waves, 1)));
    int64_t p = ceil_div(ceil_div(whole, splits), g) * g;
    p = std::max<int64_t>(std::min<int64_t>(p, whole), std::min<int64_t>(whole, kMinAutoPartitionTokens));
    *out = static_cast<int32_t>(std::min<int64_t>(p, kMaxPrefillPartitionTokens));
    return PA_OK;
}

// Scratch for pa_decode_step_noalloc: the split-K partials live in this
// file-scope device array instead of a caller's workspace.  Every GPU the
// library runs on holds its own copy from module load until the process
// ends.  Host code never passes `scratch` itself to a kernel (on the host
// that name is only a stand-in for the symbol); it passes the device address
// hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kNoallocScratchBytes = PA_DECODE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call
// made with that device current.
int noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PA_ERR_UNSUPPORTED, "device %d outside [0, %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace
}  // namespace pa

using namespace pa;

static int decode_impl(const char* fn, const pa_cache_desc_t* c, const void* k_cache,
                       const void* v_cache, const void* k_new, const void* v_new,
                       const int32_t* cow_src, const void* q,
                       const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_q_heads, int32_t max_blocks_per_seq, int32_t max_context_len,
                       float scale, void* out, void* workspace, size_t workspace_bytes_given,
                       int32_t partition_tokens, uint32_t flags, void* stream) {
    int st = check_desc(c);
    if (st) return st;
    if ((st = check_heads(c, num_seqs, num_q_heads))) return st;
    if (max_blocks_per_seq < 1) return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
    if (max_context_len < 0) return fail(PA_ERR_SHAPE, "max_context_len %d < 0", max_context_len);
    if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * c->block_size)
        return fail(PA_ERR_SHAPE, "max_context_len %d exceeds max_blocks_per_seq * block_size = %lld",
                    max_context_len, static_cast<long long>(max_blocks_per_seq) * c->block_size);
    if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "scale is not finite");
    if (flags & ~(PA_DECODE_STREAM_KV | PA_DECODE_GROUP_SHARED | PA_DECODE_PREFIX_RUNS |
                  PA_DECODE_APPEND_TILES))
        return fail(PA_ERR_UNSUPPORTED, "unknown decode flags 0x%x", flags);
    if (num_seqs == 0) return ok();
    if (!k_cache || !v_cache || !q || !block_tables || !context_lens || !out)
        return fail(PA_ERR_NULL, "%s: a required pointer is NULL", fn);
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(out))
        return fail(PA_ERR_ALIGN, "%s: caches, q and out must be 16-byte aligned", fn);
    if (k_new != nullptr || v_new != nullptr) {
        if (!k_new || !v_new) return fail(PA_ERR_NULL, "%s: k_new and v_new are both required", fn);
        if (!aligned16(k_new) || !aligned16(v_new))
            return fail(PA_ERR_ALIGN, "%s: k_new and v_new must be 16-byte aligned", fn);
    }
    int32_t part = 0;
    if ((st = resolve_partition(c, num_seqs, num_q_heads, max_context_len, partition_tokens, &part))) return st;
    const size_t need = workspace_bytes(c, num_seqs, num_q_heads, max_context_len, part);
    if (need > 0) {
        if (!workspace) return fail(PA_ERR_WORKSPACE, "pa_decode needs %zu bytes of workspace, got NULL", need);
        if (workspace_bytes_given < need)
            return fail(PA_ERR_WORKSPACE, "pa_decode needs %zu bytes of workspace, got %zu", need, workspace_bytes_given);
        if (!aligned16(workspace)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");
    }
    hipStream_t s = as_stream(stream);
    if (validate_enabled()) {
        std::vector<int32_t> lens, tables;
        if ((st = fetch(lens, context_lens, num_seqs, s))) return st;
        if ((st = fetch(tables, block_tables, static_cast<size_t>(num_seqs) * max_blocks_per_seq, s))) return st;
        for (int32_t i = 0; i < num_seqs; ++i) {
            const int32_t L = lens[i];
            if (L < 0 || L > max_context_len)
                return fail(PA_ERR_VALIDATE, "context_lens[%d] = %d outside [0, %d]", i, L, max_context_len);
            const int32_t nb = (L + c->block_size - 1) / c->block_size;
            for (int32_t j = 0; j < nb; ++j) {
                const int32_t b = tables[static_cast<size_t>(i) * max_blocks_per_seq + j];
                if (b < 0 || b >= c->num_blocks)
                    return fail(PA_ERR_VALIDATE, "block_tables[%d][%d] = %d outside [0, %lld)", i, j, b, (long long)c->num_blocks);
            }
        }
        if (cow_src) {
            // the copies: sources in range, each destination (a request's block
            // holding L-1) named once, and no destination also a source
            std::vector<int32_t> srcs;
            if ((st = fetch(srcs, cow_src, num_seqs, s))) return st;
            std::vector<int64_t> dsts;
            std::vector<int64_t> all_src;
            for (int32_t i = 0; i < num_seqs; ++i) {
                if (srcs[i] < 0) continue;
                if (srcs[i] >= c->num_blocks)
                    return fail(PA_ERR_VALIDATE, "cow_src[%d] = %d outside [0, %lld)", i, srcs[i], (long long)c->num_blocks);
                if (lens[i] <= 0)
                    return fail(PA_ERR_VALIDATE, "cow_src[%d] set for a request with no positions", i);
                dsts.push_back(tables[static_cast<size_t>(i) * max_blocks_per_seq + (lens[i] - 1) / c->block_size]);
                all_src.push_back(srcs[i]);
            }
            std::vector<int64_t> d2 = dsts;
            std::sort(d2.begin(), d2.end());
            if (std::adjacent_find(d2.begin(), d2.end()) != d2.end())
                return fail(PA_ERR_VALIDATE, "two copy-on-write destinations are the same block");
            std::sort(all_src.begin(), all_src.end());
            for (int64_t d : dsts)
                if (std::binary_search(all_src.begin(), all_src.end(), d))
                    return fail(PA_ERR_VALIDATE, "copy-on-write destination %lld is also a source", (long long)d);
        }
    }
    const int64_t parts64 = std::max<int64_t>(1, ceil_div(max_context_len, part));
    if (parts64 > kMaxGridYZ)
        return fail(PA_ERR_SHAPE, "max_context_len %d needs %lld partitions of %d tokens (> %d)",
                    max_context_len, (long long)parts64, part, kMaxGridYZ);
    const int32_t max_parts = static_cast<int32_t>(parts64);
    DecodeArgs a;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.q = q;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_blocks = c->num_blocks;
    a.block_stride = block_stride(c);
    a.block_size = c->block_size;
    a.num_kv_heads = c->num_kv_heads;
    a.head_dim = c->head_dim;
    a.dtype = c->dtype;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.group = num_q_heads / c->num_kv_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.len_clamp = max_context_len;
    a.part_tokens = part;
    a.max_parts = max_parts;
    a.scale = scale;
    a.flags = flags;
    a.out = out;
    const size_t slots = static_cast<size_t>(num_seqs) * num_q_heads * max_parts;
    float* ws = need ? static_cast<float*>(workspace) : nullptr;
    a.ws_acc = ws;
    a.ws_m = need ? ws + slots * c->head_dim : nullptr;
    a.ws_l = need ? ws + slots * (c->head_dim + 1) : nullptr;
    a.k_new = k_new;
    a.v_new = v_new;
    a.cow_src = cow_src;
    a.stream = s;
    if ((st = launch_decode(a))) return st;
    return ok();
}


extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_NULL: return "PA_ERR_NULL";
        case PA_ERR_SHAPE: return "PA_ERR_SHAPE";
        case PA_ERR_DTYPE: return "PA_ERR_DTYPE";
        case PA_ERR_ALIGN: return "PA_ERR_ALIGN";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
        case PA_ERR_HIP: return "PA_ERR_HIP";
        case PA_ERR_VALIDATE: return "PA_ERR_VALIDATE";
        case PA_ERR_NO_SPACE: return "PA_ERR_NO_SPACE";
        case PA_ERR_NOT_FOUND: return "PA_ERR_NOT_FOUND";
        default: return "PA_ERR_UNKNOWN";
    }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_write_kv(const pa_cache_desc_t* c, void* k_cache, void* v_cache, const void* k_new,
                const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                void* stream) {
    int st = check_desc(c);
    if (st) return st;
    if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens %d < 0", num_tokens);
    if (num_tokens == 0) return ok();
    if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
        return fail(PA_ERR_NULL, "pa_write_kv: a required pointer is NULL");
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
        return fail(PA_ERR_ALIGN, "pa_write_kv: caches and new K/V must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    if (validate_enabled()) {
        std::vector<int64_t> slots;
        if ((st = fetch(slots, slot_mapping, num_tokens, s))) return st;
        const int64_t limit = c->num_blocks * c->block_size;
        std::unordered_set<int64_t> seen;
        for (int32_t t = 0; t < num_tokens; ++t) {
            const int64_t v = slots[t];
            if (v < 0) continue;
            if (v >= limit) return fail(PA_ERR_VALIDATE, "slot_mapping[%d] = %lld >= %lld", t, (long long)v, (long long)limit);
            if (!seen.insert(v).second) return fail(PA_ERR_VALIDATE, "slot %lld written twice", (long long)v);
        }
    }
    if ((st = launch_write_kv(c, k_cache, v_cache, k_new, v_new, slot_mapping, num_tokens, s))) return st;
    return ok();
}

int pa_copy_blocks(const pa_cache_desc_t* c, void* k_cache, void* v_cache,
                   const int64_t* block_pairs, int32_t num_pairs, void* stream) {
    int st = check_desc(c);
    if (st) return st;
    if (num_pairs < 0) return fail(PA_ERR_SHAPE, "num_pairs %d < 0", num_pairs);
    if (num_pairs == 0) return ok();
    if (!k_cache || !v_cache || !block_pairs) return fail(PA_ERR_NULL, "pa_copy_blocks: a required pointer is NULL");
    if (!aligned16(k_cache) || !aligned16(v_cache))
        return fail(PA_ERR_ALIGN, "pa_copy_blocks: caches must be 16-byte aligned");
    hipStream_t s = as_stream(stream);
    if (validate_enabled()) {
        std::vector<int64_t> pairs;
        if ((st = fetch(pairs, block_pairs, 2 * static_cast<size_t>(num_pairs), s))) return st;
        std::unordered_set<int64_t> dsts, srcs;
        for (int32_t i = 0; i < num_pairs; ++i) {
            const int64_t a = pairs[2 * i], b = pairs[2 * i + 1];
            if (a < 0 || a >= c->num_blocks || b < 0 || b >= c->num_blocks)
                return fail(PA_ERR_VALIDATE, "pair %d = (%lld, %lld) outside [0, %lld)", i, (long long)a, (long long)b, (long long)c->num_blocks);
            if (!dsts.insert(b).second) return fail(PA_ERR_VALIDATE, "block %lld is the destination of two pairs", (long long)b);
            srcs.insert(a);
        }
        for (int64_t b : dsts)
            if (srcs.count(b)) return fail(PA_ERR_VALIDATE, "block %lld is both a source and a destination", (long long)b);
    }
    if ((st = launch_copy_blocks(c, k_cache, v_cache, block_pairs, num_pairs, s))) return st;
    return ok();
}

int pa_slot_mapping(int32_t block_size, const int32_t* block_tables, int32_t num_seqs,
                    int32_t max_blocks_per_seq, const int32_t* seq_ids,
                    const int32_t* positions, int32_t num_tokens, int64_t* slot_mapping,
                    void* stream) {
    if (block_size < 1) return fail(PA_ERR_SHAPE, "block_size %d < 1", block_size);
    if (num_seqs < 0 || max_blocks_per_seq < 1 || num_tokens < 0)
        return fail(PA_ERR_SHAPE, "pa_slot_mapping: need num_seqs >= 0, max_blocks_per_seq >= 1, num_tokens >= 0");
    if (num_tokens == 0) return ok();
    if (!positions || !slot_mapping || (num_seqs > 0 && !block_tables))
        return fail(PA_ERR_NULL, "pa_slot_mapping: a required pointer is NULL");
    int st = launch_slot_mapping(block_size, block_tables, num_seqs, max_blocks_per_seq, seq_ids,
                                 positions, num_tokens, slot_mapping, as_stream(stream));
    return st ? st : ok();
}

int pa_gather_kv(const pa_cache_desc_t* c, const void* k_cache, const void* v_cache,
                 const int32_t* block_table, int32_t context_len, void* k_out, void* v_out,
                 void* stream) {
    int st = check_desc(c);
    if (st) return st;
    if (context_len < 0) return fail(PA_ERR_SHAPE, "context_len %d < 0", context_len);
    if (context_len == 0) return ok();
    if (!k_cache || !v_cache || !block_table || !k_out || !v_out)
        return fail(PA_ERR_NULL, "pa_gather_kv: a required pointer is NULL");
    hipStream_t s = as_stream(stream);
    if (validate_enabled()) {
        std::vector<int32_t> table;
        const size_t n = static_cast<size_t>((context_len + c->block_size - 1) / c->block_size);
        if ((st = fetch(table, block_table, n, s))) return st;
        for (size_t i = 0; i < n; ++i)
            if (table[i] < 0 || table[i] >= c->num_blocks)
                return fail(PA_ERR_VALIDATE, "block_table[%zu] = %d outside [0, %lld)", i, table[i], (long long)c->num_blocks);
    }
    if ((st = launch_gather_kv(c, k_cache, v_cache, block_table, context_len, k_out, v_out, s))) return st;
    return ok();
}

int32_t pa_decode_partition_tokens(const pa_cache_desc_t* c, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_context_len) {
    if (check_desc(c) || check_heads(c, num_seqs, num_q_heads)) return -1;
    return plan_partition(c, num_seqs, num_q_heads, max_context_len);
}

size_t pa_decode_workspace_bytes(const pa_cache_desc_t* c, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_context_len,
                                 int32_t partition_tokens) {
    if (check_desc(c) || check_heads(c, num_seqs, num_q_heads)) return 0;
    int32_t part = 0;
    if (resolve_partition(c, num_seqs, num_q_heads, max_context_len, partition_tokens, &part)) return 0;
    return workspace_bytes(c, num_seqs, num_q_heads, max_context_len, part);
}

int pa_decode(const pa_cache_desc_t* c, const void* k_cache, const void* v_cache,
              const void* q, const int32_t* block_tables, const int32_t* context_lens,
              int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
              int32_t max_context_len, float scale, void* out, void* workspace,
              size_t workspace_bytes, int32_t partition_tokens, uint32_t flags, void* stream) {
    return decode_impl("pa_decode", c, k_cache, v_cache, nullptr, nullptr, nullptr, q, block_tables,
                       context_lens, num_seqs, num_q_heads, max_blocks_per_seq, max_context_len,
                       scale, out, workspace, workspace_bytes, partition_tokens, flags, stream);
}

size_t pa_prefill_workspace_bytes(const pa_cache_desc_t* c, int32_t num_seqs, int32_t total_q,
                                  int32_t max_q_len, int32_t num_q_heads,
                                  int32_t max_context_len, int32_t partition_tokens) {
    if (check_desc(c) || check_heads(c, num_seqs, num_q_heads) || total_q < 0 || max_q_len < 0)
        return 0;
    int32_t part = 0;
    if (!prefill_mfma_ok(c, num_q_heads / c->num_kv_heads, max_q_len)) {
        if (resolve_partition(c, total_q, num_q_heads, max_context_len, partition_tokens, &part))
            return 0;
        return prefill_rows_workspace(c, total_q, num_q_heads, max_context_len, part);
    }
    if (prefill_partition(c, num_seqs, max_q_len, num_q_heads, max_context_len, partition_tokens, &part))
        return 0;
    return prefill_workspace(c, total_q, num_q_heads, max_context_len, part);
}

int pa_prefill(const pa_cache_desc_t* c, const void* k_cache, const void* v_cache,
               const void* q, const int32_t* q_start, const int32_t* block_tables,
               const int32_t* context_lens, int32_t num_seqs, int32_t total_q,
               int32_t max_q_len, int32_t num_q_heads, int32_t max_blocks_per_seq,
               int32_t max_context_len, float scale, void* out, void* workspace,
               size_t workspace_bytes_given, int32_t partition_tokens, uint32_t flags,
               void* stream) {
    int st = check_desc(c);
    if (st) return st;
    if ((st = check_heads(c, num_seqs, num_q_heads))) return st;
    const int group = num_q_heads / c->num_kv_heads;
    // outside the MFMA prefill kernels' set, each query row is a decode request
    const bool as_rows = !prefill_mfma_ok(c, group, max_q_len);
    if (total_q < 0 || total_q > kMaxGridYZ)
        return fail(PA_ERR_SHAPE, "total_q %d outside [0, %d]", total_q, kMaxGridYZ);
    if (max_q_len < 0) return fail(PA_ERR_SHAPE, "max_q_len %d < 0", max_q_len);
    if (max_blocks_per_seq < 1) return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
    if (max_context_len < 0) return fail(PA_ERR_SHAPE, "max_context_len %d < 0", max_context_len);
    if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * c->block_size)
        return fail(PA_ERR_SHAPE, "max_context_len %d exceeds max_blocks_per_seq * block_size = %lld",
                    max_context_len, static_cast<long long>(max_blocks_per_seq) * c->block_size);
    if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "scale is not finite");
    if (flags != 0) return fail(PA_ERR_UNSUPPORTED, "unknown prefill flags 0x%x", flags);
    const int64_t rows = as_rows ? 0 : prefill_waves_rows(num_seqs, max_q_len, group);
    if (rows > kMaxGridYZ)
        return fail(PA_ERR_SHAPE, "num_seqs * ceil(max_q_len / %d) = %lld exceeds %d", 16 / group,
                    (long long)rows, kMaxGridYZ);
    if (num_seqs == 0 || total_q == 0) return ok();
    if (!k_cache || !v_cache || !q || !q_start || !block_tables || !context_lens || !out)
        return fail(PA_ERR_NULL, "pa_prefill: a required pointer is NULL");
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(out))
        return fail(PA_ERR_ALIGN, "pa_prefill: caches, q and out must be 16-byte aligned");
    int32_t part = 0;
    if (as_rows) {
        if ((st = resolve_partition(c, total_q, num_q_heads, max_context_len, partition_tokens, &part)))
            return st;
    } else if ((st = prefill_partition(c, num_seqs, max_q_len, num_q_heads, max_context_len,
                                       partition_tokens, &part))) {
        return st;
    }
    const size_t need = as_rows ? prefill_rows_workspace(c, total_q, num_q_heads, max_context_len, part)
                                : prefill_workspace(c, total_q, num_q_heads, max_context_len, part);
    if (need > 0) {
        if (!workspace) return fail(PA_ERR_WORKSPACE, "pa_prefill needs %zu bytes of workspace, got NULL", need);
        if (workspace_bytes_given < need)
            return fail(PA_ERR_WORKSPACE, "pa_prefill needs %zu bytes of workspace, got %zu", need,
                        workspace_bytes_given);
        if (!aligned16(workspace)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");
    }
    hipStream_t s = as_stream(stream);
    if (validate_enabled()) {
        std::vector<int32_t> starts, lens, tables;
        if ((st = fetch(starts, q_start, static_cast<size_t>(num_seqs) + 1, s))) return st;
        if ((st = fetch(lens, context_lens, num_seqs, s))) return st;
        if ((st = fetch(tables, block_tables, static_cast<size_t>(num_seqs) * max_blocks_per_seq, s))) return st;
        if (starts[0] != 0 || starts[num_seqs] != total_q)
            return fail(PA_ERR_VALIDATE, "q_start must run from 0 to total_q = %d", total_q);
        for (int32_t i = 0; i < num_seqs; ++i) {
            const int32_t n = starts[i + 1] - starts[i];
            if (n < 0 || n > max_q_len)
                return fail(PA_ERR_VALIDATE, "request %d has %d query tokens (max_q_len %d)", i, n, max_q_len);
            const int32_t L = lens[i];
            if (L < 0 || L > max_context_len)
                return fail(PA_ERR_VALIDATE, "context_lens[%d] = %d outside [0, %d]", i, L, max_context_len);
            const int32_t nb = (L + c->block_size - 1) / c->block_size;
            for (int32_t j = 0; j < nb; ++j) {
                const int32_t b = tables[static_cast<size_t>(i) * max_blocks_per_seq + j];
                if (b < 0 || b >= c->num_blocks)
                    return fail(PA_ERR_VALIDATE, "block_tables[%d][%d] = %d outside [0, %lld)", i, j, b,
                                (long long)c->num_blocks);
            }
        }
    }
    const int64_t parts64 = std::max<int64_t>(1, ceil_div(max_context_len, part));
    if (parts64 > kMaxGridYZ)
        return fail(PA_ERR_SHAPE, "max_context_len %d needs %lld partitions of %d tokens (> %d)",
                    max_context_len, (long long)parts64, part, kMaxGridYZ);
    if (as_rows) {
        const int32_t row_blocks = prefill_row_blocks(c, max_context_len);
        char* base = static_cast<char*>(workspace);
        int32_t* row_tables = reinterpret_cast<int32_t*>(base);
        base += round16(static_cast<size_t>(total_q) * row_blocks * sizeof(int32_t));
        int32_t* row_lens = reinterpret_cast<int32_t*>(base);
        base += round16(static_cast<size_t>(total_q) * sizeof(int32_t));
        if ((st = launch_prefill_rows(q_start, block_tables, context_lens, num_seqs, total_q,
                                      max_blocks_per_seq, row_blocks, max_context_len, row_tables,
                                      row_lens, s)))
            return st;
        DecodeArgs a;
        a.k_cache = k_cache;
        a.v_cache = v_cache;
        a.q = q;
        a.block_tables = row_tables;
        a.context_lens = row_lens;
        a.num_blocks = c->num_blocks;
        a.block_stride = block_stride(c);
        a.block_size = c->block_size;
        a.num_kv_heads = c->num_kv_heads;
        a.head_dim = c->head_dim;
        a.dtype = c->dtype;
        a.num_seqs = total_q;
        a.num_q_heads = num_q_heads;
        a.group = group;
        a.max_blocks_per_seq = row_blocks;
        a.len_clamp = max_context_len;
        a.part_tokens = part;
        a.max_parts = static_cast<int32_t>(parts64);
        a.scale = scale;
        a.flags = 0;
        a.out = out;
        const size_t slots = static_cast<size_t>(total_q) * num_q_heads * a.max_parts;
        const bool split = workspace_bytes(c, total_q, num_q_heads, max_context_len, part) > 0;
        float* ws = split ? reinterpret_cast<float*>(base) : nullptr;
        a.ws_acc = ws;
        a.ws_m = split ? ws + slots * c->head_dim : nullptr;
        a.ws_l = split ? ws + slots * (c->head_dim + 1) : nullptr;
        a.k_new = nullptr;
        a.v_new = nullptr;
        a.cow_src = nullptr;
        a.stream = s;
        if ((st = launch_decode(a))) return st;
        return ok();
    }
    PrefillArgs p;
    DecodeArgs& a = p.d;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.q = q;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_blocks = c->num_blocks;
    a.block_stride = block_stride(c);
    a.block_size = c->block_size;
    a.num_kv_heads = c->num_kv_heads;
    a.head_dim = c->head_dim;
    a.dtype = c->dtype;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.group = group;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.len_clamp = max_context_len;
    a.part_tokens = part;
    a.max_parts = static_cast<int32_t>(parts64);
    a.scale = scale;
    a.flags = 0;
    a.out = out;
    const size_t slots = static_cast<size_t>(total_q) * num_q_heads * a.max_parts;
    float* ws = need ? static_cast<float*>(workspace) : nullptr;
    a.ws_acc = ws;
    a.ws_m = need ? ws + slots * c->head_dim : nullptr;
    a.ws_l = need ? ws + slots * (c->head_dim + 1) : nullptr;
    a.k_new = nullptr;
    a.v_new = nullptr;
    a.stream = s;
    p.q_start = q_start;
    p.total_q = total_q;
    p.max_q_len = max_q_len;
    p.ws_len = need ? reinterpret_cast<int32_t*>(ws + slots * (c->head_dim + 2)) : nullptr;
    if ((st = launch_prefill(p))) return st;
    return ok();
}

int pa_decode_append(const pa_cache_desc_t* c, void* k_cache, void* v_cache, const void* k_new,
                     const void* v_new, const void* q, const int32_t* block_tables,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                     int32_t max_blocks_per_seq, int32_t max_context_len, float scale, void* out,
                     void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                     uint32_t flags, void* stream) {
    if (num_seqs > 0 && (!k_new || !v_new))
        return fail(PA_ERR_NULL, "pa_decode_append: k_new and v_new are required");
    return decode_impl("pa_decode_append", c, k_cache, v_cache, k_new, v_new, nullptr, q,
                       block_tables, context_lens, num_seqs, num_q_heads, max_blocks_per_seq,
                       max_context_len, scale, out, workspace, workspace_bytes, partition_tokens,
                       flags, stream);
}

int pa_decode_step(const pa_cache_desc_t* c, void* k_cache, void* v_cache, const void* k_new,
                   const void* v_new, const int32_t* cow_src, const void* q,
                   const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                   int32_t num_q_heads, int32_t max_blocks_per_seq, int32_t max_context_len,
                   float scale, void* out, void* workspace, size_t workspace_bytes,
                   int32_t partition_tokens, uint32_t flags, void* stream) {
    if (num_seqs > 0 && (!k_new || !v_new))
        return fail(PA_ERR_NULL, "pa_decode_step: k_new and v_new are required");
    return decode_impl("pa_decode_step", c, k_cache, v_cache, k_new, v_new, cow_src, q,
                       block_tables, context_lens, num_seqs, num_q_heads, max_blocks_per_seq,
                       max_context_len, scale, out, workspace, workspace_bytes, partition_tokens,
                       flags, stream);
}

int pa_decode_step_noalloc(const pa_cache_desc_t* c, void* k_cache, void* v_cache,
                           const void* k_new, const void* v_new, const int32_t* cow_src,
                           const void* q, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                           int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                           void* out, int32_t partition_tokens, uint32_t flags, void* stream) {
    int st = check_desc(c);
    if (st) return st;
    if ((st = check_heads(c, num_seqs, num_q_heads))) return st;
    if (num_seqs > 0 && (!k_new || !v_new))
        return fail(PA_ERR_NULL, "pa_decode_step_noalloc: k_new and v_new are required");
    int32_t part = 0;
    if ((st = resolve_partition(c, num_seqs, num_q_heads, max_context_len, partition_tokens, &part)))
        return st;
    const size_t need = workspace_bytes(c, num_seqs, num_q_heads, max_context_len, part);
    if (need > kNoallocScratchBytes)
        return fail(PA_ERR_WORKSPACE,
                    "pa_decode_step_noalloc: this call needs %zu bytes of split-K partials; the "
                    "static scratch holds %zu (use pa_decode_step with a workspace)",
                    need, kNoallocScratchBytes);
    void* ws = nullptr;
    if (need > 0 && (st = noalloc_scratch(&ws))) return st;
    return decode_impl("pa_decode_step_noalloc", c, k_cache, v_cache, k_new, v_new, cow_src, q,
                       block_tables, context_lens, num_seqs, num_q_heads, max_blocks_per_seq,
                       max_context_len, scale, out, ws, need ? kNoallocScratchBytes : 0,
                       partition_tokens, flags, stream);
}

}  // extern "C"
