// pa_debug.hip -- PA_DEBUG: device-side checks of the preconditions on values
// that live on the device (slots, block ids, context lengths, block pairs,
// query starts, groups).
//
// Without PA_DEBUG these values are trusted: the kernels clamp or skip any
// that would take an access out of its buffer, and the result for such
// inputs is unspecified.  With PA_DEBUG on (environment variable PA_DEBUG=1
// when the library first needs it, or pa_set_debug) every entry point first
// runs the checks below on the caller's stream, waits for them, and returns
// PA_ERR_INVALID_ARG naming each violated precondition instead of launching
// anything.  The pages' own convention for an out-of-range index is an error
// raised to the caller (the ValueError of the per-request offset helper,
// [論文解説: vAttention, 技術的詳細 › リクエスト単位のKVキャッシュインデキシング]).
//
// The checks allocate a small scratch buffer and wait on the stream: debug
// mode is for finding bad inputs, not for the serving loop, and it is refused
// while the stream is being captured into a graph.
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <string>

#include "../../include/pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

std::atomic<int> g_debug{-1};  // -1: not decided yet (read PA_DEBUG at first use)

enum : unsigned {
    kBadCtx = 1u,          // context length < 0 or > max_blocks_per_seq * B
    kBadBlock = 2u,        // a table entry the context uses is outside [0, num_blocks)
    kBadSlot = 4u,         // a slot >= num_blocks * B
    kDupSlot = 8u,         // two tokens of one call with the same slot
    kBadPair = 16u,        // a block pair id outside its pool
    kDupDst = 32u,         // two pairs with the same destination
    kDstIsSrc = 64u,       // a destination that is also a source (same pools)
    kBadQueryStart = 128u, // query_start not 0 .. num_tokens non-decreasing, or a chunk
                           // longer than its context or than max_query_len
    kBadGroup = 256u,      // group_start / prefix_blocks inconsistent with the sequences
    kXcdSplit = 512u,      // the units of one split row ran on more than one XCD
};

const char *const kFlagText[] = {
    "a context length is negative or exceeds max_blocks_per_seq * block_size",
    "a block-table entry within a context is outside [0, num_blocks)",
    "a slot is >= num_blocks * block_size",
    "two tokens of the call have the same slot",
    "a block id of block_mapping is outside its pool",
    "two pairs of block_mapping have the same destination",
    "a destination of block_mapping is also a source",
    "query_start is not non-decreasing from 0 to num_tokens, or a chunk is longer than its "
    "context or than max_query_len",
    "group_start / prefix_blocks do not describe consecutive groups sharing their prefix blocks",
    "the work units of one (sequence, kv head) ran on more than one XCD, so the in-kernel merge "
    "of that call may have read stale partials; pass PA_DECODE_MERGE_KERNEL on this device",
};

__device__ __forceinline__ void raise(unsigned *flags, unsigned bit) { atomicOr(flags, bit); }

__device__ __forceinline__ int64_t gtid() {
    return (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
}
__device__ __forceinline__ int64_t gstride() { return (int64_t)gridDim.x * blockDim.x; }

__global__ void check_tables_kernel(const int32_t *bt, const int32_t *ctx, int S, int MB, int B,
                                    int64_t NB, unsigned *flags) {
    const int64_t cap = (int64_t)MB * B;
    for (int64_t s = gtid(); s < S; s += gstride()) {
        const int c = ctx[s];
        if (c < 0 || c > cap) raise(flags, kBadCtx);
    }
    for (int64_t i = gtid(); i < (int64_t)S * MB; i += gstride()) {
        const int64_t s = i / MB, e = i % MB;
        const int64_t c = ctx[s] < 0 ? 0 : (ctx[s] > cap ? cap : ctx[s]);
        if (e < (c + B - 1) / B) {
            const int32_t b = bt[i];
            if (b < 0 || b >= NB) raise(flags, kBadBlock);
        }
    }
}

// bitmap: one bit per slot, zero before the launch
__global__ void check_slots_kernel(const int64_t *slots, int64_t T, int64_t num_slots,
                                   unsigned *bitmap, unsigned *flags) {
    for (int64_t t = gtid(); t < T; t += gstride()) {
        const int64_t s = slots[t];
        if (s < 0) continue;  // skipped by the write
        if (s >= num_slots) {
            raise(flags, kBadSlot);
            continue;
        }
        const unsigned bit = 1u << (s & 31);
        if (atomicOr(bitmap + (s >> 5), bit) & bit) raise(flags, kDupSlot);
    }
}

// first pass: ranges, and a bit per source block (src_map)
__global__ void check_pairs_src_kernel(const int64_t *pairs, int64_t n, int64_t src_blocks,
                                       int64_t dst_blocks, unsigned *src_map, unsigned *flags) {
    for (int64_t i = gtid(); i < n; i += gstride()) {
        const int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
        if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) {
            raise(flags, kBadPair);
            continue;
        }
        atomicOr(src_map + (src >> 5), 1u << (src & 31));
    }
}

// second pass (after the first on the stream): distinct destinations, and
// with one pool pair, no destination among the sources
__global__ void check_pairs_dst_kernel(const int64_t *pairs, int64_t n, int64_t src_blocks,
                                       int64_t dst_blocks, int same_pool,
                                       const unsigned *src_map, unsigned *dst_map,
                                       unsigned *flags) {
    for (int64_t i = gtid(); i < n; i += gstride()) {
        const int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
        if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) continue;
        const unsigned bit = 1u << (dst & 31);
        if (atomicOr(dst_map + (dst >> 5), bit) & bit) raise(flags, kDupDst);
        if (same_pool && dst < src_blocks && (src_map[dst >> 5] & bit)) raise(flags, kDstIsSrc);
    }
}

__global__ void check_query_start_kernel(const int32_t *qs, const int32_t *ctx, int S, int T,
                                         int max_query_len, unsigned *flags) {
    for (int64_t s = gtid(); s < S; s += gstride()) {
        const int q0 = qs[s], q1 = qs[s + 1];
        const int n = q1 - q0;
        if ((s == 0 && q0 != 0) || (s == S - 1 && q1 != T) || n < 0 || n > max_query_len ||
            n > ctx[s])
            raise(flags, kBadQueryStart);
    }
}

// thread per (sequence, prefix entry): each member of group k (sequences
// gs[k] .. gs[k+1]-1) has a context covering the group's prefix blocks and
// the same physical blocks there as the group's first member
__global__ void check_groups_kernel(const int32_t *gs, const int32_t *pblk, const int32_t *bt,
                                    const int32_t *ctx, int NG, int S, int MB, int max_group,
                                    unsigned *flags) {
    for (int64_t k = gtid(); k < NG; k += gstride()) {
        const int g0 = gs[k], g1 = gs[k + 1];
        if ((k == 0 && g0 != 0) || (k == NG - 1 && g1 != S) || g1 <= g0 || g1 - g0 > max_group ||
            pblk[k] < 0 || pblk[k] > MB)
            raise(flags, kBadGroup);
    }
    // entries: only where the group description itself is in range
    for (int64_t i = gtid(); i < (int64_t)NG * MB; i += gstride()) {
        const int64_t k = i / MB, e = i % MB;
        const int g0 = gs[k], g1 = gs[k + 1], pb = pblk[k];
        if (g0 < 0 || g1 > S || g1 <= g0 || pb < 0 || pb > MB || e >= pb) continue;
        const int32_t first = bt[(int64_t)g0 * MB + e];
        for (int s = g0; s < g1; ++s) {
            if (bt[(int64_t)s * MB + e] != first || (int64_t)pb * 16 > ctx[s]) {
                raise(flags, kBadGroup);
                break;
            }
        }
    }
}

__global__ void check_xcd_kernel(const unsigned *seen, int64_t rows, unsigned *flags) {
    for (int64_t r = gtid(); r < rows; r += gstride())
        if (__popc(seen[r]) > 1) raise(flags, kXcdSplit);
}

int grid_for(int64_t n) {
    const int64_t g = (n + 255) / 256;
    return (int)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

// Scratch for one check: flags word + bitmaps, zeroed on the stream, freed
// after the wait.
struct Scratch {
    void *p = nullptr;
    size_t bytes = 0;
    bool owned = true;
    ~Scratch() {
        if (p && owned) (void)hipFree(p);
    }
};

int begin(const char *who, hipStream_t stream, size_t bitmap_words, Scratch &sc,
          unsigned **flags, unsigned **bitmaps, unsigned *given = nullptr) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return api_hip_fail(e, who);
    if (cs != hipStreamCaptureStatusNone) {
        std::string m = std::string(who) + ": PA_DEBUG checks wait for the stream, which is "
                        "being captured; switch PA_DEBUG off for graph capture";
        return api_fail(PA_ERR_INVALID_ARG, m.c_str());
    }
    sc.bytes = (1 + bitmap_words) * sizeof(unsigned);
    if (given && bitmap_words == 0) {  // the caller's word: nothing to allocate
        sc.p = given;
        sc.owned = false;
        e = hipMemsetAsync(sc.p, 0, sc.bytes, stream);
        if (e != hipSuccess) return api_hip_fail(e, who);
        *flags = given;
        *bitmaps = nullptr;
        return PA_OK;
    }
    e = hipMalloc(&sc.p, sc.bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        sc.p = nullptr;
        std::string m = std::string(who) + ": PA_DEBUG scratch: " + hipGetErrorString(e);
        return api_fail(PA_ERR_NO_MEMORY, m.c_str());
    }
    e = hipMemsetAsync(sc.p, 0, sc.bytes, stream);
    if (e != hipSuccess) return api_hip_fail(e, who);
    *flags = (unsigned *)sc.p;
    *bitmaps = (unsigned *)sc.p + 1;
    return PA_OK;
}

int finish(const char *who, hipStream_t stream, Scratch &sc) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return api_hip_fail(e, who);
    unsigned flags = 0;
    e = hipMemcpyAsync(&flags, sc.p, sizeof flags, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return api_hip_fail(e, who);
    if (!flags) return PA_OK;
    std::string m = std::string(who) + ": PA_DEBUG:";
    for (unsigned i = 0; i < sizeof kFlagText / sizeof kFlagText[0]; ++i)
        if (flags & (1u << i)) m += std::string(" ") + kFlagText[i] + ";";
    return api_fail(PA_ERR_INVALID_ARG, m.c_str());
}

}  // namespace

bool debug_enabled() {
    int d = g_debug.load(std::memory_order_relaxed);
    if (d < 0) {
        const char *env = getenv("PA_DEBUG");
        d = (env && *env && strcmp(env, "0") != 0) ? 1 : 0;
        int expect = -1;
        if (!g_debug.compare_exchange_strong(expect, d)) d = expect;
    }
    return d > 0;
}

int debug_set(int on) {
    const int prev = debug_enabled() ? 1 : 0;
    g_debug.store(on ? 1 : 0);
    return prev;
}

int debug_check_tables(const char *who, const int32_t *bt, const int32_t *ctx, int S, int MB,
                       int B, int64_t NB, hipStream_t stream, unsigned *flags_buf) {
    if (S <= 0) return PA_OK;
    Scratch sc;
    unsigned *flags, *bm;
    int rc = begin(who, stream, 0, sc, &flags, &bm, flags_buf);
    if (rc != PA_OK) return rc;
    check_tables_kernel<<<grid_for((int64_t)S * (MB > 0 ? MB : 1)), 256, 0, stream>>>(
        bt, ctx, S, MB, B, NB, flags);
    return finish(who, stream, sc);
}

int debug_check_slots(const char *who, const int64_t *slots, int64_t T, int64_t num_slots,
                      hipStream_t stream) {
    if (T <= 0) return PA_OK;
    Scratch sc;
    unsigned *flags, *bm;
    int rc = begin(who, stream, (size_t)((num_slots + 31) / 32), sc, &flags, &bm);
    if (rc != PA_OK) return rc;
    check_slots_kernel<<<grid_for(T), 256, 0, stream>>>(slots, T, num_slots, bm, flags);
    return finish(who, stream, sc);
}

int debug_check_pairs(const char *who, const int64_t *pairs, int64_t n, int64_t src_blocks,
                      int64_t dst_blocks, bool same_pool, hipStream_t stream) {
    if (n <= 0) return PA_OK;
    Scratch sc;
    unsigned *flags, *bm;
    const size_t src_words = (size_t)((src_blocks + 31) / 32);
    const size_t dst_words = (size_t)((dst_blocks + 31) / 32);
    int rc = begin(who, stream, src_words + dst_words, sc, &flags, &bm);
    if (rc != PA_OK) return rc;
    check_pairs_src_kernel<<<grid_for(n), 256, 0, stream>>>(pairs, n, src_blocks, dst_blocks,
                                                             bm, flags);
    check_pairs_dst_kernel<<<grid_for(n), 256, 0, stream>>>(pairs, n, src_blocks, dst_blocks,
                                                             same_pool ? 1 : 0, bm,
                                                             bm + src_words, flags);
    return finish(who, stream, sc);
}

int debug_check_query_start(const char *who, const int32_t *qs, const int32_t *ctx, int S, int T,
                            int max_query_len, hipStream_t stream) {
    if (S <= 0) return PA_OK;
    Scratch sc;
    unsigned *flags, *bm;
    int rc = begin(who, stream, 0, sc, &flags, &bm);
    if (rc != PA_OK) return rc;
    check_query_start_kernel<<<grid_for(S), 256, 0, stream>>>(qs, ctx, S, T, max_query_len,
                                                               flags);
    return finish(who, stream, sc);
}

int debug_check_groups(const char *who, const int32_t *gs, const int32_t *pblk, const int32_t *bt,
                       const int32_t *ctx, int NG, int S, int MB, int max_group,
                       hipStream_t stream) {
    if (NG <= 0) return PA_OK;
    Scratch sc;
    unsigned *flags, *bm;
    int rc = begin(who, stream, 0, sc, &flags, &bm);
    if (rc != PA_OK) return rc;
    check_groups_kernel<<<grid_for((int64_t)NG * (MB > 0 ? MB : 1)), 256, 0, stream>>>(
        gs, pblk, bt, ctx, NG, S, MB, max_group, flags);
    return finish(who, stream, sc);
}

int debug_check_xcd(const char *who, const unsigned *seen, int64_t rows, hipStream_t stream,
                    unsigned *flags_buf) {
    if (rows <= 0) return PA_OK;
    Scratch sc;
    unsigned *flags, *bm;
    int rc = begin(who, stream, 0, sc, &flags, &bm, flags_buf);
    if (rc != PA_OK) return rc;
    check_xcd_kernel<<<grid_for(rows), 256, 0, stream>>>(seen, rows, flags);
    return finish(who, stream, sc);
}

}  // namespace pa

extern "C" int pa_set_debug(int on) { return pa::debug_set(on); }
