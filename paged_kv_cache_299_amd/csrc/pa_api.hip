// pa_api.hip -- the extern "C" entry points of libpa (declared in include/pa.h).
//
// Host work per call: check every argument the host can see, plan the launch
// from host-known sizes only (context lengths stay on the device), make sure
// the split workspace exists, and enqueue the kernels on the caller's stream.
#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char *where) {
    return fail(PA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

int elem_bytes(int dtype) {
    switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    default: return 0;
    }
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

namespace pa {
int api_fail(int status, const char *msg) {
    g_last_error = msg;
    return status;
}
int api_hip_fail(hipError_t e, const char *where) { return hip_fail(e, where); }
}  // namespace pa

namespace {

// ---- split workspace: one grow-only buffer per (device, stream) ------------
// A buffer that a larger one replaces is kept, not freed, until
// pa_release_workspaces: work already queued on the stream, and HIP graphs that
// captured a launch, keep using the buffer they were given.
struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
    std::vector<void *> retired;
};
std::mutex g_ws_mutex;
// kind kPartials: the split partials (any contents between calls).  kind
// kTickets: the in-kernel merge's row counters, zeroed when allocated and left
// at zero by every call -- a buffer of its own, so that no partial of a later
// call with other sizes ever lands on a counter.
enum WorkspaceKind { kPartials = 0, kTickets = 1 };
std::map<std::tuple<int, hipStream_t, int>, Workspace> g_ws;

// The stream's buffer of `kind`, grown to `need` bytes.  may_grow false (the
// stream is being captured): *out is null when the buffer is too small.
int workspace_for(hipStream_t stream, size_t need, void **out, int kind = kPartials,
                  bool may_grow = true) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace &w = g_ws[{dev, stream, kind}];
    if (w.bytes < need) {
        if (!may_grow) {
            *out = nullptr;
            return PA_OK;
        }
        const size_t least = kind == kTickets ? (size_t)(64 << 10) : (size_t)(1 << 20);
        size_t bytes = need < least ? least : need;
        if (bytes < 2 * w.bytes) bytes = 2 * w.bytes;  // geometric growth
        void *p = nullptr;
        e = hipMalloc(&p, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(PA_ERR_NO_MEMORY, "workspace of %zu bytes: %s", bytes,
                        hipGetErrorString(e));
        }
        if (kind == kTickets) {
            e = hipMemset(p, 0, bytes);  // synchronous: done before anything is queued
            if (e != hipSuccess) {
                (void)hipFree(p);
                return hip_fail(e, "workspace hipMemset");
            }
        }
        if (w.ptr) w.retired.push_back(w.ptr);
        w.ptr = p;
        w.bytes = bytes;
    }
    *out = w.ptr;
    return PA_OK;
}

// ---- allocation-free decode: the split workspace in a static device array ----
// For callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc): pa_decode_noalloc keeps its
// partials in this array, one copy per GPU, held until the process ends.
// Every call on a GPU shares that GPU's copy, so such calls must not overlap
// in time on one GPU.  In host code `scratch` is a stand-in, not a device
// address: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is used.
// Layout: [0, 256) the PA_DEBUG flags word; then the in-kernel merge's row
// counters (zero between calls: the array starts at zero and every call
// leaves them so) and PA_DEBUG's per-row XCD bits, 2,048 rows each; then the
// partials.
constexpr size_t kScratchBytes = (size_t)32 << 20;  // 32 MiB
constexpr size_t kScratchRows = 2048;
constexpr size_t kScratchTickets = 256;
constexpr size_t kScratchSeen = kScratchTickets + kScratchRows * sizeof(int);
constexpr size_t kScratchPartials = kScratchSeen + kScratchRows * sizeof(unsigned);  // 16,640
static_assert(kScratchPartials % 256 == 0, "partials stay 256-byte aligned");
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on its first use).
int scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "pa_decode_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_noalloc: device %d (at most %d devices)", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(PA_ERR_HIP, "pa_decode_noalloc: hipGetSymbolAddress: %s",
                        hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PA_OK;
}

// ---- in-kernel merge: the dispatcher rule it relies on, probed per device ----
std::mutex g_xcd_mutex;
int g_xcd_state[kMaxDevices] = {};  // 0 not probed, 1 the rule holds, 2 it does not

// Whether workgroups congruent mod 8 run on one XCD on the current device
// (pa::probe_xcd_dispatch, once per device: X XCDs dealt in turn, X dividing
// 8).  A stream under capture does not probe: its calls use the merge kernel
// until a call outside capture has probed.
bool xcd_rule_holds(bool capturing) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return false;
    }
    std::lock_guard<std::mutex> lock(g_xcd_mutex);
    if (g_xcd_state[dev] == 0) {
        if (capturing) return false;
        int X = 0;
        bool ok = false;
        if (pa::probe_xcd_dispatch(&X, &ok) != hipSuccess) {
            (void)hipGetLastError();
            ok = false;
        }
        g_xcd_state[dev] = ok && X >= 1 && 8 % X == 0 ? 1 : 2;
    }
    return g_xcd_state[dev] == 1;
}

// A PA_DEBUG buffer of one call: the stream is drained before it is freed.
struct DeviceBuffer {
    void *p = nullptr;
    hipStream_t stream = nullptr;
    ~DeviceBuffer() {
        if (p) {
            (void)hipStreamSynchronize(stream);
            (void)hipFree(p);
        }
    }
};

// The address a kernel uses for p: device memory as it is, pinned host memory
// (hipHostMalloc; torch's pin_memory) through its device mapping.  Pageable
// host memory cannot be reached by a kernel: PA_ERR_INVALID_ARG.
int device_view(const void *p, const char *what, const void **out) {
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e == hipErrorInvalidValue) {  // memory HIP does not know (older runtimes)
        (void)hipGetLastError();
        return fail(PA_ERR_INVALID_ARG,
                    "pa_swap_blocks: %s is neither device memory nor pinned host memory", what);
    }
    if (e != hipSuccess) return hip_fail(e, "pa_swap_blocks: hipPointerGetAttributes");
    if (attr.type == hipMemoryTypeHost) {
        void *dp = nullptr;
        e = hipHostGetDevicePointer(&dp, const_cast<void *>(p), 0);
        if (e != hipSuccess || !dp) {
            (void)hipGetLastError();
            return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: %s is host memory without a device "
                        "mapping", what);
        }
        *out = dp;
        return PA_OK;
    }
    if (attr.type == hipMemoryTypeUnregistered)
        return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: %s is pageable host memory", what);
    *out = p;
    return PA_OK;
}

constexpr int kBlock = 16;
constexpr int kMaxPartition = 1024;  // a unit keeps its table slice in one VGPR per lane
constexpr int kMaxPartitions = 1 << 16;

// Partition length when the caller leaves it to the library (the host cannot
// see the real lengths and counts units for full tables; rows = sequences x
// kv heads on MFMA, x query heads on VALU).  Both kernels run one wave per
// unit with one block requested ahead; a decode step streams fastest with
// about 40 KiB of reads outstanding per compute unit and with every compute
// unit busy to the end.  Measured on MI355X:
//  * rows >= 2048 (e.g. 64 sequences x 40 heads): the rows alone fill the
//    machine, and short units (P = 256) keep it evenly loaded to the end
//    (more units than resident waves, so finished ones are replaced):
//    OPT-13B-shaped MHA 156 us at P = 256 vs 162 us at P = 1024 -- unless
//    the tables hold at most 1024 tokens: then one pass per row needs no
//    merge (512 sequences of U{128..600} tokens, tables of 640: 132.4 us in
//    one pass against 148.0 at P = 256 and 139.5 at P = 512);
//  * fewer rows (32 sequences x 8 kv heads): rows must be split for
//    parallelism, and long units cut the partials the merge reads: the
//    longest P <= 1024 with >= 1024 units (Llama-3-8B-shaped: P = 1024,
//    53.7 us vs 54.9 at 512 and 58.1 at 256);
//  * the VALU kernel (fp32 data or more than 16 query heads per kv head)
//    does more arithmetic per byte and takes P <= 512 with >= 2048 units.
int auto_partition(bool mfma, int64_t rows, int max_tokens) {
    if (mfma && rows >= 2048) return max_tokens <= kMaxPartition ? kMaxPartition : 256;
    const int longest = mfma ? 1024 : 512;
    const int64_t min_units = mfma ? 1024 : 2048;
    for (int P = longest; P > 256; P /= 2)
        if (rows * (((int64_t)max_tokens + P - 1) / P) >= min_units) return P;
    return 256;
}

// Compute units of the current device (cached per device; 256 if unknown).
int device_cus() {
    static std::mutex mu;
    static std::map<int, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    cache[dev] = cus;
    return cus;
}

int64_t num_partitions(int max_tokens, int P) {
    int64_t np = ((int64_t)max_tokens + P - 1) / P;
    return np < 1 ? 1 : np;
}

}  // namespace

extern "C" {

const char *pa_status_str(int status) {
    switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_NO_MEMORY: return "PA_ERR_NO_MEMORY";
    default: return "PA_ERR_UNKNOWN";
    }
}

const char *pa_last_error(void) { return g_last_error.c_str(); }

int pa_version(void) { return 100; }

int pa_write_kv(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                const int64_t *slot_mapping, int64_t num_tokens, int num_kv_heads, int head_dim,
                int block_size, int64_t num_blocks, int dtype, void *stream) {
    const int e = elem_bytes(dtype);
    if (e == 0) return fail(PA_ERR_INVALID_ARG, "pa_write_kv: unknown dtype %d", dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG,
                    "pa_write_kv: sizes must be positive (tokens %lld, kv heads %d, head_dim %d, "
                    "block %d, blocks %lld)",
                    (long long)num_tokens, num_kv_heads, head_dim, block_size,
                    (long long)num_blocks);
    const int x = 16 / e;
    if (head_dim % x != 0 || head_dim > 512)
        return fail(PA_ERR_INVALID_ARG, "pa_write_kv: head_dim %d must be a multiple of %d, <= 512",
                    head_dim, x);
    if (num_tokens == 0) return PA_OK;
    const int64_t tile_tokens = 256 / (head_dim / x);  // tokens per workgroup
    if ((num_tokens + tile_tokens - 1) / tile_tokens * num_kv_heads > 0x7fffffff)
        return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: %lld tokens x %d kv heads in one call",
                    (long long)num_tokens, num_kv_heads);
    if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "pa_write_kv: null pointer");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
        ((uintptr_t)slot_mapping & 7u))
        return fail(PA_ERR_INVALID_ARG, "pa_write_kv: data pointers must be 16-byte aligned");
    if (pa::debug_enabled()) {
        const int rc = pa::debug_check_slots("pa_write_kv", slot_mapping, num_tokens,
                                             num_blocks * block_size, (hipStream_t)stream);
        if (rc != PA_OK) return rc;
    }
    hipError_t err = pa::launch_write_kv(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens,
                                         num_kv_heads, head_dim, block_size, num_blocks, e,
                                         (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "pa_write_kv launch");
    return PA_OK;
}

int pa_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping, int64_t num_pairs,
                   int num_kv_heads, int head_dim, int block_size, int64_t num_blocks, int dtype,
                   void *stream) {
    const int e = elem_bytes(dtype);
    if (e == 0) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: unknown dtype %d", dtype);
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: sizes must be positive");
    const int64_t block_bytes = (int64_t)num_kv_heads * head_dim * block_size * e;
    if (block_bytes % 16 != 0)
        return fail(PA_ERR_INVALID_ARG,
                    "pa_copy_blocks: a block of %lld bytes is not a multiple of 16",
                    (long long)block_bytes);
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !block_mapping)
        return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: null pointer");
    if (!aligned16(k_cache) || !aligned16(v_cache) || ((uintptr_t)block_mapping & 7u))
        return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: pools must be 16-byte aligned");
    if (pa::debug_enabled()) {
        const int rc = pa::debug_check_pairs("pa_copy_blocks", block_mapping, num_pairs,
                                             num_blocks, num_blocks, true, (hipStream_t)stream);
        if (rc != PA_OK) return rc;
    }
    hipError_t err = pa::launch_copy_blocks(k_cache, v_cache, k_cache, v_cache, block_mapping,
                                            num_pairs, num_blocks, num_blocks, block_bytes,
                                            (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "pa_copy_blocks launch");
    return PA_OK;
}

int pa_swap_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                   const int64_t *block_mapping, int64_t num_pairs, int num_kv_heads,
                   int head_dim, int block_size, int64_t num_src_blocks, int64_t num_dst_blocks,
                   int dtype, void *stream) {
    const int e = elem_bytes(dtype);
    if (e == 0) return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: unknown dtype %d", dtype);
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_src_blocks <= 0 || num_dst_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: sizes must be positive");
    const int64_t block_bytes = (int64_t)num_kv_heads * head_dim * block_size * e;
    if (block_bytes % 16 != 0)
        return fail(PA_ERR_INVALID_ARG,
                    "pa_swap_blocks: a block of %lld bytes is not a multiple of 16",
                    (long long)block_bytes);
    if (num_pairs == 0) return PA_OK;
    if (!src_k || !src_v || !dst_k || !dst_v || !block_mapping)
        return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: null pointer");
    if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v) ||
        ((uintptr_t)block_mapping & 7u))
        return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: pools must be 16-byte aligned");
    const void *d[5];
    const void *h[5] = {src_k, src_v, dst_k, dst_v, block_mapping};
    const char *names[5] = {"src_k", "src_v", "dst_k", "dst_v", "block_mapping"};
    for (int i = 0; i < 5; ++i) {
        const int rc = device_view(h[i], names[i], &d[i]);
        if (rc != PA_OK) return rc;
    }
    if (pa::debug_enabled()) {
        const int rc = pa::debug_check_pairs("pa_swap_blocks", (const int64_t *)d[4], num_pairs,
                                             num_src_blocks, num_dst_blocks,
                                             d[0] == d[2] || d[1] == d[3], (hipStream_t)stream);
        if (rc != PA_OK) return rc;
    }
    hipError_t err = pa::launch_copy_blocks(d[0], d[1], (void *)d[2], (void *)d[3],
                                            (const int64_t *)d[4], num_pairs, num_src_blocks,
                                            num_dst_blocks, block_bytes, (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "pa_swap_blocks launch");
    return PA_OK;
}

int pa_decode_plan(const int32_t *context_lens, int num_seqs, int num_heads, int num_kv_heads,
                   int block_size, int max_blocks_per_seq, int dtype, int *partition_tokens) {
    if (!partition_tokens) return fail(PA_ERR_INVALID_ARG, "pa_decode_plan: null output");
    *partition_tokens = 0;
    if (elem_bytes(dtype) == 0) return fail(PA_ERR_INVALID_ARG, "pa_decode_plan: unknown dtype");
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || block_size <= 0 ||
        max_blocks_per_seq < 0 || num_heads % num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_plan: bad sizes");
    if (num_seqs > 0 && !context_lens)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_plan: null context_lens");
    const bool mfma = dtype != PA_F32 && num_heads / num_kv_heads <= 16;
    const int64_t rows = (int64_t)num_seqs * num_kv_heads;
    // where the plan does not apply, 0: the library's automatic choice
    if (num_seqs == 0 || !mfma || (block_size != kBlock && block_size != 32) || rows >= 2048)
        return PA_OK;
    // Every unit of the split is resident at once, so each compute unit runs
    // about ceil(units / CUs) of them and the step lasts about as long as
    // that many of the longest; take the length that makes this product
    // smallest (ties: the longer partitions, fewer partials to merge).
    const int64_t cus = device_cus();
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    int best = 0;
    int64_t best_cost = INT64_MAX;
    for (int P = 512; P <= kMaxPartition; P += 128) {
        int64_t units = 0, longest = 0;
        for (int s = 0; s < num_seqs; ++s) {
            const int64_t c = std::min<int64_t>(std::max<int32_t>(context_lens[s], 0), cap);
            const int64_t n = c > P ? (c + P - 1) / P : 1;
            const int64_t nb = (c + block_size - 1) / block_size;
            units += n * num_kv_heads;
            longest = std::max(longest, (nb + n - 1) / n);
        }
        const int64_t cost = (units + cus - 1) / cus * longest;
        if (cost <= best_cost) best_cost = cost, best = P;
    }
    *partition_tokens = best;
    return PA_OK;
}

int64_t pa_decode_workspace_bytes(int num_seqs, int num_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int partition_tokens) {
    if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks_per_seq <= 0)
        return 0;
    const int max_tokens = max_blocks_per_seq * block_size;
    // an upper bound: the smallest partition length the library picks itself
    // (plus the 256 bytes a length planned on the device keeps beside them)
    int P = partition_tokens > 0 ? partition_tokens : 256;
    if (P >= max_tokens) return 0;
    const int64_t np = num_partitions(max_tokens, P);
    return (int64_t)num_seqs * num_heads * np * (head_dim + 2) * (int64_t)sizeof(float) +
           (partition_tokens > 0 ? 0 : 256);
}

}  // extern "C"

namespace pa {

// The partitioning a decode call takes (arguments already validated).
struct DecodeShape {
    bool mfma;       // matrix-core partition kernel
    int P;           // partition length in tokens
    int64_t NP;      // partitions per row for full tables
    int64_t units;   // work units for full tables (the grid)
    bool fused;      // merge inside the partition kernel (subject to the dispatch probe)
    bool plan;       // P chosen on the device (device_plan); P, NP, units: for 512 tokens
};

// Automatic partitions planned on the device from the context lengths: the
// matrix-core kernel at B = 16 with fewer than 2,048 rows (sequences x kv
// heads; more rows fill the machine at 256 tokens), at most 256 sequences
// (every workgroup holds all context lengths in four registers), and tables
// longer than the shortest candidate (512 tokens; shorter ones take one pass
// anyway) and of at most 2^20 tokens (the plan's integer quotients go
// through fp32).
constexpr int kPlanMaxSeqs = 256;
constexpr int kPlanShortest = 512;
constexpr int kPlanLongest = 1 << 20;

DecodeShape decode_shape(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int dtype,
                         int partition_tokens, int flags) {
    DecodeShape sh{};
    const int G = num_heads / num_kv_heads;
    const int max_tokens = max_blocks_per_seq * block_size;
    // block size 8: a unit's table slice is 64 entries = 512 tokens
    const int max_part = block_size == 8 ? 512 : kMaxPartition;
    sh.mfma = dtype != PA_F32 && G <= 16 && !(flags & PA_DECODE_FORCE_VALU);
    sh.plan = partition_tokens == 0 && sh.mfma && block_size == kBlock &&
              (int64_t)num_seqs * num_kv_heads < 2048 && num_seqs <= kPlanMaxSeqs &&
              max_tokens > kPlanShortest && max_tokens <= kPlanLongest;
    int P = sh.plan ? kPlanShortest
            : partition_tokens > 0
                ? partition_tokens
                : std::min(auto_partition(sh.mfma,
                                          (int64_t)num_seqs * (sh.mfma ? num_kv_heads : num_heads),
                                          max_tokens),
                           // block 32: a wave has a whole 16 KiB block in flight, and
                           // shorter units stream better (Llama-3-8B step: 53.2 us at
                           // 512 against 54.5 at 1024 and 57.4 at 256)
                           block_size == 32 ? 512 : max_part);
    int64_t NP = 1;
    if (P < max_tokens) {
        NP = num_partitions(max_tokens, P);
    } else {
        // one partition covers every sequence; keep P a multiple of 16 that does
        P = max_tokens < kBlock ? kBlock : (max_tokens + kBlock - 1) / kBlock * kBlock;
        if (P > max_part) P = max_part, NP = num_partitions(max_tokens, P);
    }
    sh.P = P;
    sh.NP = NP;
    sh.units = NP * (int64_t)num_seqs * (sh.mfma ? num_kv_heads : num_heads);
    // In-kernel merge (merge_row_in_l2 in pa_decode.hip): the matrix-core
    // kernel at B = 8 or 16; kv heads a multiple of 8, so that a row's units
    // are congruent mod 8 and share an XCD; at most kFusedMaxParts partitions
    // and 512 outputs per row, which the last unit reads back in one round
    // trip; and every unit resident at once (kFusedMaxUnits: 3 waves per SIMD
    // at the kernel's ~144 VGPRs hold 3,072), since a unit that keeps its slot
    // through the ticket round trip would otherwise hold back queued units
    // (OPT-13B-shaped step, ~6,000 units: 1 us slower than the merge kernel).
    sh.fused = NP > 1 && sh.mfma && block_size != 32 && num_kv_heads % 8 == 0 &&
               NP <= kFusedMaxParts && G * head_dim <= 512 && sh.units <= kFusedMaxUnits &&
               !(flags & PA_DECODE_MERGE_KERNEL);
    return sh;
}

// pa_decode_ex, and the decode over virtual-memory storage (block_tables ==
// nullptr, a Contiguous description instead).
int decode_impl(const void *q, const void *k_cache, const void *v_cache,
                const int32_t *block_tables, const int32_t *context_lens, float scale,
                void *out, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                int block_size, int max_blocks_per_seq, int64_t num_blocks, int dtype,
                int partition_tokens, int flags, void *stream, const Contiguous *contig,
                const void *k_new, const void *v_new, int *read_sink, bool no_alloc) {
    const int e = elem_bytes(dtype);
    if (e == 0) return fail(PA_ERR_INVALID_ARG, "pa_decode: unknown dtype %d", dtype);
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq < 0 || num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode: sizes must be positive");
    if (num_heads % num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode: num_heads %d is not a multiple of %d",
                    num_heads, num_kv_heads);
    if (!isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "pa_decode: scale is not finite");
    if (flags & ~(PA_DECODE_SHARED_BLOCKS | PA_DECODE_FORCE_VALU | PA_DECODE_MERGE_KERNEL))
        return fail(PA_ERR_INVALID_ARG, "pa_decode: unknown flags 0x%x", flags);
    const bool force_valu = (flags & PA_DECODE_FORCE_VALU) != 0;
    if (force_valu && (block_size != kBlock || k_new || v_new))
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: PA_DECODE_FORCE_VALU takes block_size 16 "
                    "and no appended token");
    if (partition_tokens < 0 || (partition_tokens > 0 && (partition_tokens % kBlock != 0 ||
                                                          partition_tokens > kMaxPartition)))
        return fail(PA_ERR_INVALID_ARG,
                    "pa_decode: partition_tokens %d must be 0 or a multiple of 16 in [16, %d]",
                    partition_tokens, kMaxPartition);
    const bool mfma_ok = dtype != PA_F32 && num_heads / num_kv_heads <= 16;
    if ((k_new || v_new) && !(mfma_ok && block_size == kBlock && !contig))
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_append: 16-bit data, at most 16 query heads "
                    "per kv head and block_size 16 only");
    if (block_size != kBlock && !((block_size == 8 || block_size == 32) && mfma_ok && !contig))
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: block_size %d (16 is built for every case; "
                    "8 and 32 for 16-bit data with at most 16 query heads per kv head)",
                    block_size);
    // block size 8: a unit's table slice is 64 entries = 512 tokens, and the
    // kernel addresses the pool with 32-bit offsets
    const int max_part = block_size == 8 ? 512 : kMaxPartition;
    if (block_size == 8 && partition_tokens > max_part)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: block_size 8 takes partition_tokens <= 512");
    if (block_size == 32 && partition_tokens % 32 != 0)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: block_size 32 takes partition_tokens that "
                    "are multiples of 32");
    if (block_size == 8 &&
        num_blocks * (int64_t)num_kv_heads * head_dim * block_size * e > 0x7fff0000LL)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: block_size 8 takes pools under 2 GiB");
    if (head_dim != 64 && head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: head_dim %d (64 and 128 are built)",
                    head_dim);
    if ((int64_t)max_blocks_per_seq * block_size > (int64_t)1 << 30)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: max_blocks_per_seq too large");
    if (num_seqs == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !(block_tables || contig) || !context_lens || !out ||
        (contig && (!contig->req || !contig->mapped)) || (!k_new != !v_new))
        return fail(PA_ERR_INVALID_ARG, "pa_decode: null pointer");
    if ((k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)))
        return fail(PA_ERR_INVALID_ARG, "pa_decode_append: new tokens must be 16-byte aligned");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u) ||
        (contig && ((uintptr_t)contig->req & 3u)))
        return fail(PA_ERR_INVALID_ARG, "pa_decode: data pointers must be 16-byte aligned");

    const int G = num_heads / num_kv_heads;
    const DecodeShape sh = decode_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                        max_blocks_per_seq, dtype, partition_tokens, flags);
    const bool mfma = sh.mfma;
    int P = sh.P;
    const int64_t NP = sh.NP;
    if (NP > kMaxPartitions)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: %lld partitions (max %d)", (long long)NP,
                    kMaxPartitions);
    const int64_t units = sh.units;
    if (units > (int64_t)0x7fffffff - 4096)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode: %lld work units", (long long)units);

    pa::DecodeArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.bt = block_tables;
    a.ctx = context_lens;
    a.out = out;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.scale_log2_abs = fabsf(scale) * 1.4426950408889634f;
    a.q_xor = scale < 0.f ? (int)0x80008000u : 0;
    a.S = num_seqs;
    a.Hq = num_heads;
    a.Hkv = num_kv_heads;
    a.G = G;
    a.MB = max_blocks_per_seq;
    a.NP = (int)NP;
    a.P = P;
    a.plan = sh.plan ? 1 : 0;
    a.cus = device_cus();
    a.NB = num_blocks;
    a.BS = block_size;
    a.num_units = (int)units;
    a.shared_blocks = (flags & PA_DECODE_SHARED_BLOCKS) != 0;
    a.k_new = k_new;
    a.v_new = v_new;
    if (contig) {
        a.bt = nullptr;
        a.req = contig->req;
        a.mapped = contig->mapped;
        a.req_stride = contig->req_stride;
        a.num_req = contig->num_req;
    }
    // a planned launch keeps its length after the partials, for the merge kernel
    const size_t plan_bytes = sh.plan ? 256 : 0;
    const size_t part_bytes =
        NP > 1 ? (size_t)num_seqs * num_heads * NP * (head_dim + 2) * sizeof(float) + plan_bytes
               : 0;
    void *fixed = nullptr;  // pa_decode_noalloc: the static scratch
    if (no_alloc) {
        if (part_bytes > kScratchBytes - kScratchPartials)
            return fail(PA_ERR_UNSUPPORTED,
                        "pa_decode_noalloc: %zu bytes of partials (%d sequences x %d heads x %lld "
                        "partitions) exceed the %zu-byte static workspace; use pa_decode",
                        part_bytes, num_seqs, num_heads, (long long)NP,
                        kScratchBytes - kScratchPartials);
        const int rc = scratch_address(&fixed);
        if (rc != PA_OK) return rc;
    }
    if (pa::debug_enabled() && !contig) {
        const int rc = pa::debug_check_tables(read_sink ? "pa_read_tiles" : "pa_decode",
                                              block_tables, context_lens, num_seqs,
                                              max_blocks_per_seq, block_size, num_blocks,
                                              (hipStream_t)stream, (unsigned *)fixed);
        if (rc != PA_OK) return rc;
    }
    if (read_sink) {  // pa_read_tiles: the partition kernel's loads alone
        hipError_t err = pa::launch_read_tiles(a, head_dim, read_sink, (hipStream_t)stream);
        if (err != hipSuccess) return hip_fail(err, "pa_read_tiles launch");
        return PA_OK;
    }
    DeviceBuffer seen_owned;  // PA_DEBUG's per-row XCD bits (in-kernel merge)
    const int64_t rows = (int64_t)num_seqs * num_kv_heads;
    if (NP > 1) {
        void *ws = nullptr;
        const size_t o_bytes = (size_t)num_seqs * num_heads * NP * head_dim * sizeof(float);
        if (fixed) {
            ws = (char *)fixed + kScratchPartials;
        } else {
            const int rc = workspace_for((hipStream_t)stream, part_bytes, &ws);
            if (rc != PA_OK) return rc;
        }
        a.part_o = (float *)ws;
        a.part_ml = (float *)((char *)ws + o_bytes);
        if (sh.plan) a.plan_slot = (int *)((char *)ws + part_bytes - plan_bytes);
        if (sh.fused) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            hipError_t ce = hipStreamIsCapturing((hipStream_t)stream, &cs);
            if (ce != hipSuccess) return hip_fail(ce, "pa_decode: hipStreamIsCapturing");
            const bool capturing = cs != hipStreamCaptureStatusNone;
            void *tk = nullptr;
            if (xcd_rule_holds(capturing)) {
                if (fixed) {
                    tk = (char *)fixed + kScratchTickets;  // rows <= units <= kScratchRows
                } else {
                    // a stream under capture does not allocate: merge kernel instead
                    const int rc = workspace_for((hipStream_t)stream, (size_t)rows * sizeof(int),
                                                 &tk, kTickets, !capturing);
                    if (rc != PA_OK) return rc;
                }
            }
            if (tk) {
                a.fuse_merge = 1;
                a.ticket = (int *)tk;
                if (pa::debug_enabled() && !capturing) {
                    void *seen = nullptr;
                    if (fixed) {
                        seen = (char *)fixed + kScratchSeen;
                    } else {
                        hipError_t me = hipMalloc(&seen, (size_t)rows * sizeof(unsigned));
                        if (me != hipSuccess) {
                            (void)hipGetLastError();
                            return fail(PA_ERR_NO_MEMORY, "pa_decode: PA_DEBUG scratch: %s",
                                        hipGetErrorString(me));
                        }
                        seen_owned.p = seen;
                        seen_owned.stream = (hipStream_t)stream;
                    }
                    hipError_t me = hipMemsetAsync(seen, 0, (size_t)rows * sizeof(unsigned),
                                                   (hipStream_t)stream);
                    if (me != hipSuccess) return hip_fail(me, "pa_decode: PA_DEBUG memset");
                    a.xcd_seen = (unsigned *)seen;
                }
            }
        }
    }
    hipError_t err = pa::launch_decode(a, dtype, head_dim,
                                       mfma ? pa::DecodeKernel::kMfma : pa::DecodeKernel::kValu,
                                       (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "pa_decode launch");
    if (a.xcd_seen)
        return pa::debug_check_xcd(k_new ? "pa_decode_append" : "pa_decode", a.xcd_seen, rows,
                                   (hipStream_t)stream, (unsigned *)fixed);
    return PA_OK;
}

}  // namespace pa

extern "C" {

int pa_decode_merge_mode(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int dtype,
                         int partition_tokens, int flags) {
    if (elem_bytes(dtype) == 0 || num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || block_size <= 0 || max_blocks_per_seq < 0 ||
        num_heads % num_kv_heads != 0 || partition_tokens < 0 ||
        (partition_tokens > 0 &&
         (partition_tokens % kBlock != 0 || partition_tokens > kMaxPartition)) ||
        (flags & ~(PA_DECODE_SHARED_BLOCKS | PA_DECODE_FORCE_VALU | PA_DECODE_MERGE_KERNEL))) {
        fail(PA_ERR_INVALID_ARG, "pa_decode_merge_mode: bad arguments");
        return -PA_ERR_INVALID_ARG;
    }
    if (num_seqs == 0) return PA_MERGE_NONE;
    const pa::DecodeShape sh = pa::decode_shape(num_seqs, num_heads, num_kv_heads, head_dim,
                                                block_size, max_blocks_per_seq, dtype,
                                                partition_tokens, flags);
    if (sh.NP <= 1) return PA_MERGE_NONE;
    return sh.fused && xcd_rule_holds(false) ? PA_MERGE_IN_KERNEL : PA_MERGE_KERNEL;
}

int pa_decode_ex(const void *q, const void *k_cache, const void *v_cache,
                 const int32_t *block_tables, const int32_t *context_lens, float scale,
                 void *out, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                 int block_size, int max_blocks_per_seq, int64_t num_blocks, int dtype,
                 int partition_tokens, int flags, void *stream) {
    return pa::decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                           num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                           max_blocks_per_seq, num_blocks, dtype, partition_tokens, flags, stream,
                           nullptr);
}

int pa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, float scale,
                      void *out, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                      int block_size, int max_blocks_per_seq, int64_t num_blocks, int dtype,
                      int partition_tokens, int flags, void *stream) {
    return pa::decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                           num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                           max_blocks_per_seq, num_blocks, dtype, partition_tokens, flags, stream,
                           nullptr, nullptr, nullptr, nullptr, true);
}

int pa_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache,
                     void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                     float scale, void *out, int num_seqs, int num_heads, int num_kv_heads,
                     int head_dim, int block_size, int max_blocks_per_seq, int64_t num_blocks,
                     int dtype, int partition_tokens, void *stream) {
    if (num_seqs > 0 && (!k_new || !v_new))
        return fail(PA_ERR_INVALID_ARG, "pa_decode_append: null pointer");
    return pa::decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                           num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                           num_blocks, dtype, partition_tokens, 0, stream, nullptr, k_new, v_new);
}

int pa_read_tiles(const void *k_cache, const void *v_cache, const int32_t *block_tables,
                  const int32_t *context_lens, int32_t *sink, int num_seqs, int num_heads,
                  int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                  int64_t num_blocks, int dtype, int partition_tokens, void *stream) {
    if (dtype == PA_F32 || (num_kv_heads > 0 && num_heads / num_kv_heads > 16) ||
        block_size != kBlock)
        return fail(PA_ERR_UNSUPPORTED, "pa_read_tiles: the matrix-core decode configuration "
                    "only (16-bit data, at most 16 query heads per kv head, block_size 16)");
    if (num_seqs > 0 && (!sink || ((uintptr_t)sink & 3u)))
        return fail(PA_ERR_INVALID_ARG, "pa_read_tiles: sink must be a 4-byte aligned pointer");
    // q and out are not touched: the K pool stands in for them in the checks
    return pa::decode_impl(k_cache, k_cache, v_cache, block_tables, context_lens, 1.f,
                           (void *)k_cache, num_seqs, num_heads, num_kv_heads, head_dim,
                           block_size, max_blocks_per_seq, num_blocks, dtype, partition_tokens, 0,
                           stream, nullptr, nullptr, nullptr, sink);
}

int pa_decode(const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, const int32_t *context_lens, float scale, void *out,
              int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
              int max_blocks_per_seq, int64_t num_blocks, int dtype, void *stream) {
    return pa_decode_ex(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                        num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        num_blocks, dtype, 0, 0, stream);
}

int pa_decode_cascade(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens,
                      const int32_t *group_start, const int32_t *prefix_blocks, int num_groups,
                      int max_group_size, float scale, void *out, int num_seqs, int num_heads,
                      int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                      int64_t num_blocks, int dtype, int partition_tokens, void *stream) {
    const int e = elem_bytes(dtype);
    if (e == 0) return fail(PA_ERR_INVALID_ARG, "pa_decode_cascade: unknown dtype %d", dtype);
    if (num_seqs < 0 || num_groups < 0 || max_group_size < 0 || num_heads <= 0 ||
        num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq < 0 ||
        num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_cascade: sizes must be positive");
    if (num_heads % num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARG,
                    "pa_decode_cascade: num_heads %d is not a multiple of %d", num_heads,
                    num_kv_heads);
    if (!isfinite(scale))
        return fail(PA_ERR_INVALID_ARG, "pa_decode_cascade: scale is not finite");
    if ((num_seqs > 0) != (num_groups > 0) || num_groups > num_seqs ||
        (num_seqs > 0 && (max_group_size < 1 || max_group_size > num_seqs)))
        return fail(PA_ERR_INVALID_ARG, "pa_decode_cascade: %d groups of at most %d sequences "
                    "cannot cover %d sequences", num_groups, max_group_size, num_seqs);
    if (partition_tokens < 0 || (partition_tokens > 0 && (partition_tokens % kBlock != 0 ||
                                                          partition_tokens > kMaxPartition)))
        return fail(PA_ERR_INVALID_ARG,
                    "pa_decode_cascade: partition_tokens %d must be 0 or a multiple of 16 in "
                    "[16, %d]", partition_tokens, kMaxPartition);
    if (dtype == PA_F32)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_cascade: fp32 (the matrix-core path takes "
                    "16-bit data)");
    if (block_size != kBlock)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_cascade: block_size %d (only 16 is built)",
                    block_size);
    if (head_dim != 64 && head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_cascade: head_dim %d (64 and 128 are built)",
                    head_dim);
    if ((int64_t)max_blocks_per_seq * block_size > (int64_t)1 << 30)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_cascade: max_blocks_per_seq too large");
    if (num_seqs == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !group_start ||
        !prefix_blocks || !out)
        return fail(PA_ERR_INVALID_ARG, "pa_decode_cascade: null pointer");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u) ||
        ((uintptr_t)group_start & 3u) || ((uintptr_t)prefix_blocks & 3u))
        return fail(PA_ERR_INVALID_ARG,
                    "pa_decode_cascade: data pointers must be 16-byte aligned");

    const int G = num_heads / num_kv_heads;
    // default: the longest partitions (fewest partials to merge; parallel
    // sampling 108 us at 1024 against 117 at 256, 113 at 512)
    const int P = partition_tokens > 0 ? partition_tokens : kMaxPartition;
    const int64_t max_tokens = (int64_t)max_blocks_per_seq * kBlock;
    const int64_t np = max_tokens > 0 ? (max_tokens + P - 1) / P : 1;
    const int64_t tiles = ((int64_t)max_group_size * G + 15) / 16;
    // units: prefix (group, partition, tile, kv head) + suffix (sequence, partition, kv head)
    const int64_t units = ((int64_t)num_groups * tiles + num_seqs) * np * num_kv_heads;
    if (units > (int64_t)0x7fffffff - 65536 || (int64_t)num_seqs * num_heads > 0x7fffffff / 64)
        return fail(PA_ERR_UNSUPPORTED, "pa_decode_cascade: %lld work units",
                    (long long)units);
    // one wave per workgroup; up to 8192 workgroups take a unit each (the
    // dispatcher then balances units of different lengths), beyond that they
    // walk the list in rounds (measured on the parallel-sampling step: 8192
    // 116.5 us, 16384 117.9 us, 4096 123 us)
    const int grid = (int)(units < 8192 ? (units > 0 ? units : 1) : 8192);

    pa::CascadeArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.bt = block_tables;
    a.ctx = context_lens;
    a.gs = group_start;
    a.pblk = prefix_blocks;
    a.out = out;
    a.scale_log2_abs = fabsf(scale) * 1.4426950408889634f;
    a.q_xor = scale < 0.f ? (int)0x80008000u : 0;
    a.S = num_seqs;
    a.NG = num_groups;
    a.Hq = num_heads;
    a.Hkv = num_kv_heads;
    a.G = G;
    a.MB = max_blocks_per_seq;
    a.P = P;
    a.NPP = (int)np;
    a.NPT = (int)(2 * np);
    a.NB = num_blocks;
    if (pa::debug_enabled()) {
        int rc = pa::debug_check_tables("pa_decode_cascade", block_tables, context_lens,
                                        num_seqs, max_blocks_per_seq, block_size, num_blocks,
                                        (hipStream_t)stream);
        if (rc == PA_OK)
            rc = pa::debug_check_groups("pa_decode_cascade", group_start, prefix_blocks,
                                        block_tables, context_lens, num_groups, num_seqs,
                                        max_blocks_per_seq, max_group_size, (hipStream_t)stream);
        if (rc != PA_OK) return rc;
    }
    void *ws = nullptr;
    const size_t rows = (size_t)num_seqs * num_heads;
    const size_t o_bytes = rows * a.NPT * head_dim * sizeof(float);
    const size_t ml_bytes = rows * a.NPT * 2 * sizeof(float);
    int rc = workspace_for((hipStream_t)stream, o_bytes + ml_bytes, &ws);
    if (rc != PA_OK) return rc;
    a.part_o = (float *)ws;
    a.part_ml = (float *)((char *)ws + o_bytes);
    hipError_t err = pa::launch_cascade(a, dtype, head_dim, grid, (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "pa_decode_cascade launch");
    return PA_OK;
}

int pa_prefill(const void *q, const void *k_cache, const void *v_cache,
               const int32_t *block_tables, const int32_t *context_lens,
               const int32_t *query_start, float scale, void *out, int num_seqs, int num_tokens,
               int max_query_len, int num_heads, int num_kv_heads, int head_dim, int block_size,
               int max_blocks_per_seq, int64_t num_blocks, int dtype, void *stream) {
    const int e = elem_bytes(dtype);
    if (e == 0) return fail(PA_ERR_INVALID_ARG, "pa_prefill: unknown dtype %d", dtype);
    if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || num_heads <= 0 ||
        num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq < 0 ||
        num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "pa_prefill: sizes must be positive");
    if (num_heads % num_kv_heads != 0)
        return fail(PA_ERR_INVALID_ARG, "pa_prefill: num_heads %d is not a multiple of %d",
                    num_heads, num_kv_heads);
    if (!isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "pa_prefill: scale is not finite");
    if (max_query_len > num_tokens)
        return fail(PA_ERR_INVALID_ARG, "pa_prefill: max_query_len %d exceeds num_tokens %d",
                    max_query_len, num_tokens);
    if (dtype == PA_F32)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: fp32 (the matrix-core path takes 16-bit "
                    "data)");
    if (block_size != kBlock)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: block_size %d (only 16 is built)",
                    block_size);
    if (head_dim != 64 && head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: head_dim %d (64 and 128 are built)",
                    head_dim);
    if ((int64_t)max_blocks_per_seq * block_size > (int64_t)1 << 30)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: max_blocks_per_seq too large");
    const int G = num_heads / num_kv_heads;
    if ((int64_t)max_query_len * G > (int64_t)1 << 30 || num_seqs > 65535 ||
        pa::prefill_row_tiles(max_query_len, G) > 65535 ||
        pa::prefill_row_tiles(max_query_len, G) * num_seqs * num_kv_heads > INT32_MAX)
        return fail(PA_ERR_UNSUPPORTED, "pa_prefill: %d sequences x %d queries x %d heads per "
                    "kv head exceed the launch grid", num_seqs, max_query_len, G);
    if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
        return fail(PA_ERR_INVALID_ARG, "pa_prefill: null pointer");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u) ||
        ((uintptr_t)query_start & 3u))
        return fail(PA_ERR_INVALID_ARG, "pa_prefill: data pointers must be 16-byte aligned");

    if (pa::debug_enabled()) {
        int rc = pa::debug_check_tables("pa_prefill", block_tables, context_lens, num_seqs,
                                        max_blocks_per_seq, block_size, num_blocks,
                                        (hipStream_t)stream);
        if (rc == PA_OK)
            rc = pa::debug_check_query_start("pa_prefill", query_start, context_lens, num_seqs,
                                             num_tokens, max_query_len, (hipStream_t)stream);
        if (rc != PA_OK) return rc;
    }
    pa::PrefillArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.bt = block_tables;
    a.ctx = context_lens;
    a.qs = query_start;
    a.out = out;
    a.scale_log2_abs = fabsf(scale) * 1.4426950408889634f;
    a.q_xor = scale < 0.f ? (int)0x80008000u : 0;
    a.S = num_seqs;
    a.T = num_tokens;
    a.Hq = num_heads;
    a.Hkv = num_kv_heads;
    a.G = G;
    a.MB = max_blocks_per_seq;
    a.NB = num_blocks;
    hipError_t err = pa::launch_prefill(a, dtype, head_dim, max_query_len, (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "pa_prefill launch");
    return PA_OK;
}

int pa_release_workspaces(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int rc = PA_OK;
    int prev = 0;
    (void)hipGetDevice(&prev);
    for (auto it = g_ws.begin(); it != g_ws.end();) {
        Workspace &w = it->second;
        (void)hipSetDevice(std::get<0>(it->first));
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) {  // keep the buffers: work may still use them
            rc = hip_fail(e, "pa_release_workspaces");
            ++it;
            continue;
        }
        if (w.ptr) w.retired.push_back(w.ptr);
        for (void *p : w.retired) {
            e = hipFree(p);
            if (e != hipSuccess) rc = hip_fail(e, "pa_release_workspaces");
        }
        it = g_ws.erase(it);
    }
    (void)hipSetDevice(prev);
    return rc;
}

}  // extern "C"
