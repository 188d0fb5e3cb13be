// pa_internal.h -- host-side declarations shared by the libpa translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Everything one decode launch needs; passed by value as the kernel argument.
struct DecodeArgs {
    const void *q;          // [S][Hq][D]
    const void *k;          // K pool [NB][Hkv][D/x][B][x]
    const void *v;          // V pool [NB][Hkv][D][B]
    const int *bt;          // [S][MB]
    const int *ctx;         // [S]
    void *out;              // [S][Hq][D]
    float *part_o;          // [S][Hq][NP][D]   (split path only)
    float *part_ml;         // [S][Hq][NP][2]   (m in log2 units, l)
    float scale_log2;       // scale * log2(e)
    float scale_log2_abs;   // |scale| * log2(e)
    int q_xor;              // 0x80008000 when scale < 0: flips the sign of 16-bit q
    int S, Hq, Hkv, G, MB, NP, P;
    // plan != 0: the partition length is chosen by every workgroup from the
    // context lengths (device_plan in pa_decode.hip) among 512, 640, ...,
    // 1024 tokens; P and NP then describe the shortest, which sizes the grid
    // and the partials.  cus: compute units of the device, for that choice.
    int plan;
    int cus;
    int *plan_slot;         // plan: workgroup 0 of the partition kernel stores P here for the merge
    int BS;                 // tokens per block: 16, or 8 / 32 (matrix-core kernel only)
    int64_t NB;
    int num_units;          // workgroups of the launch: an upper bound on the units
    int shared_blocks;      // MFMA kernel: K/V with cacheable loads (blocks read by several sequences)
    // Contiguous layout (bt == nullptr): sequence s uses request slot req[s],
    // whose blocks are req[s] * req_stride + 0, 1, ...; mapped[r] tokens of
    // slot r are backed by memory (virtual-memory KV storage).
    const int *req;         // [S]
    const int *mapped;      // [num_req]
    int req_stride;
    int num_req;
    // Append (k_new != nullptr): token ctx - 1 of every sequence is new; its
    // K/V ([S][Hkv][D]) are stored into its slot by the unit that reads it.
    const void *k_new;
    const void *v_new;
    // In-kernel merge of split rows (matrix-core kernel, B = 8 or 16): the
    // unit of a row that finishes last merges the row's partials through the
    // L2 of the XCD that ran all of the row's units (merge_row_in_l2).
    int fuse_merge;
    int *ticket;            // [S][Hkv] finished-unit counters, zero between calls
    unsigned *xcd_seen;     // PA_DEBUG: [S][Hkv] bit x set by each unit run on XCD x, or null
};

// In-kernel merge limits: partitions per row, and work units per launch
// (all resident at once).
constexpr int kFusedMaxParts = 8;
constexpr int64_t kFusedMaxUnits = 2048;

enum class DecodeKernel { kValu, kMfma };

// Launch the partition kernel (and, when NP > 1 without fuse_merge, the merge kernel).
hipError_t launch_decode(const DecodeArgs &a, int dtype, int head_dim, DecodeKernel kind,
                         hipStream_t stream);

// Workgroup b of a launch runs on the XCD numbered (b + r) mod X for some r,
// where X is the number of XCDs: checked once per device by a probe launch of
// 4,096 workgroups that read their XCD's id (the hardware dispatcher deals
// workgroups to the XCDs in turn).  Writes the XCD count to *num_xcd and
// whether the rule held to *ok; the probe runs on its own stream and is waited for.
hipError_t probe_xcd_dispatch(int *num_xcd, bool *ok);

// Loads only: the K/V tiles the matrix-core partition kernel would read for
// these arguments (16-bit data, B = 16), for measuring the access pattern.
hipError_t launch_read_tiles(const DecodeArgs &a, int head_dim, int *sink, hipStream_t stream);

// Everything one prefill launch needs (16-bit data, B = 16).
struct PrefillArgs {
    const void *q;          // [T][Hq][D], rows of sequence s at qs[s] .. qs[s+1]-1
    const void *k;          // K pool [NB][Hkv][D/x][B][x]
    const void *v;          // V pool [NB][Hkv][D][B]
    const int *bt;          // [S][MB]
    const int *ctx;         // [S]
    const int *qs;          // [S+1]
    void *out;              // [T][Hq][D]
    float scale_log2_abs;   // |scale| * log2(e)
    int q_xor;              // 0x80008000 when scale < 0
    int S, T, Hq, Hkv, G, MB;
    int64_t NB;
};

// Workgroup rows along the query axis for max_query_len queries of G heads.
int64_t prefill_row_tiles(int64_t max_query_len, int G);

hipError_t launch_prefill(const PrefillArgs &a, int dtype, int head_dim, int max_query_len,
                          hipStream_t stream);

// Decode with shared prefixes (16-bit data, B = 16).
struct CascadeArgs {
    const void *q;          // [S][Hq][D]
    const void *k;          // K pool
    const void *v;          // V pool
    const int *bt;          // [S][MB]
    const int *ctx;         // [S]
    const int *gs;          // [NG+1] first sequence of each group
    const int *pblk;        // [NG] shared blocks of each group
    void *out;              // [S][Hq][D]
    float *part_o;          // [S][Hq][NPT][D]
    float *part_ml;         // [S][Hq][NPT][2]
    float scale_log2_abs;
    int q_xor;
    int S, NG, Hq, Hkv, G, MB, P;
    int NPP;                // partial slots per row for the prefix (ceil(MB * 16 / P))
    int NPT;                // partial slots per row in all (prefix + suffix)
    int64_t NB;
};

hipError_t launch_cascade(const CascadeArgs &a, int dtype, int head_dim, int grid,
                          hipStream_t stream);

// mapped != nullptr: a slot is stored only if its request slot
// (slot / (req_stride * B)) has memory behind its position (< mapped[r] tokens).
hipError_t launch_write_kv(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                           const int64_t *slots, int64_t T, int Hkv, int D, int B, int64_t NB,
                           int elem_bytes, hipStream_t stream, const int *mapped = nullptr,
                           int req_stride = 0, int num_req = 0);

hipError_t launch_copy_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                              const int64_t *pairs, int64_t n, int64_t src_blocks,
                              int64_t dst_blocks, int64_t block_bytes, hipStream_t stream);

// Contiguous (virtual-memory) KV layout for decode_impl.
struct Contiguous {
    const int *req;     // [S] request slot of each sequence (device)
    const int *mapped;  // [num_req] tokens with memory behind them (device)
    int req_stride;     // blocks between consecutive request slots
    int num_req;
};

int decode_impl(const void *q, const void *k_cache, const void *v_cache,
                const int32_t *block_tables, const int32_t *context_lens, float scale,
                void *out, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                int block_size, int max_blocks_per_seq, int64_t num_blocks, int dtype,
                int partition_tokens, int flags, void *stream, const Contiguous *contig,
                const void *k_new = nullptr, const void *v_new = nullptr,
                int *read_sink = nullptr, bool no_alloc = false);

// Record the message pa_last_error() returns on this thread; returns status.
int api_fail(int status, const char *msg);
int api_hip_fail(hipError_t e, const char *where);

// PA_DEBUG (pa_debug.hip): checks of the device-resident preconditions, run
// on the stream and waited for; PA_OK, or PA_ERR_INVALID_ARG naming what is
// violated.  `who` prefixes the message.
bool debug_enabled();
int debug_set(int on);
// flags_buf: a device word to use instead of allocating one (allocation-free callers)
int debug_check_tables(const char *who, const int32_t *bt, const int32_t *ctx, int S, int MB,
                       int B, int64_t NB, hipStream_t stream, unsigned *flags_buf = nullptr);
int debug_check_slots(const char *who, const int64_t *slots, int64_t T, int64_t num_slots,
                      hipStream_t stream);
int debug_check_pairs(const char *who, const int64_t *pairs, int64_t n, int64_t src_blocks,
                      int64_t dst_blocks, bool same_pool, hipStream_t stream);
int debug_check_query_start(const char *who, const int32_t *qs, const int32_t *ctx, int S, int T,
                            int max_query_len, hipStream_t stream);
int debug_check_groups(const char *who, const int32_t *gs, const int32_t *pblk, const int32_t *bt,
                       const int32_t *ctx, int NG, int S, int MB, int max_group,
                       hipStream_t stream);
// After a decode with the in-kernel merge: every row's units ran on one XCD
// (`seen`: the kernel's [rows] XCD bit sets, zeroed before it; flags_buf as above).
int debug_check_xcd(const char *who, const unsigned *seen, int64_t rows, hipStream_t stream,
                    unsigned *flags_buf = nullptr);

}  // namespace pa
