/*
 * pa.h -- C ABI of libpa, paged decode attention for AMD Instinct MI355X (gfx950).
 *
 * The operation is the decode step of PagedAttention: every sequence keeps its
 * keys and values in fixed-size physical blocks of B tokens that may sit
 * anywhere in a pool, a per-sequence block table maps logical block i to a
 * physical block, and the query of the newest token is scored against every
 * cached token with a streaming (max / sum-of-exponentials) softmax.
 *   [論文解説: PagedAttention — 仮想メモリ着想のKVキャッシュ管理でLLMサービングを高効率化,
 *    技術的詳細 › PagedAttentionアルゴリズム: block definition, block table,
 *    decode equation]
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers are DEVICE pointers unless stated; the caller owns every buffer and
 * the library never frees or retains them.  All work is enqueued on `stream`
 * (a hipStream_t passed as void*, NULL = the null stream) and the calls return
 * without waiting for it.  Calls on one stream are ordered, so
 * pa_copy_blocks -> pa_write_kv -> pa_decode needs no extra fence.
 *
 * Element type `dtype` (pa_dtype): one type for q, caches, new tokens and out.
 * Arithmetic is fp32 inside the kernels; out is rounded to nearest-even.
 *
 * Storage format (B = block_size, D = head_dim, x = 16 / element bytes):
 *   k_cache  [num_blocks][num_kv_heads][D / x][B][x]
 *            element (block b, head g, token offset o, dim d) at
 *            (((b * Hkv + g) * (D / x) + d / x) * B + o) * x + d % x
 *   v_cache  [num_blocks][num_kv_heads][D][B]
 *            element (b, g, o, d) at ((b * Hkv + g) * D + d) * B + o
 *   q, out   [num_seqs][num_heads][D]
 *   query head h reads kv head h / (num_heads / num_kv_heads).
 *
 * Errors: each call returns a pa_status.  Arguments the host can see (sizes,
 * dtype, null or misaligned pointers) are checked before anything is
 * enqueued; a failing check enqueues nothing.  Values that live on the device
 * (slots, block ids, context lengths, block pairs, query starts, groups) are
 * preconditions, listed with each call: by default the kernels clamp or skip
 * out-of-range values so that no access leaves the buffers, and the result for
 * such inputs is unspecified.  With PA_DEBUG on (pa_set_debug below) every
 * call first checks them on the device, waits for the check, and returns
 * PA_ERR_INVALID_ARG naming each violated precondition without launching
 * anything.  pa_last_error() gives a message for the last failure on the
 * calling thread.
 */
#ifndef PA_H
#define PA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1, /* a size, pointer or dtype the call cannot accept */
    PA_ERR_UNSUPPORTED = 2, /* valid, but not a shape the library implements */
    PA_ERR_HIP = 3,         /* the HIP runtime reported an error */
    PA_ERR_NO_MEMORY = 4    /* the library could not allocate its workspace */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/*
 * pa_write_kv -- store the keys and values of new tokens in their slots.
 * A token's slot names a physical block and an offset in it:
 * slot = block * B + offset (blocks are filled token by token,
 * [論文解説: PagedAttention, 技術的詳細 › PagedAttentionアルゴリズム, block table example]).
 *
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim], device
 *   k_cache, v_cache  pools in the storage format above, device, updated in place
 *   slot_mapping   int64 [num_tokens], device.  slot < 0 skips the token.
 *                  Non-negative slots must be distinct and < num_blocks * B.
 *
 * Every element is copied bit for bit; slots not named are left untouched.
 * Supports head_dim a multiple of x up to 512, any block_size >= 1.
 * Errors: PA_ERR_INVALID_ARG for non-positive sizes, null pointers, unknown
 * dtype, head_dim not a multiple of x, or data pointers not 16-byte aligned.
 */
int pa_write_kv(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                const int64_t *slot_mapping, int64_t num_tokens, int num_kv_heads,
                int head_dim, int block_size, int64_t num_blocks, int dtype, void *stream);

/*
 * pa_decode -- paged decode attention for one new query token per sequence.
 *   out[s][h][:] = sum_{i < ctx_s} softmax_i(scale * <q[s][h], k_i>) * v_i
 * where token i of sequence s sits in physical block block_tables[s][i / B] at
 * offset i % B.  [論文解説: PagedAttention, 技術的詳細 › PagedAttentionアルゴリズム,
 * decode equation; the page fixes scale = 1/sqrt(d), here it is an argument]
 *
 *   q              [num_seqs][num_heads][head_dim], device
 *   k_cache, v_cache  pools (storage format above), device, read only
 *   block_tables   int32 [num_seqs][max_blocks_per_seq], device; entries at
 *                  or past ceil(ctx / B) are never read
 *   context_lens   int32 [num_seqs], device; 0 <= ctx <= max_blocks_per_seq * B.
 *                  ctx == 0 gives out = 0.  Slots of the last block at or past
 *                  ctx may hold any bits (NaN included) and do not matter.
 *   scale          host float, multiplies every dot product
 *   out            [num_seqs][num_heads][head_dim], device, written
 *
 * Long contexts are split into partitions whose partial results are merged
 * with log-sum-exp weights.  The partition length is automatic: with bf16 /
 * fp16 data, at most 16 query heads per kv head, block_size 16, fewer than
 * 2,048 (sequence, kv head) rows, at most 256 sequences and tables of 513 to
 * 2^20 tokens, the kernels choose it on the device from context_lens by the
 * rule of pa_decode_plan (same length, same bits as pa_decode_ex with the
 * length pa_decode_plan gives for the same lengths); otherwise it follows
 * from the sizes alone.  The library keeps a grow-only workspace for the
 * partials per (device, stream) (PA_ERR_NO_MEMORY if it cannot be allocated).  A
 * workspace buffer is never freed before pa_release_workspaces, so a HIP graph
 * that captured pa_decode stays valid; the first call on a stream that needs
 * a larger workspace allocates one (hipMalloc), so make that call before
 * capturing.  Every call on one stream, and every graph captured on it,
 * uses that stream's one buffer: such calls and graph replays must not run
 * at the same time (stream order keeps eager calls apart; two graphs
 * captured on one stream -- torch.cuda.graph uses one capture stream for
 * all captures unless it is given one -- must not be replayed concurrently
 * with each other or with work on that stream).  Give concurrent graphs
 * their own capture streams.  Results are bit-identical from run to run and
 * do not depend on where the physical blocks sit.
 * Supports head_dim 64 or 128 and num_heads a multiple of num_kv_heads;
 * block_size 16 for every dtype and head ratio, and 8 or 32 for bf16 / fp16
 * with at most 16 query heads per kv head (block_size 8: pools under 2 GiB);
 * PA_ERR_UNSUPPORTED otherwise.
 */
int pa_decode(const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, const int32_t *context_lens, float scale, void *out,
              int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
              int max_blocks_per_seq, int64_t num_blocks, int dtype, void *stream);

/*
 * pa_decode_append -- one decode step in one call: store the newest token of
 * every sequence, then attend.  For each sequence s with ctx = context_lens[s]
 * >= 1, token ctx - 1 is the new one: its keys and values k_new[s], v_new[s]
 * ([num_seqs][num_kv_heads][head_dim], device) go to its slot, block
 * block_tables[s][(ctx - 1) / 16] at offset (ctx - 1) % 16, exactly as
 * pa_write_kv would store them, and the output is pa_decode's over the ctx
 * tokens.  The unit of the decode kernel that reads that block stores the
 * token into the pool and waits for the store before it loads that block, so
 * there is no separate write kernel.  A new token whose table entry is out of
 * range ([0, num_blocks)) is not stored.
 *   [論文解説: PagedAttention, 技術的詳細 › PagedAttentionアルゴリズム (block
 *    table, decode equation)]
 * Preconditions as pa_write_kv and pa_decode (the block of slot ctx - 1 is
 * the sequence's own: copy-on-write copies come first).  16-bit data, at most
 * 16 query heads per kv head, block_size 16; PA_ERR_UNSUPPORTED otherwise.
 * partition_tokens as pa_decode_ex.
 */
int pa_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache,
                     void *v_cache, const int32_t *block_tables, const int32_t *context_lens,
                     float scale, void *out, int num_seqs, int num_heads, int num_kv_heads,
                     int head_dim, int block_size, int max_blocks_per_seq, int64_t num_blocks,
                     int dtype, int partition_tokens, void *stream);

/* Flags of pa_decode_ex. */
enum pa_decode_flags {
    /* Hint: physical blocks of this call are read by several sequences
     * (shared prompt prefixes, parallel sampling; reference count > 1).  K/V
     * are then read with cacheable loads so that the sequences sharing a
     * block hit in L2; without the hint they are streamed with nontemporal
     * loads, which is faster when every block is read once.  Results are
     * bit-identical either way. */
    PA_DECODE_SHARED_BLOCKS = 1,
    /* For testing and measurement: run the one-query-head VALU kernel (dot
     * products and P.V on the vector ALUs) on 16-bit data too, where the
     * matrix-core kernel would run; same results within the tolerance.
     * block_size 16 only (PA_ERR_UNSUPPORTED otherwise). */
    PA_DECODE_FORCE_VALU = 2,
    /* Merge split contexts with the separate merge kernel even where the
     * partition kernel would merge them itself (pa_decode_merge_mode); same
     * bits either way. */
    PA_DECODE_MERGE_KERNEL = 4
};

/*
 * pa_decode_ex -- pa_decode with an explicit partition length and flags.
 *   partition_tokens  0 = choose automatically (what pa_decode does);
 *                     otherwise a multiple of 16 in [16, 1024]: a sequence
 *                     of ctx tokens is cut into the fewest runs of at most
 *                     that many tokens, ceil(ctx / partition_tokens), all of
 *                     the same number of whole blocks but a shorter last one;
 *                     each run is reduced on its own and the runs are merged.
 *                     A value >= max_blocks_per_seq * B gives the single-pass
 *                     kernel.
 *   flags             0, or PA_DECODE_SHARED_BLOCKS (a hint, see above),
 *                     PA_DECODE_FORCE_VALU, PA_DECODE_MERGE_KERNEL or'd;
 *                     other bits give PA_ERR_INVALID_ARG.
 * The split is exact up to rounding: the streaming softmax is associative.
 *   [論文解説: PagedAttention, 技術的詳細 › PagedAttentionアルゴリズム,
 *    online softmax ("FlashAttention style")]
 */
int pa_decode_ex(const void *q, const void *k_cache, const void *v_cache,
                 const int32_t *block_tables, const int32_t *context_lens, float scale,
                 void *out, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                 int block_size, int max_blocks_per_seq, int64_t num_blocks, int dtype,
                 int partition_tokens, int flags, void *stream);

/*
 * pa_decode_noalloc -- pa_decode_ex that allocates nothing, for callers that
 * cannot call hipMalloc: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, same kernels, and the
 * same bits as pa_decode_ex with the same partition length; the partials of
 * split contexts go to a static device array of 32 MiB in the library (one
 * per GPU, held until the process ends) instead of the per-stream workspace,
 * and so do the in-kernel merge's row counters.
 *   Limit: num_seqs * num_heads * ceil(max_blocks_per_seq * B / P) *
 *   (head_dim + 2) * 4 bytes of partials at most 32 MiB - 16,640
 *   (PA_ERR_UNSUPPORTED beyond, before anything is enqueued; at head_dim 128,
 *   e.g. 32 sequences x 32 heads with tables of up to 63,488 tokens at
 *   P = 1024, or 128 x 32 of up to 3,840 tokens at P = 256).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (on different streams, or
 * graph replays running concurrently) race and give wrong results.  Nothing
 * in the array needs to start at zero.  With PA_DEBUG on, the checks use the
 * array too (they still wait for the stream).
 */
int pa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, float scale,
                      void *out, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                      int block_size, int max_blocks_per_seq, int64_t num_blocks, int dtype,
                      int partition_tokens, int flags, void *stream);

/*
 * pa_read_tiles -- a measurement aid, not part of the attention path: reads
 * exactly the K/V tiles that pa_decode_ex would read for these arguments, with
 * the same work units and load instructions, and does nothing else (no
 * scores, no softmax, no output).  Its time is the ceiling of the decode's
 * access pattern on the machine at hand; the decode's time over it is the
 * cost of everything else.  [論文解説: vAttention, 実験結果 › Decode性能:
 * decode is bound by memory, so the reads alone bound it]
 *   sink  device int32, 4-byte aligned; written only in the (practically
 *         impossible) case that the XOR of all loaded words equals a fixed
 *         constant, which keeps the loads from being optimised away.
 * Other arguments as pa_decode_ex (q, out, scale and flags are not taken).
 * The matrix-core configuration only: 16-bit data, at most 16 query heads per
 * kv head, block_size 16; PA_ERR_UNSUPPORTED otherwise.
 */
int pa_read_tiles(const void *k_cache, const void *v_cache, const int32_t *block_tables,
                  const int32_t *context_lens, int32_t *sink, int num_seqs, int num_heads,
                  int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                  int64_t num_blocks, int dtype, int partition_tokens, void *stream);

/*
 * pa_decode_cascade -- pa_decode for sequences that share prefix blocks,
 * reading each shared block once per group instead of once per sequence.
 * Under parallel sampling (or beam search) the samples of one prompt keep
 * the prompt's blocks physically shared through copy-on-write.
 *   [論文解説: PagedAttention, 技術的詳細 › Copy-on-Write KVキャッシュ共有]
 *
 * Arguments as pa_decode, plus:
 *   group_start     int32 [num_groups + 1], device: group i is sequences
 *                   group_start[i] .. group_start[i+1]-1 (consecutive),
 *                   group_start[0] = 0, group_start[num_groups] = num_seqs
 *                   (a sequence that shares nothing is a group of one)
 *   prefix_blocks   int32 [num_groups], device: the first prefix_blocks[i]
 *                   block-table entries are the same physical blocks in every
 *                   member of group i, and every member's context covers them
 *                   (prefix_blocks[i] * 16 <= context_lens[s]); 0 = nothing
 *                   shared
 *   max_group_size  host bound on the members of a group (sizes the launch)
 *   partition_tokens  0 (1024) or a multiple of 16 in [16, 1024]: shared
 *                   prefixes and private suffixes are cut into runs of at
 *                   most that many tokens
 * The result is the attention pa_decode computes, up to rounding: the shared
 * keys are scored against the queries of every member of the group at once
 * (one read of each shared block per group and kv head), each sequence's own
 * keys against its own queries, and the partial results are merged with
 * log-sum-exp weights (the streaming softmax is associative).
 * bf16 and fp16; fp32 is PA_ERR_UNSUPPORTED.  Uses the same per-stream
 * workspace as pa_decode: num_seqs * num_heads * 2 * ceil(max_blocks_per_seq
 * * 16 / P) * (head_dim + 2) floats.
 * Errors: as pa_decode; PA_ERR_INVALID_ARG also when groups cannot cover the
 * sequences (num_groups > num_seqs, max_group_size outside [1, num_seqs]).
 */
int pa_decode_cascade(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens,
                      const int32_t *group_start, const int32_t *prefix_blocks, int num_groups,
                      int max_group_size, float scale, void *out, int num_seqs, int num_heads,
                      int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                      int64_t num_blocks, int dtype, int partition_tokens, void *stream);

/*
 * pa_prefill -- paged prefill attention: the queries of a chunk of new tokens
 * attend causally over their sequence's tokens in the pool.  The same block
 * gather as decode serves the prefill phase.
 *   [論文解説: PagedAttention, 実装のポイント › CUDAカーネル実装]
 *
 *   q, out         [num_tokens][num_heads][D], device; the rows of sequence s
 *                  are query_start[s] .. query_start[s+1]-1 (packed, in order)
 *   block_tables   int32 [num_seqs][max_blocks_per_seq], device
 *   context_lens   int32 [num_seqs], device: tokens of the sequence in the
 *                  pool, the chunk's own included (write them with
 *                  pa_write_kv first)
 *   query_start    int32 [num_seqs + 1], device, query_start[0] = 0,
 *                  query_start[num_seqs] = num_tokens
 *   max_query_len  host bound on query_start[s+1] - query_start[s] (sizes the
 *                  launch grid)
 * With n = query_start[s+1] - query_start[s] <= ctx = context_lens[s], query
 * i of sequence s is the token at position ctx - n + i and its output is
 *   sum_{j <= ctx - n + i} softmax_j(scale * q . k_j) v_j.
 * n = ctx is a whole prompt, n < ctx a chunk after a cached prefix, n = 0
 * leaves the sequence out.  bf16 and fp16; fp32 is PA_ERR_UNSUPPORTED.
 * Arithmetic: scores and the softmax in fp32; P.V on the matrix cores with
 * each weight split into two 16-bit parts (hi + lo), fp32 accumulation.
 * Preconditions (device values): query_start non-decreasing, n <= ctx,
 * ctx <= max_blocks_per_seq * 16, block ids in range.
 * Errors: PA_ERR_INVALID_ARG for bad sizes, dtype, scale, pointers, or
 * max_query_len > num_tokens; PA_ERR_UNSUPPORTED for fp32, block_size != 16,
 * head_dim not 64 or 128, or a grid past the launch limits (num_seqs > 65535).
 * Allocates nothing.
 */
int pa_prefill(const void *q, const void *k_cache, const void *v_cache,
               const int32_t *block_tables, const int32_t *context_lens,
               const int32_t *query_start, float scale, void *out, int num_seqs, int num_tokens,
               int max_query_len, int num_heads, int num_kv_heads, int head_dim, int block_size,
               int max_blocks_per_seq, int64_t num_blocks, int dtype, void *stream);

/*
 * pa_copy_blocks -- copy whole physical blocks, the copy step of
 * copy-on-write: a block shared by several sequences (reference count > 1) is
 * copied to a fresh block before one of them writes into it.
 *   [論文解説: PagedAttention, 技術的詳細 › Copy-on-Write KVキャッシュ共有]
 *
 *   k_cache, v_cache  pools, device, updated in place
 *   block_mapping  int64 [num_pairs][2] = (src, dst), device
 * Copies every kv head, every slot, of K and of V, bit for bit.
 * Preconditions: ids in [0, num_blocks); destinations distinct; no
 * destination is also a source in the same call (then the result equals
 * reading every source before writing any destination).
 * Errors: PA_ERR_INVALID_ARG for non-positive sizes, null pointers, unknown
 * dtype or pools not 16-byte aligned.
 */
int pa_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping, int64_t num_pairs,
                   int num_kv_heads, int head_dim, int block_size, int64_t num_blocks, int dtype,
                   void *stream);

/*
 * pa_swap_blocks -- move whole physical blocks between two pool pairs, the
 * data step of preemption by swapping: when GPU memory runs short, the
 * scheduler moves a preempted sequence's KV blocks out to a pool in CPU
 * memory, and back into free GPU blocks when it resumes.
 *   [論文解説: PagedAttention, 実装のポイント › スケジューラ]
 *
 *   src_k, src_v   source pools, num_src_blocks blocks each, read only
 *   dst_k, dst_v   destination pools, num_dst_blocks blocks each, updated
 *   block_mapping  int64 [num_pairs][2] = (src block, dst block)
 * Each pool pair has the layout above with the same num_kv_heads, head_dim,
 * block_size and dtype; the pools are pointers of the caller, who keeps
 * ownership.  Every pointer may be device memory or pinned host memory
 * (hipHostMalloc, or torch's pin_memory): one kernel launch moves every pair,
 * reading and writing host memory directly over the host link, so swap-out
 * (device -> host), swap-in (host -> device) and moves within one memory are
 * the same call.  Copies every kv head and slot of K and V, bit for bit.
 * Asynchronous on `stream`: host pools must not be touched by the host until
 * the stream has reached this call.
 * Preconditions: ids in range; destinations distinct; when source and
 * destination are the same pools, no destination is also a source.
 * Errors: PA_ERR_INVALID_ARG for non-positive sizes, null pointers, unknown
 * dtype, pools not 16-byte aligned, or a pointer to pageable host memory
 * (checked with hipPointerGetAttributes before anything is enqueued).
 */
int pa_swap_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                   const int64_t *block_mapping, int64_t num_pairs, int num_kv_heads,
                   int head_dim, int block_size, int64_t num_src_blocks, int64_t num_dst_blocks,
                   int dtype, void *stream);

/*
 * ---- KV storage on virtual memory (the vAttention design) -----------------
 * Virtual address space is reserved up front for every (layer, K/V) buffer:
 * max_batch request slots of max_context_len tokens each, contiguous per
 * slot.  Physical pages are created and mapped into a slot's range only when
 * its sequence grows (pa_vkv_step), and stay mapped after the request ends
 * until pa_vkv_reclaim (deferred reclamation), so a new request on that slot
 * reuses them.  Decode and writes then address a sequence's tokens by
 * arithmetic (slot r, position i), with no block table.
 *   [論文解説: vAttention, 技術的詳細 › CUDA Virtual Memory Management APIの
 *    活用; 仮想メモリの事前予約; リクエスト単位のKVキャッシュインデキシング;
 *    Demand Paging vs Pre-allocation; 実装のポイント (init / alloc_reqid /
 *    step / free_reqid)]
 *
 * Inside a slot's range tokens keep the library's storage format: position
 * i of slot r is in block r * request_stride_blocks + i / 16 of the K and V
 * pools of pa_vkv_layer, at offset i % 16 (the pools described above, with
 * num_blocks = max_batch * request_stride_blocks and B = 16).
 * All calls are host calls on the device current at pa_vkv_create; a pa_vkv
 * is not thread-safe.  Mapping is synchronous (pa_vkv_step returns when the
 * new pages are usable); pa_vkv_reclaim and pa_vkv_destroy synchronize the
 * device before unmapping.  Reading a position that no page backs would be a
 * memory fault: pa_vkv_write_kv skips, and pa_vkv_decode clamps each context
 * to, the tokens mapped for the slot.
 */
typedef struct pa_vkv pa_vkv;

/* Reserve the virtual ranges.  page_bytes 0 = the device's recommended
 * allocation granularity (hipMemGetAllocationGranularity) doubled up to at
 * least 2 MiB, else a multiple of the minimum granularity.
 * max_context_len a multiple of 16.  Every page is a physical allocation of
 * its own, and the runtime holds about 32K of them per process (the
 * 32,757th hipMemCreate fails on MI355X with ROCm 7.2): a storage whose
 * pages, mapped in every slot of its 2 * num_layers buffers, would number
 * more than 24,576 is refused, with the smallest page size that fits in the
 * message (64 KiB pages fit 1.5 GiB of mapped storage).  Errors:
 * PA_ERR_INVALID_ARG (sizes, dtype, page size), PA_ERR_UNSUPPORTED (no
 * virtual memory management on the device, pages and 16-token blocks that
 * do not tile a slot, or too many pages), PA_ERR_HIP. */
int pa_vkv_create(int num_layers, int max_batch, int max_context_len, int num_kv_heads,
                  int head_dim, int dtype, int64_t page_bytes, pa_vkv **out);

/* Sizes and counters (each output pointer may be NULL): the page size, the
 * slot stride in 16-token blocks, the bytes currently mapped over all
 * buffers, and the mean host time of hipMemCreate and of hipMemMap +
 * hipMemSetAccess per page so far. */
int pa_vkv_info(const pa_vkv *v, int64_t *page_bytes, int64_t *request_stride_blocks,
                int64_t *mapped_bytes, double *create_us_per_page, double *map_us_per_page);

/* Base addresses of layer `layer`'s K and V pools (device virtual addresses). */
int pa_vkv_layer(const pa_vkv *v, int layer, void **k_cache, void **v_cache);

/* Take a free slot, preferring one whose pages are still mapped.
 * PA_ERR_NO_MEMORY when every slot is in use. */
int pa_vkv_alloc_reqid(pa_vkv *v, int *req_id);

/* Map pages so that slot r holds seq_lens[r] tokens (host int32
 * [max_batch]) in every layer.  Never unmaps.  PA_ERR_NO_MEMORY when the
 * device runs out of memory, or the process out of page allocations (pages
 * mapped before the failure stay). */
int pa_vkv_step(pa_vkv *v, const int32_t *seq_lens);

/* Release a slot; its pages stay mapped until pa_vkv_reclaim. */
int pa_vkv_free_reqid(pa_vkv *v, int req_id);

/* Unmap and release the pages of every free slot (synchronizes the device). */
int pa_vkv_reclaim(pa_vkv *v);

/* Synchronize the device, unmap everything and free the reservations. */
int pa_vkv_destroy(pa_vkv *v);

/* pa_write_kv into layer `layer`: slot = r * request_stride_blocks * 16 + i
 * for position i of slot r (int64, device); slots < 0 and positions without
 * a mapped page are skipped. */
int pa_vkv_write_kv(const pa_vkv *v, int layer, const void *k_new, const void *v_new,
                    const int64_t *slot_mapping, int64_t num_tokens, void *stream);

/* pa_decode over layer `layer` without a block table: sequence s reads slot
 * req_ids[s] (int32 [num_seqs], device), positions 0 .. context_lens[s]-1.
 * Same arithmetic and kernels as pa_decode; q / out as there.
 * partition_tokens as pa_decode_ex (0 = automatic). */
int pa_vkv_decode(const pa_vkv *v, int layer, const void *q, const int32_t *req_ids,
                  const int32_t *context_lens, float scale, void *out, int num_seqs,
                  int num_heads, int partition_tokens, void *stream);

/* Name of a status code (static string, never NULL). */
const char *pa_status_str(int status);

/* Message for the last failing call on this thread ("" if none). */
const char *pa_last_error(void);

/*
 * pa_decode_plan -- host-side planning of the split: the partition length to
 * pass to pa_decode_ex for this batch, from the context lengths as the
 * caller's scheduler holds them (host memory; the decode itself reads them
 * from the device).
 *   context_lens  host int32 [num_seqs], clamped to [0, max_blocks_per_seq * B]
 *   *partition_tokens  out: a multiple of 128 in [512, 1024], or 0 where the
 *                  plan does not apply and the library's automatic choice is
 *                  the one to take (fp32 data or more than 16 query heads per
 *                  kv head, block_size other than 16 and 32, or num_seqs * kv
 *                  heads >= 2048, where short partitions keep the machine
 *                  evenly loaded).
 * All units of a decode are resident together, so a compute unit runs about
 * ceil(units / compute units) of them; the plan takes the length that makes
 * that count times the longest unit (in blocks of block_size tokens)
 * smallest, ties to the longer length.  A partition is still the unit of the online softmax, merged with
 * log-sum-exp weights.  [論文解説: PagedAttention, 技術的詳細 ›
 * PagedAttentionアルゴリズム, online softmax; 論文解説: vAttention, 背景と動機:
 * the host prepares the block tables of each decode step]
 * Returns PA_OK, or PA_ERR_INVALID_ARG for bad sizes, dtype or null pointers.
 * Touches no device memory; queries the current device's compute-unit count.
 */
int pa_decode_plan(const int32_t *context_lens, int num_seqs, int num_heads, int num_kv_heads,
                   int block_size, int max_blocks_per_seq, int dtype, int *partition_tokens);

/*
 * pa_decode_merge_mode -- how pa_decode_ex merges split contexts for these
 * sizes, partition length and flags on the current device, for a stream that
 * is not being captured:
 *   PA_MERGE_NONE (0)       one partition covers every table: nothing to merge;
 *   PA_MERGE_KERNEL (1)     a merge kernel follows the partition kernel;
 *   PA_MERGE_IN_KERNEL (2)  the unit of each split (sequence, kv head) that
 *                           finishes last merges it inside the partition
 *                           kernel, through the L2 of the one XCD that ran all
 *                           of that row's units.  Taken for the matrix-core
 *                           kernel at block size 8 or 16 when num_kv_heads is
 *                           a multiple of 8, rows have at most 8 partitions
 *                           and 512 outputs (G * head_dim), the launch has at
 *                           most 2,048 work units (num_seqs * num_kv_heads *
 *                           partitions), PA_DECODE_MERGE_KERNEL is not set,
 *                           and the device's dispatcher places workgroups b
 *                           and b + 8 of a launch on one XCD (checked once per
 *                           device by a small probe launch, which this call
 *                           or the first decode makes and waits for).  A
 *                           stream under capture, or one whose counter buffer
 *                           would have to grow during capture, takes the merge
 *                           kernel instead.
 * Same bits in every mode: the partitions are folded in the same order.
 * A negative value is -(status) for bad arguments (PA_ERR_INVALID_ARG).
 */
enum pa_merge_mode { PA_MERGE_NONE = 0, PA_MERGE_KERNEL = 1, PA_MERGE_IN_KERNEL = 2 };
int pa_decode_merge_mode(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int dtype,
                         int partition_tokens, int flags);

/* Bytes of workspace pa_decode_ex would use for these sizes (0 = none); for
 * partition_tokens 0, an upper bound over the automatic choices. */
int64_t pa_decode_workspace_bytes(int num_seqs, int num_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int partition_tokens);

/* Frees the library-owned decode workspaces (including buffers that larger
 * ones replaced) after synchronising each device that holds one.  Call only
 * when no pa_decode work is pending and no captured graph that uses them will
 * be replayed again. */
int pa_release_workspaces(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int pa_version(void);

/*
 * pa_set_debug -- switch PA_DEBUG on (nonzero) or off (0) for every later
 * call in the process; returns the previous setting.  Without a call, the
 * environment variable PA_DEBUG (set and not "0") decides, read when the
 * library first needs it.  The pages' convention for an index out of range is
 * an error raised to the caller (the per-request offset helper raises
 * ValueError, [論文解説: vAttention, 技術的詳細 ›
 * リクエスト単位のKVキャッシュインデキシング]); with PA_DEBUG on, each call
 * checks the preconditions on its device-resident arguments before it
 * launches anything, and a violation gives PA_ERR_INVALID_ARG (ValueError in
 * the Python binding) with a message naming it:
 *   pa_write_kv       slots < num_blocks * B (negative = skip), distinct;
 *   pa_decode, _ex, _append, pa_read_tiles, pa_prefill, pa_decode_cascade
 *                     0 <= context_lens[s] <= max_blocks_per_seq * B, and the
 *                     first ceil(ctx / B) table entries in [0, num_blocks);
 *   pa_prefill        query_start from 0 to num_tokens, non-decreasing, each
 *                     chunk at most max_query_len and at most its context;
 *   pa_decode_cascade groups consecutive from 0 to num_seqs, each of at most
 *                     max_group_size members, prefix_blocks within the table,
 *                     every member's context covering them and its entries
 *                     there equal to the group's first member's;
 *   pa_copy_blocks    ids in [0, num_blocks), destinations distinct, none a
 *                     source;
 *   pa_swap_blocks    ids in range of their pools, destinations distinct, and
 *                     with one pool pair none a source.
 * The checks run on the call's stream and are waited for (the call returns
 * only when they are done), allocate a small scratch buffer (hipMalloc) and
 * are refused with PA_ERR_INVALID_ARG while the stream is being captured into
 * a graph.  For finding bad inputs, not for the serving loop.  The virtual-
 * memory storage calls (pa_vkv_*) are not checked.
 */
int pa_set_debug(int on);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
