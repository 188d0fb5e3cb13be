// pa_decode.hip -- paged decode attention kernels for gfx950.
//
// What is computed, per sequence s and query head h (kv head g = h / G):
//   out[s][h] = sum_{i < ctx} softmax_i(scale * <q, k_i>) v_i,
// token i living in physical block bt[s][i / 16], offset i % 16, reduced with
// a streaming softmax that keeps a running maximum m and a running sum l and
// rescales the accumulator by exp(m_old - m_new) when m grows.
// [論文解説: PagedAttention, 技術的詳細 › PagedAttentionアルゴリズム: block
//  table and decode equation; "online softmax (FlashAttention style)"]
//
// Work unit = (sequence, partition p, kv head or query head), one wave64 per
// unit.  A sequence longer than P tokens is cut into the fewest partitions of
// at most P tokens, equal in whole blocks (blocks_per_partition); each
// writes (m, l, unnormalised o), and the partitions are recombined with
// log-sum-exp weights -- the streaming softmax is associative, so the split
// only changes rounding -- either inside the partition kernel by the row's
// last unit (merge_row_in_l2) or by a merge kernel after it.  A sequence that
// fits one partition is normalised and written by its single unit directly.
//
// Two partition kernels:
//  * decode_mfma_kernel (bf16/fp16, 1..16 query heads per kv head): the G
//    query heads of one kv head form a small dense contraction (at G = 1 the
//    MFMA is mostly idle, but a block still costs far fewer instructions than
//    on VALU).  Per block of
//    16 tokens: S^T[16 tok x 16 cols] = K[16 x D] . Q^T on v_mfma_f32_16x16x32
//    and O^T[D x 16 cols] += V^T[D x 16 tok] . P^T on v_mfma_f32_16x16x16
//    (heads padded to 16 columns), with the weights split into a high and a
//    low 16-bit part so they keep ~16 significant bits.
//  * decode_valu_kernel (one query head per unit; fp32, or G > 16): dot
//    products with v_dot2 / FMA on 16-byte loads, cross-lane reductions, and
//    P.V with the 16 weights broadcast through SGPRs.
// Both read each (block, kv head) tile of K and of V exactly once per unit,
// as 16-byte (K) and 8/16-byte (V) loads that cover the tile in order, and
// keep one block requested ahead of the one being reduced.
#include <math.h>

#include <vector>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// ---------------------------------------------------------------------------
// Work units in launch order.  Unit = (sequence s, partition p, head group g),
// sequence-major, g fastest; a sequence has max(1, ceil(ctx / P)) partitions
// (an empty context still gets one unit, which writes zeros).  Workgroup b
// takes the b-th unit of this list, so the units that exist fill the front of
// the grid and the workgroups past the end (the host sizes the grid for full
// tables) exit at once: with all units resident, every compute unit then holds
// the same number of units (a grid with holes left some compute units with
// more streaming waves than others, and the decode step ran at the pace of the
// busiest ones).  Consecutive units have consecutive g, so the 8 XCDs
// (workgroup b runs on XCD b % 8) each take every 8th head of every partition.
// Returns false past the last unit; otherwise s, its clamped context length
// and the unit's rank r within its sequence (p = r / groups, g = r % groups).
// ---------------------------------------------------------------------------
// Context length of sequence s clamped to what its storage holds: the block
// table's capacity, and with the contiguous layout the tokens mapped for its
// request slot (a slot out of range holds none).
__device__ __forceinline__ int seq_ctx(const DecodeArgs &a, int s) {
    int cap = a.MB * a.BS;
    if (!a.bt) {
        const int r = a.req[s];
        cap = (r >= 0 && r < a.num_req) ? min(cap, a.mapped[r]) : 0;
    }
    return clamp_ctx(a.ctx[s], cap);
}

// Physical block of logical block blk of sequence s (0 past the table).
__device__ __forceinline__ int table_entry(const DecodeArgs &a, int s, int blk) {
    if (blk >= a.MB) return 0;
    if (a.bt) return a.bt[(int64_t)s * a.MB + blk];
    return a.req[s] * a.req_stride + blk;  // only read when seq_ctx(s) > 0: r in range
}

__device__ __forceinline__ bool find_unit(int b, const DecodeArgs &a, int P, int groups,
                                          int &s_out, int &ctx_out, int &r_out) {
    const int S = a.S;
    const int lane = threadIdx.x & 63;
    int base = 0;
    for (int c0 = 0; c0 < S; c0 += 64) {
        const int s = c0 + lane;
        int u = 0;
        const int c = s < S ? seq_ctx(a, s) : 0;
        if (s < S) u = groups * (c > P ? (c + P - 1) / P : 1);
        // inclusive prefix sum over the wave
        int incl = u;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(incl, d, 64);
            if (lane >= d) incl += t;
        }
        // (readlane: results the compiler knows to be wave-uniform, so that
        // addresses derived from them stay scalar)
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (b < base + total) {
            const uint64_t past = __ballot(base + incl > b);  // lanes whose units end after b
            const int first = __builtin_amdgcn_readfirstlane(__builtin_ctzll(past));
            s_out = c0 + first;
            ctx_out = __builtin_amdgcn_readlane(c, first);
            r_out = b - (base + __builtin_amdgcn_readlane(incl - u, first));
            return true;
        }
        base += total;
    }
    return false;
}

// ---------------------------------------------------------------------------
// Partition length planned on the device (DecodeArgs::plan: automatic
// partitions of the matrix-core kernel at B = 16 with fewer than 2,048 rows,
// at most 256 sequences and tables of at most 2^20 tokens).  Every unit of
// the split is resident at once, so a compute unit runs about ceil(units /
// CUs) of them and the call lasts about as long as that many of the longest;
// of 512, 640, ..., 1024 tokens the length that makes this product smallest is
// taken, ties to the longer (fewer partials to merge) -- the rule
// pa_decode_plan applies on the host, here to the context lengths the kernels
// read anyway.  Each wave computes it for itself from one load of the lengths
// (sequences lane, 64 + lane, 128 + lane, 192 + lane), and all get the same
// value; all 64 lanes must be active.
// ---------------------------------------------------------------------------
constexpr int kPlanChunks = 4;       // 256 sequences
constexpr int kPlanCandidates = 5;   // 512, 640, ..., 1024 tokens

// t / d for t < 2^24 and t / d < 2^21: the quotient through the float
// reciprocal is off by at most one, and one step corrects it.
__device__ __forceinline__ unsigned udiv_small(unsigned t, unsigned d) {
    unsigned q = (unsigned)((float)t * __builtin_amdgcn_rcpf((float)d));
    const int rem = (int)(t - q * d);
    return rem < 0 ? q - 1 : (rem >= (int)d ? q + 1 : q);
}

// Context lengths of this lane's sequences (-1: no sequence).
__device__ __forceinline__ void plan_lengths(const DecodeArgs &a, int (&c)[kPlanChunks]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kPlanChunks; ++i) {
        const int s = 64 * i + lane;
        c[i] = -1;
        if (64 * i < a.S && s < a.S) c[i] = seq_ctx(a, s);
    }
}

// Units at 512 tokens, summed over the wave (x groups): no candidate makes more.
__device__ __forceinline__ int plan_max_units(const DecodeArgs &a, const int (&c)[kPlanChunks],
                                              int groups) {
    int u = 0;
#pragma unroll
    for (int i = 0; i < kPlanChunks; ++i) {
        if (64 * i >= a.S) break;  // (uniform)
        u += c[i] < 0 ? 0 : (c[i] > 512 ? (c[i] + 511) >> 9 : 1);
    }
    return __builtin_amdgcn_readfirstlane(wave_sum_i32(u)) * groups;
}

__device__ __forceinline__ int plan_choose(const DecodeArgs &a, const int (&c)[kPlanChunks],
                                           int units512) {
    unsigned units[kPlanCandidates], longest[kPlanCandidates];
#pragma unroll
    for (int k = 0; k < kPlanCandidates; ++k) units[k] = 0, longest[k] = 0;
#pragma unroll
    for (int i = 0; i < kPlanChunks; ++i) {
        if (64 * i >= a.S) break;  // (uniform)
        const bool in = c[i] >= 0;
        const unsigned cc = in ? (unsigned)c[i] : 0u;
        const unsigned nb = (cc + kB - 1) / kB;
#pragma unroll
        for (int k = 0; k < kPlanCandidates; ++k) {
            const unsigned P = 512 + 128 * k;
            const unsigned np = cc > P ? (cc + P - 1) / P : 1u;
            if (k > 0) units[k] += in ? np : 0u;
            longest[k] = max(longest[k], udiv_small(nb + np - 1, np));  // ceil(nb / np)
        }
    }
    int best = 0;
    unsigned best_cost = ~0u;
#pragma unroll
    for (int k = 0; k < kPlanCandidates; ++k) {
        // units * Hkv < 2^22 (fewer than 2,048 rows of at most 2,048 partitions)
        const unsigned u = k == 0 ? (unsigned)units512
                                  : (unsigned)wave_sum_i32((int)units[k]) * (unsigned)a.Hkv;
        const unsigned lg = (unsigned)wave_max_i32((int)longest[k]);
        const unsigned cost = udiv_small(u + a.cus - 1, a.cus) * lg;
        if (cost <= best_cost) best_cost = cost, best = 512 + 128 * k;
    }
    return __builtin_amdgcn_readfirstlane(best);
}

// The partition length of a merge kernel's launch: a planned one reads what
// the partition kernel before it chose (its workgroup 0 stores it).
__device__ __forceinline__ int merge_partition_len(const DecodeArgs &a) {
    return a.plan ? *a.plan_slot : a.P;
}

// Unit search of a planned launch: the lengths are loaded once; workgroups
// past the units at 512 tokens (no candidate makes more) leave before the
// plan -- tables far longer than the contexts leave most of the grid, which
// is sized for full tables at 512, without a unit; then the plan, then the
// b-th unit at the chosen length, as find_unit.
__device__ __forceinline__ bool plan_find_unit(int b, const DecodeArgs &a, int groups, int &P_out,
                                               int &s_out, int &ctx_out, int &r_out) {
    const int lane = threadIdx.x & 63;
    int c[kPlanChunks];
    plan_lengths(a, c);
    const int u512 = plan_max_units(a, c, groups);
    if (b >= u512) return false;
    const int P = plan_choose(a, c, u512);
    P_out = P;
    int base = 0;
#pragma unroll
    for (int i = 0; i < kPlanChunks; ++i) {
        if (64 * i >= a.S) break;
        const int ci = c[i];
        const int u = ci < 0 ? 0
                             : groups * (ci > P ? (int)udiv_small((unsigned)(ci + P - 1),
                                                                  (unsigned)P) : 1);
        int incl = u;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(incl, d, 64);
            if (lane >= d) incl += t;
        }
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (b < base + total) {
            const uint64_t past = __ballot(base + incl > b);
            const int first = __builtin_amdgcn_readfirstlane(__builtin_ctzll(past));
            s_out = 64 * i + first;
            ctx_out = __builtin_amdgcn_readlane(ci, first);
            r_out = b - (base + __builtin_amdgcn_readlane(incl - u, first));
            return true;
        }
        base += total;
    }
    return false;
}

// The unit of workgroup b and the partition length, planned or not.
__device__ __forceinline__ bool unit_of(int b, const DecodeArgs &a, int groups, int &P, int &s,
                                        int &ctx, int &r) {
    if (a.plan) return plan_find_unit(b, a, groups, P, s, ctx, r);
    P = a.P;
    return find_unit(b, a, P, groups, s, ctx, r);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the partitions of one (sequence, query head):
//   M' = max(M, m_q),  L' = L 2^(M-M') + l_q 2^(m_q-M'),  o' likewise,
// over the partitions q = 0 .. np - 1 in order; out = o / L.  Every merge
// here folds the partitions in this order, so the in-kernel merge and the
// merge kernels give the same bits.
// ---------------------------------------------------------------------------
struct LseState {
    float M = -INFINITY, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // fold in a partition (m_q finite: every partition has a token)
    __device__ __forceinline__ void add(float mq, float lq, const f32x4 &oq) {
        const float Mn = fmaxf(M, mq);
        const float ca = fast_exp2(M - Mn), cb = fast_exp2(mq - Mn);
        L = L * ca + lq * cb;
        acc = acc * ca + oq * cb;
        M = Mn;
    }
};

// ---------------------------------------------------------------------------
// In-kernel merge of a split row (matrix-core kernel).
//
// Row (s, g) = sequence s, kv head g, cut into npart partitions.  With Hkv a
// multiple of 8, the row's units are workgroups b = base_s + p Hkv + g
// (base_s a multiple of Hkv), all congruent to g mod 8; the dispatcher deals
// workgroup b to XCD (b + r) mod 8 (probe_xcd_dispatch checks this once per
// device), so one XCD runs all of them, and its L2 is their point of
// coherence.  Each unit has stored its partial with plain stores (the L1 writes
// through); it waits until the L2 has them all, then adds one to the row's
// counter with an L2 atomic.  The unit that draws npart - 1 is the last: it
// zeroes the counter for the next call, reads the npart partials of the G
// heads with L1-bypassing (sc0) loads in one round trip, and writes the
// outputs.  Nobody waits for anybody.  No cross-XCD coherence is needed, so
// no L2 write-back or invalidate is issued: a device-scope version of the
// same protocol (sc1 stores, loads and atomic) made the Llama-3-8B-shaped step
// slower than a separate merge kernel, this one makes it 1.2-2 us faster.
// The host takes this path only when all units are resident at once (a unit
// that holds its slot through the ticket round trip would delay the units
// queued behind it) and rows have at most kFusedMaxParts partitions.
// ---------------------------------------------------------------------------
constexpr int kL1Bypass = 1;  // sc0 on a buffer load: served by the L2, not the L1

__device__ __forceinline__ unsigned xcc_id() {
    return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 15u;  // hwreg(XCC_ID, 0, 4)
}

template <int DT, int D>
__device__ __forceinline__ void merge_row_in_l2(const DecodeArgs &a, int s, int g, int npart) {
    const int lane = threadIdx.x;
    const int64_t row = (int64_t)s * a.Hkv + g;
    if (a.xcd_seen && lane == 0)  // PA_DEBUG: which XCDs ran the row's units
        __hip_atomic_fetch_or(a.xcd_seen + row, 1u << xcc_id(), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    // this wave's partial is in the L2 before its ticket
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int t = 0;
    if (lane == 0)
        t = __hip_atomic_fetch_add(a.ticket + row, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    t = __builtin_amdgcn_readfirstlane(t);
    if (t != npart - 1) return;
    if (lane == 0) a.ticket[row] = 0;

    // the G * D outputs of the row as f32x4 pieces: piece k = lane + 64 i is
    // head k / (D / 4), dims 4 (k % (D / 4)) .. + 3 (the host takes this path
    // only for G * D <= 512)
    const int G = a.G;
    const int items = G * (D / 4);
    const int64_t h0 = (int64_t)s * a.Hq + g * G;  // first query head of the row
    const auto ro = tile_rsrc((const char *)(a.part_o + h0 * a.NP * D), G * a.NP * D * 4);
    const auto rml = tile_rsrc((const char *)(a.part_ml + h0 * a.NP * 2), G * a.NP * 8);
    constexpr int kNone = 0x7ffffff0;  // outside the descriptor: no request
    f32x4 ov[2][kFusedMaxParts];
    f32x2 mlv[2][kFusedMaxParts];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int k = lane + 64 * i;
        const int hh = k / (D / 4);
        const int d0 = 4 * (k % (D / 4));
#pragma unroll
        for (int q = 0; q < kFusedMaxParts; ++q) {
            const bool in = k < items && q < npart;
            ov[i][q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                ro, in ? ((hh * a.NP + q) * D + d0) * 4 : kNone, 0, kL1Bypass));
            mlv[i][q] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(
                rml, in ? (hh * a.NP + q) * 8 : kNone, 0, kL1Bypass));
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int k = lane + 64 * i;
        if (k >= items) continue;
        const int hh = k / (D / 4);
        const int d0 = 4 * (k % (D / 4));
        LseState st;
#pragma unroll
        for (int q = 0; q < kFusedMaxParts; ++q)
            if (q < npart) st.add(mlv[i][q][0], mlv[i][q][1], ov[i][q]);
        store4<DT>((char *)a.out + ((h0 + hh) * D + d0) * Elem<DT>::bytes, st.acc, 1.f / st.L);
    }
}

// ---------------------------------------------------------------------------
// GQA partition kernel on MFMA.
//
// Lane l = 16 j + n.  Column n of every product is query head n of the group
// (heads padded to 16 with q = 0).  Per block of 16 tokens:
//  * S^T[16 tok x 16 col] = K[16 x D] . Q^T on v_mfma_f32_16x16x32: lane l
//    supplies K[token n][8 dims of run 4c + j] (instruction c of the wave
//    reads bytes [1024 c, 1024 c + 1024) of the [D/8][16][8] K tile) and
//    Q^T[same dims][col n], and gets back the scores of tokens 4j..4j+3 of
//    column n;
//  * O^T[D x 16 col] += V^T[D x 16 tok] . P^T on v_mfma_f32_16x16x16: lane l
//    supplies V^T[dim 16t + n][tokens 4j..4j+3] (8 bytes of the [D][16] V
//    tile) and exactly the four weights it computed, and O^T[dims 16t +
//    4j..4j+3][col n] stays in the lane across blocks.
// The weights enter the product as two 16-bit parts, hi = RNE(p) and lo =
// RNE(p - hi), so they keep ~16 significant bits.  When 2G <= 16 both parts
// ride in one product: columns G..2G-1 carry the same heads as columns 0..G-1
// (same q, so the same scores and weights) and take the lo parts; the two
// column halves are added once at the end.  Otherwise hi and lo take one
// product each.
//
// One wave per unit, one block of K and V (8 KiB) requested ahead: the next
// block is requested as soon as the scores of the current one are in.  On
// MI355X a compute unit streams best with ~40 KiB of reads outstanding (more
// only queues and slows the step), which the usual decode grid of ~1000-1500
// units gives at one block per wave.  Loads go through one buffer descriptor
// per tile whose range is empty past the unit's last block, so the request
// needs no branch and the one past the end makes no memory traffic.
// ---------------------------------------------------------------------------
//
// Block size 8 (BS): the kernel still works in steps of 16 tokens; a step
// spans two blocks, and each lane addresses the block of its own tokens
// through a whole-pool descriptor (32-bit offsets: pools under 2 GiB), a step
// past the end getting offsets outside the descriptor's range.  (Block size
// 32 has a kernel of its own below, with whole-block steps.)
//
// APPEND: the unit that holds a sequence's last token (position ctx - 1, the
// new one) stores its K/V for kv head g into the pool before it loads any
// block: no other unit reads that slot, so no ordering between workgroups is
// needed.  (Keeping the new token in registers and patching the loaded
// operands instead took 28 more registers and a wave per SIMD: 56.8 us on
// the Llama-3-8B step against 51.5 for the decode alone.)
//
// PLAN: the partition length is planned in the kernel (DecodeArgs::plan); a
// kernel of its own, so that launches with a given length carry no plan code.
template <int DT, int D, bool SPLIT, int POLICY, int BS = 16, bool APPEND = false,
          bool PLAN = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8)))
void decode_mfma_kernel(const DecodeArgs a) {
    static_assert(DT == kBF16 || DT == kF16, "MFMA path takes 16-bit data");
    static_assert(D % 32 == 0, "head_dim must be a multiple of 32");
    static_assert(BS == 8 || BS == 16, "block size");
    static_assert(!APPEND || BS == 16, "append takes 16-token blocks");
    constexpr int NKC = D / 32;       // QK steps, 32 dims each
    constexpr int NVT = D / 16;       // P.V output tiles, 16 dims each
    constexpr int TILE = D * BS * 2;  // bytes of one (block, kv head) tile

    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int j = lane >> 4;
    int P, s, ctx, r;
    if constexpr (PLAN) {
        if (!plan_find_unit(blockIdx.x, a, a.Hkv, P, s, ctx, r)) return;
        if (blockIdx.x == 0 && lane == 0) *a.plan_slot = P;  // for the merge kernel
    } else {
        P = a.P;
        if (!find_unit(blockIdx.x, a, P, a.Hkv, s, ctx, r)) return;
    }
    const int g = r % a.Hkv;
    const int p = r / a.Hkv;
    const int per = blocks_per_partition(ctx, P);
    const int blk0 = p * per;  // in steps of 16 tokens
    const int t0 = blk0 * kB;
    const int e0 = t0 / BS;    // the unit's first table entry
    int my_bt = table_entry(a, s, e0 + lane);

    // column n -> query head of the group; in SPLIT mode columns G..2G-1
    // repeat heads 0..G-1 (they take the lo parts of the weights)
    const bool hi_col = n < a.G;
    const bool col_ok = SPLIT ? n < 2 * a.G : hi_col;
    const int hn = hi_col ? n : (col_ok ? n - a.G : 0);
    const int h = g * a.G + hn;
    uint16_t *outp = (uint16_t *)a.out + ((int64_t)s * a.Hq + h) * D;
    if (ctx == 0) {  // empty context (its only unit): the output is zero
        if (hi_col) {
#pragma unroll
            for (int t = 0; t < NVT; ++t) *(i32x2 *)(outp + 16 * t + 4 * j) = i32x2{0, 0};
        }
        return;
    }
    const int t1 = min(ctx, t0 + per * kB);
    const int nblk = (t1 - t0 + kB - 1) / kB;  // 16-token steps, 1..64 (1..32 at BS = 8)
    const int nent = (t1 + BS - 1) / BS - e0;  // table entries of the unit
    // entries past the context are never used; out-of-range ids are clamped so
    // that no read leaves the pool (and the append below stores nothing into
    // a block whose id was out of range)
    const int bt_ok = my_bt >= 0 && (int64_t)my_bt < a.NB;
    if (lane >= nent || !bt_ok) my_bt = 0;

    const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)s * a.Hq + h) * D;
    i32x4 qf[NKC];
#pragma unroll
    for (int c = 0; c < NKC; ++c)
        qf[c] = col_ok ? ld16(qrow + (4 * c + j) * 8) ^ a.q_xor : i32x4{0, 0, 0, 0};
    const float cs = a.scale_log2_abs;  // the sign of the scale went into q

    const char *kbase = (const char *)a.k + (int64_t)g * TILE;
    const char *vbase = (const char *)a.v + (int64_t)g * TILE;
    const int64_t blk_stride = (int64_t)a.Hkv * TILE;

    float m = -INFINITY;  // reference maximum of the column, log2 units
    float l = 0.f;        // this lane's share of the softmax denominator
    f32x4 o[NVT];
#pragma unroll
    for (int t = 0; t < NVT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the new token: stored into its slot before the unit requests any block;
    // the stores are waited for (they reach L2, where the block's loads are
    // served), so the loads see them.  (Waiting only before the last block's
    // loads measured slower: 58.6 against 56.0 us on the Llama-3-8B step.)
    if constexpr (APPEND) {
        if (t1 == ctx && __builtin_amdgcn_readlane(bt_ok, nblk - 1)) {
            const int noff = (ctx - 1) & (kB - 1);
            const uint16_t *knp = (const uint16_t *)a.k_new + ((int64_t)s * a.Hkv + g) * D;
            const uint16_t *vnp = (const uint16_t *)a.v_new + ((int64_t)s * a.Hkv + g) * D;
            const int64_t tile = (int64_t)__builtin_amdgcn_readlane(my_bt, nblk - 1) * blk_stride +
                                 (int64_t)g * TILE;
            char *kt = (char *)a.k + tile;
            char *vt = (char *)a.v + tile;
            if (lane < D / 8) *(i32x4 *)(kt + (lane * kB + noff) * 16) = ld16(knp + lane * 8);
#pragma unroll
            for (int d = lane; d < D; d += 64) *(uint16_t *)(vt + (d * kB + noff) * 2) = vnp[d];
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    }

    struct Blk {
        i32x4 k[NKC];
        i32x2 v[NVT];
    };
    Blk b0, b1;
    // (BS = 8: descriptors over the rest of the pool from this kv head's first tile)
    const int pool_left = BS == 8 ? (int)min<int64_t>(a.NB * blk_stride - (int64_t)g * TILE,
                                                        0x7fffffff)
                                  : 0;
    const auto rk8 = tile_rsrc(kbase, pool_left);
    const auto rv8 = tile_rsrc(vbase, pool_left);
    auto load = [&](Blk &x, int i) {
        const bool in = i < nblk;
        if constexpr (BS == 16) {
            const int phys = __builtin_amdgcn_readlane(my_bt, in ? i : 0);
            const int64_t off = (int64_t)phys * blk_stride;
            const auto rk = tile_rsrc(kbase + off, in ? TILE : 0);
            const auto rv = tile_rsrc(vbase + off, in ? TILE : 0);
#pragma unroll
            for (int c = 0; c < NKC; ++c) x.k[c] = bload16<POLICY>(rk, (64 * c + lane) * 16);
#pragma unroll
            for (int t = 0; t < NVT; ++t)
                x.v[t] = bload8<POLICY>(rv, ((16 * t + n) * kB + 4 * j) * 2);
        } else {
            const int tok = t0 + kB * i;
            const int e = in ? tok / BS - e0 : 0;  // the step's two blocks: e, e + 1
            const int p0 = __builtin_amdgcn_readlane(my_bt, e);
            const int p1 = __builtin_amdgcn_readlane(my_bt, in ? e + 1 : 0);
            // tokens n < 8 (K) and 4j < 8 (V) are in the first block
            const int kofs = (n < 8 ? p0 : p1) * (int)blk_stride;
            const int vofs = (j < 2 ? p0 : p1) * (int)blk_stride;
            const int none = 0x7fffffff;  // outside the descriptor: zeros, no traffic
#pragma unroll
            for (int c = 0; c < NKC; ++c)
                x.k[c] = bload16<POLICY>(rk8, in ? kofs + ((4 * c + j) * BS + (n & 7)) * 16 : none);
#pragma unroll
            for (int t = 0; t < NVT; ++t)
                x.v[t] = bload8<POLICY>(rv8, in ? vofs + ((16 * t + n) * BS + 4 * (j & 1)) * 2 : none);
        }
        issue_point();
    };

    // One online-softmax step over block i (held in x); the next block goes
    // into y.  Only the unit's last block can hold empty slots; there they are
    // masked (score -inf, weight 0, V zeroed since it may hold NaN) in a
    // branch of its own.  The reference maximum m moves only when the block
    // maximum exceeds it by more than 8 (a factor 2^8): weights exp2(s - m)
    // then stay <= 256 and the rescale of O and l is skipped for most blocks.
    auto step = [&](Blk &x, Blk &y, int i) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKC; ++c) sc = mfma32<DT>(x.k[c], qf[c], sc);
        load(y, i + 1);
        const bool tail = i == nblk - 1;
        int nv = kB;
        if (tail) {
            nv = t1 - (t0 + i * kB);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * j + e >= nv) sc[e] = -INFINITY;
        }
        // The running maximum moves only when a score passes it by more than 8
        // (log2 units): each lane tests its own scores, and the row maximum
        // over the lane groups is formed only when some lane is over.
        const float lm = max4f(sc[0], sc[1], sc[2], sc[3]);
        if (__any(lm * cs > m + 8.f)) {
            const float bm = xor32_max(xor16_max(lm)) * cs;  // the block has a valid token
            const bool grow = bm > m + 8.f;
            const float mn = grow ? bm : m;
            const float alpha = fast_exp2(m - mn);  // 0 on the first step (m = -inf)
#pragma unroll
            for (int t = 0; t < NVT; ++t) o[t] *= alpha;
            l *= alpha;
            m = mn;
        }
        const float nm = -m;
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[e] = fast_exp2(fmaf(sc[e], cs, nm));
        if (tail) {  // (-inf) * 0 is NaN when the scale is 0
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * j + e >= nv) pe[e] = 0.f;
            const uint32_t m0 = (4 * j + 0 < nv ? 0x0000ffffu : 0u) | (4 * j + 1 < nv ? 0xffff0000u : 0u);
            const uint32_t m1 = (4 * j + 2 < nv ? 0x0000ffffu : 0u) | (4 * j + 3 < nv ? 0xffff0000u : 0u);
#pragma unroll
            for (int t = 0; t < NVT; ++t)
                x.v[t] = i32x2{(int)((uint32_t)x.v[t][0] & m0), (int)((uint32_t)x.v[t][1] & m1)};
        }
        l += (pe[0] + pe[1]) + (pe[2] + pe[3]);
        // P = hi + lo, both 16-bit: hi = RNE(p), lo = RNE(p - hi) (p - hi is exact)
        const uint32_t h0 = pack2<DT>(pe[0], pe[1]);
        const uint32_t h1 = pack2<DT>(pe[2], pe[3]);
        const uint32_t l0 = pack2<DT>(pe[0] - elem_lo<DT>(h0), pe[1] - elem_hi<DT>(h0));
        const uint32_t l1 = pack2<DT>(pe[2] - elem_lo<DT>(h1), pe[3] - elem_hi<DT>(h1));
        if constexpr (SPLIT) {
            const i32x2 pw = hi_col ? i32x2{(int)h0, (int)h1} : i32x2{(int)l0, (int)l1};
#pragma unroll
            for (int t = 0; t < NVT; ++t) o[t] = mfma16<DT>(x.v[t], pw, o[t]);
        } else {
            const i32x2 phi = {(int)h0, (int)h1}, plo = {(int)l0, (int)l1};
#pragma unroll
            for (int t = 0; t < NVT; ++t) {
                o[t] = mfma16<DT>(x.v[t], phi, o[t]);
                o[t] = mfma16<DT>(x.v[t], plo, o[t]);
            }
        }
    };

    // One exit, at the loop test (an exit between the two steps would give the
    // loop head a second predecessor with another load order, and the wait
    // counts there would have to cover both).
    load(b0, 0);
    int i = 0;
    for (; i + 2 <= nblk; i += 2) {
        step(b0, b1, i);
        step(b1, b0, i + 1);
    }
    if (i < nblk) step(b0, b1, i);

    if constexpr (SPLIT) {
        // add the lo columns G..2G-1 into the hi columns 0..G-1
#pragma unroll
        for (int t = 0; t < NVT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[t][e] += __shfl_down(o[t][e], a.G, 16);
    }
    const float lt = xor32_sum(xor16_sum(l));  // all lanes take part in the swaps
    if (t0 == 0 && t1 == ctx) {  // the unit covers the whole context
        if (!hi_col) return;
        const float inv = 1.f / lt;
#pragma unroll
        for (int t = 0; t < NVT; ++t) store4<DT>(outp + 16 * t + 4 * j, o[t], inv);
        return;
    }
    if (hi_col) {
        const int64_t part = ((int64_t)s * a.Hq + h) * a.NP + p;
        float *po = a.part_o + part * D;
#pragma unroll
        for (int t = 0; t < NVT; ++t) *(f32x4 *)(po + 16 * t + 4 * j) = o[t];
        if (j == 0) *(float2 *)(a.part_ml + 2 * part) = float2{m, lt};
    }
    if (a.fuse_merge) merge_row_in_l2<DT, D>(a, s, g, (ctx + P - 1) / P);
}

// ---------------------------------------------------------------------------
// Block size 32 on MFMA: a step is one whole block.  The scores of its two
// 16-token halves come from two products per 32 dims; the P.V product is one
// 16x16x32 per output tile whose k slots 8j .. 8j+7 hold keys 4j .. 4j+3 of
// the first half and of the second, which is what lane group j holds of P^T
// and what its two 8-byte V reads at the same keys give (both halves of each
// V row in one step).  Partitions are whole blocks: P is a multiple of 32.
// ---------------------------------------------------------------------------
template <int DT, int D, bool SPLIT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8)))
void decode_mfma_b32_kernel(const DecodeArgs a) {
    static_assert(DT == kBF16 || DT == kF16, "MFMA path takes 16-bit data");
    constexpr int BS = 32;
    constexpr int NKC = D / 32;
    constexpr int NVT = D / 16;
    constexpr int TILE = D * BS * 2;

    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int j = lane >> 4;
    int s, ctx, r;
    if (!find_unit(blockIdx.x, a, a.P, a.Hkv, s, ctx, r)) return;
    const int g = r % a.Hkv;
    const int p = r / a.Hkv;
    // ceil(ctx / P) partitions of equal whole blocks (ceil(nb / per) of them are
    // non-empty, which is that count since P is a multiple of the block)
    const int nb = (ctx + BS - 1) / BS;
    const int npart = ctx > a.P ? (ctx + a.P - 1) / a.P : 1;
    const int per = (nb + npart - 1) / npart;
    const int blk0 = p * per;
    const int t0 = blk0 * BS;
    int my_bt = table_entry(a, s, blk0 + lane);

    const bool hi_col = n < a.G;
    const bool col_ok = SPLIT ? n < 2 * a.G : hi_col;
    const int hn = hi_col ? n : (col_ok ? n - a.G : 0);
    const int h = g * a.G + hn;
    uint16_t *outp = (uint16_t *)a.out + ((int64_t)s * a.Hq + h) * D;
    if (ctx == 0) {
        if (hi_col) {
#pragma unroll
            for (int t = 0; t < NVT; ++t) *(i32x2 *)(outp + 16 * t + 4 * j) = i32x2{0, 0};
        }
        return;
    }
    const int t1 = min(ctx, t0 + per * BS);
    const int nblk = (t1 - t0 + BS - 1) / BS;  // 1..32
    if (lane >= nblk || my_bt < 0 || (int64_t)my_bt >= a.NB) my_bt = 0;

    const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)s * a.Hq + h) * D;
    i32x4 qf[NKC];
#pragma unroll
    for (int c = 0; c < NKC; ++c)
        qf[c] = col_ok ? ld16(qrow + (4 * c + j) * 8) ^ a.q_xor : i32x4{0, 0, 0, 0};
    const float cs = a.scale_log2_abs;

    const char *kbase = (const char *)a.k + (int64_t)g * TILE;
    const char *vbase = (const char *)a.v + (int64_t)g * TILE;
    const int64_t blk_stride = (int64_t)a.Hkv * TILE;

    float m = -INFINITY;
    float l = 0.f;
    f32x4 o[NVT];
#pragma unroll
    for (int t = 0; t < NVT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    struct Blk {
        i32x4 k[2][NKC];
        i32x4 v[NVT];
    };
    Blk b0, b1;
    auto load = [&](Blk &x, int i) {
        const bool in = i < nblk;
        const int phys = __builtin_amdgcn_readlane(my_bt, in ? i : 0);
        const int64_t off = (int64_t)phys * blk_stride;
        const auto rk = tile_rsrc(kbase + off, in ? TILE : 0);
        const auto rv = tile_rsrc(vbase + off, in ? TILE : 0);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int c = 0; c < NKC; ++c)
                x.k[hh][c] = bload16<kCachePolicyNT>(rk, ((4 * c + j) * BS + kB * hh + n) * 16);
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            const int row = (16 * t + n) * BS + 4 * j;
            const i32x2 lo = bload8<kCachePolicyNT>(rv, row * 2);
            const i32x2 hi = bload8<kCachePolicyNT>(rv, (row + kB) * 2);
            x.v[t] = i32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        issue_point();
    };

    auto step = [&](Blk &x, Blk &y, int i) {
        f32x4 sc[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            sc[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NKC; ++c) sc[hh] = mfma32<DT>(x.k[hh][c], qf[c], sc[hh]);
        }
        load(y, i + 1);
        const bool tail = i == nblk - 1;
        int nv = BS;
        float sv[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[4 * hh + e] = sc[hh][e];
        if (tail) {
            nv = t1 - (t0 + i * BS);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (kB * hh + 4 * j + e >= nv) sv[4 * hh + e] = -INFINITY;
        }
        // lazy row maximum, as in the 16-token kernel
        const float lm = __builtin_elementwise_maximum(max4f(sv[0], sv[1], sv[2], sv[3]),
                                                       max4f(sv[4], sv[5], sv[6], sv[7]));
        if (__any(lm * cs > m + 8.f)) {
            const float bm = xor32_max(xor16_max(lm)) * cs;  // the block has a valid token
            const bool grow = bm > m + 8.f;
            const float mn = grow ? bm : m;
            const float alpha = fast_exp2(m - mn);
#pragma unroll
            for (int t = 0; t < NVT; ++t) o[t] *= alpha;
            l *= alpha;
            m = mn;
        }
        const float nm = -m;
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(fmaf(sv[e], cs, nm));
        if (tail) {
            uint32_t vm[4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int kb = kB * hh + 4 * j;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (kb + e >= nv) pe[4 * hh + e] = 0.f;
                vm[2 * hh] = (kb + 0 < nv ? 0x0000ffffu : 0u) | (kb + 1 < nv ? 0xffff0000u : 0u);
                vm[2 * hh + 1] = (kb + 2 < nv ? 0x0000ffffu : 0u) | (kb + 3 < nv ? 0xffff0000u : 0u);
            }
#pragma unroll
            for (int t = 0; t < NVT; ++t)
                x.v[t] = i32x4{(int)((uint32_t)x.v[t][0] & vm[0]), (int)((uint32_t)x.v[t][1] & vm[1]),
                               (int)((uint32_t)x.v[t][2] & vm[2]), (int)((uint32_t)x.v[t][3] & vm[3])};
        }
        l += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            hw[w] = pack2<DT>(pe[2 * w], pe[2 * w + 1]);
            lw[w] = pack2<DT>(pe[2 * w] - elem_lo<DT>(hw[w]), pe[2 * w + 1] - elem_hi<DT>(hw[w]));
        }
        const i32x4 phi = {(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3]};
        const i32x4 plo = {(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3]};
        if constexpr (SPLIT) {
            const i32x4 pw = hi_col ? phi : plo;
#pragma unroll
            for (int t = 0; t < NVT; ++t) o[t] = mfma32<DT>(x.v[t], pw, o[t]);
        } else {
#pragma unroll
            for (int t = 0; t < NVT; ++t) {
                o[t] = mfma32<DT>(x.v[t], phi, o[t]);
                o[t] = mfma32<DT>(x.v[t], plo, o[t]);
            }
        }
    };

    load(b0, 0);
    int i = 0;
    for (; i + 2 <= nblk; i += 2) {
        step(b0, b1, i);
        step(b1, b0, i + 1);
    }
    if (i < nblk) step(b0, b1, i);

    if constexpr (SPLIT) {
#pragma unroll
        for (int t = 0; t < NVT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[t][e] += __shfl_down(o[t][e], a.G, 16);
    }
    const float lt = xor32_sum(xor16_sum(l));
    if (!hi_col) return;
    if (t0 == 0 && t1 == ctx) {
        const float inv = 1.f / lt;
#pragma unroll
        for (int t = 0; t < NVT; ++t) store4<DT>(outp + 16 * t + 4 * j, o[t], inv);
        return;
    }
    const int64_t part = ((int64_t)s * a.Hq + h) * a.NP + p;
    float *po = a.part_o + part * D;
#pragma unroll
    for (int t = 0; t < NVT; ++t) *(f32x4 *)(po + 16 * t + 4 * j) = o[t];
    if (j == 0) *(float2 *)(a.part_ml + 2 * part) = float2{m, lt};
}

// ---------------------------------------------------------------------------
// One-query-head partition kernel on VALU.
//
// Lane l = 16 j + n.  Load c of the K tile gives lane l the 16-byte run 4c + j
// of token n; the lane's partial dot products are summed over j (xor 16,
// xor 32), so every lane ends with the score of token n.  For P.V lane l owns
// dims l, l + 64, ...: it loads the 16 tokens of each such dim row of the
// [D][16] V tile and accumulates sum_t p_t v_t with p_t read from lane t
// (v_readlane into an SGPR).  Plain (cacheable) loads: each 32-byte V row is
// read in two halves by two instructions, and blocks shared by several
// sequences (copy-on-write prefixes) are read by several units, so L2 reuse
// matters here; the MFMA kernel streams its tiles with nontemporal loads.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float dot16(const i32x4 &q, const i32x4 &k) {
    if constexpr (DT == kF32) {
        float r = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) r = fmaf(__int_as_float(q[e]), __int_as_float(k[e]), r);
        return r;
    } else if constexpr (DT == kBF16) {
        // Pairs are taken with shufflevector from the whole 16-byte vector:
        // bit-casting single dwords of it to a 2 x bf16 vector was observed to
        // compile to one reused dword.
        const bf16x8 a = __builtin_bit_cast(bf16x8, q);
        const bf16x8 b = __builtin_bit_cast(bf16x8, k);
        float r = 0.f;
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1),
                                            __builtin_shufflevector(b, b, 0, 1), r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3),
                                            __builtin_shufflevector(b, b, 2, 3), r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5),
                                            __builtin_shufflevector(b, b, 4, 5), r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7),
                                            __builtin_shufflevector(b, b, 6, 7), r, false);
        return r;
    } else {
        const f16x8 a = __builtin_bit_cast(f16x8, q);
        const f16x8 b = __builtin_bit_cast(f16x8, k);
        float r = 0.f;
        r = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 0, 1),
                                   __builtin_shufflevector(b, b, 0, 1), r, false);
        r = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 2, 3),
                                   __builtin_shufflevector(b, b, 2, 3), r, false);
        r = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 4, 5),
                                   __builtin_shufflevector(b, b, 4, 5), r, false);
        r = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 6, 7),
                                   __builtin_shufflevector(b, b, 6, 7), r, false);
        return r;
    }
}

// Element t (0..15) of a 16-token V row held as E 16-byte words.
template <int DT> __device__ __forceinline__ float v_elem(const i32x4 *w, int t) {
    if constexpr (DT == kF32) {
        return __int_as_float(w[t >> 2][t & 3]);
    } else {
        const uint32_t x = (uint32_t)w[t >> 3][(t >> 1) & 3];
        return (t & 1) ? elem_hi<DT>(x) : elem_lo<DT>(x);
    }
}

// fp32 rows at D = 128 need more registers than four waves per SIMD allow
template <int DT, int D>
__global__ __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(DT == kF32 && D == 128 ? 3 : 4, 8)))
void decode_valu_kernel(const DecodeArgs a) {
    constexpr int E = Elem<DT>::bytes;
    constexpr int X = 16 / E;     // elements per 16-byte run
    constexpr int NC = D / X;     // runs per token
    constexpr int KL = NC / 4;    // K loads per lane per block
    constexpr int DPL = D / 64;   // V dims per lane
    constexpr int VW = E;         // 16-byte words per 16-token V row
    constexpr int TILE = D * kB * E;
    static_assert(NC % 4 == 0 && D % 64 == 0, "unsupported head_dim");

    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int j = lane >> 4;

    // Units in the order of find_unit (sequence-major, head fastest).  With a
    // multiple of 8 heads, head h of a sequence runs on XCD (offset + h) % 8.
    int s, ctx, r;
    if (!find_unit(blockIdx.x, a, a.P, a.Hq, s, ctx, r)) return;
    const int h = r % a.Hq;
    const int p = r / a.Hq;
    const int g = h / a.G;

    const int per = blocks_per_partition(ctx, a.P);
    const int blk0 = p * per;
    const int t0 = blk0 * kB;
    int my_bt = table_entry(a, s, blk0 + lane);
    char *outp = (char *)a.out + ((int64_t)s * a.Hq + h) * D * E;
    if (t0 >= ctx) {
        if (p == 0) {
#pragma unroll
            for (int w = 0; w < DPL; ++w) store1<DT>(outp + (lane + 64 * w) * E, 0.f);
        }
        return;
    }
    const int t1 = min(ctx, t0 + per * kB);
    const int nblk = (t1 - t0 + kB - 1) / kB;
    if (lane >= nblk || my_bt < 0 || (int64_t)my_bt >= a.NB) my_bt = 0;

    const char *qrow = (const char *)a.q + ((int64_t)s * a.Hq + h) * D * E;
    i32x4 qf[KL];
#pragma unroll
    for (int c = 0; c < KL; ++c) qf[c] = ld16(qrow + (4 * c + j) * 16);

    const char *kbase = (const char *)a.k + (int64_t)g * TILE;
    const char *vbase = (const char *)a.v + (int64_t)g * TILE;
    const int64_t blk_stride = (int64_t)a.Hkv * TILE;

    float m = -INFINITY;
    float l = 0.f;
    float o[DPL];
#pragma unroll
    for (int w = 0; w < DPL; ++w) o[w] = 0.f;

    i32x4 kf[KL];
    i32x4 vf[DPL][VW];

    auto load_k = [&](int i) {
        const char *kt = kbase + (int64_t)__builtin_amdgcn_readlane(my_bt, i) * blk_stride;
#pragma unroll
        for (int c = 0; c < KL; ++c) kf[c] = ld16(kt + (64 * c + lane) * 16);
        issue_point();
    };
    auto load_v = [&](int i) {
        const char *vt = vbase + (int64_t)__builtin_amdgcn_readlane(my_bt, i) * blk_stride;
#pragma unroll
        for (int w = 0; w < DPL; ++w)
#pragma unroll
            for (int x = 0; x < VW; ++x) vf[w][x] = ld16(vt + (lane + 64 * w) * (kB * E) + 16 * x);
        issue_point();
    };
    auto scores = [&]() {
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < KL; ++c) part += dot16<DT>(qf[c], kf[c]);
        part += shfl_xor(part, 16);
        part += shfl_xor(part, 32);
        return part;
    };
    auto update = [&](float part, int nv, bool tail) {
        const float sc = (!tail || n < nv) ? part * a.scale_log2 : -INFINITY;
        const float bm = row16_max(sc);
        const float mn = fmaxf(m, bm);
        const float alpha = fast_exp2(m - mn);
        m = mn;
        const float pt = fast_exp2(sc - mn);
        l = l * alpha + pt;
#pragma unroll
        for (int w = 0; w < DPL; ++w) {
            float acc0 = o[w] * alpha, acc1 = 0.f;
#pragma unroll
            for (int t = 0; t < kB; ++t) {
                const float pw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pt), t));
                float vv = v_elem<DT>(vf[w], t);
                if (tail && t >= nv) vv = 0.f;  // empty slot: may hold NaN
                if (t & 1)
                    acc1 = fmaf(pw, vv, acc1);
                else
                    acc0 = fmaf(pw, vv, acc0);
            }
            o[w] = acc0 + acc1;
        }
    };

    load_k(0);
    load_v(0);
    for (int i = 0; i < nblk - 1; ++i) {
        const float part = scores();
        load_k(i + 1);
        update(part, kB, false);
        load_v(i + 1);
    }
    {
        const float part = scores();
        update(part, t1 - (t0 + (nblk - 1) * kB), true);
    }

    const float lt = row16_sum(l);  // each row of 16 lanes holds the 16 tokens
    if (t0 == 0 && t1 == ctx) {
        const float inv = 1.f / lt;
#pragma unroll
        for (int w = 0; w < DPL; ++w) store1<DT>(outp + (lane + 64 * w) * E, o[w] * inv);
        return;
    }
    const int64_t part = ((int64_t)s * a.Hq + h) * a.NP + p;
    float *po = a.part_o + part * D;
#pragma unroll
    for (int w = 0; w < DPL; ++w) po[lane + 64 * w] = o[w];
    if (lane == 0) {
        a.part_ml[2 * part] = m;
        a.part_ml[2 * part + 1] = lt;
    }
}

// ---------------------------------------------------------------------------
// Loads only, for measurement: the K/V tiles decode_mfma_kernel reads, with
// its work units, its load instructions (16-byte K runs, 8-byte V pieces,
// nontemporal) and one block requested ahead, folded into an XOR so that no
// load can be dropped, and nothing else.  Its time is what the decode would
// take if the reduction cost nothing: the ceiling of this access pattern on
// the machine at hand.  (The fold is stored only if it equals a constant, so
// the kernel writes nothing in practice.)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void read_tiles_kernel(const DecodeArgs a, int *sink) {
    constexpr int NKC = D / 32;
    constexpr int NVT = D / 16;
    constexpr int TILE = D * kB * 2;
    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int j = lane >> 4;
    int P, s, ctx, r;
    if (!unit_of(blockIdx.x, a, a.Hkv, P, s, ctx, r)) return;
    if (ctx == 0) return;
    const int g = r % a.Hkv;
    const int p = r / a.Hkv;
    const int per = blocks_per_partition(ctx, P);
    const int t0 = p * per * kB;
    const int t1 = min(ctx, t0 + per * kB);
    const int nblk = (t1 - t0 + kB - 1) / kB;
    int my_bt = table_entry(a, s, p * per + lane);
    if (lane >= nblk || my_bt < 0 || (int64_t)my_bt >= a.NB) my_bt = 0;
    const char *kbase = (const char *)a.k + (int64_t)g * TILE;
    const char *vbase = (const char *)a.v + (int64_t)g * TILE;
    const int64_t blk_stride = (int64_t)a.Hkv * TILE;
    struct Blk {
        i32x4 k[NKC];
        i32x2 v[NVT];
    };
    Blk b0, b1;
    auto load = [&](Blk &x, int i) {
        const bool in = i < nblk;
        const int phys = __builtin_amdgcn_readlane(my_bt, in ? i : 0);
        const int64_t off = (int64_t)phys * blk_stride;
        const auto rk = tile_rsrc(kbase + off, in ? TILE : 0);
        const auto rv = tile_rsrc(vbase + off, in ? TILE : 0);
#pragma unroll
        for (int c = 0; c < NKC; ++c) x.k[c] = bload16<kCachePolicyNT>(rk, (64 * c + lane) * 16);
#pragma unroll
        for (int t = 0; t < NVT; ++t)
            x.v[t] = bload8<kCachePolicyNT>(rv, ((16 * t + n) * kB + 4 * j) * 2);
        issue_point();
    };
    int acc = 0;
    auto step = [&](Blk &x, Blk &y, int i) {
        load(y, i + 1);
#pragma unroll
        for (int c = 0; c < NKC; ++c) acc ^= x.k[c][0] ^ x.k[c][1] ^ x.k[c][2] ^ x.k[c][3];
#pragma unroll
        for (int t = 0; t < NVT; ++t) acc ^= x.v[t][0] ^ x.v[t][1];
    };
    load(b0, 0);
    int i = 0;
    for (; i + 2 <= nblk; i += 2) {
        step(b0, b1, i);
        step(b1, b0, i + 1);
    }
    if (i < nblk) step(b0, b1, i);
    if (acc == 0x5eed1e55) *sink = acc;
}

hipError_t launch_read_tiles(const DecodeArgs &a, int head_dim, int *sink, hipStream_t stream) {
    if (a.num_units <= 0) return hipSuccess;
    if (head_dim == 64)
        read_tiles_kernel<64><<<a.num_units, 64, 0, stream>>>(a, sink);
    else
        read_tiles_kernel<128><<<a.num_units, 64, 0, stream>>>(a, sink);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge kernels: the log-sum-exp merge (LseState) of every split row, run
// after the partition kernel when the in-kernel merge does not apply; np
// follows from the context length.
//
// merge_kernel (rows of at most 16 partitions): D/4 lanes per row, four dims
// each.  The (m, l, o) of the first kSpec = 2 partitions are requested
// together with the context length; the remaining ones (np - 2 <= 14) follow
// in blocks of 8 requested at once.  Requesting more partitions ahead of the
// context length reads the slots of partitions that do not exist for short
// contexts, and those bytes cost more than the extra round trip: on the
// Llama-3-8B-shaped step (partitions of 640 tokens, up to 7 per row) the
// decode took 49.0 us with 8 requested ahead, 48.2 with 4 and 47.6-47.8 with
// 1, 2 or 3 (steady state, MI355X); 2 lanes per dim pair or 1 dim per lane
// were slower.
//
// merge_wide_kernel (more than 16 partitions per row: long contexts): one
// workgroup per row; its 256 / (D/4) lane groups take every n-th partition,
// 8 requests in flight each, and combine their states through LDS in group
// order.  (With a row per D/4 lanes, the 4-sequence long-context step ran its
// merge on 32 workgroups, a few dozen dependent round trips each.)
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 128;   // 4 rows at D = 128
constexpr int kMergeWideThreads = 256;
constexpr int kMergeWideMaxParts = 16;  // rows with more partitions take the wide merge

template <int DT, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const DecodeArgs a) {
    constexpr int LPR = D / 4;                // lanes per row
    constexpr int RPB = kMergeThreads / LPR;  // rows per workgroup
    constexpr int kSpec = 2;
    constexpr int kRest = kMergeWideMaxParts - kSpec;
    const int tid = threadIdx.x;
    const int row = blockIdx.x * RPB + tid / LPR;  // s * Hq + h
    const int d0 = (tid % LPR) * 4;
    const int P = merge_partition_len(a);
    if (row >= a.S * a.Hq) return;
    const int s = row / a.Hq;
    const float *pml = a.part_ml + (int64_t)row * a.NP * 2;
    const float *po = a.part_o + (int64_t)row * a.NP * D + d0;
    float2 ml[kSpec];
    f32x4 ov[kSpec];
#pragma unroll
    for (int q = 0; q < kSpec; ++q) {
        if (q < a.NP) {
            ml[q] = *(const float2 *)(pml + 2 * q);
            ov[q] = *(const f32x4 *)(po + (int64_t)q * D);
        }
    }
    const int ctx = seq_ctx(a, s);
    const int np = ctx > P ? (ctx + P - 1) / P : 1;
    if (np <= 1) return;  // written by the partition kernel
    LseState st;
#pragma unroll
    for (int q = 0; q < kSpec; ++q)
        if (q < np) st.add(ml[q].x, ml[q].y, ov[q]);
    // the rest (np <= 16: the host takes the wide merge otherwise), in blocks of 8
#pragma unroll
    for (int q0 = kSpec; q0 < kSpec + kRest; q0 += 8) {
        if (q0 >= np) break;
        float2 m2[8];
        f32x4 o2[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (q0 + q < np) {
                m2[q] = *(const float2 *)(pml + 2 * (q0 + q));
                o2[q] = *(const f32x4 *)(po + (int64_t)(q0 + q) * D);
            }
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (q0 + q < np) st.add(m2[q].x, m2[q].y, o2[q]);
    }
    store4<DT>((char *)a.out + ((int64_t)row * D + d0) * Elem<DT>::bytes, st.acc, 1.f / st.L);
}

template <int DT, int D>
__global__ __launch_bounds__(kMergeWideThreads) void merge_wide_kernel(const DecodeArgs a) {
    constexpr int LPR = D / 4;                       // lanes per group: one row's D outputs
    constexpr int NGRP = kMergeWideThreads / LPR;    // lane groups
    constexpr int kIn = 8;                           // partitions in flight per group
    __shared__ float sm_ml[NGRP][2];
    __shared__ f32x4 sm_o[NGRP][LPR];
    const int row = blockIdx.x;  // s * Hq + h
    const int tid = threadIdx.x;
    const int grp = tid / LPR, lg = tid % LPR, d0 = lg * 4;
    const int s = row / a.Hq;
    const int P = merge_partition_len(a);
    const int ctx = seq_ctx(a, s);
    const int np = ctx > P ? (ctx + P - 1) / P : 1;
    if (np <= 1) return;  // the whole workgroup: written by the partition kernel
    const float *pml = a.part_ml + (int64_t)row * a.NP * 2;
    const float *po = a.part_o + (int64_t)row * a.NP * D + d0;
    // group k folds partitions k, k + NGRP, k + 2 NGRP, ... in order
    LseState st;
    for (int q0 = grp; q0 < np; q0 += NGRP * kIn) {
        float2 m2[kIn];
        f32x4 o2[kIn];
#pragma unroll
        for (int q = 0; q < kIn; ++q) {
            const int qq = q0 + q * NGRP;
            if (qq < np) {
                m2[q] = *(const float2 *)(pml + 2 * qq);
                o2[q] = *(const f32x4 *)(po + (int64_t)qq * D);
            }
        }
#pragma unroll
        for (int q = 0; q < kIn; ++q)
            if (q0 + q * NGRP < np) st.add(m2[q].x, m2[q].y, o2[q]);
    }
    if (lg == 0) {
        sm_ml[grp][0] = st.M;
        sm_ml[grp][1] = st.L;
    }
    sm_o[grp][lg] = st.acc;
    __syncthreads();
    if (grp != 0) return;
    // groups 0 .. min(np, NGRP) - 1 hold partitions; combine them in order
    LseState tot;
    const int ng = np < NGRP ? np : NGRP;
    for (int k = 0; k < ng; ++k) tot.add(sm_ml[k][0], sm_ml[k][1], sm_o[k][lg]);
    store4<DT>((char *)a.out + ((int64_t)row * D + d0) * Elem<DT>::bytes, tot.acc, 1.f / tot.L);
}

// ---------------------------------------------------------------------------
template <int DT, int D, int POLICY, bool APPEND, bool PLAN>
static void launch_mfma16(const DecodeArgs &a, bool split, int grid, hipStream_t stream) {
    if (split)
        decode_mfma_kernel<DT, D, true, POLICY, 16, APPEND, PLAN><<<grid, 64, 0, stream>>>(a);
    else
        decode_mfma_kernel<DT, D, false, POLICY, 16, APPEND, PLAN><<<grid, 64, 0, stream>>>(a);
}

template <int DT, int D>
static hipError_t launch_typed(const DecodeArgs &a, DecodeKernel kind, hipStream_t stream) {
    // one workgroup per possible unit (the host plans for full tables); the
    // ones past the real units exit at once
    const int grid = a.num_units;
    if (grid > 0) {
        if constexpr (DT != kF32) {
            if (kind == DecodeKernel::kMfma && a.BS != kB) {
                const bool split = 2 * a.G <= 16;
                if (a.BS == 32) {
                    if (split)
                        decode_mfma_b32_kernel<DT, D, true><<<grid, 64, 0, stream>>>(a);
                    else
                        decode_mfma_b32_kernel<DT, D, false><<<grid, 64, 0, stream>>>(a);
                } else {
                    if (split)
                        decode_mfma_kernel<DT, D, true, kCachePolicyNT, 8><<<grid, 64, 0, stream>>>(a);
                    else
                        decode_mfma_kernel<DT, D, false, kCachePolicyNT, 8><<<grid, 64, 0, stream>>>(a);
                }
            } else if (kind == DecodeKernel::kMfma) {
                const bool split = 2 * a.G <= 16;
                if (a.k_new) {
                    if (a.plan)
                        launch_mfma16<DT, D, kCachePolicyNT, true, true>(a, split, grid, stream);
                    else
                        launch_mfma16<DT, D, kCachePolicyNT, true, false>(a, split, grid, stream);
                } else if (a.shared_blocks) {
                    if (a.plan)
                        launch_mfma16<DT, D, kCachePolicyPlain, false, true>(a, split, grid, stream);
                    else
                        launch_mfma16<DT, D, kCachePolicyPlain, false, false>(a, split, grid, stream);
                } else {
                    if (a.plan)
                        launch_mfma16<DT, D, kCachePolicyNT, false, true>(a, split, grid, stream);
                    else
                        launch_mfma16<DT, D, kCachePolicyNT, false, false>(a, split, grid, stream);
                }
            } else {
                decode_valu_kernel<DT, D><<<dim3(grid), dim3(64), 0, stream>>>(a);
            }
        } else {
            decode_valu_kernel<DT, D><<<dim3(grid), dim3(64), 0, stream>>>(a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.NP > 1 && a.S > 0 && !a.fuse_merge) {
        const int rows = a.S * a.Hq;
        if (a.NP > kMergeWideMaxParts) {
            merge_wide_kernel<DT, D><<<dim3(rows), dim3(kMergeWideThreads), 0, stream>>>(a);
        } else {
            const int rows_per_block = kMergeThreads / (D / 4);
            merge_kernel<DT, D><<<dim3((rows + rows_per_block - 1) / rows_per_block),
                                   dim3(kMergeThreads), 0, stream>>>(a);
        }
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs &a, int dtype, int head_dim, DecodeKernel kind,
                         hipStream_t stream) {
    switch (dtype) {
    case kF32:
        return head_dim == 64 ? launch_typed<kF32, 64>(a, kind, stream)
                              : launch_typed<kF32, 128>(a, kind, stream);
    case kF16:
        return head_dim == 64 ? launch_typed<kF16, 64>(a, kind, stream)
                              : launch_typed<kF16, 128>(a, kind, stream);
    default:
        return head_dim == 64 ? launch_typed<kBF16, 64>(a, kind, stream)
                              : launch_typed<kBF16, 128>(a, kind, stream);
    }
}

// ---------------------------------------------------------------------------
// Dispatch probe for the in-kernel merge: each workgroup records the XCD it
// runs on.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void xcd_probe_kernel(unsigned *xcd) {
    if (threadIdx.x == 0) xcd[blockIdx.x] = xcc_id();
}

hipError_t probe_xcd_dispatch(int *num_xcd, bool *ok) {
    constexpr int kWorkgroups = 4096;
    *num_xcd = 0;
    *ok = false;
    unsigned *d = nullptr;
    hipError_t e = hipMalloc(&d, kWorkgroups * sizeof(unsigned));
    if (e != hipSuccess) return e;
    hipStream_t st = nullptr;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    std::vector<unsigned> h(kWorkgroups, ~0u);
    if (e == hipSuccess) {
        xcd_probe_kernel<<<kWorkgroups, 64, 0, st>>>(d);
        e = hipGetLastError();
        if (e == hipSuccess)
            e = hipMemcpyAsync(h.data(), d, kWorkgroups * sizeof(unsigned),
                               hipMemcpyDeviceToHost, st);
        const hipError_t e2 = hipStreamSynchronize(st);
        if (e == hipSuccess) e = e2;
        (void)hipStreamDestroy(st);
    }
    (void)hipFree(d);
    if (e != hipSuccess) return e;
    // X distinct ids in the first X workgroups, then the same cycle throughout
    int X = 0;
    while (X < 16 && X < kWorkgroups) {
        bool seen = false;
        for (int i = 0; i < X; ++i) seen |= h[i] == h[X];
        if (seen) break;
        ++X;
    }
    bool cyclic = X >= 1 && X <= 16;
    for (int b = X; cyclic && b < kWorkgroups; ++b) cyclic = h[b] == h[b % X];
    *num_xcd = X;
    *ok = cyclic;
    return hipSuccess;
}

}  // namespace pa
