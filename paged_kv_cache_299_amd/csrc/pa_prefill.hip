// pa_prefill.hip -- paged prefill attention on the matrix cores (gfx950).
//
// The queries of a chunk of new tokens attend causally over their sequence's
// cached tokens, read through the block table: the i-th of n queries of a
// sequence with ctx cached tokens (the chunk's own K/V included) sits at
// position ctx - n + i and sees positions 0 .. ctx - n + i.  n == ctx is a
// whole prompt, n < ctx a chunk after a cached prefix, n == 1 a decode step.
// [論文解説: PagedAttention, 実装のポイント › CUDAカーネル実装: one kernel
//  gathers the scattered blocks for both the prefill and the decode phase]
//
// Work: a workgroup of 4 waves takes 128 consecutive "rows" of one
// (sequence, kv head); row r is query r / G of the chunk with query head
// r % G of the group, so the G heads that share a kv head share every K/V
// operand.  Each wave owns 32 rows as two 16-row tiles and walks the keys 32
// at a time (two blocks), up to its last row's position.
//
// Per 32 keys and 16-row tile, with lane l = 16 j + n:
//  * S^T = K . Q^T on v_mfma_f32_16x16x32 (4 per block at D = 128): the A
//    operand is the K tile's 16-byte run 4c + j of token n, read straight from
//    the pool (64 lanes read 1 KiB in order), the B operand the row's q.  Lane
//    l receives keys 4j .. 4j+3 of the block for row n.
//  * online softmax per row (log2 domain, lazy rescale when the maximum grows
//    by more than 8), causal and tail masking only in the iterations that
//    need it;
//  * O^T += V^T . P^T on v_mfma_f32_16x16x32 over the 32 keys: the k slots
//    8j .. 8j+7 of lane group j are keys 8j .. 8j+7, one 16-byte read of the
//    transposed V tile (half a 16-token row of one block).  Two lane swaps
//    (v_permlane32_swap, v_permlane16_swap) move the weights from the score
//    layout to that one.  The weights go in as hi + lo 16-bit parts
//    (hi = RNE(p), lo = RNE(p - hi)), so P keeps about 16 significant bits.
// K/V go through one set of operand registers (221 VGPRs, two waves per
// SIMD): the next K is requested as soon as the scores are in, the next V as
// soon as the P.V products have read the current one.  The address unit
// costs about the same per load instruction whatever its width, so every
// operand load is 16 bytes a lane.  Plain (cacheable) loads: the other waves
// of the workgroup and the other row tiles of the sequence read the same
// tiles.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kPrefillWaves = 4;
constexpr int kRowTiles = 2;                                 // 16-row tiles per wave
constexpr int kRowsPerWave = 16 * kRowTiles;                 // 32
constexpr int kRowsPerGroup = kPrefillWaves * kRowsPerWave;  // 128
constexpr int kBtChunk = 64;                                 // table entries per lane load

template <int DT, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(const PrefillArgs a) {
    static_assert(DT == kBF16 || DT == kF16, "MFMA path takes 16-bit data");
    static_assert(D % 32 == 0, "head_dim must be a multiple of 32");
    constexpr int NKC = D / 32;       // QK steps of 32 dims
    constexpr int NVT = D / 16;       // output tiles of 16 dims
    constexpr int TILE = D * kB * 2;  // bytes of one (block, kv head) tile

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int j = lane >> 4;
    // Workgroups start in linear order, dealt round-robin to the eight XCDs,
    // each with its own L2.  Linear id L takes kv head L % Hkv (so one head
    // per XCD when Hkv is a multiple of 8), then the tiles of one sequence,
    // longest first: the workgroups that run together on an XCD read the same
    // K/V, which stays in that L2 (95% hits against 83% with the tiles of all
    // sequences interleaved, and 21% less time on 8 prompts of 1-4k tokens).
    const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int g = L % gridDim.x;
    const int r = L / gridDim.x;
    const int s = r / gridDim.z;
    const int tile = gridDim.z - 1 - (r - s * gridDim.z);

    // The sequence's queries and context, clamped so that no access leaves
    // the buffers whatever the device holds.
    int q0 = __builtin_amdgcn_readfirstlane(a.qs[s]);
    int q1 = __builtin_amdgcn_readfirstlane(a.qs[s + 1]);
    q0 = min(max(q0, 0), a.T);
    q1 = min(max(q1, q0), a.T);
    int ctx = __builtin_amdgcn_readfirstlane(a.ctx[s]);
    ctx = min(max(ctx, 0), a.MB * kB);
    const int nq = min(q1 - q0, ctx);
    const int rows = nq * a.G;
    const int R0 = tile * kRowsPerGroup + wave * kRowsPerWave;
    if (R0 >= rows) return;
    const int pos0 = ctx - nq;  // position of the chunk's first query

    // this lane's rows: a row past the end repeats the last one (computed, never stored)
    int prow[kRowTiles];
    int64_t orow[kRowTiles];
    bool keep[kRowTiles];
    i32x4 qf[kRowTiles][NKC];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        const int R = R0 + 16 * rt + n;
        const int Rc = min(R, rows - 1);
        const int ql = Rc / a.G;
        const int hl = Rc - ql * a.G;
        prow[rt] = pos0 + ql;
        orow[rt] = ((int64_t)(q0 + ql) * a.Hq + g * a.G + hl) * D;
        keep[rt] = R < rows;
        const uint16_t *qp = (const uint16_t *)a.q + orow[rt];
#pragma unroll
        for (int c = 0; c < NKC; ++c) qf[rt][c] = ld16(qp + (4 * c + j) * 8) ^ a.q_xor;
    }
    const float cs = a.scale_log2_abs;  // the sign of the scale went into q

    // keys this wave needs: positions 0 .. p_max; no row masks keys <= p_min
    const int p_min = pos0 + R0 / a.G;
    const int p_max = pos0 + (min(R0 + kRowsPerWave, rows) - 1) / a.G;
    const int nblk = p_max / kB + 1;
    const int iters = (nblk + 1) / 2;

    const char *kbase = (const char *)a.k + (int64_t)g * TILE;
    const char *vbase = (const char *)a.v + (int64_t)g * TILE;
    const int64_t blk_stride = (int64_t)a.Hkv * TILE;
    const int *btrow = a.bt + (int64_t)s * a.MB;
    int my_bt = 0;  // table entries kBtChunk * chunk + lane

    float m[kRowTiles], l[kRowTiles];
    f32x4 o[kRowTiles][NVT];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        m[rt] = -INFINITY;
        l[rt] = 0.f;
#pragma unroll
        for (int t = 0; t < NVT; ++t) o[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // One set of operand registers: the K of the next two blocks is requested
    // as soon as the scores of the current ones are in, their V as soon as
    // the current P.V products have read theirs.  (A second set, to request a
    // whole iteration ahead, took the kernel to 352 registers and one wave
    // per SIMD.)
    i32x4 kk[2][NKC];
    i32x4 vv[NVT];
    // Iteration it reads blocks 2 it and 2 it + 1; a block past the wave's
    // last one gets a zero-range descriptor (zeros, no memory traffic).
    auto tile_off = [&](int it, int b, bool &in) {
        const int blk = 2 * it + b;
        in = blk < nblk;
        const int phys = __builtin_amdgcn_readlane(my_bt, in ? (blk & (kBtChunk - 1)) : 0);
        return (int64_t)phys * blk_stride;
    };
    auto load_table = [&](int it) {  // the slice of the block table from block 2 it on
        const int e = 2 * it + lane;
        int id = e < nblk ? btrow[e] : 0;
        if (id < 0 || (int64_t)id >= a.NB) id = 0;
        my_bt = id;
    };
    auto load_k = [&](int it) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            bool in;
            const int64_t off = tile_off(it, b, in);
            const auto rk = tile_rsrc(kbase + off, in ? TILE : 0);
#pragma unroll
            for (int c = 0; c < NKC; ++c)
                kk[b][c] = bload16<kCachePolicyPlain>(rk, (64 * c + lane) * 16);
        }
        issue_point();
    };
    // V: lane group j reads keys 8 j .. 8 j + 7 of the 32, i.e. half j & 1 of
    // the 16-token row of block j >> 1: one 16-byte load per 16 dims.  The two
    // blocks sit anywhere in the pool, so these are global loads with a lane
    // address; a block past the wave's last one is replaced by the first (a
    // valid tile whose keys all get weight 0).
    auto load_v = [&](int it) {
        bool in0, in1;
        const int64_t off0 = tile_off(it, 0, in0);
        const int64_t off1 = tile_off(it, 1, in1);
        const char *vp = vbase + ((j >> 1) && in1 ? off1 : off0) + n * (kB * 2) + (j & 1) * 16;
        const __attribute__((address_space(1))) i32x4 *gp =
            (const __attribute__((address_space(1))) i32x4 *)vp;
#pragma unroll
        for (int t = 0; t < NVT; ++t) vv[t] = gp[t * kB * 2];  // 16 rows of 32 bytes further
        issue_point();
    };

    // One step: the 32 keys of blocks 2 it, 2 it + 1 for the wave's 32 rows.
    // FULL steps mask no key for any row (every key precedes every row's
    // position and the sequence's tail): they have no masking code, and one
    // rarely taken branch (the rescale) in the middle, so that the compiler
    // can lay the exponentials and weight packing of one row tile between the
    // P.V products of the other.
    auto step = [&](int it, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        if (((it + 1) & (kBtChunk / 2 - 1)) == 0) load_table(it + 1);
        f32x4 sc[kRowTiles][2];
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                sc[rt][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < NKC; ++c) sc[rt][b] = mfma32<DT>(kk[b][c], qf[rt][c], sc[rt][b]);
            }
        load_k(it + 1);
        const int key0 = 32 * it;
        if constexpr (!FULL) {
            // slots at or past ctx (the tail of the sequence's last block) may
            // hold NaN: their V is zeroed, since a zero weight does not cancel a NaN
            if (key0 + 32 > ctx) {
                const int kb = key0 + 8 * j;
                uint32_t mk[4];
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    mk[w] = (kb + 2 * w < ctx ? 0x0000ffffu : 0u) |
                            (kb + 2 * w + 1 < ctx ? 0xffff0000u : 0u);
#pragma unroll
                for (int t = 0; t < NVT; ++t)
#pragma unroll
                    for (int w = 0; w < 4; ++w) vv[t][w] = (int)((uint32_t)vv[t][w] & mk[w]);
            }
        }
        // The running maximum only moves when a score passes it by more than 8
        // (log2 units), so each lane first tests its own 8 scores per row tile,
        // and a row's maximum over the four lane groups is formed only when
        // some lane of the wave is over.
        float sv[kRowTiles][8], lm[kRowTiles];
        bool over = false;
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[rt][4 * b + e] = sc[rt][b][e];
            if constexpr (!FULL) {
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (key0 + 16 * b + 4 * j + e > prow[rt]) sv[rt][4 * b + e] = -INFINITY;
            }
            lm[rt] = __builtin_elementwise_maximum(max4f(sv[rt][0], sv[rt][1], sv[rt][2], sv[rt][3]),
                                                   max4f(sv[rt][4], sv[rt][5], sv[rt][6], sv[rt][7]));
            over = over | (lm[rt] * cs > m[rt] + 8.f);
        }
        if (__any(over)) {
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) {
                const float bm = xor32_max(xor16_max(lm[rt])) * cs;  // -inf: the row sees none of these keys
                const bool grow = bm > m[rt] + 8.f;
                if (__any(grow)) {
                    const float mn = grow ? bm : m[rt];
                    const float alpha = fast_exp2(m[rt] - mn);  // 0 on a row's first keys
#pragma unroll
                    for (int t = 0; t < NVT; ++t) o[rt][t] *= alpha;
                    l[rt] *= alpha;
                    m[rt] = mn;
                }
            }
        }
        uint32_t hi[kRowTiles][4], lo[kRowTiles][4];
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) {
            const float nm = -m[rt];
            float pe[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(fmaf(sv[rt][e], cs, nm));
            if constexpr (!FULL) {  // (-inf) * 0 is NaN when the scale is 0
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (key0 + 16 * b + 4 * j + e > prow[rt]) pe[4 * b + e] = 0.f;
            }
            l[rt] += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                hi[rt][w] = pack2<DT>(pe[2 * w], pe[2 * w + 1]);
                lo[rt][w] = pack2<DT>(pe[2 * w] - elem_lo<DT>(hi[rt][w]),
                                      pe[2 * w + 1] - elem_hi<DT>(hi[rt][w]));
            }
        }
        // The scores left lane group j with keys 4j .. 4j+3 of each block
        // (words 0, 1: block 0; words 2, 3: block 1).  Two lane swaps give it
        // keys 8j .. 8j+7 of the 32, the k slots of its V operand: the upper
        // half-wave's block-0 words trade with the lower half-wave's block-1
        // words, then odd lane groups trade with even ones.
        auto regroup = [](uint32_t (&w)[4]) {
            const auto r0 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
            const auto r1 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
            const auto s0 = __builtin_amdgcn_permlane16_swap(r0[0], r0[1], false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(r1[0], r1[1], false, false);
            w[0] = s0[0];
            w[1] = s1[0];
            w[2] = s0[1];
            w[3] = s1[1];
        };
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) {
            regroup(hi[rt]);
            regroup(lo[rt]);
        }
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            const i32x4 va = vv[t];
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) {
                const i32x4 phi = {(int)hi[rt][0], (int)hi[rt][1], (int)hi[rt][2], (int)hi[rt][3]};
                const i32x4 plo = {(int)lo[rt][0], (int)lo[rt][1], (int)lo[rt][2], (int)lo[rt][3]};
                o[rt][t] = mfma32<DT>(va, phi, o[rt][t]);
                o[rt][t] = mfma32<DT>(va, plo, o[rt][t]);
            }
        }
        load_v(it + 1);
    };

    load_table(0);
    load_k(0);
    load_v(0);
    // steps 0 .. nfull - 1 end at or before the wave's first row: key0 + 31 <= p_min
    const int nfull = min(iters, p_min >= 31 ? (p_min - 31) / 32 + 1 : 0);
    int it = 0;
    for (; it < nfull; ++it) step(it, std::true_type{});
    for (; it < iters; ++it) step(it, std::false_type{});

#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
        const float lt = xor32_sum(xor16_sum(l[rt]));  // all lanes take part in the swaps
        if (keep[rt]) {
            const float inv = 1.f / lt;
            uint16_t *op = (uint16_t *)a.out + orow[rt];
#pragma unroll
            for (int t = 0; t < NVT; ++t) store4<DT>(op + 16 * t + 4 * j, o[rt][t], inv);
        }
    }
}

template <int DT>
hipError_t launch_typed(const PrefillArgs &a, int head_dim, dim3 grid, hipStream_t stream) {
    if (head_dim == 128) {
        prefill_mfma_kernel<DT, 128><<<grid, dim3(64 * kPrefillWaves), 0, stream>>>(a);
    } else {
        prefill_mfma_kernel<DT, 64><<<grid, dim3(64 * kPrefillWaves), 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

int64_t prefill_row_tiles(int64_t max_query_len, int G) {
    return (max_query_len * G + kRowsPerGroup - 1) / kRowsPerGroup;
}

hipError_t launch_prefill(const PrefillArgs &a, int dtype, int head_dim, int max_query_len,
                          hipStream_t stream) {
    const int64_t tiles = prefill_row_tiles(max_query_len, a.G);
    if (tiles == 0 || a.S == 0) return hipSuccess;
    const dim3 grid((unsigned)a.Hkv, (unsigned)a.S, (unsigned)tiles);
    return dtype == kBF16 ? launch_typed<kBF16>(a, head_dim, grid, stream)
                          : launch_typed<kF16>(a, head_dim, grid, stream);
}

}  // namespace pa
