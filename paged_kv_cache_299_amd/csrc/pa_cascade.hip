// pa_cascade.hip -- decode that reads each shared prefix block once for all
// the sequences that share it.
//
// Sequences that share their first blocks (the samples of one prompt under
// parallel sampling or beam search; copy-on-write keeps those blocks
// physically shared) form a group.  [論文解説: PagedAttention, 技術的詳細 ›
// Copy-on-Write KVキャッシュ共有]  pa_decode streams a shared block once per
// sequence; here the attention is cut at the end of the shared blocks:
//  * prefix units: the group's shared keys against the queries of all its
//    members at once (rows = members x query heads of one kv head, as the
//    columns of the matrix-core tiles), so each shared block is read once
//    per group and kv head;
//  * suffix units: each sequence's own keys against its own G heads;
//  * both write partial (max, sum, unnormalised output) states per query row,
//    and a merge kernel combines them with log-sum-exp weights.
// The split is exact up to rounding: the streaming softmax is associative.
// [論文解説: PagedAttention, 技術的詳細 › PagedAttentionアルゴリズム, online
//  softmax]
//
// A "row group" is either the prefix of group r (r < NG) or the suffix of
// sequence s (r = NG + s).  Units = (row group, key partition of at most P
// tokens in equal whole blocks, 16-row column tile, kv head), kv head
// fastest.  The workgroups (one wave each) walk the unit list with a stride
// of the grid size; a wave-wide prefix sum over the row groups finds a unit.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

// The group of sequence s: the last r with gs[r] <= s (gs non-decreasing,
// gs[0] = 0); wave-uniform arguments give a scalar search.
__device__ __forceinline__ int group_of(const int *gs, int NG, int s) {
    int lo = 0, hi = NG - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (gs[mid] <= s) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Row group r, with every device value clamped so that no access leaves the
// buffers: first sequence, member count and the key range [k0, k1).
struct RowGroup {
    int seq0, members, k0, k1;
};

__device__ __forceinline__ RowGroup row_group(const CascadeArgs &a, int r) {
    const int cap_blocks = a.MB;
    RowGroup g;
    if (r < a.NG) {
        const int s0 = min(max(a.gs[r], 0), a.S);
        const int s1 = min(max(a.gs[r + 1], s0), a.S);
        const int pb = min(max(a.pblk[r], 0), cap_blocks);
        g.seq0 = s0;
        g.members = s1 - s0;
        g.k0 = 0;
        g.k1 = g.members > 0 ? pb * kB : 0;
    } else {
        const int s = r - a.NG;
        const int gi = group_of(a.gs, a.NG, s);
        const int pb = min(max(a.pblk[gi], 0), cap_blocks);
        const int ctx = clamp_ctx(a.ctx[s], a.MB * kB);
        g.seq0 = s;
        g.members = 1;
        g.k0 = pb * kB;
        g.k1 = max(ctx, g.k0);
    }
    return g;
}

__device__ __forceinline__ int partitions(int len, int P) { return len > 0 ? (len + P - 1) / P : 0; }

// Unit b of the list: its row group r and rank within it.  False past the end.
__device__ __forceinline__ bool find_cascade_unit(const CascadeArgs &a, int b, int &r_out,
                                                  int &rank_out) {
    const int lane = threadIdx.x & 63;
    const int R = a.NG + a.S;
    int base = 0;
    for (int c0 = 0; c0 < R; c0 += 64) {
        const int r = c0 + lane;
        int u = 0;
        if (r < R) {
            const RowGroup g = row_group(a, r);
            const int tiles = (g.members * a.G + 15) / 16;
            u = a.Hkv * tiles * partitions(g.k1 - g.k0, a.P);
        }
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
            r_out = c0 + first;
            rank_out = b - (base + __builtin_amdgcn_readlane(incl - u, first));
            return true;
        }
        base += total;
    }
    return false;
}

// One unit: keys [t0, t1) of the row group against one 16-row column tile of
// one kv head.  Lane l = 16 j + n; column n is row ct * 16 + n of the group
// (member n' / G, query head n' % G of kv head g).  The block loop is the
// decode kernel's: S^T = K . Q^T on 16x16x32, the weights as hi + lo 16-bit
// parts into two 16x16x16 products per output tile, one block requested
// ahead through per-tile buffer descriptors.
template <int DT, int D>
__device__ __forceinline__ void cascade_unit(const CascadeArgs &a, int r, int rank) {
    constexpr int NKC = D / 32;
    constexpr int NVT = D / 16;
    constexpr int TILE = D * kB * 2;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int j = lane >> 4;

    const RowGroup rg = row_group(a, r);
    const int rows = rg.members * a.G;
    const int tiles = (rows + 15) / 16;
    const int g = rank % a.Hkv;
    const int ct = (rank / a.Hkv) % tiles;
    const int p = rank / (a.Hkv * tiles);
    const int len = rg.k1 - rg.k0;
    const int per = blocks_per_partition(len, a.P);
    const int blk0 = rg.k0 / kB + p * per;  // k0 is a whole number of blocks
    const int t0 = blk0 * kB;
    const int t1 = min(rg.k1, t0 + per * kB);
    const int nblk = (t1 - t0 + kB - 1) / kB;  // 1..64
    // the prefix is read through its first member's table
    int my_bt = blk0 + lane < a.MB ? a.bt[(int64_t)rg.seq0 * a.MB + blk0 + lane] : 0;
    if (lane >= nblk || my_bt < 0 || (int64_t)my_bt >= a.NB) my_bt = 0;

    const int R = ct * 16 + n;
    const bool col_ok = R < rows;
    const int m_idx = col_ok ? R / a.G : 0;
    const int hl = col_ok ? R - m_idx * a.G : 0;
    const int seq = rg.seq0 + m_idx;
    const int h = g * a.G + hl;
    const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)seq * a.Hq + h) * D;
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
            const float bm = xor32_max(xor16_max(lm)) * cs;
            const bool grow = bm > m + 8.f;
            const float mn = grow ? bm : m;
            const float alpha = fast_exp2(m - mn);
#pragma unroll
            for (int t = 0; t < NVT; ++t) o[t] *= alpha;
            l *= alpha;
            m = mn;
        }
        const float nm = -m;
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[e] = fast_exp2(fmaf(sc[e], cs, nm));
        if (tail) {
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
        const uint32_t h0 = pack2<DT>(pe[0], pe[1]);
        const uint32_t h1 = pack2<DT>(pe[2], pe[3]);
        const uint32_t l0 = pack2<DT>(pe[0] - elem_lo<DT>(h0), pe[1] - elem_hi<DT>(h0));
        const uint32_t l1 = pack2<DT>(pe[2] - elem_lo<DT>(h1), pe[3] - elem_hi<DT>(h1));
        const i32x2 phi = {(int)h0, (int)h1}, plo = {(int)l0, (int)l1};
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            o[t] = mfma16<DT>(x.v[t], phi, o[t]);
            o[t] = mfma16<DT>(x.v[t], plo, o[t]);
        }
    };

    load(b0, 0);
    int i = 0;
    for (; i + 2 <= nblk; i += 2) {
        step(b0, b1, i);
        step(b1, b0, i + 1);
    }
    if (i < nblk) step(b0, b1, i);

    const float lt = xor32_sum(xor16_sum(l));  // all lanes take part in the swaps
    if (!col_ok) return;
    // prefix partitions take slots 0 .. NPP-1 of the row, suffix ones NPP ..
    const int slot = (r < a.NG ? 0 : a.NPP) + p;
    const int64_t part = ((int64_t)seq * a.Hq + h) * a.NPT + slot;
    float *po = a.part_o + part * D;
#pragma unroll
    for (int t = 0; t < NVT; ++t) *(f32x4 *)(po + 16 * t + 4 * j) = o[t];
    if (j == 0) *(float2 *)(a.part_ml + 2 * part) = float2{m, lt};
}

template <int DT, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8)))
void cascade_kernel(const CascadeArgs a) {
    // Rounds of gridDim.x units, in alternating directions: the list holds
    // the (longer) prefix units first, so a wave that took a prefix unit in
    // one round takes one of the last units of the next.
    for (int round = 0;; ++round) {
        const int b = round * gridDim.x + ((round & 1) ? gridDim.x - 1 - blockIdx.x : blockIdx.x);
        int r, rank;
        if (!find_cascade_unit(a, b, r, rank)) return;
        cascade_unit<DT, D>(a, r, rank);
    }
}

// Merge of one query row's partial states: its group's prefix partitions and
// its own suffix partitions, with log-sum-exp weights; D/4 lanes per row, four
// dims each.  A row with no keys (empty context) gets zeros.
constexpr int kMergeThreads = 128;

template <int DT, int D>
__global__ __launch_bounds__(kMergeThreads) void cascade_merge_kernel(const CascadeArgs a) {
    constexpr int LPR = D / 4;
    const int row = blockIdx.x * (kMergeThreads / LPR) + threadIdx.x / LPR;
    const int d4 = (threadIdx.x % LPR) * 4;
    if (row >= a.S * a.Hq) return;
    const int s = row / a.Hq;
    const int gi = group_of(a.gs, a.NG, s);
    const int pb = min(max(a.pblk[gi], 0), a.MB);
    const int ctx = clamp_ctx(a.ctx[s], a.MB * kB);
    const int npp = partitions(pb * kB, a.P);  // the group has a member: this row
    const int nsp = partitions(max(ctx, pb * kB) - pb * kB, a.P);
    const int64_t base = (int64_t)row * a.NPT;
    float M = -INFINITY, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < npp + nsp; ++k) {
        const int slot = k < npp ? k : a.NPP + (k - npp);
        const float2 ml = *(const float2 *)(a.part_ml + 2 * (base + slot));
        const f32x4 ov = *(const f32x4 *)(a.part_o + (base + slot) * D + d4);
        const float Mn = fmaxf(M, ml.x);
        const float wo = fast_exp2(M - Mn);   // 0 on the first partial (M = -inf)
        const float wn = fast_exp2(ml.x - Mn);
        acc = acc * wo + ov * wn;
        L = L * wo + ml.y * wn;
        M = Mn;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    store4<DT>((uint16_t *)a.out + (int64_t)row * D + d4, acc, inv);
}

template <int DT>
hipError_t launch_typed(const CascadeArgs &a, int head_dim, int grid, hipStream_t stream) {
    const int rows_per_block = kMergeThreads / (head_dim / 4);
    const int mgrid = (a.S * a.Hq + rows_per_block - 1) / rows_per_block;
    if (head_dim == 128) {
        cascade_kernel<DT, 128><<<grid, 64, 0, stream>>>(a);
        cascade_merge_kernel<DT, 128><<<mgrid, kMergeThreads, 0, stream>>>(a);
    } else {
        cascade_kernel<DT, 64><<<grid, 64, 0, stream>>>(a);
        cascade_merge_kernel<DT, 64><<<mgrid, kMergeThreads, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_cascade(const CascadeArgs &a, int dtype, int head_dim, int grid,
                          hipStream_t stream) {
    if (a.S == 0) return hipSuccess;
    return dtype == kBF16 ? launch_typed<kBF16>(a, head_dim, grid, stream)
                          : launch_typed<kF16>(a, head_dim, grid, stream);
}

}  // namespace pa
