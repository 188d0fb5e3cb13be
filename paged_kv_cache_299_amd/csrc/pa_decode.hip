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
// Work unit = (partition p of P tokens, kv head or query head, sequence), one
// wave64 per unit.  A sequence longer than P is cut into partitions; each
// writes (m, l, unnormalised o) and merge_kernel recombines the partitions with
// log-sum-exp weights -- the streaming softmax is associative, so the split
// only changes rounding.  A sequence that fits one partition is normalised and
// written by its single unit directly.
//
// Two partition kernels:
//  * decode_mfma_kernel (bf16/fp16, 2..16 query heads per kv head): the G
//    query heads of one kv head form a small dense contraction.  Per block of
//    16 tokens: S^T[16 tok x 16 heads] = K[16 x D] . Q^T on
//    v_mfma_f32_16x16x32 (heads padded to 16); per pair of blocks:
//    O^T[D x 16] += V^T[D x 32 tok] . P^T, again on v_mfma_f32_16x16x32, with
//    P split into a high and a low 16-bit part so the weights keep ~16
//    significant bits.
//  * decode_valu_kernel (one query head per unit; fp32, or G == 1): dot
//    products with v_dot2 / FMA on 16-byte loads, cross-lane reductions, and
//    P.V with the 16 weights broadcast through SGPRs.
// Both read each (block, kv head) tile of K and of V exactly once per unit,
// as 16-byte (K) and 8/16-byte (V) loads that cover the tile in order.  One
// register set holds a block: the next block's K is requested as soon as the
// scores have consumed K, its V as soon as P.V has consumed V, so every wave
// keeps about one block in flight, and the register budget allows three (MFMA
// kernel) or four (VALU kernel) waves per SIMD, so that all units of a decode
// step are resident at once.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kB = 16;  // tokens per block (the only block size these kernels take)

// ---------------------------------------------------------------------------
// MFMA helper: D = A . B + C on v_mfma_f32_16x16x32 (bf16 or f16).  Lane l
// supplies A[l % 16][8 (l / 16) .. +8] and B[8 (l / 16) .. +8][l % 16] and
// receives D[4 (l / 16) .. +4][l % 16] (checked on the hardware).
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ f32x4 mfma32(const i32x4 &a, const i32x4 &b, const f32x4 &c) {
    if constexpr (DT == kBF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

template <int DT> __device__ __forceinline__ float from_bits16(uint32_t b) {
    return DT == kBF16 ? bf16_lo(b) : f16_lo(b);
}

// Store 4 consecutive outputs (fp32 values times `mul`) in the output type.
template <int DT> __device__ __forceinline__ void store4(void *dst, const f32x4 &v, float mul) {
    if constexpr (DT == kF32) {
        *(f32x4 *)dst = v * mul;
    } else {
        const uint32_t a = to_bits16<DT>(v[0] * mul) | ((uint32_t)to_bits16<DT>(v[1] * mul) << 16);
        const uint32_t b = to_bits16<DT>(v[2] * mul) | ((uint32_t)to_bits16<DT>(v[3] * mul) << 16);
        *(i32x2 *)dst = i32x2{(int)a, (int)b};
    }
}

template <int DT> __device__ __forceinline__ void store1(void *dst, float v) {
    if constexpr (DT == kF32) {
        *(float *)dst = v;
    } else {
        *(uint16_t *)dst = to_bits16<DT>(v);
    }
}

// Placed right after a prefetch.  The empty asm (no instruction) keeps the
// optimiser from merging the loads of the loop's first block with those of
// the next-block prefetch into one load at the loop head; the scheduling
// barrier keeps the instruction scheduler from sinking the prefetch below the
// reduction of the current block.  Without them no block would be in flight
// while the current one is reduced.
__device__ __forceinline__ void issue_point() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Clamp a context length read from the device to what the block table holds.
__device__ __forceinline__ int clamp_ctx(int c, int cap) { return c < 0 ? 0 : (c > cap ? cap : c); }

// ---------------------------------------------------------------------------
// GQA partition kernel on MFMA.
//
// Lane l = 16 j + n.  In the QK product lane l supplies K[token n][8 dims of
// run 4c + j] (one 16-byte load of the [D/8][16][8] K tile: instruction c of
// the wave reads bytes [1024 c, 1024 c + 1024) of the tile) and
// Q^T[same dims][head n]; it gets back the scores of tokens 4j..4j+3 for
// query head n of the group.  Those four scores are exactly the B operand it
// supplies to the P.V product, whose A operand is V^T[dim 16t + n][tokens
// 4j..4j+3] (8 bytes of the [D][16] V tile), and whose result O^T[dims 16t +
// 4j..4j+3][head n] stays in the lane across blocks.
// ---------------------------------------------------------------------------
template <int DT, int D, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 8)))
void decode_mfma_kernel(const DecodeArgs a) {
    static_assert(DT == kBF16 || DT == kF16, "MFMA path takes 16-bit data");
    static_assert(D % 32 == 0, "head_dim must be a multiple of 32");
    constexpr int NKC = D / 32;       // QK steps, 32 dims each
    constexpr int NVT = D / 16;       // P.V output tiles, 16 dims each
    constexpr int TILE = D * kB * 2;  // bytes of one (block, kv head) tile

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;  // wave of the unit: it takes block pairs wv, wv + W, ...
    const int n = lane & 15;
    const int j = lane >> 4;

    // Unit order (partition, sequence, kv head), head fastest: workgroup b runs
    // on XCD b % 8, so with a multiple of 8 kv heads every XCD gets one head of
    // every (sequence, partition) and the same share of work whatever the
    // context lengths (sequence-fastest order tied each XCD to fixed sequences).
    int u = xcd_unit(blockIdx.x, a.run);
    if (u >= a.num_units) return;
    const int g = u % a.Hkv;
    u /= a.Hkv;
    const int s = u % a.S;
    const int p = u / a.S;

    const int t0 = p * a.P;
    const int blk0 = t0 / kB;
    // The table slice of this partition does not depend on the context length:
    // request it together with ctx (one round trip instead of two).
    int my_bt = blk0 + lane < a.MB ? a.bt[(int64_t)s * a.MB + blk0 + lane] : 0;
    const int ctx = clamp_ctx(a.ctx[s], a.MB * kB);
    const bool head_ok = n < a.G;
    const int h = g * a.G + (head_ok ? n : 0);
    uint16_t *outp = (uint16_t *)a.out + ((int64_t)s * a.Hq + h) * D;
    if (t0 >= ctx) {
        if (p == 0 && head_ok) {  // empty context: the output is zero
#pragma unroll
            for (int t = 0; t < NVT; ++t) *(i32x2 *)(outp + 16 * t + 4 * j) = i32x2{0, 0};
        }
        return;
    }
    const int t1 = min(ctx, t0 + a.P);
    const int nblk = (t1 - t0 + kB - 1) / kB;  // 1..64
    // entries past the context are never used; out-of-range ids are clamped so
    // that no read leaves the pool
    if (lane >= nblk || my_bt < 0 || (int64_t)my_bt >= a.NB) my_bt = 0;

    const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)s * a.Hq + h) * D;
    i32x4 qf[NKC];
#pragma unroll
    for (int c = 0; c < NKC; ++c)
        qf[c] = head_ok ? ld16(qrow + (4 * c + j) * 8) : i32x4{0, 0, 0, 0};

    const char *kbase = (const char *)a.k + (int64_t)g * TILE;
    const char *vbase = (const char *)a.v + (int64_t)g * TILE;
    const int64_t blk_stride = (int64_t)a.Hkv * TILE;

    float m = -INFINITY;
    float l = 0.f;
    f32x4 o[NVT];
#pragma unroll
    for (int t = 0; t < NVT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // K operand slices of a pair of blocks, and V operand slices of a pair.
    struct KRegs {
        i32x4 a[NKC], b[NKC];
    };
    struct VRegs {
        i32x2 a[NVT], b[NVT];
    };
    KRegs kr;
    VRegs v0, v1;

    // Valid tokens of block b of the unit (16 except in its last block).
    auto valid = [&](int b) {
        const int v = t1 - (t0 + b * kB);
        return v < 0 ? 0 : (v > kB ? kB : v);
    };
    // Second block of pair q; an absent one (odd block count) re-reads the
    // first block's tile and is masked out, so every pair issues the same loads.
    auto second = [&](int q) { return min(2 * q + 1, nblk - 1); };

    auto load_k = [&](int q) {
        const char *ka = kbase + (int64_t)__builtin_amdgcn_readlane(my_bt, 2 * q) * blk_stride;
        const char *kb = kbase + (int64_t)__builtin_amdgcn_readlane(my_bt, second(q)) * blk_stride;
#pragma unroll
        for (int c = 0; c < NKC; ++c) kr.a[c] = ld16_stream(ka + (64 * c + lane) * 16);
#pragma unroll
        for (int c = 0; c < NKC; ++c) kr.b[c] = ld16_stream(kb + (64 * c + lane) * 16);
        issue_point();
    };
    auto load_v = [&](VRegs &r, int q) {
        const char *va = vbase + (int64_t)__builtin_amdgcn_readlane(my_bt, 2 * q) * blk_stride;
        const char *vb = vbase + (int64_t)__builtin_amdgcn_readlane(my_bt, second(q)) * blk_stride;
#pragma unroll
        for (int t = 0; t < NVT; ++t) r.a[t] = ld8_stream(va + ((16 * t + n) * kB + 4 * j) * 2);
#pragma unroll
        for (int t = 0; t < NVT; ++t) r.b[t] = ld8_stream(vb + ((16 * t + n) * kB + 4 * j) * 2);
        issue_point();
    };
    // Scores of both blocks of the pair in kr.
    auto scores = [&](f32x4 &sa, f32x4 &sb) {
        sa = f32x4{0.f, 0.f, 0.f, 0.f};
        sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
            sa = mfma32<DT>(kr.a[c], qf[c], sa);
            sb = mfma32<DT>(kr.b[c], qf[c], sb);
        }
    };
    // Mask of the 16-bit V elements of tokens 4j..4j+3 that are valid (< nv).
    auto vmask = [&](int nv, uint32_t &m0, uint32_t &m1) {
        m0 = (4 * j + 0 < nv ? 0x0000ffffu : 0u) | (4 * j + 1 < nv ? 0xffff0000u : 0u);
        m1 = (4 * j + 2 < nv ? 0x0000ffffu : 0u) | (4 * j + 3 < nv ? 0xffff0000u : 0u);
    };
    // One online-softmax step over a pair of blocks A (nva valid tokens) and B
    // (nvb valid).  P.V runs on v_mfma_f32_16x16x32: lane group j supplies the
    // k-slots 8j..8j+7 = tokens 4j..4j+3 of A, then of B, which is both how its
    // two 8-byte V slices concatenate and how its two sets of four scores do.
    // Empty slots (only in the unit's last pair) are masked: score -inf, V
    // zeroed (they may hold NaN).
    //
    // The reference maximum m moves only when a lane's block maximum exceeds it
    // by more than 8 (a factor 2^8): weights exp2(s - m) then stay <= 256, and
    // the rescale of O and l by exp2(m_old - m_new) is skipped for most steps.
    auto update2 = [&](const VRegs &V, const f32x4 &sa, const f32x4 &sb, int nva, int nvb,
                       bool mask) {
        float sv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sv[e] = (!mask || 4 * j + e < nva) ? sa[e] * a.scale_log2 : -INFINITY;
            sv[4 + e] = (!mask || 4 * j + e < nvb) ? sb[e] * a.scale_log2 : -INFINITY;
        }
        float bm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        bm = xor32_max(xor16_max(bm));
        const bool grow = bm > m + 8.f;
        if (__any(grow)) {
            const float mn = grow ? bm : m;
            const float alpha = fast_exp2(m - mn);  // 0 on the first step (m = -inf)
#pragma unroll
            for (int t = 0; t < NVT; ++t) o[t] *= alpha;
            l *= alpha;
            m = mn;
        }
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(sv[e] - m);
        l += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
        // P = hi + lo, both 16-bit: hi = RNE(p), lo = RNE(p - hi).
        uint32_t hb[8], lb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            hb[e] = to_bits16<DT>(pe[e]);
            lb[e] = to_bits16<DT>(pe[e] - from_bits16<DT>(hb[e]));
        }
        const i32x4 phi = {(int)(hb[0] | (hb[1] << 16)), (int)(hb[2] | (hb[3] << 16)),
                           (int)(hb[4] | (hb[5] << 16)), (int)(hb[6] | (hb[7] << 16))};
        const i32x4 plo = {(int)(lb[0] | (lb[1] << 16)), (int)(lb[2] | (lb[3] << 16)),
                           (int)(lb[4] | (lb[5] << 16)), (int)(lb[6] | (lb[7] << 16))};
        uint32_t ma0 = 0xffffffffu, ma1 = 0xffffffffu, mb0 = 0xffffffffu, mb1 = 0xffffffffu;
        if (mask) {
            vmask(nva, ma0, ma1);
            vmask(nvb, mb0, mb1);
        }
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            const i32x4 vv = {(int)((uint32_t)V.a[t][0] & ma0), (int)((uint32_t)V.a[t][1] & ma1),
                              (int)((uint32_t)V.b[t][0] & mb0), (int)((uint32_t)V.b[t][1] & mb1)};
            o[t] = mfma32<DT>(vv, phi, o[t]);
            o[t] = mfma32<DT>(vv, plo, o[t]);
        }
    };
    auto last_step = [&](const VRegs &V, int q) {
        f32x4 sa, sb;
        scores(sa, sb);
        update2(V, sa, sb, valid(2 * q), 2 * q + 1 < nblk ? valid(2 * q + 1) : 0, true);
    };

    // Pairs of this wave: q = wv, wv + W, ...  One K register set and two V
    // sets: right after the scores of pair q consume K, both K and V of the
    // wave's next pair are requested (V into the other set), so a whole pair
    // is in flight while pair q is reduced.  The loop is unrolled by two so the
    // V sets alternate without copies, and issues its loads without conditions
    // so the wait counts stay exact; the wave's last pair is masked.
    const int npairs = (nblk + 1) / 2;
    const int nk = npairs > wv ? (npairs - wv + W - 1) / W : 0;  // pairs of this wave
    if (nk > 0) {
        int q = wv;
        int k = 0;
        load_k(q);
        load_v(v0, q);
        for (; k + 2 < nk; k += 2, q += 2 * W) {  // pairs q, q + W full; q + 2W exists
            f32x4 sa, sb;
            scores(sa, sb);
            load_k(q + W);
            load_v(v1, q + W);
            update2(v0, sa, sb, kB, kB, false);
            scores(sa, sb);
            load_k(q + 2 * W);
            load_v(v0, q + 2 * W);
            update2(v1, sa, sb, kB, kB, false);
        }
        if (nk - k == 2) {
            f32x4 sa, sb;
            scores(sa, sb);
            load_k(q + W);
            load_v(v1, q + W);
            update2(v0, sa, sb, kB, kB, false);
            last_step(v1, q + W);
        } else {
            last_step(v0, q);
        }
    }

    if constexpr (W > 1) {
        // Combine the W running states of the unit in wave 0 (same lane layout
        // in every wave): M = max m_w, weights exp2(m_w - M).
        __shared__ float sh_o[W - 1][NVT * 4][64];
        __shared__ float sh_m[W - 1][64];
        __shared__ float sh_l[W - 1][64];
        if (wv > 0) {
#pragma unroll
            for (int t = 0; t < NVT; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) sh_o[wv - 1][4 * t + e][lane] = o[t][e];
            sh_m[wv - 1][lane] = m;
            sh_l[wv - 1][lane] = l;
        }
        __syncthreads();
        if (wv > 0) return;
#pragma unroll
        for (int w = 0; w < W - 1; ++w) {
            const float m2 = sh_m[w][lane];
            const float mn = fmaxf(m, m2);  // finite: wave 0 always has pair 0
            const float ca = fast_exp2(m - mn), cb = fast_exp2(m2 - mn);
            l = l * ca + sh_l[w][lane] * cb;
#pragma unroll
            for (int t = 0; t < NVT; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) o[t][e] = o[t][e] * ca + sh_o[w][4 * t + e][lane] * cb;
            m = mn;
        }
    }

    const float lt = xor32_sum(xor16_sum(l));
    if (t0 == 0 && t1 == ctx) {
        if (!head_ok) return;
        const float inv = 1.f / lt;
#pragma unroll
        for (int t = 0; t < NVT; ++t) store4<DT>(outp + 16 * t + 4 * j, o[t], inv);
        return;
    }
    const int64_t part = ((int64_t)s * a.Hq + h) * a.NP + p;
    if (head_ok) {
        float *po = a.part_o + part * D;
#pragma unroll
        for (int t = 0; t < NVT; ++t) *(f32x4 *)(po + 16 * t + 4 * j) = o[t];
        if (j == 0) {
            a.part_ml[2 * part] = m;
            a.part_ml[2 * part + 1] = lt;
        }
    }
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

template <int DT, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4, 8)))
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

    // Unit order (partition, sequence, query head), head fastest (see the MFMA
    // kernel).  With a multiple of 8 heads, head h of every sequence runs on
    // XCD h % 8, so sequences that share prefix blocks share that XCD's L2.
    int u = xcd_unit(blockIdx.x, a.run);
    if (u >= a.num_units) return;
    const int h = u % a.Hq;
    u /= a.Hq;
    const int s = u % a.S;
    const int p = u / a.S;
    const int g = h / a.G;

    const int t0 = p * a.P;
    const int blk0 = t0 / kB;
    int my_bt = blk0 + lane < a.MB ? a.bt[(int64_t)s * a.MB + blk0 + lane] : 0;
    const int ctx = clamp_ctx(a.ctx[s], a.MB * kB);
    char *outp = (char *)a.out + ((int64_t)s * a.Hq + h) * D * E;
    if (t0 >= ctx) {
        if (p == 0) {
#pragma unroll
            for (int w = 0; w < DPL; ++w) store1<DT>(outp + (lane + 64 * w) * E, 0.f);
        }
        return;
    }
    const int t1 = min(ctx, t0 + a.P);
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
// Log-sum-exp merge of the partitions of one (sequence, query head).
// 256 threads = PG partition lanes x D/4 four-dim groups.  Each thread merges
// partitions pg, pg + PG, ... of its four dims with a running log-sum-exp
//   M' = max(M, m_q),  L' = L e^(M-M') + l_q e^(m_q-M'),  o' likewise,
// so the loads of all its partitions are independent and go out together;
// the PG running states are then combined the same way through LDS.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void merge_kernel(const DecodeArgs a) {
    constexpr int E = Elem<DT>::bytes;
    constexpr int DQ = D / 4;        // four-dim groups
    constexpr int PG = 256 / DQ;     // partition lanes
    const int tid = threadIdx.x;
    const int dq = tid % DQ;
    const int pg = tid / DQ;
    const int sh = blockIdx.x;       // s * Hq + h
    const int s = sh / a.Hq;
    const int ctx = clamp_ctx(a.ctx[s], a.MB * kB);
    const int np = (ctx + a.P - 1) / a.P;
    if (np <= 1) return;  // written by the partition kernel

    __shared__ f32x4 o_sh[PG][DQ];
    __shared__ float m_sh[PG][DQ];
    __shared__ float l_sh[PG][DQ];

    const float *pml = a.part_ml + (int64_t)sh * a.NP * 2;
    const float *po = a.part_o + (int64_t)sh * a.NP * D + dq * 4;
    float M = -INFINITY, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int q = pg; q < np; q += PG) {
        const float mq = pml[2 * q];
        const float lq = pml[2 * q + 1];
        const f32x4 oq = *(const f32x4 *)(po + (int64_t)q * D);
        const float Mn = fmaxf(M, mq);
        const float ca = fast_exp2(M - Mn), cb = fast_exp2(mq - Mn);
        L = L * ca + lq * cb;
        acc = acc * ca + oq * cb;
        M = Mn;
    }
    o_sh[pg][dq] = acc;
    m_sh[pg][dq] = M;
    l_sh[pg][dq] = L;
    __syncthreads();
    if (pg == 0) {
        float Mt = m_sh[0][dq];
        for (int r = 1; r < PG; ++r) Mt = fmaxf(Mt, m_sh[r][dq]);
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
        for (int r = 0; r < PG; ++r) {
            // a lane that got no partition holds M = -inf, L = 0, o = 0
            const float w = fast_exp2(m_sh[r][dq] - Mt);
            lsum += l_sh[r][dq] * w;
            sum += o_sh[r][dq] * w;
        }
        store4<DT>((char *)a.out + ((int64_t)sh * D + dq * 4) * E, sum, 1.f / lsum);
    }
}

// ---------------------------------------------------------------------------
template <int DT, int D>
static hipError_t launch_typed(const DecodeArgs &a, DecodeKernel kind, hipStream_t stream) {
    const int per = 8 * a.run;
    const int grid = (a.num_units + per - 1) / per * per;
    if (grid > 0) {
        if constexpr (DT != kF32) {
            if (kind == DecodeKernel::kMfma) {
                switch (a.waves_per_unit) {
                case 4:
                    decode_mfma_kernel<DT, D, 4><<<dim3(grid), dim3(256), 0, stream>>>(a);
                    break;
                case 2:
                    decode_mfma_kernel<DT, D, 2><<<dim3(grid), dim3(128), 0, stream>>>(a);
                    break;
                default:
                    decode_mfma_kernel<DT, D, 1><<<dim3(grid), dim3(64), 0, stream>>>(a);
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
    if (a.NP > 1 && a.S > 0) {
        merge_kernel<DT, D><<<dim3(a.S * a.Hq), dim3(256), 0, stream>>>(a);
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

}  // namespace pa
