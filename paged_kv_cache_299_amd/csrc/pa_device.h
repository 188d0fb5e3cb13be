// pa_device.h -- device-side helpers shared by the libpa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Element type codes, same numbering as pa_dtype in include/pa.h.
enum : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Elem;
template <> struct Elem<kF32> { static constexpr int bytes = 4; };
template <> struct Elem<kF16> { static constexpr int bytes = 2; };
template <> struct Elem<kBF16> { static constexpr int bytes = 2; };

// ---- 16-bit <-> fp32 -----------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

template <int DT> __device__ __forceinline__ float elem_lo(uint32_t w) {
    return DT == kBF16 ? bf16_lo(w) : f16_lo(w);
}
template <int DT> __device__ __forceinline__ float elem_hi(uint32_t w) {
    return DT == kBF16 ? bf16_hi(w) : f16_hi(w);
}

// fp32 -> 16-bit bits, round to nearest even (NaN stays NaN).
template <int DT> __device__ __forceinline__ uint16_t to_bits16(float f) {
    if constexpr (DT == kBF16) {
        return __builtin_bit_cast(uint16_t, (__bf16)f);
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)f);
    }
}

// ---- cross-lane ------------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// Maximum / sum over the 16 lanes of a row (lanes 16r .. 16r+15), result in all of them.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, shfl_xor(v, 1));
    v = fmaxf(v, shfl_xor(v, 2));
    v = fmaxf(v, shfl_xor(v, 4));
    v = fmaxf(v, shfl_xor(v, 8));
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += shfl_xor(v, 1);
    v += shfl_xor(v, 2);
    v += shfl_xor(v, 4);
    v += shfl_xor(v, 8);
    return v;
}

// Reductions across lanes l and l ^ 16 (l ^ 32) with gfx950's row swaps: the
// pair the swap returns is {x_l, x_(l^16)} (resp. {x_l, x_(l^32)}) in some
// order, so max / sum of the pair is the reduction, with no LDS traffic.
__device__ __forceinline__ float xor16_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// IEEE maximum of four values: no quieting of operands the compiler cannot
// prove canonical (matrix-core results), and v_maximum3_f32 takes three at once.
__device__ __forceinline__ float max4f(float a, float b, float c, float d) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b),
                                         __builtin_elementwise_maximum(c, d));
}
__device__ __forceinline__ float xor32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Integer sum / maximum over the 64 lanes of a wave, returned in every lane:
// DPP butterflies within each row of 16 (quad swaps, then the mirrors of
// half-rows and rows), then the row swaps above.  Every lane of the wave must
// be active.
__device__ __forceinline__ int wave_sum_i32(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = (int)r[0] + (int)r[1];
    r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (int)r[0] + (int)r[1];
}
__device__ __forceinline__ int wave_max_i32(int v) {
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max((int)r[0], (int)r[1]);
    r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max((int)r[0], (int)r[1]);
}

// ---- loads -----------------------------------------------------------------
__device__ __forceinline__ i32x4 ld16(const void *p) { return *(const i32x4 *)p; }
__device__ __forceinline__ i32x2 ld8(const void *p) { return *(const i32x2 *)p; }
// Streaming loads for K/V tiles, each read once per decode: the nontemporal
// hint keeps them from displacing reusable lines (measured on MI355X: random
// 4 KiB tile reads go from ~5.7 to ~6.4 TB/s with it).
__device__ __forceinline__ i32x4 ld16_stream(const void *p) {
    return __builtin_nontemporal_load((const i32x4 *)p);
}
__device__ __forceinline__ i32x2 ld8_stream(const void *p) {
    return __builtin_nontemporal_load((const i32x2 *)p);
}

// Two fp32 values -> one word of two 16-bit values (round to nearest even),
// the first in the low half: one v_cvt_pk_* on gfx950.
template <int DT> __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    if constexpr (DT == kBF16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
    }
}

// ---- buffer loads ------------------------------------------------------------
// Loads through a buffer descriptor check every lane's offset against the
// descriptor's byte range: a lane outside it reads zeros and makes no memory
// request.  A descriptor over one K or V tile (range = tile bytes, or 0 for a
// block that does not exist) lets a kernel issue the loads of a block ahead
// without a branch: past the end they cost nothing and return zeros.
// Word 3 is the gfx9-family value: 32-bit data format (untyped loads need a
// non-zero format), no swizzle, no index stride.
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the K/V tile loads: nontemporal (each tile is read once per
// decode: it should not displace reusable lines), or plain, so that several
// sequences reading the same physical block (shared prefixes) hit in L2.
constexpr int kCachePolicyNT = 2;
constexpr int kCachePolicyPlain = 0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, bytes, kRsrcWord3);
}
template <int POLICY> __device__ __forceinline__ i32x4 bload16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
}
template <int POLICY> __device__ __forceinline__ i32x2 bload8(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POLICY));
}

// ---- shared by the attention kernels ---------------------------------------
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

// D = A . B + C on v_mfma_f32_16x16x16: lane l supplies A[l % 16][4 (l / 16) .. +4]
// and B[4 (l / 16) .. +4][l % 16] and receives D[4 (l / 16) .. +4][l % 16].
template <int DT> __device__ __forceinline__ f32x4 mfma16(const i32x2 &a, const i32x2 &b, const f32x4 &c) {
    if constexpr (DT == kBF16) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                         __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    }
}

// Clamp a context length read from the device to what the block table holds.
__device__ __forceinline__ int clamp_ctx(int c, int cap) { return c < 0 ? 0 : (c > cap ? cap : c); }

// ---------------------------------------------------------------------------
// A context of ctx tokens is cut into the fewest partitions of at most P
// tokens, ceil(ctx / P), all of the same number of whole blocks except a
// shorter last one (a 1100-token context at P = 1024 gives 2 x 35 blocks, not
// 64 + 5): the partitions of a sequence then take about the same time, and
// fewer units run at the full length P.  Returns the blocks per partition;
// every partition holds at least one token (ceil(nb / ceil(nb / n)) = n for
// n = ceil(nb / PB), the partition count the units are counted with).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int blocks_per_partition(int ctx, int P) {
    const int nb = (ctx + kB - 1) / kB;
    if (ctx <= P) return nb;
    const int n = (ctx + P - 1) / P;
    return (nb + n - 1) / n;
}

}  // namespace pa
