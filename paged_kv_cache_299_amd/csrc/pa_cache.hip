// pa_cache.hip -- KV-pool maintenance kernels: slot scatter and block copy.
//
// Both are plain byte movers: the new tokens' K/V go to their slots
// (slot = physical block * B + offset) and copy-on-write copies whole physical
// blocks.  [論文解説: PagedAttention, 技術的詳細 › PagedAttentionアルゴリズム
// (block table) and › Copy-on-Write KVキャッシュ共有]
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// One thread per (token, kv head, 16-byte run of the head vector).  The K run
// of x dims lands as one 16-byte store in the [D/x][B][x] tile; the same run
// of V is x separate elements, one per dim row of the [D][B] tile.
template <int E>
__global__ __launch_bounds__(256) void write_kv_kernel(const char *__restrict__ k_new,
                                                       const char *__restrict__ v_new,
                                                       char *__restrict__ k_cache,
                                                       char *__restrict__ v_cache,
                                                       const int64_t *__restrict__ slots,
                                                       int64_t num_tokens, int Hkv, int D, int B,
                                                       int64_t num_slots) {
    constexpr int X = 16 / E;
    const int NC = D / X;
    const int64_t total = num_tokens * Hkv * NC;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % NC);
        const int64_t rest = idx / NC;
        const int g = (int)(rest % Hkv);
        const int64_t t = rest / Hkv;
        const int64_t slot = slots[t];
        if (slot < 0 || slot >= num_slots) continue;  // padding, or out of range
        const int64_t blk = slot / B;
        const int off = (int)(slot % B);
        const int64_t src = ((t * Hkv + g) * D) * E + (int64_t)c * 16;
        const int64_t tile = (blk * Hkv + g) * (int64_t)D * B;  // elements
        const i32x4 kv = ld16(k_new + src);
        *(i32x4 *)(k_cache + (tile + ((int64_t)c * B + off) * X) * E) = kv;
        const i32x4 vv = ld16(v_new + src);
        const char *vb = (const char *)&vv;
#pragma unroll
        for (int e = 0; e < X; ++e) {
            char *dst = v_cache + (tile + (int64_t)(c * X + e) * B + off) * E;
            if constexpr (E == 4) {
                *(uint32_t *)dst = *(const uint32_t *)(vb + 4 * e);
            } else {
                *(uint16_t *)dst = *(const uint16_t *)(vb + 2 * e);
            }
        }
    }
}

// grid.y walks the pairs, grid.x the 16-byte runs of one block of one pool.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char *__restrict__ k_cache,
                                                          char *__restrict__ v_cache,
                                                          const int64_t *__restrict__ pairs,
                                                          int64_t num_pairs, int64_t num_blocks,
                                                          int64_t block_bytes) {
    for (int64_t i = blockIdx.y; i < num_pairs; i += gridDim.y) {
        const int64_t src = pairs[2 * i];
        const int64_t dst = pairs[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
        const char *ks = k_cache + src * block_bytes;
        const char *vs = v_cache + src * block_bytes;
        char *kd = k_cache + dst * block_bytes;
        char *vd = v_cache + dst * block_bytes;
        for (int64_t off = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; off < block_bytes;
             off += (int64_t)gridDim.x * blockDim.x * 16) {
            const i32x4 a = ld16(ks + off);
            const i32x4 b = ld16(vs + off);
            *(i32x4 *)(kd + off) = a;
            *(i32x4 *)(vd + off) = b;
        }
    }
}

hipError_t launch_write_kv(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                           const int64_t *slots, int64_t T, int Hkv, int D, int B, int64_t NB,
                           int elem_bytes, hipStream_t stream) {
    const int X = 16 / elem_bytes;
    const int64_t total = T * Hkv * (D / X);
    if (total == 0) return hipSuccess;
    const int threads = 256;
    int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    if (elem_bytes == 4) {
        write_kv_kernel<4><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
            (const char *)k_new, (const char *)v_new, (char *)k_cache, (char *)v_cache, slots, T,
            Hkv, D, B, NB * B);
    } else {
        write_kv_kernel<2><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
            (const char *)k_new, (const char *)v_new, (char *)k_cache, (char *)v_cache, slots, T,
            Hkv, D, B, NB * B);
    }
    return hipGetLastError();
}

hipError_t launch_copy_blocks(void *k_cache, void *v_cache, const int64_t *pairs, int64_t n,
                              int64_t NB, int64_t block_bytes, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int threads = 256;
    int64_t runs = block_bytes / 16;
    int64_t gx = (runs + threads - 1) / threads;
    if (gx > 64) gx = 64;
    int64_t gy = n < 65535 ? n : 65535;
    copy_blocks_kernel<<<dim3((unsigned)gx, (unsigned)gy), dim3(threads), 0, stream>>>(
        (char *)k_cache, (char *)v_cache, pairs, n, NB, block_bytes);
    return hipGetLastError();
}

}  // namespace pa
