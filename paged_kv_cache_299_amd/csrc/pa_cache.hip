// pa_cache.hip -- KV-pool maintenance kernels: slot scatter and block copy.
//
// Both are plain byte movers: the new tokens' K/V go to their slots
// (slot = physical block * B + offset) and copy-on-write copies whole physical
// blocks.  [論文解説: PagedAttention, 技術的詳細 › PagedAttentionアルゴリズム
// (block table) and › Copy-on-Write KVキャッシュ共有]
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// A 256-thread workgroup stores a tile of TT consecutive tokens of one kv
// head, TT = 256 / (16-byte runs per head vector).  Workgroup b takes head
// b % Hkv of token tile b / Hkv: neighbouring workgroups read the adjacent
// head slices of the same tokens (one contiguous stretch of k_new / v_new)
// and fill the adjacent head tiles of the same blocks.  (With the head as the
// slow index, each pass over the tokens read 256 of every Hkv * 256 bytes,
// and a bulk write ran at 2.6 TB/s.)  Each thread loads one 16-byte run of K
// and of V.  The K run is one 16-byte store into the [D/x][B][x] tile.  V is
// transposed in the pool ([D][B] per tile), so the runs go through LDS and are
// stored element by element with the token as the fastest lane index: when
// consecutive tokens go to consecutive slots (prompt fill, appends) 16 lanes
// write one contiguous 16-slot row segment, which L2 merges into whole lines
// (storing aligned 8-token runs as 16-byte pieces instead measured no faster
// on a 290 MB bulk write and slower on one-token appends).
// A slot splits into (block, offset) once per token: a power-of-two block size
// (every layout the decode reads) takes a shift and a mask, any other size
// one 64-bit division.
__device__ inline void split_slot(int64_t slot, int B, int log2B, int64_t &blk, int &off) {
    if (log2B >= 0) {
        blk = slot >> log2B;
        off = (int)(slot & (B - 1));
    } else {
        blk = slot / B;
        off = (int)(slot - blk * B);
    }
}

template <int E>
__global__ __launch_bounds__(256) void write_kv_kernel(const char *__restrict__ k_new,
                                                       const char *__restrict__ v_new,
                                                       char *__restrict__ k_cache,
                                                       char *__restrict__ v_cache,
                                                       const int64_t *__restrict__ slots,
                                                       int64_t num_tokens, int Hkv, int D, int B,
                                                       int log2B, int64_t num_slots,
                                                       const int *__restrict__ mapped,
                                                       int req_stride, int num_req) {
    constexpr int X = 16 / E;
    // TT rows of D*E/4 words plus one pad word each: TT * D*E/4 <= 1024 and TT <= 256
    __shared__ uint32_t vtile[1024 + 256];
    // per token: element offset of its (block, kv head) tile plus its offset in
    // the block, or -1 for a token that is skipped
    __shared__ int64_t base_sh[256];
    const int NC = D / X;        // 16-byte runs per head vector (1..128)
    const int TT = 256 / NC;     // tokens per tile
    const int tid = threadIdx.x;
    const int g = (int)(blockIdx.x % (unsigned)Hkv);
    const int64_t t_base = (int64_t)(blockIdx.x / (unsigned)Hkv) * TT;
    // row stride in 32-bit words: one pad word, so that reading one dim of
    // consecutive tokens walks different LDS banks
    const int row_words = D * E / 4 + 1;

    // 1. loads: thread -> (token tt, run c)
    const int tt = tid / NC, c = tid % NC;
    const int64_t t = t_base + tt;
    int64_t slot = -1;
    i32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (tt < TT && t < num_tokens) {
        const int64_t src = ((t * Hkv + g) * D) * E + (int64_t)c * 16;
        slot = slots[t];
        kv = ld16(k_new + src);
        vv = ld16(v_new + src);
    }
    bool ok = slot >= 0 && slot < num_slots;
    if (ok && mapped) {  // virtual-memory storage: only positions with memory behind them
        const int64_t per_req = (int64_t)req_stride * B;
        const int64_t r = slot / per_req;
        ok = r < num_req && slot - r * per_req < mapped[r];
    }
    int64_t blk = 0;
    int off = 0;
    if (ok) split_slot(slot, B, log2B, blk, off);
    const int64_t tile = (blk * Hkv + g) * (int64_t)D * B;  // elements
    if (ok) *(i32x4 *)(k_cache + (tile + ((int64_t)c * B + off) * X) * E) = kv;
    if (tt < TT) {
        if (c == 0) base_sh[tt] = ok ? tile + off : -1;
        uint32_t *row = vtile + tt * row_words + c * 4;
        row[0] = (uint32_t)vv[0];
        row[1] = (uint32_t)vv[1];
        row[2] = (uint32_t)vv[2];
        row[3] = (uint32_t)vv[3];
    }
    __syncthreads();
    // 2. V stores: element e -> (token e % TT, dim e / TT)
    const int64_t tiles_left = num_tokens - t_base;
    const int ntok = tiles_left < TT ? (int)tiles_left : TT;
    for (int e = tid; e < TT * D; e += 256) {
        const int et = e % TT, d = e / TT;
        if (et >= ntok) continue;
        const int64_t base = base_sh[et];
        if (base < 0) continue;
        char *dst = v_cache + (base + (int64_t)d * B) * E;
        const char *src = (const char *)(vtile + et * row_words) + d * E;
        if constexpr (E == 4) {
            *(uint32_t *)dst = *(const uint32_t *)src;
        } else {
            *(uint16_t *)dst = *(const uint16_t *)src;
        }
    }
}

// Few tokens (a decode step): one wave takes 64 / NC tokens of one kv head,
// lane -> (token, 16-byte run), and stores its run's x V elements itself, x
// two-byte stores at a stride of one B-slot row, with no LDS round trip and
// no barrier.  The tokens of a decode step go to scattered slots, so the
// V stores could not merge in L2 anyway; more, smaller workgroups spread the
// stores over more compute units.
template <int E>
__global__ __launch_bounds__(64) void write_kv_few_kernel(const char *__restrict__ k_new,
                                                          const char *__restrict__ v_new,
                                                          char *__restrict__ k_cache,
                                                          char *__restrict__ v_cache,
                                                          const int64_t *__restrict__ slots,
                                                          int64_t num_tokens, int Hkv, int D,
                                                          int B, int log2B, int64_t num_slots,
                                                          const int *__restrict__ mapped,
                                                          int req_stride, int num_req) {
    constexpr int X = 16 / E;
    const int NC = D / X;      // 16-byte runs per head vector (1..64)
    const int TW = 64 / NC;    // tokens per wave
    const int lane = threadIdx.x;
    const int g = (int)(blockIdx.x % (unsigned)Hkv);
    const int tt = lane / NC, c = lane % NC;
    const int64_t t = (int64_t)(blockIdx.x / (unsigned)Hkv) * TW + tt;
    if (tt >= TW || t >= num_tokens) return;
    const int64_t src = ((t * Hkv + g) * D) * E + (int64_t)c * 16;
    const int64_t slot = slots[t];
    const i32x4 kv = ld16(k_new + src);
    const i32x4 vv = ld16(v_new + src);
    bool ok = slot >= 0 && slot < num_slots;
    if (ok && mapped) {
        const int64_t per_req = (int64_t)req_stride * B;
        const int64_t r = slot / per_req;
        ok = r < num_req && slot - r * per_req < mapped[r];
    }
    if (!ok) return;
    int64_t blk;
    int off;
    split_slot(slot, B, log2B, blk, off);
    const int64_t tile = (blk * Hkv + g) * (int64_t)D * B;  // elements
    *(i32x4 *)(k_cache + (tile + ((int64_t)c * B + off) * X) * E) = kv;
    char *vd = v_cache + (tile + (int64_t)c * X * B + off) * E;
    if constexpr (E == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) *(uint32_t *)(vd + (int64_t)e * B * 4) = (uint32_t)vv[e];
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = (uint32_t)vv[e >> 1];
            *(uint16_t *)(vd + (int64_t)e * B * 2) = (uint16_t)((e & 1) ? (w >> 16) : w);
        }
    }
}

// grid.y walks the pairs, grid.x the 16-byte runs of one block of one pool.
// Block src of the source pools goes to block dst of the destination pools.
// The pools may be the same allocations (copy-on-write: no destination is a
// source, so no byte is both read and written) or different ones (swapping
// between device memory and pinned host memory, which the kernel reads and
// writes directly over the host link, every pair in one launch).
__global__ __launch_bounds__(256) void copy_blocks_kernel(const char *__restrict__ src_k,
                                                          const char *__restrict__ src_v,
                                                          char *__restrict__ dst_k,
                                                          char *__restrict__ dst_v,
                                                          const int64_t *__restrict__ pairs,
                                                          int64_t num_pairs, int64_t src_blocks,
                                                          int64_t dst_blocks, int64_t block_bytes) {
    for (int64_t i = blockIdx.y; i < num_pairs; i += gridDim.y) {
        const int64_t src = pairs[2 * i];
        const int64_t dst = pairs[2 * i + 1];
        if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) continue;
        const char *ks = src_k + src * block_bytes;
        const char *vs = src_v + src * block_bytes;
        char *kd = dst_k + dst * block_bytes;
        char *vd = dst_v + dst * block_bytes;
        for (int64_t off = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; off < block_bytes;
             off += (int64_t)gridDim.x * blockDim.x * 16) {
            const i32x4 a = ld16(ks + off);
            const i32x4 b = ld16(vs + off);
            *(i32x4 *)(kd + off) = a;
            *(i32x4 *)(vd + off) = b;
        }
    }
}

// Up to this many tokens (a decode step's batch) take the one-wave kernel.
constexpr int64_t kFewTokens = 1024;

hipError_t launch_write_kv(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                           const int64_t *slots, int64_t T, int Hkv, int D, int B, int64_t NB,
                           int elem_bytes, hipStream_t stream, const int *mapped, int req_stride,
                           int num_req) {
    if (T == 0) return hipSuccess;
    const int NC = D * elem_bytes / 16;  // <= 64 (head_dim <= 512 at 2 bytes, 256 at 4)
    const int TT = 256 / NC;
    const int64_t tiles = (T + TT - 1) / TT;
    if (tiles * Hkv > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(tiles * Hkv));
    const int log2B = (B & (B - 1)) == 0 ? __builtin_ctz((unsigned)B) : -1;
    if (T <= kFewTokens && NC <= 64) {
        const int TW = 64 / NC;
        const dim3 fgrid((unsigned)(((T + TW - 1) / TW) * Hkv));
        if (elem_bytes == 4) {
            write_kv_few_kernel<4><<<fgrid, dim3(64), 0, stream>>>(
                (const char *)k_new, (const char *)v_new, (char *)k_cache, (char *)v_cache, slots,
                T, Hkv, D, B, log2B, NB * B, mapped, req_stride, num_req);
        } else {
            write_kv_few_kernel<2><<<fgrid, dim3(64), 0, stream>>>(
                (const char *)k_new, (const char *)v_new, (char *)k_cache, (char *)v_cache, slots,
                T, Hkv, D, B, log2B, NB * B, mapped, req_stride, num_req);
        }
        return hipGetLastError();
    }
    if (elem_bytes == 4) {
        write_kv_kernel<4><<<grid, dim3(256), 0, stream>>>(
            (const char *)k_new, (const char *)v_new, (char *)k_cache, (char *)v_cache, slots, T,
            Hkv, D, B, log2B, NB * B, mapped, req_stride, num_req);
    } else {
        write_kv_kernel<2><<<grid, dim3(256), 0, stream>>>(
            (const char *)k_new, (const char *)v_new, (char *)k_cache, (char *)v_cache, slots, T,
            Hkv, D, B, log2B, NB * B, mapped, req_stride, num_req);
    }
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                              const int64_t *pairs, int64_t n, int64_t src_blocks,
                              int64_t dst_blocks, int64_t block_bytes, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int threads = 256;
    int64_t runs = block_bytes / 16;
    int64_t gx = (runs + threads - 1) / threads;
    if (gx > 64) gx = 64;
    int64_t gy = n < 65535 ? n : 65535;
    copy_blocks_kernel<<<dim3((unsigned)gx, (unsigned)gy), dim3(threads), 0, stream>>>(
        (const char *)src_k, (const char *)src_v, (char *)dst_k, (char *)dst_v, pairs, n,
        src_blocks, dst_blocks, block_bytes);
    return hipGetLastError();
}

}  // namespace pa
