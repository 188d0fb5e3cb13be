/*
 * pa_oracle.c -- plain, slow CPU oracle for paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * never links, includes or calls it, and this file includes nothing from it.
 *
 * Everything here is computed in fp64 from the exact values of the stored
 * 16/32-bit inputs, in the most direct form of each definition:
 *
 *   oracle_decode             dense softmax attention of one query row over the
 *                             first ctx tokens of a sequence, the tokens being
 *                             fetched through the block table.
 *                             [論文解説: PagedAttention, 技術的詳細 ›
 *                              PagedAttentionアルゴリズム: block definition,
 *                              block table, decode equation]
 *   oracle_decode_partitioned the same quantity taken per run of P tokens as
 *                             (max, sum of exponentials, unnormalised output)
 *                             and recombined with log-sum-exp weights.  This is
 *                             the associativity of the streaming softmax named
 *                             in the same section ("online softmax,
 *                             FlashAttention style"), written out for whole
 *                             partitions.
 *   oracle_prefill            the queries of a chunk of new tokens, each over
 *                             the cached tokens up to its own position (causal),
 *                             fetched through the same block table.
 *                             [論文解説: PagedAttention, 実装のポイント ›
 *                              CUDAカーネル実装: one kernel for prefill and
 *                              decode]
 *   oracle_write_kv           scatter of new tokens' K/V into slots
 *                             (slot = physical block * B + offset).
 *   oracle_copy_blocks        copy of whole physical blocks, the copy step of
 *                             copy-on-write.  [論文解説: PagedAttention,
 *                             技術的詳細 › Copy-on-Write KVキャッシュ共有]
 *   oracle_swap_blocks        copy of whole blocks from one pair of pools to
 *                             another (device pools to a host pool and back),
 *                             the swapping the scheduler uses to preempt a
 *                             sequence.  [論文解説: PagedAttention,
 *                             実装のポイント › スケジューラ]
 *
 * Readings where the page is silent (each also listed in the design notes):
 *   - only tokens i < ctx contribute; the rest of the last block is ignored
 *     whatever bits it holds;
 *   - ctx == 0 gives an all-zero output;
 *   - prefill: the chunk's own K/V are in the pool before the call, the i-th
 *     of n queries sits at position ctx - n + i and sees positions up to its
 *     own (causal); q / out rows are packed per sequence (query_start);
 *   - query head h reads kv head h / (Hq / Hkv) (contiguous groups);
 *   - `scale` multiplies the dot products (the page fixes 1/sqrt(d));
 *   - write: slot < 0 means "skip"; non-negative slots must be distinct;
 *   - copy: every source is read before any destination is written;
 *     destinations must be distinct and must not be sources.
 *
 * Cache layout (the library's documented storage format, re-derived here):
 *   K pool: [NB][Hkv][D/x][B][x]  with x = k_x elements (x divides D)
 *           element (b, g, o, d) at (((b*Hkv + g)*(D/x) + d/x)*B + o)*x + d%x
 *   V pool: [NB][Hkv][D][B]
 *           element (b, g, o, d) at ((b*Hkv + g)*D + d)*B + o
 *   q, out: [S][Hq][D]; block_tables: int32 [S][MB]; context_lens int32 [S].
 *
 * Return codes: 0 on success, a negative value when a precondition is broken
 * (the oracle checks every precondition strictly; it is the reference).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

enum {
    OR_OK = 0,
    OR_BAD_DIMS = -1,
    OR_BAD_DTYPE = -2,
    OR_BAD_CTX = -3,
    OR_BAD_BLOCK = -4,
    OR_BAD_SLOT = -5,
    OR_DUP_SLOT = -6,
    OR_BAD_PAIR = -7,
    OR_NO_MEM = -8,
};

int oracle_elem_bytes(int dtype) {
    switch (dtype) {
    case OR_F32: return 4;
    case OR_F16: return 2;
    case OR_BF16: return 2;
    default: return 0;
    }
}

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/2^10) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int64_t idx, int dtype) {
    if (dtype == OR_F32) {
        float f;
        memcpy(&f, (const char *)base + idx * 4, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, (const char *)base + idx * 2, 2);
    return dtype == OR_F16 ? oracle_f16_to_double(h) : oracle_bf16_to_double(h);
}

static int64_t k_index(int64_t b, int64_t g, int64_t o, int64_t d, int64_t Hkv, int64_t D,
                       int64_t B, int64_t x) {
    return (((b * Hkv + g) * (D / x) + d / x) * B + o) * x + d % x;
}

static int64_t v_index(int64_t b, int64_t g, int64_t o, int64_t d, int64_t Hkv, int64_t D,
                       int64_t B) {
    return ((b * Hkv + g) * D + d) * B + o;
}

static int check_decode_args(const int32_t *block_tables, const int32_t *context_lens, int64_t S,
                             int64_t Hq, int64_t Hkv, int64_t D, int64_t B, int64_t MB, int64_t NB,
                             int64_t k_x, int dtype) {
    if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || B <= 0 || MB < 0 || NB < 0 || k_x <= 0)
        return OR_BAD_DIMS;
    if (Hq % Hkv != 0 || D % k_x != 0) return OR_BAD_DIMS;
    if (oracle_elem_bytes(dtype) == 0) return OR_BAD_DTYPE;
    for (int64_t s = 0; s < S; ++s) {
        int64_t n = context_lens[s];
        if (n < 0 || n > MB * B) return OR_BAD_CTX;
        int64_t used = (n + B - 1) / B; /* ceil(T / B) blocks hold T tokens */
        for (int64_t j = 0; j < used; ++j) {
            int64_t b = block_tables[s * MB + j];
            if (b < 0 || b >= NB) return OR_BAD_BLOCK;
        }
    }
    return OR_OK;
}

/* Position i of a sequence lives in logical block i / B at offset i % B;
 * the block table turns the logical block into a physical one. */
static int64_t phys_block(const int32_t *block_tables, int64_t s, int64_t MB, int64_t B,
                          int64_t i) {
    return block_tables[s * MB + i / B];
}

/* Dense softmax attention of query row (s, h) over tokens [t0, t1) of
 * sequence s.  Writes the unnormalised output sum_i w_i v_i with
 * w_i = exp(x_i - m), and returns m = max_i x_i and l = sum_i w_i.  For an
 * empty range m = -inf, l = 0 and the output is zero. */
static void attend_range(const void *q, int64_t qrow /* element offset of the row */,
                         const void *k_cache, const void *v_cache,
                         const int32_t *block_tables, double scale, int64_t s, int64_t h,
                         int64_t t0, int64_t t1, int64_t Hq, int64_t Hkv, int64_t D, int64_t B,
                         int64_t MB, int64_t k_x, int dtype, double *x /* scratch [t1-t0] */,
                         double *o /* [D] */, double *m_out, double *l_out) {
    int64_t G = Hq / Hkv;
    int64_t g = h / G;
    double m = -INFINITY;
    for (int64_t i = t0; i < t1; ++i) {
        int64_t b = phys_block(block_tables, s, MB, B, i);
        int64_t off = i % B;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += load_elem(q, qrow + d, dtype) *
                   load_elem(k_cache, k_index(b, g, off, d, Hkv, D, B, k_x), dtype);
        x[i - t0] = scale * dot;
        if (x[i - t0] > m) m = x[i - t0];
    }
    double l = 0.0;
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t i = t0; i < t1; ++i) {
        double w = exp(x[i - t0] - m);
        l += w;
        int64_t b = phys_block(block_tables, s, MB, B, i);
        int64_t off = i % B;
        for (int64_t d = 0; d < D; ++d)
            o[d] += w * load_elem(v_cache, v_index(b, g, off, d, Hkv, D, B), dtype);
    }
    *m_out = m;
    *l_out = l;
}

/* out[s][h][:] = sum_i softmax_i(scale * q.k_i) v_i over the first
 * context_lens[s] tokens of sequence s, in fp64. */
int oracle_decode(const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, const int32_t *context_lens, double scale,
                  double *out, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t B,
                  int64_t MB, int64_t NB, int64_t k_x, int dtype) {
    int rc = check_decode_args(block_tables, context_lens, S, Hq, Hkv, D, B, MB, NB, k_x, dtype);
    if (rc != OR_OK) return rc;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t sh = 0; sh < S * Hq; ++sh) {
        int64_t s = sh / Hq, h = sh % Hq;
        int64_t n = context_lens[s];
        double *dst = out + sh * D;
        if (n == 0) {
            for (int64_t d = 0; d < D; ++d) dst[d] = 0.0;
            continue;
        }
        double *x = (double *)malloc(sizeof(double) * (size_t)n);
        if (!x) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double m, l;
        attend_range(q, (s * Hq + h) * D, k_cache, v_cache, block_tables, scale, s, h, 0, n, Hq,
                     Hkv, D, B, MB, k_x,
                     dtype, x, dst, &m, &l);
        for (int64_t d = 0; d < D; ++d) dst[d] /= l;
        free(x);
    }
    return failed ? OR_NO_MEM : OR_OK;
}

/* Paged prefill: the queries of a chunk of new tokens attend causally over
 * the sequence's cached tokens.  Sequence s owns query rows
 * query_start[s] .. query_start[s+1]-1 of q and out ([T][Hq][D]); with
 * n = query_start[s+1] - query_start[s] <= ctx = context_lens[s], its i-th
 * query is the token at position ctx - n + i, whose K/V are already in the
 * pool, and it attends over positions 0 .. ctx - n + i (itself included):
 *   out[t][h] = sum_{j <= p} softmax_j(scale * q.k_j) v_j,  p = ctx - n + i.
 * n == ctx is a whole prompt, n < ctx a chunk after a cached prefix, n == 1
 * one decode step.  The same kernel serves both phases.
 * [論文解説: PagedAttention, 実装のポイント › CUDAカーネル実装; causal
 *  attention of the new tokens is the standard prefill the page names] */
int oracle_prefill(const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *block_tables, const int32_t *context_lens,
                   const int32_t *query_start, double scale, double *out, int64_t S, int64_t T,
                   int64_t Hq, int64_t Hkv, int64_t D, int64_t B, int64_t MB, int64_t NB,
                   int64_t k_x, int dtype) {
    int rc = check_decode_args(block_tables, context_lens, S, Hq, Hkv, D, B, MB, NB, k_x, dtype);
    if (rc != OR_OK) return rc;
    if (T < 0 || (S > 0 && query_start[0] != 0) || (S == 0 && T != 0)) return OR_BAD_DIMS;
    for (int64_t s = 0; s < S; ++s) {
        int64_t n = (int64_t)query_start[s + 1] - query_start[s];
        if (n < 0 || n > context_lens[s]) return OR_BAD_CTX;
    }
    if (S > 0 && query_start[S] != T) return OR_BAD_DIMS;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t th = 0; th < T * Hq; ++th) {
        int64_t t = th / Hq, h = th % Hq;
        int64_t s = 0;
        while (query_start[s + 1] <= t) ++s; /* the sequence that owns row t */
        int64_t n = (int64_t)query_start[s + 1] - query_start[s];
        int64_t p = context_lens[s] - n + (t - query_start[s]);
        double *dst = out + th * D;
        double *x = (double *)malloc(sizeof(double) * (size_t)(p + 1));
        if (!x) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double m, l;
        attend_range(q, th * D, k_cache, v_cache, block_tables, scale, s, h, 0, p + 1, Hq, Hkv,
                     D, B, MB, k_x, dtype, x, dst, &m, &l);
        for (int64_t d = 0; d < D; ++d) dst[d] /= l;
        free(x);
    }
    return failed ? OR_NO_MEM : OR_OK;
}

/* The same attention taken over runs of P tokens.  Run p covers tokens
 * [p*P, min((p+1)*P, ctx)) and yields (m_p, l_p, o_p); the runs are merged as
 *   M = max_p m_p,  w_p = exp(m_p - M),
 *   out = (sum_p w_p o_p) / (sum_p w_p l_p).
 * Optionally returns the per-run triples in part_m / part_l [S][Hq][NP] and
 * part_o [S][Hq][NP][D] with NP = ceil(MB*B / P) (runs past ctx are left as
 * m = -inf, l = 0, o = 0). */
int oracle_decode_partitioned(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *context_lens,
                              double scale, double *out, int64_t S, int64_t Hq, int64_t Hkv,
                              int64_t D, int64_t B, int64_t MB, int64_t NB, int64_t k_x, int dtype,
                              int64_t P, double *part_m, double *part_l, double *part_o) {
    int rc = check_decode_args(block_tables, context_lens, S, Hq, Hkv, D, B, MB, NB, k_x, dtype);
    if (rc != OR_OK) return rc;
    if (P <= 0) return OR_BAD_DIMS;
    int64_t NP = (MB * B + P - 1) / P;
    if (NP < 1) NP = 1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t sh = 0; sh < S * Hq; ++sh) {
        int64_t s = sh / Hq, h = sh % Hq;
        int64_t n = context_lens[s];
        int64_t np = (n + P - 1) / P;
        double *dst = out + sh * D;
        double *x = (double *)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1));
        double *ms = (double *)malloc(sizeof(double) * (size_t)NP);
        double *ls = (double *)malloc(sizeof(double) * (size_t)NP);
        double *os = (double *)malloc(sizeof(double) * (size_t)(NP * D));
        if (!x || !ms || !ls || !os) {
#pragma omp atomic write
            failed = 1;
            free(x); free(ms); free(ls); free(os);
            continue;
        }
        for (int64_t p = 0; p < NP; ++p) {
            ms[p] = -INFINITY;
            ls[p] = 0.0;
            for (int64_t d = 0; d < D; ++d) os[p * D + d] = 0.0;
        }
        for (int64_t p = 0; p < np; ++p) {
            int64_t t0 = p * P, t1 = t0 + P < n ? t0 + P : n;
            attend_range(q, (s * Hq + h) * D, k_cache, v_cache, block_tables, scale, s, h, t0, t1,
                         Hq, Hkv, D, B,
                         MB, k_x, dtype, x, os + p * D, &ms[p], &ls[p]);
        }
        if (part_m && part_l && part_o) {
            for (int64_t p = 0; p < NP; ++p) {
                part_m[sh * NP + p] = ms[p];
                part_l[sh * NP + p] = ls[p];
                for (int64_t d = 0; d < D; ++d) part_o[(sh * NP + p) * D + d] = os[p * D + d];
            }
        }
        if (np == 0) {
            for (int64_t d = 0; d < D; ++d) dst[d] = 0.0;
        } else {
            double M = -INFINITY;
            for (int64_t p = 0; p < np; ++p)
                if (ms[p] > M) M = ms[p];
            double L = 0.0;
            for (int64_t d = 0; d < D; ++d) dst[d] = 0.0;
            for (int64_t p = 0; p < np; ++p) {
                double w = exp(ms[p] - M);
                L += w * ls[p];
                for (int64_t d = 0; d < D; ++d) dst[d] += w * os[p * D + d];
            }
            for (int64_t d = 0; d < D; ++d) dst[d] /= L;
        }
        free(x); free(ms); free(ls); free(os);
    }
    return failed ? OR_NO_MEM : OR_OK;
}

/* For every t with slot_mapping[t] >= 0: token t's K/V for every kv head go
 * to physical block slot / B, offset slot % B.  Whole elements are copied as
 * raw bytes. */
int oracle_write_kv(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                    const int64_t *slot_mapping, int64_t T, int64_t Hkv, int64_t D, int64_t B,
                    int64_t NB, int64_t k_x, int dtype) {
    int64_t e = oracle_elem_bytes(dtype);
    if (e == 0) return OR_BAD_DTYPE;
    if (T < 0 || Hkv <= 0 || D <= 0 || B <= 0 || NB < 0 || k_x <= 0 || D % k_x != 0)
        return OR_BAD_DIMS;
    for (int64_t t = 0; t < T; ++t) {
        int64_t sl = slot_mapping[t];
        if (sl >= NB * B) return OR_BAD_SLOT;
        if (sl < 0) continue;
        for (int64_t u = t + 1; u < T; ++u)
            if (slot_mapping[u] == sl) return OR_DUP_SLOT;
    }
    for (int64_t t = 0; t < T; ++t) {
        int64_t sl = slot_mapping[t];
        if (sl < 0) continue;
        int64_t b = sl / B, off = sl % B;
        for (int64_t g = 0; g < Hkv; ++g) {
            for (int64_t d = 0; d < D; ++d) {
                int64_t src = (t * Hkv + g) * D + d;
                memcpy((char *)k_cache + k_index(b, g, off, d, Hkv, D, B, k_x) * e,
                       (const char *)k_new + src * e, (size_t)e);
                memcpy((char *)v_cache + v_index(b, g, off, d, Hkv, D, B) * e,
                       (const char *)v_new + src * e, (size_t)e);
            }
        }
    }
    return OR_OK;
}

/* block_mapping is int64 [n][2] = (src, dst).  Every source block (all kv
 * heads, all B slots, K and V) is read before any destination is written. */
int oracle_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping, int64_t n,
                       int64_t Hkv, int64_t D, int64_t B, int64_t NB, int dtype) {
    int64_t e = oracle_elem_bytes(dtype);
    if (e == 0) return OR_BAD_DTYPE;
    if (n < 0 || Hkv <= 0 || D <= 0 || B <= 0 || NB < 0) return OR_BAD_DIMS;
    for (int64_t i = 0; i < n; ++i) {
        int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        if (src < 0 || src >= NB || dst < 0 || dst >= NB) return OR_BAD_PAIR;
        for (int64_t j = 0; j < n; ++j) {
            if (j != i && block_mapping[2 * j + 1] == dst) return OR_BAD_PAIR;
            if (block_mapping[2 * j] == dst) return OR_BAD_PAIR;
        }
    }
    size_t block_bytes = (size_t)(Hkv * B * D * e);
    char *snap = (char *)malloc(block_bytes * 2 * (size_t)(n > 0 ? n : 1));
    if (!snap) return OR_NO_MEM;
    for (int64_t i = 0; i < n; ++i) {
        int64_t src = block_mapping[2 * i];
        memcpy(snap + (2 * i) * block_bytes, (char *)k_cache + src * block_bytes, block_bytes);
        memcpy(snap + (2 * i + 1) * block_bytes, (char *)v_cache + src * block_bytes,
               block_bytes);
    }
    for (int64_t i = 0; i < n; ++i) {
        int64_t dst = block_mapping[2 * i + 1];
        memcpy((char *)k_cache + dst * block_bytes, snap + (2 * i) * block_bytes, block_bytes);
        memcpy((char *)v_cache + dst * block_bytes, snap + (2 * i + 1) * block_bytes,
               block_bytes);
    }
    free(snap);
    return OR_OK;
}

/* Copy block src of the source pools to block dst of the destination pools,
 * for every (src, dst) pair: all kv heads, all slots, K and V, byte for byte.
 * The two pool pairs are different allocations (swap-out: device to host;
 * swap-in: host to device), so there is no overlap to order; destinations
 * must still be distinct (two pairs may not write one block). */
int oracle_swap_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                       const int64_t *block_mapping, int64_t n, int64_t Hkv, int64_t D, int64_t B,
                       int64_t src_blocks, int64_t dst_blocks, int dtype) {
    int64_t e = oracle_elem_bytes(dtype);
    if (e == 0) return OR_BAD_DTYPE;
    if (n < 0 || Hkv <= 0 || D <= 0 || B <= 0 || src_blocks < 0 || dst_blocks < 0)
        return OR_BAD_DIMS;
    for (int64_t i = 0; i < n; ++i) {
        int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return OR_BAD_PAIR;
        for (int64_t j = 0; j < i; ++j)
            if (block_mapping[2 * j + 1] == dst) return OR_BAD_PAIR;
    }
    size_t block_bytes = (size_t)(Hkv * B * D * e);
    for (int64_t i = 0; i < n; ++i) {
        int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        memcpy((char *)dst_k + dst * block_bytes, (const char *)src_k + src * block_bytes,
               block_bytes);
        memcpy((char *)dst_v + dst * block_bytes, (const char *)src_v + src * block_bytes,
               block_bytes);
    }
    return OR_OK;
}

/* KV-cache bytes for t tokens of a model with L layers, H heads of size
 * D_h, at `elem_bytes` per element: one K and one V vector per token, layer
 * and head.  [論文解説: PagedAttention, 技術的詳細 › KVキャッシュのメモリ要件]
 * With 2-byte elements this is the page's 4 * t * L * H * D_h. */
int64_t oracle_kv_cache_bytes(int64_t t, int64_t L, int64_t H, int64_t D_h, int64_t elem_bytes) {
    return 2 * elem_bytes * t * L * H * D_h;
}

/* Logical block count for T tokens at B tokens per block: ceil(T / B).
 * [論文解説: PagedAttention, 技術的詳細 › PagedAttentionアルゴリズム, block definition] */
int64_t oracle_blocks_for_tokens(int64_t T, int64_t B) { return (T + B - 1) / B; }

/* Slot of logical position i through one block-table row. */
int64_t oracle_slot_of(const int32_t *block_table_row, int64_t B, int64_t i) {
    return (int64_t)block_table_row[i / B] * B + i % B;
}

/* Threads the OpenMP loops above will use (for reporting the CPU baseline). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Sets the thread count of the calling thread's later OpenMP loops (n >= 1);
 * returns the previous count.  Each output is computed by one thread, so the
 * results do not depend on it. */
int oracle_set_num_threads(int n) {
    int prev = omp_get_max_threads();
    if (n >= 1) omp_set_num_threads(n);
    return prev;
}
