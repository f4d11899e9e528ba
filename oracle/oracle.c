/*
 * Paged-attention decode oracle: a plain, slow, obviously-correct CPU
 * reference in fp64.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this library. It shares no code, header, constant
 * table or helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes (no blocking, fusion or reordering beyond the definitions):
 *
 *  ora_write_kv_cache -- slot-mapped write of new K/V tokens into the paged
 *      pool. Source: "How pakanor/low-latency-distributed-llm-serving-
 *      infrastructure-custom-k8s-control-plane works", Connections (the
 *      engine writes the KV cache; paged attention maps cache slots), and the
 *      Continuous-Batching-LLM-Inference-Engine README, feature list (a pool
 *      of fixed-size physical blocks with a per-sequence page table).
 *      Float caches: a bit copy. int8 cache ("How vrajpatel105/paged-
 *      inference-engine works", summary: paged INT8 KV storage):
 *      q = clamp(rint(x / s), -127, 127), x / s the correctly rounded fp32
 *      quotient.
 *
 *  ora_decode -- for every sequence and query head, scaled dot-product
 *      softmax attention of the one query token over every cached token of
 *      that sequence, gathered through its logical->physical block table with
 *      no compaction copy (Continuous-Batching-LLM-Inference-Engine README,
 *      feature list, PagedAttention kernel; the decoder reads the block table
 *      in "How vrajpatel105/paged-inference-engine works", Connections).
 *      Two passes: the max, then the exponentials and sums. No online
 *      rescaling.
 *
 *  ora_decode_partials / ora_splitk_reduce -- the same attention split over
 *      context partitions of P tokens, each partition's normalised output with
 *      its max and sum, and the log-sum-exp combination of the partitions.
 *
 *  ora_prefill -- several new query tokens per sequence at once: the target
 *      model's scoring of K drafted tokens in one batched pass for
 *      speculative decoding (Continuous-Batching-LLM-Inference-Engine README,
 *      feature list) and the prefill chunks that continuous batches mix with
 *      decode tokens ("How brave30/mini-inference-engine works", summary and
 *      Model Compute: prefill attention). The n_s query tokens of sequence s
 *      are its newest tokens, already written to the cache, so query j sits
 *      at position L_s - n_s + j and attends to the cached tokens 0 .. that
 *      position: the causal reading of a prefix followed by new tokens. Each
 *      row is plain decode attention over a truncated context.
 *
 *  ora_copy_blocks -- the copy step of the block pool's copy-on-write
 *      reference counting (Continuous-Batching-LLM-Inference-Engine README,
 *      feature list): for each (src, dst) pair, every byte of physical block
 *      src -- the K and V tiles of every kv head and, for an int8 cache, its
 *      per-(block, kv head) scales -- is copied into block dst. No block may
 *      be the destination of two pairs or both a source and a destination.
 *
 * Conventions (readings where the pages are silent): context_lens counts the
 * newly written token; query head h reads kv head h / (Hq / Hkv); the cache is
 * [num_blocks][Hkv][block_size][D] row-major; L = 0 gives zeros; slots < 0 are
 * skipped; block-table entries at or past ceil(L / block_size) are never read.
 *
 * Dtype codes: 0 = fp32, 1 = bf16 (raw 16-bit patterns), 2 = int8.
 * Return codes: 0 ok, -1 bad argument, -2 index out of range.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORA_F32 0
#define ORA_BF16 1
#define ORA_I8 2

/* Exact widening of one stored element to double. */
static double load_elem(const void *base, int64_t i, int dtype)
{
    if (dtype == ORA_F32)
        return (double)((const float *)base)[i];
    if (dtype == ORA_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const int8_t *)base)[i];
}

static int elem_size(int dtype)
{
    return dtype == ORA_F32 ? 4 : dtype == ORA_BF16 ? 2 : 1;
}

int ora_num_threads(void) { return omp_get_max_threads(); }
void ora_set_num_threads(int n) { omp_set_num_threads(n); }

/* ------------------------------------------------------------------------ */
/* Slot-mapped write                                                        */
/* ------------------------------------------------------------------------ */

/* int8 code of x for scale s: the fp32 quotient x / s rounded correctly
 * (double rounding through fp64 is innocuous for one division, since
 * 53 >= 2 * 24 + 2), then rounded to the nearest integer with ties to even,
 * then clamped to [-127, 127]. A NaN quotient gives 0. */
static int8_t quantize(double x, float s)
{
    float t = (float)(x / (double)s);
    if (isnan(t))
        return 0;
    float r = nearbyintf(t);
    if (r > 127.0f)
        r = 127.0f;
    if (r < -127.0f)
        r = -127.0f;
    return (int8_t)r;
}

int ora_write_kv_cache(const void *key, const void *value, void *k_cache, void *v_cache,
                       const int64_t *slot_mapping, const float *k_scale, const float *v_scale,
                       int64_t num_tokens, int num_kv_heads, int head_dim, int block_size,
                       int64_t num_blocks, int act_dtype, int cache_dtype)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return -1;
    if (act_dtype != ORA_F32 && act_dtype != ORA_BF16)
        return -1;
    if (cache_dtype == ORA_I8) {
        if (!k_scale || !v_scale)
            return -1;
    } else if (cache_dtype != act_dtype) {
        return -1;
    }
    const int64_t Hkv = num_kv_heads, D = head_dim, B = block_size;
    const int esz = elem_size(cache_dtype);
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        int64_t b = slot / B, o = slot % B;
        if (b >= num_blocks)
            return -2;
        for (int64_t g = 0; g < Hkv; ++g) {
            for (int64_t d = 0; d < D; ++d) {
                int64_t src = (i * Hkv + g) * D + d;
                int64_t dst = ((b * Hkv + g) * B + o) * D + d;
                if (cache_dtype == ORA_I8) {
                    ((int8_t *)k_cache)[dst] = quantize(load_elem(key, src, act_dtype), k_scale[b * Hkv + g]);
                    ((int8_t *)v_cache)[dst] = quantize(load_elem(value, src, act_dtype), v_scale[b * Hkv + g]);
                } else {
                    memcpy((char *)k_cache + dst * esz, (const char *)key + src * esz, esz);
                    memcpy((char *)v_cache + dst * esz, (const char *)value + src * esz, esz);
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Copy-on-write block copy                                                 */
/* ------------------------------------------------------------------------ */

int ora_copy_blocks(void *k_cache, void *v_cache, float *k_scale, float *v_scale,
                    const int64_t *block_mapping, int64_t num_pairs, int num_kv_heads,
                    int head_dim, int block_size, int64_t num_blocks, int cache_dtype)
{
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return -1;
    if (cache_dtype != ORA_F32 && cache_dtype != ORA_BF16 && cache_dtype != ORA_I8)
        return -1;
    if (cache_dtype == ORA_I8 && (!k_scale || !v_scale))
        return -1;
    /* every index in range; destinations distinct and never a source */
    char *role = calloc((size_t)num_blocks, 1);     /* 1 source, 2 destination */
    if (!role)
        return -1;
    for (int64_t i = 0; i < num_pairs; ++i) {
        int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) {
            free(role);
            return -2;
        }
        role[src] |= 1;
    }
    for (int64_t i = 0; i < num_pairs; ++i) {
        int64_t dst = block_mapping[2 * i + 1];
        if (role[dst]) {
            free(role);
            return -2;
        }
        role[dst] = 2;
    }
    free(role);
    const int64_t bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_size(cache_dtype);
    for (int64_t i = 0; i < num_pairs; ++i) {
        int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
        memcpy((char *)k_cache + dst * bytes, (const char *)k_cache + src * bytes, (size_t)bytes);
        memcpy((char *)v_cache + dst * bytes, (const char *)v_cache + src * bytes, (size_t)bytes);
        if (cache_dtype == ORA_I8) {
            for (int64_t g = 0; g < num_kv_heads; ++g) {
                k_scale[dst * num_kv_heads + g] = k_scale[src * num_kv_heads + g];
                v_scale[dst * num_kv_heads + g] = v_scale[src * num_kv_heads + g];
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Decode                                                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
    const void *q, *k_cache, *v_cache;
    const int32_t *block_tables, *context_lens;
    const float *k_scale, *v_scale;
    double scale;
    int64_t S, Hq, Hkv, D, B, MB, NB;
    int q_dtype, cache_dtype;
} problem;

/* Element index of (physical block b, kv head g, offset o, dim d). */
static int64_t cache_index(const problem *p, int64_t b, int64_t g, int64_t o, int64_t d)
{
    return ((b * p->Hkv + g) * p->B + o) * p->D + d;
}

/* Physical block holding logical token t of sequence s (-1 if out of range). */
static int64_t phys_block(const problem *p, int64_t s, int64_t t)
{
    int64_t b = p->block_tables[s * p->MB + t / p->B];
    return (b < 0 || b >= p->NB) ? -1 : b;
}

/* Dequantised cache element: exact widening for float caches; for int8 the
 * product code * scale of its (block, kv head), exact in fp64. */
static double cache_value(const problem *p, const void *cache, const float *sc,
                          int64_t b, int64_t g, int64_t o, int64_t d)
{
    double x = load_elem(cache, cache_index(p, b, g, o, d), p->cache_dtype);
    if (p->cache_dtype == ORA_I8)
        x *= (double)sc[b * p->Hkv + g];
    return x;
}

/* logit of query row r, head h against logical token t held in physical
 * block b: scale * sum_d q[r][h][d] k_t[d]. */
static double logit(const problem *p, int64_t r, int64_t h, int64_t t, int64_t b)
{
    int64_t g = h / (p->Hq / p->Hkv);
    int64_t o = t % p->B;
    double acc = 0.0;
    for (int64_t d = 0; d < p->D; ++d)
        acc += load_elem(p->q, (r * p->Hq + h) * p->D + d, p->q_dtype) *
               cache_value(p, p->k_cache, p->k_scale, b, g, o, d);
    return p->scale * acc;
}

/* Attention of query row r, head h over logical tokens [t0, t1) of sequence
 * s: writes the normalised output to o_out[D] and returns the max logit and
 * the sum of exponentials. Returns 0, or -2 on a bad block id. (Decode: the
 * query row of sequence s is row s.) */
static int attend_range(const problem *p, int64_t s, int64_t r, int64_t h, int64_t t0,
                        int64_t t1, double *o_out, double *m_out, double *l_out, double *x)
{
    int64_t g = h / (p->Hq / p->Hkv);
    /* pass 1: logits and their max */
    double M = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t b = phys_block(p, s, t);
        if (b < 0)
            return -2;
        x[t - t0] = logit(p, r, h, t, b);
        if (x[t - t0] > M)
            M = x[t - t0];
    }
    /* pass 2: weights, their sum, the weighted sum of V */
    double Z = 0.0;
    for (int64_t d = 0; d < p->D; ++d)
        o_out[d] = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        double w = exp(x[t - t0] - M);
        Z += w;
        int64_t b = phys_block(p, s, t);
        for (int64_t d = 0; d < p->D; ++d)
            o_out[d] += w * cache_value(p, p->v_cache, p->v_scale, b, g, t % p->B, d);
    }
    for (int64_t d = 0; d < p->D; ++d)
        o_out[d] /= Z;
    *m_out = M;
    *l_out = Z;
    return 0;
}

static int check_problem(const problem *p)
{
    if (!p->q || !p->k_cache || !p->v_cache || !p->block_tables || !p->context_lens)
        return -1;
    if (p->S < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Hq % p->Hkv || p->D <= 0 || p->B <= 0 ||
        p->MB <= 0 || p->NB <= 0)
        return -1;
    if (p->q_dtype != ORA_F32 && p->q_dtype != ORA_BF16)
        return -1;
    if (p->cache_dtype == ORA_I8) {
        if (!p->k_scale || !p->v_scale)
            return -1;
    } else if (p->cache_dtype != ORA_F32 && p->cache_dtype != ORA_BF16) {
        return -1;
    }
    for (int64_t s = 0; s < p->S; ++s)
        if (p->context_lens[s] < 0 || p->context_lens[s] > p->MB * p->B)
            return -2;
    return 0;
}

int ora_decode(double *out, const void *q, const void *k_cache, const void *v_cache,
               const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
               const float *k_scale, const float *v_scale, float scale, int num_seqs,
               int num_heads, int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
               int q_dtype, int cache_dtype)
{
    problem p = {q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                 (double)scale, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                 max_blocks_per_seq, num_blocks, q_dtype, cache_dtype};
    int rc = check_problem(&p);
    if (rc)
        return rc;
    int64_t maxL = 0;
    for (int64_t s = 0; s < p.S; ++s)
        if (context_lens[s] > maxL)
            maxL = context_lens[s];
    int err = 0;
#pragma omp parallel
    {
        double *x = malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
        double m, l;
#pragma omp for schedule(dynamic)
        for (int64_t sh = 0; sh < p.S * p.Hq; ++sh) {
            int64_t s = sh / p.Hq, h = sh % p.Hq;
            double *o = out + sh * p.D;
            int64_t L = context_lens[s];
            if (L == 0) {
                for (int64_t d = 0; d < p.D; ++d)
                    o[d] = 0.0;
                continue;
            }
            if (attend_range(&p, s, s, h, 0, L, o, &m, &l, x)) {
#pragma omp atomic write
                err = -2;
            }
        }
        free(x);
    }
    return err;
}

int ora_decode_partials(double *o_part, double *m_part, double *l_part, int num_partitions,
                        const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, int max_blocks_per_seq,
                        const int32_t *context_lens, const float *k_scale, const float *v_scale,
                        float scale, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                        int block_size, int64_t num_blocks, int partition_size, int q_dtype,
                        int cache_dtype)
{
    problem p = {q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                 (double)scale, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                 max_blocks_per_seq, num_blocks, q_dtype, cache_dtype};
    int rc = check_problem(&p);
    if (rc)
        return rc;
    if (partition_size <= 0 || num_partitions < 0)
        return -1;
    const int64_t P = partition_size, NP = num_partitions;
    for (int64_t s = 0; s < p.S; ++s)
        if ((context_lens[s] + P - 1) / P > NP)
            return -1;
    int err = 0;
#pragma omp parallel
    {
        double *x = malloc(sizeof(double) * (size_t)P);
#pragma omp for schedule(dynamic)
        for (int64_t sh = 0; sh < p.S * p.Hq; ++sh) {
            int64_t s = sh / p.Hq, h = sh % p.Hq;
            int64_t L = context_lens[s];
            for (int64_t j = 0; j * P < L; ++j) {
                int64_t t1 = (j + 1) * P < L ? (j + 1) * P : L;
                if (attend_range(&p, s, s, h, j * P, t1, o_part + (sh * NP + j) * p.D,
                                 m_part + sh * NP + j, l_part + sh * NP + j, x)) {
#pragma omp atomic write
                    err = -2;
                }
            }
        }
        free(x);
    }
    return err;
}

/* Log-sum-exp combination: M = max_j m_j, W_j = l_j exp(m_j - M),
 * out = sum_j W_j o_j / sum_j W_j over the partitions j < ceil(L / P). */
int ora_splitk_reduce(double *out, const double *o_part, const double *m_part,
                      const double *l_part, const int32_t *context_lens, int num_seqs,
                      int num_heads, int head_dim, int partition_size, int num_partitions)
{
    if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || partition_size <= 0 || num_partitions < 0)
        return -1;
    const int64_t P = partition_size, NP = num_partitions, D = head_dim, H = num_heads;
    for (int64_t s = 0; s < num_seqs; ++s)
        if (context_lens[s] < 0 || (context_lens[s] + P - 1) / P > NP)
            return -1;
#pragma omp parallel for schedule(dynamic)
    for (int64_t sh = 0; sh < (int64_t)num_seqs * H; ++sh) {
        int64_t s = sh / H;
        int64_t n = (context_lens[s] + P - 1) / P;
        double *o = out + sh * D;
        for (int64_t d = 0; d < D; ++d)
            o[d] = 0.0;
        if (n == 0)
            continue;
        double M = -INFINITY;
        for (int64_t j = 0; j < n; ++j)
            if (m_part[sh * NP + j] > M)
                M = m_part[sh * NP + j];
        double Wsum = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double W = l_part[sh * NP + j] * exp(m_part[sh * NP + j] - M);
            Wsum += W;
            for (int64_t d = 0; d < D; ++d)
                o[d] += W * o_part[(sh * NP + j) * D + d];
        }
        for (int64_t d = 0; d < D; ++d)
            o[d] /= Wsum;
    }
    return 0;
}

/* Several query tokens per sequence. Rows query_start_loc[s] ..
 * query_start_loc[s + 1] - 1 of q and out belong to sequence s; with n_s
 * rows and L_s = context_lens[s] (which counts them), row query_start_loc[s]
 * + j attends to the tokens 0 .. L_s - n_s + j. Requires 0 = qsl[0] <= qsl[1]
 * <= ... <= qsl[S] = num_query_tokens and n_s <= L_s. */
int ora_prefill(double *out, const void *q, const void *k_cache, const void *v_cache,
                const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                const int32_t *query_start_loc, const float *k_scale, const float *v_scale,
                float scale, int num_seqs, int num_query_tokens, int num_heads,
                int num_kv_heads, int head_dim, int block_size, int64_t num_blocks, int q_dtype,
                int cache_dtype)
{
    problem p = {q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                 (double)scale, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                 max_blocks_per_seq, num_blocks, q_dtype, cache_dtype};
    int rc = check_problem(&p);
    if (rc)
        return rc;
    if (!query_start_loc || num_query_tokens < 0 || query_start_loc[0] != 0 ||
        query_start_loc[num_seqs] != num_query_tokens)
        return -1;
    for (int64_t s = 0; s < p.S; ++s) {
        int64_t n = (int64_t)query_start_loc[s + 1] - query_start_loc[s];
        if (n < 0 || n > context_lens[s])
            return -1;
    }
    int64_t maxL = 0;
    for (int64_t s = 0; s < p.S; ++s)
        if (context_lens[s] > maxL)
            maxL = context_lens[s];
    int err = 0;
#pragma omp parallel
    {
        double *x = malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
        double m, l;
#pragma omp for schedule(dynamic)
        for (int64_t rh = 0; rh < (int64_t)num_query_tokens * p.Hq; ++rh) {
            int64_t r = rh / p.Hq, h = rh % p.Hq;
            int64_t s = 0;
            while (query_start_loc[s + 1] <= r)        /* the sequence holding row r */
                ++s;
            int64_t n = query_start_loc[s + 1] - query_start_loc[s];
            int64_t pos = context_lens[s] - n + (r - query_start_loc[s]);
            if (attend_range(&p, s, r, h, 0, pos + 1, out + rh * p.D, &m, &l, x)) {
#pragma omp atomic write
                err = -2;
            }
        }
        free(x);
    }
    return err;
}
