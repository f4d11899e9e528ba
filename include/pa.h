/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-attention decode library, libpa.so.
 *
 * The method: during decode, every running sequence holds its keys and values
 * in fixed-size physical blocks of a shared pool, found through a per-sequence
 * logical->physical block table ("Paged KV-cache" and "PagedAttention kernel",
 * Continuous-Batching-LLM-Inference-Engine README, feature list). Each step
 *   1. writes the new token's K/V into the slot the scheduler mapped for it
 *      ("LLM engine -> KV cache manager: writes KV cache" and "Paged attention
 *      -> KV cache manager: maps cache slots", "How pakanor/low-latency-
 *      distributed-llm-serving-infrastructure-custom-k8s-control-plane works",
 *      Connections), optionally as int8 ("paged INT8 KV storage", "How
 *      vrajpatel105/paged-inference-engine works", summary);
 *   2. runs decode attention of the one new query token per sequence over its
 *      cached tokens, gathering K/V from the non-contiguous blocks inside the
 *      kernel with no compaction copy (README feature list; "Decoder model ->
 *      Block allocator: reads block table", paged-inference-engine,
 *      Connections; "Llama forward -> Paged decode attention", "How
 *      brave30/mini-inference-engine works", Connections);
 *   3. for long contexts, splits each sequence's context into partitions and
 *      combines the per-partition results with a log-sum-exp reduce (not on
 *      the pages: the flash-decoding split-K of the decode step's
 *      specification; see pa_decode_splitk_reduce).
 *
 * Math of step 2, for sequence s, query head h, kv head g = h / (Hq / Hkv):
 *   x_t   = scale * sum_d q[s,h,d] * k_t[d]          t = 0 .. L_s - 1
 *   out   = sum_t exp(x_t - max x) v_t / sum_t exp(x_t - max x)
 * with k_t, v_t row t % block_size of block block_tables[s][t / block_size],
 * dequantised as code * scale[block, g] for an int8 cache.
 *
 * Conventions used by every entry point
 *  - All data pointers are DEVICE pointers owned by the caller. The library
 *    allocates nothing, keeps no state between calls (beyond a cache of grid
 *    sizes per kernel and device), and may be called from several host
 *    threads at once -- except pa_write_decode_balanced_noalloc, whose
 *    workspace is one static array per GPU, so its calls must not overlap.
 *  - Precision: dot products and sums accumulate in fp32. The MFMA kernels
 *    (4 or 8 query heads per kv head with a bf16 cache, and pa_prefill) round
 *    the softmax weights to bf16 for the P V product and sum those same
 *    rounded weights; the VALU kernels (1 or 2 query heads per kv head) and
 *    the decode kernels on an int8 cache keep the weights, and the V scale,
 *    in fp32.
 *  - All tensors are dense, row-major, with the layouts given per argument.
 *    The KV pool is [num_blocks][num_kv_heads][block_size][head_dim]: the
 *    block_size x head_dim tile of one (block, kv head) is contiguous.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and is asynchronous. Calls on one stream run in order; in a decode step
 *    pa_write_kv_cache must precede pa_decode, because context_lens counts the
 *    newly written token.
 *  - dtypes: PA_F32 (fp32), PA_BF16 (bfloat16), PA_I8 (int8 cache codes).
 *  - Return value: PA_OK (0) or a negative pa_status. Arguments that the host
 *    can check are checked before anything is enqueued; on any error nothing
 *    is enqueued. Values held in device memory (block ids, slots, lengths)
 *    are trusted: out-of-range values are undefined behaviour, unless the
 *    environment variable PA_CHECK=1 is set, in which case they are copied to
 *    the host (synchronising the stream) and checked first (PA_ERR_INDEX).
 *  - No C++ exception crosses this interface.
 */
#ifndef PA_H
#define PA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_I8 = 2 } pa_dtype;

typedef enum {
    PA_OK = 0,
    PA_ERR_NULL = -1,        /* a required pointer is NULL */
    PA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    PA_ERR_DTYPE = -3,       /* unknown dtype or unsupported dtype combination */
    PA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    PA_ERR_UNSUPPORTED = -5, /* valid arguments that no kernel instance covers */
    PA_ERR_LAUNCH = -6,      /* the HIP runtime reported an error at launch */
    PA_ERR_INDEX = -7        /* PA_CHECK=1 found a device index out of range */
} pa_status;

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int pa_version(void);

/* Static text for a pa_status value ("unknown status" for others). */
const char *pa_status_string(int status);

/* Number of context partitions of `partition_size` tokens that cover
 * `max_context_len` tokens: ceil(max_context_len / partition_size), or 0 when
 * either is <= 0. Sizes the split-K workspace of pa_decode. */
int pa_num_partitions(int max_context_len, int partition_size);

/*
 * pa_write_kv_cache -- slot-mapped write of new tokens' keys and values
 * ("writes KV cache", "maps cache slots": pakanor ... control-plane page,
 * Connections; int8 storage: paged-inference-engine page, summary).
 *
 * For every token i with slot = slot_mapping[i] >= 0, with b = slot /
 * block_size and o = slot % block_size, for every kv head g and dim d:
 *   float cache: k_cache[b][g][o][d] = key[i][g][d] (bit copy; act_dtype must
 *                equal cache_dtype), likewise value -> v_cache;
 *   int8 cache:  k_cache[b][g][o][d] = clamp(rint(key[i][g][d] / k_scale[b][g]),
 *                -127, 127), where the quotient is the correctly rounded fp32
 *                quotient, rint rounds half to even and a NaN quotient gives 0;
 *                likewise value with v_scale.
 * Tokens with slot < 0 are skipped. Every other byte of the pool, and the
 * scales, are left untouched. Two tokens mapped to one slot: undefined.
 *
 *   key, value      [num_tokens][num_kv_heads][head_dim], act_dtype (F32/BF16)
 *   k_cache,v_cache [num_blocks][num_kv_heads][block_size][head_dim], cache_dtype
 *   slot_mapping    [num_tokens] int64
 *   k_scale,v_scale [num_blocks][num_kv_heads] fp32, read only; required (non-NULL)
 *                   iff cache_dtype == PA_I8, ignored otherwise. The caller
 *                   chooses them (e.g. absmax / 127 of the block) before the write.
 * Requirements: num_tokens >= 0 (0 = no-op), num_kv_heads >= 1, head_dim a
 * multiple of 8 in [8, 1024], block_size >= 1, num_blocks >= 1; key, value,
 * k_cache, v_cache 16-byte aligned.
 */
int pa_write_kv_cache(const void *key, const void *value, void *k_cache, void *v_cache,
                      const int64_t *slot_mapping, const float *k_scale, const float *v_scale,
                      int num_tokens, int num_kv_heads, int head_dim, int block_size,
                      int64_t num_blocks, pa_dtype act_dtype, pa_dtype cache_dtype, void *stream);

/*
 * pa_decode -- paged decode attention ("PagedAttention kernel ... gathers KV
 * data from non-contiguous physical blocks in-kernel, no compaction copy",
 * README feature list; "Paged decode attention", mini-inference-engine page,
 * Model Compute).
 *
 *   out           [num_seqs][num_heads][head_dim], q_dtype. Written only when
 *                 partition_size == 0.
 *   q             [num_seqs][num_heads][head_dim], q_dtype (F32 or BF16)
 *   k_cache, v_cache  pool as above, cache_dtype
 *   block_tables  [num_seqs][max_blocks_per_seq] int32 physical block ids;
 *                 only entries < ceil(context_lens[s] / block_size) are read
 *   context_lens  [num_seqs] int32, 0 <= L_s <= max_context_len; counts the
 *                 newly written token. L_s = 0 gives an all-zero output.
 *   k_scale, v_scale  [num_blocks][num_kv_heads] fp32, required iff int8 cache
 *   scale         softmax scale applied to q . k (usually 1 / sqrt(head_dim))
 *   num_heads     query heads Hq; num_kv_heads Hkv divides it; query head h
 *                 reads kv head h / (Hq / Hkv)
 *   max_context_len  host-side bound on every L_s; must not exceed
 *                 max_blocks_per_seq * block_size
 *   partition_size   0: one pass over each whole context, result in `out`.
 *                 > 0 (a multiple of block_size): split-K. Partition j of
 *                 sequence s covers tokens [j P, min(L_s, (j+1) P)) and stores
 *                   tmp_out[s][h][j][:] = that partition's normalised output,
 *                   tmp_max[s][h][j]    = its largest logit x_t (natural units),
 *                   tmp_sum[s][h][j]    = sum_t exp(x_t - tmp_max),
 *                 for j < ceil(L_s / P) only; `out` is not touched. Combine with
 *                 pa_decode_splitk_reduce.
 *   tmp_out       [num_seqs][num_heads][NP][head_dim] fp32, tmp_max and tmp_sum
 *                 [num_seqs][num_heads][NP] fp32, NP = pa_num_partitions(
 *                 max_context_len, partition_size); caller-owned workspace,
 *                 required iff partition_size > 0.
 * Supported instances (others return PA_ERR_UNSUPPORTED):
 *   group size G = Hq / Hkv in {1, 2}: VALU kernel; head_dim 64 or 128;
 *     (q, cache) = (F32, F32), (BF16, BF16), (F32, I8), (BF16, I8).
 *   G in {4, 8}: MFMA kernel; head_dim 128; q BF16; cache BF16 or I8.
 *   block_size 16 or 32.
 * Alignment: out, q, k_cache, v_cache, tmp_out 16-byte aligned.
 */
int pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
              const float *k_scale, const float *v_scale, float scale, int num_seqs,
              int num_heads, int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
              int max_context_len, int partition_size, float *tmp_out, float *tmp_max,
              float *tmp_sum, pa_dtype q_dtype, pa_dtype cache_dtype, void *stream);

/*
 * pa_decode_balanced -- the same decode attention as pa_decode, scheduled so
 * that every workgroup streams the same amount of KV whatever the mix of
 * context lengths, with the log-sum-exp combination of split contexts done
 * in the same launch; writes `out` directly (no separate reduce).
 *
 * Schedule: all (sequence, kv head) contexts are laid end to end as one list
 * of 16-token chunks; a persistent grid (resident workgroups per CU times the
 * CU count) splits it into one contiguous range of about equal cost per wave,
 * each at least min_piece_tokens / 16 chunks. A context inside one range is
 * finished in place. A context cut by range ends leaves one partial per piece
 * in the workspace; the wave that completes its last piece (an atomic counter
 * per (sequence, kv head)) combines the pieces exactly as
 * pa_decode_splitk_reduce would, writes `out`, and resets the counter. With 8
 * query heads per kv head on a bf16 cache (and at most 4096 sequences) the
 * list holds pairs of neighbouring sequences instead, the 16 query heads of a
 * pair filling one 16-column MFMA tile: the leading chunks that both block
 * tables place on the same physical blocks (copy-on-write prefixes) are read
 * and computed once for the two, the other chunks for their own sequence.
 *
 *   out, q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
 *   scale, num_seqs .. max_context_len, q_dtype, cache_dtype: as pa_decode.
 *   min_piece_tokens  smallest piece a range may be cut to, a multiple of 16.
 *   tmp_out       [slots][G][head_dim] fp32, tmp_max and tmp_sum [slots][G] fp32,
 *                 G = num_heads / num_kv_heads, slots as pa_balanced_workspace
 *                 reports for the stream's device. Contents on return are
 *                 unspecified.
 *   counters      int32 [counters as pa_balanced_workspace reports], all zero
 *                 before the call; the call leaves them all zero again (zero
 *                 them once, reuse).
 * Calls that share `counters` or the workspace must not overlap in time
 * (e.g. run them on one stream). Supported instances: as pa_decode.
 * Alignment: out, q, k_cache, v_cache, tmp_out 16-byte aligned.
 */
int pa_decode_balanced(void *out, const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, int max_blocks_per_seq,
                       const int32_t *context_lens, const float *k_scale, const float *v_scale,
                       float scale, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                       int block_size, int64_t num_blocks, int max_context_len,
                       int min_piece_tokens, float *tmp_out, float *tmp_max, float *tmp_sum,
                       int32_t *counters, pa_dtype q_dtype, pa_dtype cache_dtype, void *stream);

/*
 * pa_write_decode_balanced -- one decode step in one call: the slot-mapped
 * write of every sequence's new token (as pa_write_kv_cache with
 * num_tokens = num_seqs) followed by pa_decode_balanced. For the MFMA
 * instances (bf16 q, G = 4 or 8, head_dim 128) both run in one launch: the
 * wave that consumes the chunk holding a sequence's new token loads the
 * token's rows with it, stores them into the slot and uses them in place of
 * the chunk's old row (int8: the codes of the chunk's block scales), so the
 * kernel never reads back what it stores. Otherwise the two kernels run one
 * after the other on `stream`.
 *
 *   key, value    [num_seqs][num_kv_heads][head_dim], q_dtype: row s is the new
 *                 token of sequence s.
 *   slot_mapping  [num_seqs] int64: its slot, or < 0 to write nothing. For a
 *                 non-empty context it must be the slot of logical position
 *                 context_lens[s] - 1 of sequence s (the token is part of its
 *                 own context); PA_CHECK=1 verifies this.
 *   k_cache, v_cache are written; all other arguments as pa_decode_balanced.
 * Result and pool contents are bit-identical to the two calls.
 */
int pa_write_decode_balanced(const void *key, const void *value, const int64_t *slot_mapping,
                             void *out, const void *q, void *k_cache, void *v_cache,
                             const int32_t *block_tables, int max_blocks_per_seq,
                             const int32_t *context_lens, const float *k_scale,
                             const float *v_scale, float scale, int num_seqs, int num_heads,
                             int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                             int max_context_len, int min_piece_tokens, float *tmp_out,
                             float *tmp_max, float *tmp_sum, int32_t *counters, pa_dtype q_dtype,
                             pa_dtype cache_dtype, void *stream);

/*
 * pa_write_decode_balanced_noalloc -- pa_write_decode_balanced for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same step, with the workspace
 * (partials, maxima, sums, counters) in a static array of the library instead
 * of caller buffers. It calls no hipMalloc or hipFree and allocates nothing.
 *
 * The array is 72 MiB per GPU (held by every device that loads the library
 * until the process ends): a 1 MiB region of int32 counters, cleared by a
 * kernel on `stream` at the first call on each device and left zero by every
 * call, then the partial states. Shapes whose workspace (pa_balanced_workspace)
 * does not fit -- more than 262144 (sequence, kv head) counters, or partial
 * slots beyond the rest of the array -- return PA_ERR_SHAPE before anything is
 * enqueued (on a 256-CU device every kernel instance's slots fit). Every call on
 * one GPU uses that GPU's array: calls that overlap in time on one GPU (two
 * streams, two host threads) race and must not be made. Arguments, results and
 * errors otherwise as pa_write_decode_balanced.
 */
int pa_write_decode_balanced_noalloc(const void *key, const void *value,
                                     const int64_t *slot_mapping, void *out, const void *q,
                                     void *k_cache, void *v_cache, const int32_t *block_tables,
                                     int max_blocks_per_seq, const int32_t *context_lens,
                                     const float *k_scale, const float *v_scale, float scale,
                                     int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                     int block_size, int64_t num_blocks, int max_context_len,
                                     int min_piece_tokens, pa_dtype q_dtype, pa_dtype cache_dtype,
                                     void *stream);

/*
 * pa_copy_blocks -- the copy step of copy-on-write block sharing
 * ("Continuous-Batching-LLM-Inference-Engine" README, feature list: the paged
 * KV cache's block pool with copy-on-write reference counts): before a
 * sequence writes into a block it shares, the block manager gives it a private
 * copy. For each pair i, every byte of physical block block_mapping[2i] of
 * k_cache and of v_cache (all kv heads) -- and, for an int8 cache, its
 * k_scale / v_scale entries -- is copied into block block_mapping[2i+1].
 *
 *   k_cache, v_cache  [num_blocks][num_kv_heads][block_size][head_dim], cache_dtype,
 *                     16-byte aligned, written in place.
 *   k_scale, v_scale  [num_blocks][num_kv_heads] fp32, int8 cache only (else ignored).
 *   block_mapping     [num_pairs][2] int64 (src, dst), device. Every id must be in
 *                     [0, num_blocks); no block may be the destination of two pairs,
 *                     both a source and a destination, or its own source (the
 *                     copies then do not depend on their order). PA_CHECK=1 verifies.
 * head_dim * element size must be a multiple of 16 bytes; num_pairs <= 65535.
 * Enqueued on `stream`; num_pairs = 0 does nothing. Rolling a sequence back
 * (e.g. rejected draft tokens) needs no device work: the caller lowers its
 * context length and releases the blocks past it.
 */
int pa_copy_blocks(void *k_cache, void *v_cache, float *k_scale, float *v_scale,
                   const int64_t *block_mapping, int num_pairs, int num_kv_heads, int head_dim,
                   int block_size, int64_t num_blocks, pa_dtype cache_dtype, void *stream);

/*
 * pa_prefill -- attention of several new query tokens per sequence over its
 * paged context: the target model scoring K drafted tokens in one batched
 * pass for speculative decoding (Continuous-Batching-LLM-Inference-Engine
 * README, feature list; the verify pass has K + 1 query tokens) and the
 * prefill chunks that continuous batches mix with decode tokens ("How
 * brave30/mini-inference-engine works", summary; Model Compute: prefill
 * attention). The new tokens' K/V are already in the cache (pa_write_kv_cache
 * with one slot per new token), and context_lens counts them.
 *
 * Sequence s owns rows qsl[s] .. qsl[s+1]-1 of q and out (qsl =
 * query_start_loc), n_s = qsl[s+1] - qsl[s] rows. Row qsl[s] + j is the new
 * token at position p = L_s - n_s + j and, for each query head h (kv head
 * h / (Hq / Hkv)), attends causally to the cached tokens 0 .. p:
 *   out[r][h][:] = sum_{t <= p} exp(x_t - max x) v_t / sum_{t <= p} exp(x_t - max x),
 *   x_t = scale * q[r][h] . k_t,
 * with k_t, v_t gathered through block_tables and dequantised as in pa_decode.
 * With n_s = 1 this is pa_decode of that sequence.
 *
 *   out             [num_query_tokens][num_heads][head_dim], q_dtype, 16-byte aligned;
 *                   written only when partition_size == 0
 *   q               [num_query_tokens][num_heads][head_dim], q_dtype
 *   k_cache, v_cache, block_tables, context_lens, k_scale, v_scale, scale:
 *                   as in pa_decode (context_lens[s] >= n_s)
 *   query_start_loc [num_seqs + 1] int32, device: 0 = qsl[0] <= qsl[1] <= ... <=
 *                   qsl[num_seqs] = num_query_tokens
 *   max_query_len   host-side bound on every n_s, at most max_context_len; it sizes
 *                   the launch (rows of sequences with more are not written)
 *   partition_size  0: one pass, result in `out`. > 0 (a multiple of 32): split-K
 *                   over each row's tokens. Partition j of row r (position p) covers
 *                   tokens [j P, min(p + 1, (j+1) P)) and stores, for j < ceil((p+1)/P),
 *                     tmp_out[r][h][j][:] = its normalised output,
 *                     tmp_max[r][h][j] = a reference max in natural units (at most
 *                                        ln 256 below its largest logit),
 *                     tmp_sum[r][h][j] = sum_t exp(x_t - tmp_max),
 *                   and row_lens[r] = p + 1; `out` is not touched. Then
 *                   pa_decode_splitk_reduce(out, tmp_out, tmp_max, tmp_sum, row_lens,
 *                   num_query_tokens, num_heads, head_dim, max_context_len,
 *                   partition_size, q_dtype, stream) gives the result: it treats each
 *                   query row as a sequence of length p + 1.
 *   tmp_out         [num_query_tokens][num_heads][NP][head_dim] fp32 (16-byte aligned),
 *   tmp_max, tmp_sum  [num_query_tokens][num_heads][NP] fp32, row_lens
 *                   [num_query_tokens] int32, NP = pa_num_partitions(max_context_len,
 *                   partition_size): caller-owned workspace, required iff
 *                   partition_size > 0 (and num_query_tokens > 0).
 * Precision: Q K^T and P V run on bf16 MFMAs with fp32 accumulation; the
 * softmax weights are rounded to bf16 for the P V product, and each row's sum
 * is the sum of those same bf16 weights. int8 caches: codes convert exactly to
 * bf16; the K scale multiplies the logits and the V scale multiplies, in fp32,
 * the P V product of the 16 tokens of its block.
 * Supported instances (others return PA_ERR_UNSUPPORTED): q BF16; cache BF16 or
 * I8; head_dim 128; block_size 16 or 32; group size Hq / Hkv in {1, 2, 4, 8, 16}.
 * num_seqs and num_kv_heads <= 65535. num_query_tokens = 0 does nothing (q and out
 * may then be NULL).
 * PA_CHECK=1 also verifies query_start_loc and n_s <= min(max_query_len, L_s).
 */
int pa_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
               const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
               const int32_t *query_start_loc, const float *k_scale, const float *v_scale,
               float scale, int num_seqs, int num_query_tokens, int max_query_len,
               int num_heads, int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
               int max_context_len, int partition_size, float *tmp_out, float *tmp_max,
               float *tmp_sum, int32_t *row_lens, pa_dtype q_dtype, pa_dtype cache_dtype,
               void *stream);

/*
 * pa_write_prefill -- pa_write_kv_cache of the new tokens followed by
 * pa_prefill, in one launch. Row r = qsl[s] + j of key and value (the layout of
 * q: [num_query_tokens][num_kv_heads][head_dim], q_dtype) is new token j of
 * sequence s, at position L_s - n_s + j, and goes to slot slot_mapping[r]
 * (int64). The kernel reads the positions of tokens with a slot >= 0 from key
 * and value, never from the cache, and stores them to their slots, so the
 * cache holds them afterwards exactly as after pa_write_kv_cache. A token with
 * a negative slot is not written, and its position is read from the cache as
 * it stands. With an int8 cache the kernel stores each new token's codes
 * under the scales of its (block, kv head), k_scale / v_scale as in
 * pa_write_kv_cache, and quantises the positions it reads from key and value
 * the same way, so the attention sees the codes the cache then holds. Result
 * and pool are therefore bit-identical to pa_write_kv_cache followed by
 * pa_prefill. context_lens counts the new tokens. Other arguments and the
 * split-K option as in pa_prefill.
 * Supported: bf16 q, key and value; bf16 or int8 cache (k_scale and v_scale
 * required for int8, ignored for bf16). key and value 16-byte aligned;
 * PA_CHECK=1 also verifies each slot against its position (the kernel takes
 * a new token's scale from the block its position maps to, the block of its
 * slot when the two agree).
 */
int pa_write_prefill(const void *key, const void *value, const int64_t *slot_mapping, void *out,
                     const void *q, void *k_cache, void *v_cache, const int32_t *block_tables,
                     int max_blocks_per_seq, const int32_t *context_lens,
                     const int32_t *query_start_loc, const float *k_scale,
                     const float *v_scale, float scale, int num_seqs,
                     int num_query_tokens, int max_query_len, int num_heads, int num_kv_heads,
                     int head_dim, int block_size, int64_t num_blocks, int max_context_len,
                     int partition_size, float *tmp_out, float *tmp_max, float *tmp_sum,
                     int32_t *row_lens, pa_dtype q_dtype, pa_dtype cache_dtype, void *stream);

/*
 * pa_balanced_workspace -- sizes of the workspace that pa_decode_balanced and
 * pa_write_decode_balanced need for these shapes on the device of `stream`
 * (any dtypes): *slots partial-state slots, i.e. tmp_out [*slots][G][head_dim]
 * and tmp_max, tmp_sum [*slots][G] fp32 with G = num_heads / num_kv_heads,
 * and *counters int32 counters (num_seqs * num_kv_heads). The slots grow
 * with the device (4 per wave of the persistent grid, 8 at G = 8, whose
 * partial states may cover a pair of sequences), not with the context
 * lengths. Returns PA_OK, PA_ERR_NULL,
 * PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (no balanced instance for head_dim and G)
 * or PA_ERR_LAUNCH (the runtime could not report the device's occupancy).
 * Allocates nothing; the caller allocates and zeroes the counters once.
 */
int pa_balanced_workspace(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                          void *stream, int64_t *slots, int64_t *counters);

/*
 * pa_decode_splitk_reduce -- log-sum-exp combination of split-K partials.
 * The pages define no long-context split: the partition of each context into
 * fixed-size pieces and this exact combination of their (normalised output,
 * max, sum) triples are the flash-decoding split-K that the decode step's
 * specification adds for long contexts; the formula is the merge of two
 * softmax states over disjoint token sets, applied to all of them at once.
 * For each (s, h), over j < n = ceil(L_s / partition_size):
 *   M = max_j tmp_max[j], W_j = tmp_sum[j] * exp(tmp_max[j] - M),
 *   out[s][h][:] = sum_j W_j tmp_out[j][:] / sum_j W_j      (0 when n = 0),
 * rounded to out_dtype (F32 or BF16, round to nearest even).
 * Arguments as in pa_decode; head_dim in [1, 1024].
 */
int pa_decode_splitk_reduce(void *out, const float *tmp_out, const float *tmp_max,
                            const float *tmp_sum, const int32_t *context_lens, int num_seqs,
                            int num_heads, int head_dim, int max_context_len, int partition_size,
                            pa_dtype out_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
