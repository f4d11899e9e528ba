// Arguments and launcher of the multi-query kernel (pa_prefill.hip): several
// new query tokens per sequence, attending causally to the paged context.
#pragma once

#include "pa_kernels.hpp"

namespace pa {

// Several new query tokens per sequence (prefill chunks, speculative verify).
struct PrefillArgs {
    void* out;                       // [T][Hq][D], q dtype
    const void* q;                   // [T][Hq][D]
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;     // [S], counts the new tokens
    const int32_t* query_start_loc;  // [S + 1]: rows of sequence s are [qsl[s], qsl[s+1])
    const float* k_scale;
    const float* v_scale;
    float scale;
    int num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
    int max_query_len;               // bound on every qsl[s+1] - qsl[s]
    Dtype q_dtype, cache;
    // split-K (partition_size > 0, a multiple of 32): partition j of a row's
    // tokens goes to slot (row * Hq + h) * num_partitions + j of the
    // workspace, and row_lens[row] = position + 1 (the reduce's lengths)
    int partition_size = 0, num_partitions = 1;
    float* tmp_out = nullptr;
    float* tmp_max = nullptr;
    float* tmp_sum = nullptr;
    int32_t* row_lens = nullptr;
    // The new tokens' K/V written by the kernel itself (key == nullptr: they are
    // already in the cache): rows [qsl[s], qsl[s+1]) of key / value [T][Hkv][D]
    // (q dtype) are the n_s newest tokens of sequence s, going to slots
    // slot_mapping[row]; their positions are read from key / value, never from
    // the cache. bf16 or int8 caches (int8: the codes under k_scale / v_scale
    // of the token's block).
    const void* key = nullptr;
    const void* value = nullptr;
    const int64_t* slot_mapping = nullptr;
    void* k_cache_w = nullptr;       // k_cache / v_cache, writable
    void* v_cache_w = nullptr;
    int row_tiles = 0;               // set by the launcher: row tiles per (sequence, kv head)
    int one_round = 0;               // set by the launcher: every workgroup resident at once
};

bool prefill_supports(const PrefillArgs& a);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);

}  // namespace pa
