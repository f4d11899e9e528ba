// Internal launch interface between the C ABI (pa_api.cpp) and the kernels.
// Arguments have been validated by the caller; launchers only enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum Dtype : int { F32 = 0, BF16 = 1, I8 = 2 };

struct WriteArgs {
    const void* key;
    const void* value;
    void* k_cache;
    void* v_cache;
    const int64_t* slot_mapping;
    const float* k_scale;
    const float* v_scale;
    int num_tokens, num_kv_heads, head_dim, block_size;
    Dtype act, cache;
};

struct DecodeArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const float* k_scale;
    const float* v_scale;
    float* tmp_out;
    float* tmp_max;
    float* tmp_sum;
    int32_t* counters;    // balanced mode only: [S][Hkv] segment counters, then the
                          // schedule's claims; all zero on entry and exit
    float scale;
    int num_seqs, num_heads, num_kv_heads, head_dim, block_size;
    int max_blocks_per_seq;
    int max_context_len;  // bound on every context length
    int partition_size;   // 0 = one pass; else partition / minimum piece, tokens
    int num_partitions;   // workspace slots per (s, h) (1 for one pass)
    Dtype q_dtype, cache;
    // New tokens written by the balanced decode itself (null: none): token s of
    // key / value [S][Hkv][D] (q dtype) goes to slot slot_mapping[s].
    const void* key = nullptr;
    const void* value = nullptr;
    const int64_t* slot_mapping = nullptr;
};

struct CopyArgs {
    void* k_cache;
    void* v_cache;
    float* k_scale;          // int8 cache: [NB][Hkv], copied with the blocks; else null
    float* v_scale;
    const int64_t* block_mapping;   // [num_pairs][2] (src, dst)
    int num_pairs, num_kv_heads;
    int64_t block_bytes;     // bytes of one block of one pool, a multiple of 16
};

struct ReduceArgs {
    void* out;
    const float* tmp_out;
    const float* tmp_max;
    const float* tmp_sum;
    const int32_t* context_lens;
    int num_seqs, num_heads, head_dim, partition_size, num_partitions;
    Dtype out_dtype;
};

enum class Schedule { Partitions, Balanced };

hipError_t launch_write_kv(const WriteArgs& a, hipStream_t st);
// Returns hipErrorNotSupported when no instance covers the arguments.
hipError_t launch_decode_valu(const DecodeArgs& a, Schedule sch, hipStream_t st);
hipError_t launch_decode_mfma(const DecodeArgs& a, Schedule sch, hipStream_t st);
// Workgroups of a balanced launch: resident workgroups per CU times CUs.
int balanced_grid(const void* kernel, int threads, hipStream_t st);
// Most waves any balanced instance for (head_dim, G) runs on the stream's
// device (0: no instance; < 0: the runtime failed).
int balanced_waves_valu(int head_dim, int G, hipStream_t st);
int balanced_waves_mfma(int head_dim, int G, hipStream_t st);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t st);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t st);

bool valu_supports(const DecodeArgs& a);
bool mfma_supports(const DecodeArgs& a);

}  // namespace pa
