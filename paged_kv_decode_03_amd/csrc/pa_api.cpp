// C ABI of libpa.so: argument validation, kernel-instance selection and
// launch on the caller's stream. Declarations and the contract of every entry
// point are in include/pa.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "pa.h"
#include "pa_kernels.hpp"
#include "pa_prefill.hpp"

namespace {

constexpr int kVersion = 10100;   // 1.1.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_act(pa_dtype d) { return d == PA_F32 || d == PA_BF16; }
bool valid_cache(pa_dtype d) { return d == PA_F32 || d == PA_BF16 || d == PA_I8; }

int launch_status(hipError_t e) {
    if (e == hipSuccess) return PA_OK;
    if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
    return PA_ERR_LAUNCH;
}

bool check_enabled() {
    const char* v = std::getenv("PA_CHECK");
    return v && v[0] == '1';
}

// Copy n elements of a device array to the host (synchronous, debug path).
template <typename T>
bool fetch(std::vector<T>& host, const T* dev, int64_t n, hipStream_t st) {
    host.resize((size_t)n);
    if (n == 0) return true;
    if (hipStreamSynchronize(st) != hipSuccess) return false;
    return hipMemcpy(host.data(), dev, sizeof(T) * (size_t)n, hipMemcpyDeviceToHost) == hipSuccess;
}

// Shared validation of the decode arguments (both schedules).
int check_decode(const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                 const float* k_scale, const float* v_scale, int num_seqs, int num_heads,
                 int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                 int max_context_len, int partition_size, pa_dtype q_dtype, pa_dtype cache_dtype) {
    if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads ||
        head_dim < 1 || block_size < 1 || max_blocks_per_seq < 1 || num_blocks < 1 ||
        max_context_len < 0 || partition_size < 0)
        return PA_ERR_SHAPE;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_SHAPE;
    if (!valid_act(q_dtype) || !valid_cache(cache_dtype)) return PA_ERR_DTYPE;
    if (cache_dtype != PA_I8 && cache_dtype != q_dtype) return PA_ERR_DTYPE;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
    if (cache_dtype == PA_I8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
    return PA_OK;
}

// PA_CHECK=1: device indices against the pool and the length bound.
int check_indices(const int32_t* block_tables, int max_blocks_per_seq,
                  const int32_t* context_lens, int num_seqs, int block_size, int64_t num_blocks,
                  int max_context_len, hipStream_t st) {
    std::vector<int32_t> lens, tables;
    if (!fetch(lens, context_lens, num_seqs, st) ||
        !fetch(tables, block_tables, (int64_t)num_seqs * max_blocks_per_seq, st))
        return PA_ERR_LAUNCH;
    for (int s = 0; s < num_seqs; ++s) {
        if (lens[s] < 0 || lens[s] > max_context_len) return PA_ERR_INDEX;
        const int nb = (lens[s] + block_size - 1) / block_size;
        for (int b = 0; b < nb; ++b) {
            const int32_t id = tables[(size_t)s * max_blocks_per_seq + b];
            if (id < 0 || id >= num_blocks) return PA_ERR_INDEX;
        }
    }
    return PA_OK;
}

// PA_CHECK=1, decodes that write the new tokens: slot s in the pool, and, for a
// non-empty context, the slot of logical position L_s - 1 of sequence s.
int check_new_slots(const int64_t* slot_mapping, const int32_t* block_tables,
                    int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                    int block_size, int64_t num_blocks, hipStream_t st) {
    std::vector<int64_t> slots;
    std::vector<int32_t> lens, tables;
    if (!fetch(slots, slot_mapping, num_seqs, st) || !fetch(lens, context_lens, num_seqs, st) ||
        !fetch(tables, block_tables, (int64_t)num_seqs * max_blocks_per_seq, st))
        return PA_ERR_LAUNCH;
    for (int s = 0; s < num_seqs; ++s) {
        const int64_t sl = slots[s];
        if (sl < 0) continue;
        if (sl / block_size >= num_blocks) return PA_ERR_INDEX;
        if (lens[s] > 0) {
            const int t = lens[s] - 1;
            const int64_t want =
                (int64_t)tables[(size_t)s * max_blocks_per_seq + t / block_size] * block_size +
                t % block_size;
            if (sl != want) return PA_ERR_INDEX;
        }
    }
    return PA_OK;
}

// PA_CHECK=1, block copies: every id in [0, num_blocks); no destination
// twice, none also a source, none its own source.
int check_copy_mapping(const int64_t* block_mapping, int num_pairs, int64_t num_blocks,
                       hipStream_t st) {
    std::vector<int64_t> m;
    if (!fetch(m, block_mapping, 2 * (int64_t)num_pairs, st)) return PA_ERR_LAUNCH;
    std::map<int64_t, int> role;                     // 1 source, 2 destination
    for (int i = 0; i < num_pairs; ++i) {
        const int64_t src = m[2 * i], dst = m[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst)
            return PA_ERR_INDEX;
        role[src] |= 1;
    }
    for (int i = 0; i < num_pairs; ++i) {
        int& r = role[m[2 * i + 1]];
        if (r) return PA_ERR_INDEX;
        r = 2;
    }
    return PA_OK;
}

// PA_CHECK=1, several query tokens per sequence: query_start_loc runs from 0
// to num_query_tokens without decreasing, and every count n_s is at most
// max_query_len and at most L_s.
int check_query_starts(const int32_t* query_start_loc, const int32_t* context_lens,
                       int num_seqs, int num_query_tokens, int max_query_len, hipStream_t st) {
    std::vector<int32_t> qsl, lens;
    if (!fetch(qsl, query_start_loc, (int64_t)num_seqs + 1, st) ||
        !fetch(lens, context_lens, num_seqs, st))
        return PA_ERR_LAUNCH;
    if (qsl[0] != 0 || qsl[num_seqs] != num_query_tokens) return PA_ERR_INDEX;
    for (int s = 0; s < num_seqs; ++s) {
        const int n = qsl[s + 1] - qsl[s];
        if (n < 0 || n > max_query_len || n > lens[s]) return PA_ERR_INDEX;
    }
    return PA_OK;
}

// PA_CHECK=1, prefill steps that write their new tokens: each row's slot is
// negative (skipped) or the slot of its position L_s - n_s + j.
int check_prefill_slots(const int64_t* slot_mapping, const int32_t* query_start_loc,
                        const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* context_lens, int num_seqs, int num_query_tokens,
                        int block_size, hipStream_t st) {
    std::vector<int64_t> slots;
    std::vector<int32_t> qsl, lens, tables;
    if (!fetch(slots, slot_mapping, num_query_tokens, st) ||
        !fetch(qsl, query_start_loc, (int64_t)num_seqs + 1, st) ||
        !fetch(lens, context_lens, num_seqs, st) ||
        !fetch(tables, block_tables, (int64_t)num_seqs * max_blocks_per_seq, st))
        return PA_ERR_LAUNCH;
    for (int s = 0; s < num_seqs; ++s) {
        const int n = qsl[s + 1] - qsl[s];
        for (int j = 0; j < n; ++j) {
            const int64_t sl = slots[(size_t)qsl[s] + j];
            if (sl < 0) continue;
            const int t = lens[s] - n + j;
            const int64_t want =
                (int64_t)tables[(size_t)s * max_blocks_per_seq + t / block_size] * block_size +
                t % block_size;
            if (sl != want) return PA_ERR_INDEX;
        }
    }
    return PA_OK;
}

}  // namespace

namespace pa {

// Resident workgroups per CU (occupancy calculator) times the CU count of the
// stream's device, remembered per (kernel, device).
int balanced_grid(const void* kernel, int threads, hipStream_t st) {
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, int> cache;
    int dev = 0;
    if (st ? hipStreamGetDevice(st, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
        return -1;
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = cache.find({kernel, dev});
        if (it != cache.end()) return it->second;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) !=
        hipSuccess)
        return -1;
    const int grid = cus * (per_cu > 0 ? per_cu : 1);
    std::lock_guard<std::mutex> lk(mu);
    cache[{kernel, dev}] = grid;
    return grid;
}

}  // namespace pa

extern "C" {

int pa_version(void) { return kVersion; }

const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "a required pointer is NULL";
        case PA_ERR_SHAPE: return "a size is out of range or inconsistent";
        case PA_ERR_DTYPE: return "unknown or unsupported dtype combination";
        case PA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case PA_ERR_UNSUPPORTED: return "no kernel instance covers these arguments";
        case PA_ERR_LAUNCH: return "the HIP runtime reported a launch error";
        case PA_ERR_INDEX: return "a device-side index is out of range (PA_CHECK)";
        default: return "unknown status";
    }
}

int pa_num_partitions(int max_context_len, int partition_size) {
    if (max_context_len <= 0 || partition_size <= 0) return 0;
    return (int)(((int64_t)max_context_len + partition_size - 1) / partition_size);
}

int pa_write_kv_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                      const int64_t* slot_mapping, const float* k_scale, const float* v_scale,
                      int num_tokens, int num_kv_heads, int head_dim, int block_size,
                      int64_t num_blocks, pa_dtype act_dtype, pa_dtype cache_dtype, void* stream) {
    if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 8 || head_dim > 1024 || head_dim % 8 ||
        block_size < 1 || num_blocks < 1)
        return PA_ERR_SHAPE;
    if (!valid_act(act_dtype) || !valid_cache(cache_dtype)) return PA_ERR_DTYPE;
    if (cache_dtype != PA_I8 && cache_dtype != act_dtype) return PA_ERR_DTYPE;
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
    if (cache_dtype == PA_I8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_ALIGN;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (check_enabled()) {
        std::vector<int64_t> slots;
        if (!fetch(slots, slot_mapping, num_tokens, st)) return PA_ERR_LAUNCH;
        for (int64_t sl : slots) {
            if (sl < 0) continue;
            if (sl / block_size >= num_blocks) return PA_ERR_INDEX;
        }
    }
    pa::WriteArgs a{key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale,
                    num_tokens, num_kv_heads, head_dim, block_size,
                    (pa::Dtype)act_dtype, (pa::Dtype)cache_dtype};
    return launch_status(pa::launch_write_kv(a, st));
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
              const float* k_scale, const float* v_scale, float scale, int num_seqs,
              int num_heads, int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
              int max_context_len, int partition_size, float* tmp_out, float* tmp_max,
              float* tmp_sum, pa_dtype q_dtype, pa_dtype cache_dtype, void* stream) {
    int rc = check_decode(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                          k_scale, v_scale, num_seqs, num_heads, num_kv_heads, head_dim,
                          block_size, num_blocks, max_context_len, partition_size, q_dtype,
                          cache_dtype);
    if (rc) return rc;
    if (partition_size > 0 && partition_size % block_size) return PA_ERR_SHAPE;
    const bool split = partition_size > 0;
    if (split ? (!tmp_out || !tmp_max || !tmp_sum) : !out) return PA_ERR_NULL;
    if (split ? !aligned16(tmp_out) : !aligned16(out)) return PA_ERR_ALIGN;
    const int np = split ? pa_num_partitions(max_context_len, partition_size) : 1;

    pa::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                     tmp_out, tmp_max, tmp_sum, nullptr, scale, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len,
                     partition_size, np, (pa::Dtype)q_dtype, (pa::Dtype)cache_dtype};
    const bool mfma = pa::mfma_supports(a);
    if (!mfma && !pa::valu_supports(a)) return PA_ERR_UNSUPPORTED;
    const int64_t nwg = (int64_t)num_kv_heads * num_seqs * np;
    if (nwg > 0x7fffffff) return PA_ERR_SHAPE;
    if (num_seqs == 0 || np == 0) return PA_OK;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (check_enabled()) {
        rc = check_indices(block_tables, max_blocks_per_seq, context_lens, num_seqs, block_size,
                           num_blocks, max_context_len, st);
        if (rc) return rc;
    }
    const pa::Schedule sch = pa::Schedule::Partitions;
    return launch_status(mfma ? pa::launch_decode_mfma(a, sch, st)
                              : pa::launch_decode_valu(a, sch, st));
}

int pa_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                   const int64_t* block_mapping, int num_pairs, int num_kv_heads, int head_dim,
                   int block_size, int64_t num_blocks, pa_dtype cache_dtype, void* stream) {
    if (num_pairs < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
        return PA_ERR_SHAPE;
    if (!valid_cache(cache_dtype)) return PA_ERR_DTYPE;
    const int elt = cache_dtype == PA_F32 ? 4 : cache_dtype == PA_BF16 ? 2 : 1;
    if (((int64_t)head_dim * elt) % 16) return PA_ERR_SHAPE;
    if (!k_cache || !v_cache || (num_pairs > 0 && !block_mapping)) return PA_ERR_NULL;
    if (cache_dtype == PA_I8 && (!k_scale || !v_scale)) return PA_ERR_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
    if (num_pairs > 65535) return PA_ERR_SHAPE;      // one grid row per pair
    if (num_pairs == 0) return PA_OK;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (check_enabled()) {
        const int rc = check_copy_mapping(block_mapping, num_pairs, num_blocks, st);
        if (rc) return rc;
    }
    pa::CopyArgs a{k_cache, v_cache, cache_dtype == PA_I8 ? k_scale : nullptr,
                   cache_dtype == PA_I8 ? v_scale : nullptr, block_mapping, num_pairs,
                   num_kv_heads, (int64_t)num_kv_heads * block_size * head_dim * elt};
    return launch_status(pa::launch_copy_blocks(a, st));
}

}  // extern "C"

namespace {

// pa_prefill, optionally writing the new tokens first (key != NULL).
int prefill(const void* key, const void* value, const int64_t* slot_mapping, void* out,
            const void* q, const void* k_cache, const void* v_cache,
            const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
            const int32_t* query_start_loc, const float* k_scale, const float* v_scale,
            float scale, int num_seqs, int num_query_tokens, int max_query_len, int num_heads,
            int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
            int max_context_len, int partition_size, float* tmp_out, float* tmp_max,
            float* tmp_sum, int32_t* row_lens, pa_dtype q_dtype, pa_dtype cache_dtype,
            void* stream);

}  // namespace

extern "C" {

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
               const int32_t* query_start_loc, const float* k_scale, const float* v_scale,
               float scale, int num_seqs, int num_query_tokens, int max_query_len,
               int num_heads, int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
               int max_context_len, int partition_size, float* tmp_out, float* tmp_max,
               float* tmp_sum, int32_t* row_lens, pa_dtype q_dtype, pa_dtype cache_dtype,
               void* stream) {
    return prefill(nullptr, nullptr, nullptr, out, q, k_cache, v_cache, block_tables,
                   max_blocks_per_seq, context_lens, query_start_loc, k_scale, v_scale, scale,
                   num_seqs, num_query_tokens, max_query_len, num_heads, num_kv_heads, head_dim,
                   block_size, num_blocks, max_context_len, partition_size, tmp_out, tmp_max,
                   tmp_sum, row_lens, q_dtype, cache_dtype, stream);
}

int pa_write_prefill(const void* key, const void* value, const int64_t* slot_mapping, void* out,
                     const void* q, void* k_cache, void* v_cache, const int32_t* block_tables,
                     int max_blocks_per_seq, const int32_t* context_lens,
                     const int32_t* query_start_loc, const float* k_scale,
                     const float* v_scale, float scale, int num_seqs,
                     int num_query_tokens, int max_query_len, int num_heads, int num_kv_heads,
                     int head_dim, int block_size, int64_t num_blocks, int max_context_len,
                     int partition_size, float* tmp_out, float* tmp_max, float* tmp_sum,
                     int32_t* row_lens, pa_dtype q_dtype, pa_dtype cache_dtype, void* stream) {
    if (num_query_tokens > 0) {
        if (!key || !value || !slot_mapping) return PA_ERR_NULL;
        if (!aligned16(key) || !aligned16(value)) return PA_ERR_ALIGN;
    }
    return prefill(num_query_tokens > 0 ? key : nullptr, value, slot_mapping, out, q, k_cache,
                   v_cache, block_tables, max_blocks_per_seq, context_lens, query_start_loc,
                   k_scale, v_scale, scale, num_seqs, num_query_tokens, max_query_len, num_heads,
                   num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                   partition_size, tmp_out, tmp_max, tmp_sum, row_lens, q_dtype, cache_dtype,
                   stream);
}

}  // extern "C"

namespace {

int prefill(const void* key, const void* value, const int64_t* slot_mapping, void* out,
            const void* q, const void* k_cache, const void* v_cache,
            const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
            const int32_t* query_start_loc, const float* k_scale, const float* v_scale,
            float scale, int num_seqs, int num_query_tokens, int max_query_len, int num_heads,
            int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
            int max_context_len, int partition_size, float* tmp_out, float* tmp_max,
            float* tmp_sum, int32_t* row_lens, pa_dtype q_dtype, pa_dtype cache_dtype,
            void* stream) {
    // with no query rows, q and out are never read and may be NULL
    const void* qc = num_query_tokens == 0 && !q ? k_cache : q;
    int rc = check_decode(qc, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                          k_scale, v_scale, num_seqs, num_heads, num_kv_heads, head_dim,
                          block_size, num_blocks, max_context_len, 0, q_dtype, cache_dtype);
    if (rc) return rc;
    if (num_query_tokens < 0 || max_query_len < 0 || max_query_len > max_context_len ||
        num_seqs > 65535 || num_kv_heads > 65535 ||
        (int64_t)max_query_len * (num_heads / num_kv_heads) > 0x7fffffff)
        return PA_ERR_SHAPE;
    if (partition_size < 0 || (partition_size > 0 && partition_size % 32)) return PA_ERR_SHAPE;
    if (!query_start_loc) return PA_ERR_NULL;
    const bool split = partition_size > 0;
    if (num_query_tokens > 0) {
        if (!split && !out) return PA_ERR_NULL;
        if (!split && !aligned16(out)) return PA_ERR_ALIGN;
        if (split && (!tmp_out || !tmp_max || !tmp_sum || !row_lens)) return PA_ERR_NULL;
        if (split && !aligned16(tmp_out)) return PA_ERR_ALIGN;
    }
    pa::PrefillArgs a{out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                      k_scale, v_scale, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                      block_size, max_blocks_per_seq, max_query_len, (pa::Dtype)q_dtype,
                      (pa::Dtype)cache_dtype};
    if (split) {
        a.partition_size = partition_size;
        a.num_partitions = pa_num_partitions(max_context_len, partition_size);
        if (a.num_partitions < 1) a.num_partitions = 1;
        a.tmp_out = tmp_out;
        a.tmp_max = tmp_max;
        a.tmp_sum = tmp_sum;
        a.row_lens = row_lens;
    }
    if (key) {
        a.key = key;
        a.value = value;
        a.slot_mapping = slot_mapping;
        a.k_cache_w = const_cast<void*>(k_cache);     // pa_write_prefill's pool is writable
        a.v_cache_w = const_cast<void*>(v_cache);
    }
    if (!pa::prefill_supports(a)) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || num_query_tokens == 0) return PA_OK;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (check_enabled()) {
        rc = check_indices(block_tables, max_blocks_per_seq, context_lens, num_seqs, block_size,
                           num_blocks, max_context_len, st);
        if (rc) return rc;
        rc = check_query_starts(query_start_loc, context_lens, num_seqs, num_query_tokens,
                                max_query_len, st);
        if (rc) return rc;
        if (key) {
            rc = check_prefill_slots(slot_mapping, query_start_loc, block_tables,
                                     max_blocks_per_seq, context_lens, num_seqs,
                                     num_query_tokens, block_size, st);
            if (rc) return rc;
        }
    }
    return launch_status(pa::launch_prefill(a, st));
}

}  // namespace

extern "C" {

int pa_balanced_workspace(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                          void* stream, int64_t* slots, int64_t* counters) {
    if (!slots || !counters) return PA_ERR_NULL;
    if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads ||
        head_dim < 1)
        return PA_ERR_SHAPE;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int G = num_heads / num_kv_heads;
    const int wv = pa::balanced_waves_valu(head_dim, G, st);
    const int wm = pa::balanced_waves_mfma(head_dim, G, st);
    if (wv < 0 || wm < 0) return PA_ERR_LAUNCH;
    const int waves = wv > wm ? wv : wm;
    if (waves == 0) return PA_ERR_UNSUPPORTED;
    // 4 partial states per wave; at G = 8 the 16x16 core's states may cover
    // two sequences (pair units), so twice as many slots of G heads
    *slots = (G == 8 ? 8 : 4) * (int64_t)waves;
    *counters = (int64_t)num_seqs * num_kv_heads;
    return PA_OK;
}

}  // extern "C"

namespace {

// pa_decode_balanced, optionally writing the new tokens first (key != NULL).
int balanced(const void* key, const void* value, const int64_t* slot_mapping, void* out,
             const void* q, const void* k_cache, const void* v_cache,
             const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
             const float* k_scale, const float* v_scale, float scale, int num_seqs, int num_heads,
             int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
             int max_context_len, int min_piece_tokens, float* tmp_out, float* tmp_max,
             float* tmp_sum, int32_t* counters, pa_dtype q_dtype, pa_dtype cache_dtype,
             void* stream) {
    int rc = check_decode(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                          k_scale, v_scale, num_seqs, num_heads, num_kv_heads, head_dim,
                          block_size, num_blocks, max_context_len, min_piece_tokens, q_dtype,
                          cache_dtype);
    if (rc) return rc;
    if (min_piece_tokens < 16 || min_piece_tokens % 16) return PA_ERR_SHAPE;
    if (!out || !tmp_out || !tmp_max || !tmp_sum || !counters) return PA_ERR_NULL;
    if (!aligned16(out) || !aligned16(tmp_out)) return PA_ERR_ALIGN;
    const bool write = slot_mapping != nullptr;
    if (write) {
        if (head_dim % 8) return PA_ERR_SHAPE;
        if (!key || !value) return PA_ERR_NULL;
        if (!aligned16(key) || !aligned16(value)) return PA_ERR_ALIGN;
    }
    pa::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                     tmp_out, tmp_max, tmp_sum, counters, scale, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len,
                     min_piece_tokens, 1, (pa::Dtype)q_dtype, (pa::Dtype)cache_dtype};
    const bool mfma = pa::mfma_supports(a);
    if (!mfma && !pa::valu_supports(a)) return PA_ERR_UNSUPPORTED;
    if ((int64_t)num_kv_heads * (((int64_t)max_context_len + 15) / 16) * num_seqs > 0x7fffffff)
        return PA_ERR_SHAPE;
    if (num_seqs == 0) return PA_OK;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (check_enabled()) {
        rc = check_indices(block_tables, max_blocks_per_seq, context_lens, num_seqs, block_size,
                           num_blocks, max_context_len, st);
        if (rc) return rc;
        if (write) {
            rc = check_new_slots(slot_mapping, block_tables, max_blocks_per_seq, context_lens,
                                 num_seqs, block_size, num_blocks, st);
            if (rc) return rc;
        }
    }
    const pa::Schedule sch = pa::Schedule::Balanced;
    if (write && mfma) {                             // one launch: the decode writes the tokens
        a.key = key;
        a.value = value;
        a.slot_mapping = slot_mapping;
        return launch_status(pa::launch_decode_mfma(a, sch, st));
    }
    if (write) {                                     // the write kernel, then the decode
        pa::WriteArgs w{key, value, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                        slot_mapping, k_scale, v_scale, num_seqs, num_kv_heads, head_dim,
                        block_size, (pa::Dtype)q_dtype, (pa::Dtype)cache_dtype};
        rc = launch_status(pa::launch_write_kv(w, st));
        if (rc) return rc;
    }
    return launch_status(mfma ? pa::launch_decode_mfma(a, sch, st)
                              : pa::launch_decode_valu(a, sch, st));
}

}  // namespace

extern "C" {

int pa_decode_balanced(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* context_lens, const float* k_scale, const float* v_scale,
                       float scale, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                       int block_size, int64_t num_blocks, int max_context_len,
                       int min_piece_tokens, float* tmp_out, float* tmp_max, float* tmp_sum,
                       int32_t* counters, pa_dtype q_dtype, pa_dtype cache_dtype, void* stream) {
    return balanced(nullptr, nullptr, nullptr, out, q, k_cache, v_cache, block_tables,
                    max_blocks_per_seq, context_lens, k_scale, v_scale, scale, num_seqs, num_heads,
                    num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                    min_piece_tokens, tmp_out, tmp_max, tmp_sum, counters, q_dtype, cache_dtype,
                    stream);
}

int pa_write_decode_balanced(const void* key, const void* value, const int64_t* slot_mapping,
                             void* out, const void* q, void* k_cache, void* v_cache,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, const float* k_scale,
                             const float* v_scale, float scale, int num_seqs, int num_heads,
                             int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                             int max_context_len, int min_piece_tokens, float* tmp_out,
                             float* tmp_max, float* tmp_sum, int32_t* counters, pa_dtype q_dtype,
                             pa_dtype cache_dtype, void* stream) {
    if (num_seqs > 0 && !slot_mapping) return PA_ERR_NULL;
    return balanced(key, value, slot_mapping, out, q, k_cache, v_cache, block_tables,
                    max_blocks_per_seq, context_lens, k_scale, v_scale, scale, num_seqs, num_heads,
                    num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                    min_piece_tokens, tmp_out, tmp_max, tmp_sum, counters, q_dtype, cache_dtype,
                    stream);
}

int pa_decode_splitk_reduce(void* out, const float* tmp_out, const float* tmp_max,
                            const float* tmp_sum, const int32_t* context_lens, int num_seqs,
                            int num_heads, int head_dim, int max_context_len, int partition_size,
                            pa_dtype out_dtype, void* stream) {
    if (num_seqs < 0 || num_heads < 1 || head_dim < 1 || head_dim > 1024 || max_context_len < 0 ||
        partition_size < 1)
        return PA_ERR_SHAPE;
    if (!valid_act(out_dtype)) return PA_ERR_DTYPE;
    if (num_seqs == 0) return PA_OK;
    const int np = pa_num_partitions(max_context_len, partition_size);
    if (!out || !context_lens || (np > 0 && (!tmp_out || !tmp_max || !tmp_sum))) return PA_ERR_NULL;
    if ((int64_t)num_seqs * num_heads > 0x7fffffff) return PA_ERR_SHAPE;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (check_enabled()) {
        std::vector<int32_t> lens;
        if (!fetch(lens, context_lens, num_seqs, st)) return PA_ERR_LAUNCH;
        for (int s = 0; s < num_seqs; ++s)
            if (lens[s] < 0 || lens[s] > max_context_len) return PA_ERR_INDEX;
    }
    pa::ReduceArgs a{out, tmp_out, tmp_max, tmp_sum, context_lens, num_seqs, num_heads, head_dim,
                     partition_size, np, (pa::Dtype)out_dtype};
    return launch_status(pa::launch_reduce(a, st));
}

}  // extern "C"

// ---- the decode step without a caller workspace ------------------------------
// The balanced step's workspace in a file-scope device array, one copy per GPU
// (each device that loads the library holds it until the process ends): the
// counters first (zeroed once per device, left zero by every call), then the
// partial states. In host code the array's name is only a stand-in: its device
// address, per device, comes from hipGetSymbolAddress and is used everywhere
// host code needs the memory.
namespace {

constexpr size_t kScratchBytes = size_t(72) << 20;           // 72 MiB per GPU
constexpr size_t kScratchCounters = size_t(1) << 18;         // int32 counters (1 MiB)
static __device__ __align__(256) char scratch[kScratchBytes];

__global__ void zero_ints(int32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// The scratch's device address on the stream's device, taken once per device
// (with that device current), its counters cleared by a kernel on the stream
// at that first call. nullptr: the runtime failed.
char* scratch_on(hipStream_t st) {
    static std::mutex mu;
    static std::map<int, char*> addr;
    int dev = 0;
    if (st ? hipStreamGetDevice(st, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
        return nullptr;
    std::lock_guard<std::mutex> lk(mu);
    auto it = addr.find(dev);
    if (it != addr.end()) return it->second;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return nullptr;
    hipLaunchKernelGGL(zero_ints, dim3(256), dim3(256), 0, st, reinterpret_cast<int32_t*>(ptr),
                       (int64_t)kScratchCounters);
    if (hipGetLastError() != hipSuccess) return nullptr;
    addr[dev] = reinterpret_cast<char*>(ptr);
    return addr[dev];
}

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace

extern "C" {

int pa_write_decode_balanced_noalloc(const void* key, const void* value,
                                     const int64_t* slot_mapping, void* out, const void* q,
                                     void* k_cache, void* v_cache, const int32_t* block_tables,
                                     int max_blocks_per_seq, const int32_t* context_lens,
                                     const float* k_scale, const float* v_scale, float scale,
                                     int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                     int block_size, int64_t num_blocks, int max_context_len,
                                     int min_piece_tokens, pa_dtype q_dtype, pa_dtype cache_dtype,
                                     void* stream) {
    if (num_seqs > 0 && !slot_mapping) return PA_ERR_NULL;
    if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads ||
        head_dim < 1)
        return PA_ERR_SHAPE;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int64_t slots = 0, counters = 0;
    int rc = pa_balanced_workspace(num_seqs, num_heads, num_kv_heads, head_dim, stream, &slots,
                                   &counters);
    if (rc) return rc;
    const size_t G = (size_t)(num_heads / num_kv_heads);
    const size_t out_bytes = round256((size_t)slots * G * (size_t)head_dim * 4);
    const size_t ml_bytes = round256((size_t)slots * G * 4);
    if ((size_t)counters > kScratchCounters ||
        kScratchCounters * 4 + out_bytes + 2 * ml_bytes > kScratchBytes)
        return PA_ERR_SHAPE;                         // beyond the static scratch
    char* base = scratch_on(st);
    if (!base) return PA_ERR_LAUNCH;
    int32_t* cnt = reinterpret_cast<int32_t*>(base);
    float* tmp_out = reinterpret_cast<float*>(base + kScratchCounters * 4);
    float* tmp_max = reinterpret_cast<float*>(base + kScratchCounters * 4 + out_bytes);
    float* tmp_sum = reinterpret_cast<float*>(base + kScratchCounters * 4 + out_bytes + ml_bytes);
    return balanced(key, value, slot_mapping, out, q, k_cache, v_cache, block_tables,
                    max_blocks_per_seq, context_lens, k_scale, v_scale, scale, num_seqs, num_heads,
                    num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                    min_piece_tokens, tmp_out, tmp_max, tmp_sum, cnt, q_dtype, cache_dtype, stream);
}

}  // extern "C"
