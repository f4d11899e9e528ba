// Slot-mapped write of new tokens' K/V into the paged pool (bit copy, or int8
// quantisation with caller-chosen per-(block, kv head) scales).
//
// Source: "How pakanor/low-latency-distributed-llm-serving-infrastructure-
// custom-k8s-control-plane works", Connections (the engine writes the KV
// cache; paged attention maps cache slots); int8 storage: "How vrajpatel105/
// paged-inference-engine works", summary.
//
// One thread moves one 16-byte vector of one (token, kv head) row: 4 fp32 or
// 8 bf16 activations. Consecutive threads take consecutive vectors of a row,
// so both the read of `key` and the write into the slot's row are coalesced.
#include "pa_write_row.hpp"

namespace pa {
namespace {

template <Dtype ACT, Dtype CACHE>
__global__ __launch_bounds__(256) void write_kv_kernel(WriteArgs a, int64_t total) {
    constexpr int VEC = (ACT == F32) ? 4 : 8;           // elements per 16-byte vector
    const int nv = a.head_dim / VEC;
    const int64_t per_tok = (int64_t)a.num_kv_heads * nv;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t tok = idx / per_tok;
        const int r = (int)(idx - tok * per_tok);
        const int g = r / nv;
        write_vector<ACT, CACHE>(a.key, a.value, a.k_cache, a.v_cache, a.slot_mapping, a.k_scale,
                                 a.v_scale, a.num_kv_heads, a.head_dim, a.block_size, tok, g,
                                 r - g * nv);
    }
}

template <Dtype ACT, Dtype CACHE>
hipError_t launch(const WriteArgs& a, hipStream_t st) {
    constexpr int VEC = (ACT == F32) ? 4 : 8;
    const int64_t total = (int64_t)a.num_tokens * a.num_kv_heads * (a.head_dim / VEC);
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;   // grid-stride loop covers the rest
    hipLaunchKernelGGL((write_kv_kernel<ACT, CACHE>), dim3((unsigned)blocks), dim3(256), 0, st, a,
                       total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_write_kv(const WriteArgs& a, hipStream_t st) {
    if (a.act == F32 && a.cache == F32) return launch<F32, F32>(a, st);
    if (a.act == BF16 && a.cache == BF16) return launch<BF16, BF16>(a, st);
    if (a.act == F32 && a.cache == I8) return launch<F32, I8>(a, st);
    if (a.act == BF16 && a.cache == I8) return launch<BF16, I8>(a, st);
    return hipErrorNotSupported;
}

}  // namespace pa
