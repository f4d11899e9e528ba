// The slot-mapped write of one 16-byte vector of a new token's K or V row,
// shared by the write kernel and the decode that writes the new tokens itself.
//
// Source: "How pakanor/low-latency-distributed-llm-serving-infrastructure-
// custom-k8s-control-plane works", Connections (the engine writes the KV
// cache; paged attention maps cache slots); int8 storage: "How vrajpatel105/
// paged-inference-engine works", summary.
#pragma once

#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

// clamp(rint(x / s), -127, 127) with the correctly rounded fp32 quotient;
// a NaN quotient gives 0.
__device__ __forceinline__ int8_t quantize_i8(float x, float s) {
    const float t = __fdiv_rn(x, s);
    if (t != t) return 0;
    const float r = fminf(fmaxf(rintf(t), -127.0f), 127.0f);
    return (int8_t)(int)r;
}

// Four int8 codes of x0..x3 packed little-endian.
__device__ __forceinline__ uint32_t codes4(float x0, float x1, float x2, float x3, float s) {
    return (uint32_t)(uint8_t)quantize_i8(x0, s) | (uint32_t)(uint8_t)quantize_i8(x1, s) << 8 |
           (uint32_t)(uint8_t)quantize_i8(x2, s) << 16 | (uint32_t)(uint8_t)quantize_i8(x3, s) << 24;
}

// The int8 codes of 8 packed bf16 values (16 bytes -> 8 bytes).
__device__ __forceinline__ uint2 codes_bf16x8(uint4 w, float s) {
    return make_uint2(codes4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y), s),
                      codes4(bf16lo(w.z), bf16hi(w.z), bf16lo(w.w), bf16hi(w.w), s));
}

// One 16-byte vector w of activations (4 fp32 or 8 bf16) into `cache` at
// element offset dst: a bit copy, or its int8 codes with scale s.
template <Dtype ACT, Dtype CACHE>
__device__ __forceinline__ void put_vector(void* cache, int64_t dst, uint4 w, float s) {
    if constexpr (CACHE != I8) {
        constexpr int E = (ACT == F32) ? 4 : 2;
        *reinterpret_cast<uint4*>((char*)cache + dst * E) = w;
    } else if constexpr (ACT == F32) {
        *reinterpret_cast<uint32_t*>((int8_t*)cache + dst) =
            codes4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                   __uint_as_float(w.w), s);
    } else {
        *reinterpret_cast<uint2*>((int8_t*)cache + dst) = codes_bf16x8(w, s);
    }
}

// Element offset of vector v of kv head g's row in cache slot `slot`.
__device__ __forceinline__ int64_t slot_row(int64_t slot, int g, int v, int vec, int num_kv_heads,
                                            int head_dim, int block_size) {
    const int64_t b = slot / block_size;
    const int64_t o = slot - b * block_size;
    return ((b * num_kv_heads + g) * block_size + o) * head_dim + (int64_t)v * vec;
}

// Vector v (16 bytes of activations) of kv head g of token `tok` into slot
// slot_mapping[tok] (skipped when negative): a bit copy, or int8 codes with the
// (block, kv head) scales.
template <Dtype ACT, Dtype CACHE>
__device__ __forceinline__ void write_vector(const void* key, const void* value, void* k_cache,
                                             void* v_cache, const int64_t* slot_mapping,
                                             const float* k_scale, const float* v_scale,
                                             int num_kv_heads, int head_dim, int block_size,
                                             int64_t tok, int g, int v) {
    constexpr int VEC = (ACT == F32) ? 4 : 8;            // elements per 16-byte vector
    constexpr int E = (ACT == F32) ? 4 : 2;
    // the activations are loaded with the slot, not after it: their addresses
    // do not depend on it, so the two loads overlap
    const int64_t src = (tok * num_kv_heads + g) * head_dim + (int64_t)v * VEC;
    const uint4 kw = ld16((const char*)key + src * E);
    const uint4 vw = ld16((const char*)value + src * E);
    const int64_t slot = slot_mapping[tok];
    if (slot < 0) return;
    const int64_t dst = slot_row(slot, g, v, VEC, num_kv_heads, head_dim, block_size);
    float ks = 1.0f, vs = 1.0f;
    if constexpr (CACHE == I8) {
        const int64_t sc = (slot / block_size) * num_kv_heads + g;
        ks = k_scale[sc];
        vs = v_scale[sc];
    }
    put_vector<ACT, CACHE>(k_cache, dst, kw, ks);
    put_vector<ACT, CACHE>(v_cache, dst, vw, vs);
}

}  // namespace pa
