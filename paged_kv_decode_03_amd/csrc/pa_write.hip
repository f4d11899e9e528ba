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
#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {
namespace {

// clamp(rint(x / s), -127, 127) with the correctly rounded fp32 quotient;
// a NaN quotient gives 0.
__device__ __forceinline__ int8_t quantize_i8(float x, float s) {
    float t = __fdiv_rn(x, s);
    if (t != t) return 0;
    float r = rintf(t);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int8_t)(int)r;
}

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
        const int v = r - g * nv;
        const int64_t slot = a.slot_mapping[tok];
        if (slot < 0) continue;
        const int64_t b = slot / a.block_size;
        const int64_t o = slot - b * a.block_size;
        const int64_t src = (tok * a.num_kv_heads + g) * a.head_dim + (int64_t)v * VEC;
        const int64_t dst = ((b * a.num_kv_heads + g) * a.block_size + o) * a.head_dim +
                            (int64_t)v * VEC;
        if constexpr (CACHE != I8) {
            constexpr int E = (ACT == F32) ? 4 : 2;
            *reinterpret_cast<uint4*>((char*)a.k_cache + dst * E) =
                ld16((const char*)a.key + src * E);
            *reinterpret_cast<uint4*>((char*)a.v_cache + dst * E) =
                ld16((const char*)a.value + src * E);
        } else {
            constexpr int E = (ACT == F32) ? 4 : 2;
            const float ks = a.k_scale[b * a.num_kv_heads + g];
            const float vs = a.v_scale[b * a.num_kv_heads + g];
            const uint4 kw = ld16((const char*)a.key + src * E);
            const uint4 vw = ld16((const char*)a.value + src * E);
            float kx[VEC], vx[VEC];
            const uint32_t kwa[4] = {kw.x, kw.y, kw.z, kw.w};
            const uint32_t vwa[4] = {vw.x, vw.y, vw.z, vw.w};
            if constexpr (ACT == F32) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kx[i] = __uint_as_float(kwa[i]);
                    vx[i] = __uint_as_float(vwa[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kx[2 * i] = bf16lo(kwa[i]);
                    kx[2 * i + 1] = bf16hi(kwa[i]);
                    vx[2 * i] = bf16lo(vwa[i]);
                    vx[2 * i + 1] = bf16hi(vwa[i]);
                }
            }
            uint32_t kq[VEC / 4], vq[VEC / 4];
#pragma unroll
            for (int w = 0; w < VEC / 4; ++w) {
                uint32_t kk = 0, vv = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kk |= (uint32_t)(uint8_t)quantize_i8(kx[4 * w + i], ks) << (8 * i);
                    vv |= (uint32_t)(uint8_t)quantize_i8(vx[4 * w + i], vs) << (8 * i);
                }
                kq[w] = kk;
                vq[w] = vv;
            }
            if constexpr (VEC == 8) {
                *reinterpret_cast<uint2*>((int8_t*)a.k_cache + dst) = make_uint2(kq[0], kq[1]);
                *reinterpret_cast<uint2*>((int8_t*)a.v_cache + dst) = make_uint2(vq[0], vq[1]);
            } else {
                *reinterpret_cast<uint32_t*>((int8_t*)a.k_cache + dst) = kq[0];
                *reinterpret_cast<uint32_t*>((int8_t*)a.v_cache + dst) = vq[0];
            }
        }
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
