// Copy-on-write block copy: for each (src, dst) pair, every byte of physical
// block src of the K and V pools (all kv heads), and for an int8 cache its
// per-(block, kv head) scales, is copied into block dst.
//
// Source: the block pool's copy-on-write reference counting
// ("Continuous-Batching-LLM-Inference-Engine" README, feature list): a block
// shared by several sequences is copied into a block of the writer's own
// before the writer changes it.
//
// HBM-bound copy. Block (pair p, pool z) is bpb = Hkv * block_size * head_dim
// * elt contiguous bytes; a workgroup of 256 threads moves kVecs 16-byte
// vectors per thread of one such block, the loads of a thread issued together
// before its stores, consecutive threads on consecutive vectors. Grid:
// (ceil(vectors per block / (256 * kVecs)), pairs, 2 pools).
#include "pa_kernels.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kVecs = 4;

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
    const int64_t pair = blockIdx.y;
    const int64_t src = ld_uniform(a.block_mapping, 2 * pair);
    const int64_t dst = ld_uniform(a.block_mapping, 2 * pair + 1);
    char* const pool = (char*)(blockIdx.z == 0 ? a.k_cache : a.v_cache);
    const int64_t bpb = a.block_bytes;
    const uint4* s = reinterpret_cast<const uint4*>(pool + src * bpb);
    uint4* d = reinterpret_cast<uint4*>(pool + dst * bpb);
    const int64_t nvec = bpb / 16;
    const int64_t v0 = (int64_t)blockIdx.x * (256 * kVecs) + threadIdx.x;
    uint4 buf[kVecs];
#pragma unroll
    for (int i = 0; i < kVecs; ++i)
        if (v0 + 256 * i < nvec) buf[i] = s[v0 + 256 * i];
#pragma unroll
    for (int i = 0; i < kVecs; ++i)
        if (v0 + 256 * i < nvec) d[v0 + 256 * i] = buf[i];
    if (a.k_scale != nullptr && blockIdx.x == 0) {
        float* const sc = blockIdx.z == 0 ? a.k_scale : a.v_scale;
        for (int g = threadIdx.x; g < a.num_kv_heads; g += 256)
            sc[dst * a.num_kv_heads + g] = sc[src * a.num_kv_heads + g];
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t st) {
    if (a.num_pairs == 0) return hipSuccess;
    const int64_t nvec = a.block_bytes / 16;
    const int64_t gx = (nvec + 256 * kVecs - 1) / (256 * kVecs);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)gx, (unsigned)a.num_pairs, 2), dim3(256),
                       0, st, a);
    return hipGetLastError();
}

}  // namespace pa
