// Log-sum-exp reduce of split-K decode partials (flash-decoding combine).
//
// For one (sequence s, query head h) with n = ceil(L_s / P) partitions:
//   M = max_j m_j, W_j = l_j e^{m_j - M}, out = sum_j W_j o_j / sum_j W_j.
// One 256-thread workgroup per (s, h). The maxima and weights of all n
// partitions are computed in parallel (weights kept in LDS); the four waves
// then take every fourth partition, lane d holding dims d, d + 64, ..., with
// several partitions' loads in flight, and add their sums in LDS. (A single
// wave walking the partitions one after another waits a full memory latency
// per partition.)
#include "pa_decode_common.hpp"

namespace pa {
namespace {

constexpr int RW = 4;                     // waves per workgroup
constexpr int WMAX = 4096;                // partitions whose weights fit in LDS

__device__ __forceinline__ float block_max(float v, float* red) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    const int wave = threadIdx.x >> 6;
    __syncthreads();                      // red is free
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < RW; ++w) v = fmaxf(v, red[w]);
    return v;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < RW; ++w) v += red[w];
    return v;
}

// NV: dims per lane (head_dim <= 64 NV)
template <int NV>
__global__ __launch_bounds__(RW * 64) void reduce_kernel(ReduceArgs a) {
    __shared__ float wts[WMAX];
    __shared__ float red[RW];
    __shared__ float part[RW - 1][NV * 64];
    const int sh_i = blockIdx.x;
    const int s = sh_i / a.num_heads;
    const int64_t sh = sh_i;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = a.head_dim;
    const int NP = a.num_partitions;
    const float* mp = a.tmp_max + sh * NP;
    const float* lp = a.tmp_sum + sh * NP;
    const float* op = a.tmp_out + sh * NP * D;
    // The first partitions' maxima, sums and (wave w combining partitions w,
    // w + RW, ..., four per round) the first round's outputs are loaded at
    // once with the context length: their addresses need only the workspace's
    // partition count, and those past the sequence's own count n are read
    // but never used.
    constexpr int U = 4;
    float x0[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int jj = wave + u * RW, d = lane + 64 * k;
            x0[u][k] = (jj < NP && d < D) ? op[(int64_t)jj * D + d] : 0.0f;
        }
    const float m0 = tid < NP ? mp[tid] : kNegInf;
    const float l0 = tid < NP ? lp[tid] : 0.0f;
    const int L = a.context_lens[s];
    const int n = (L + a.partition_size - 1) / a.partition_size;
    if (n == 0) {
        for (int d = tid; d < D; d += RW * 64) store_out(a.out, sh * D + d, 0.0f, a.out_dtype);
        return;
    }
    float M = tid < n ? m0 : kNegInf;
    for (int j = tid + RW * 64; j < n; j += RW * 64) M = fmaxf(M, mp[j]);
    M = block_max(M, red);
    const bool in_lds = n <= WMAX;
    float ws = 0.0f;
    for (int j = tid; j < n; j += RW * 64) {
        const float mj = j == tid ? m0 : mp[j], lj = j == tid ? l0 : lp[j];
        const float W = lj * __builtin_amdgcn_exp2f((mj - M) * kLog2e);
        ws += W;
        if (in_lds) wts[j] = W;
    }
    const float wsum = block_sum(ws, red);  // its barriers also publish wts
    auto weight = [&](int j) {
        return in_lds ? wts[j] : lp[j] * __builtin_amdgcn_exp2f((mp[j] - M) * kLog2e);
    };

    float acc[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k] = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int jj = wave + u * RW;
        if (jj < n) {
            const float W = weight(jj);
#pragma unroll
            for (int k = 0; k < NV; ++k) acc[k] = fmaf(W, x0[u][k], acc[k]);
        }
    }
    // the later rounds: loads first
    int j = wave + U * RW;
    for (; j + (U - 1) * RW < n; j += U * RW) {
        float x[U][NV];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int d = lane + 64 * k;
                x[u][k] = d < D ? op[(int64_t)(j + u * RW) * D + d] : 0.0f;
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float W = weight(j + u * RW);
#pragma unroll
            for (int k = 0; k < NV; ++k) acc[k] = fmaf(W, x[u][k], acc[k]);
        }
    }
    for (; j < n; j += RW) {
        const float W = weight(j);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int d = lane + 64 * k;
            if (d < D) acc[k] = fmaf(W, op[(int64_t)j * D + d], acc[k]);
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int k = 0; k < NV; ++k) part[wave - 1][k * 64 + lane] = acc[k];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int d = lane + 64 * k;
        if (d < D) {
            float v = acc[k];
#pragma unroll
            for (int w = 0; w < RW - 1; ++w) v += part[w][k * 64 + lane];
            store_out(a.out, sh * D + d, v / wsum, a.out_dtype);
        }
    }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t st) {
    const int64_t nwg = (int64_t)a.num_seqs * a.num_heads;
    if (nwg == 0) return hipSuccess;
    const dim3 grid((unsigned)nwg), block(RW * 64);
    if (a.head_dim <= 64)
        hipLaunchKernelGGL(reduce_kernel<1>, grid, block, 0, st, a);
    else if (a.head_dim <= 128)
        hipLaunchKernelGGL(reduce_kernel<2>, grid, block, 0, st, a);
    else if (a.head_dim <= 256)
        hipLaunchKernelGGL(reduce_kernel<4>, grid, block, 0, st, a);
    else if (a.head_dim <= 512)
        hipLaunchKernelGGL(reduce_kernel<8>, grid, block, 0, st, a);
    else
        hipLaunchKernelGGL(reduce_kernel<16>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace pa
