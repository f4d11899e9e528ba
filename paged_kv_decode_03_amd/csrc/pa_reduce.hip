// Log-sum-exp reduce of split-K decode partials (flash-decoding combine).
//
// For one (sequence s, query head h) with n = ceil(L_s / P) partitions:
//   M = max_j m_j, W_j = l_j e^{m_j - M}, out = sum_j W_j o_j / sum_j W_j.
// One wave per (s, h); lane d handles dims d, d + 64, ...; the per-partition
// max and sum are wave-uniform scalar loads.
#include "pa_decode_common.hpp"

namespace pa {
namespace {

__global__ __launch_bounds__(64) void reduce_kernel(ReduceArgs a) {
    const int sh_i = blockIdx.x;
    const int s = sh_i / a.num_heads;
    const int64_t sh = sh_i;
    const int L = a.context_lens[s];
    const int n = (L + a.partition_size - 1) / a.partition_size;
    const int lane = threadIdx.x;
    const int D = a.head_dim;
    if (n == 0) {
        for (int d = lane; d < D; d += 64) store_out(a.out, sh * D + d, 0.0f, a.out_dtype);
        return;
    }
    const float* mp = a.tmp_max + sh * a.num_partitions;
    const float* lp = a.tmp_sum + sh * a.num_partitions;
    const float* op = a.tmp_out + sh * a.num_partitions * D;
    float M = kNegInf;
    for (int jj = 0; jj < n; ++jj) M = fmaxf(M, mp[jj]);
    constexpr int MAXV = 16;              // head_dim <= 1024
    float acc[MAXV];
#pragma unroll
    for (int k = 0; k < MAXV; ++k) acc[k] = 0.0f;
    float wsum = 0.0f;
    for (int jj = 0; jj < n; ++jj) {
        const float W = lp[jj] * __builtin_amdgcn_exp2f((mp[jj] - M) * kLog2e);
        wsum += W;
        const float* o = op + (int64_t)jj * D;
#pragma unroll
        for (int k = 0; k < MAXV; ++k) {
            const int d = lane + 64 * k;
            if (d < D) acc[k] = fmaf(W, o[d], acc[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int d = lane + 64 * k;
        if (d < D) store_out(a.out, sh * D + d, acc[k] / wsum, a.out_dtype);
    }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t st) {
    const int64_t nwg = (int64_t)a.num_seqs * a.num_heads;
    if (nwg == 0) return hipSuccess;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)nwg), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace pa
