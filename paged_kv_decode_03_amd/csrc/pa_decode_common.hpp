// Pieces shared by the two decode kernels: merging online-softmax states and
// the workgroup epilogue that combines the per-wave states and stores either
// the final output (one pass) or one split-K partial.
//
// A softmax state over a set of tokens is (m, l, acc): m the largest logit, l
// the sum of exp(x_t - m), acc[d] the sum of exp(x_t - m) v_t[d]. Two states
// over disjoint token sets merge exactly into the state of their union:
//   M = max(m1, m2), l = l1 e^{m1-M} + l2 e^{m2-M}, acc likewise.
// The decode kernels keep m either in natural units (VALU kernel) or in base-2
// units with log2(e) folded into the logits (MFMA kernel); BASE2 says which.
#pragma once

#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

constexpr float kNegInf = -__builtin_huge_valf();

template <bool BASE2>
__device__ __forceinline__ float rel_weight(float m, float M) {
    // e^{m-M} (natural) or 2^{m-M} (base 2); 0 for an empty state.
    if (m == kNegInf) return 0.0f;
    return __builtin_amdgcn_exp2f(BASE2 ? (m - M) : (m - M) * kLog2e);
}

// Merge the state held by lane (lane ^ mask) into this lane's state.
template <bool BASE2, int N>
__device__ __forceinline__ void merge_xor(float& m, float& l, float (&acc)[N], int mask) {
    const float mo = __shfl_xor(m, mask);
    const float lo = __shfl_xor(l, mask);
    const float M = fmaxf(m, mo);
    const float a = rel_weight<BASE2>(m, M);
    const float b = rel_weight<BASE2>(mo, M);
    l = l * a + lo * b;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float ao = __shfl_xor(acc[i], mask);
        acc[i] = acc[i] * a + ao * b;
    }
    m = M;
}

__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, Dtype dt) {
    if (dt == F32)
        reinterpret_cast<float*>(out)[idx] = v;
    else
        reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
}

// LDS holding one state per wave for the G query heads of a kv head.
template <int NW, int G, int D>
struct WaveStates {
    float m[NW][G];
    float l[NW][G];
    float acc[NW][G][D];
};

// Combine the NW wave states of (sequence s, kv head g, partition j) and
// store: out[s][g*G + h][:] (one pass) or the split-K partial.
template <int NW, int G, int D, bool BASE2>
__device__ __forceinline__ void finish(const WaveStates<NW, G, D>& st, const DecodeArgs& a, int s,
                                       int g, int j) {
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, st.m[w][h]);
        float lsum = 0.0f, o = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float W = rel_weight<BASE2>(st.m[w][h], M);
            lsum += W * st.l[w][h];
            o += W * st.acc[w][h][d];
        }
        const float val = o / lsum;
        const int head = g * G + h;
        if (a.partition_size > 0) {
            const int64_t sh = (int64_t)s * a.num_heads + head;
            a.tmp_out[(sh * a.num_partitions + j) * D + d] = val;
            if (d == 0) {
                a.tmp_max[sh * a.num_partitions + j] = BASE2 ? M * kLn2 : M;
                a.tmp_sum[sh * a.num_partitions + j] = lsum;
            }
        } else {
            store_out(a.out, ((int64_t)s * a.num_heads + head) * D + d, val, a.q_dtype);
        }
    }
}

// One pass over an empty context: the output is all zeros.
template <int G, int D>
__device__ __forceinline__ void store_zeros(const DecodeArgs& a, int s, int g) {
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D;
        const int d = idx - h * D;
        store_out(a.out, ((int64_t)s * a.num_heads + g * G + h) * D + d, 0.0f, a.q_dtype);
    }
}

// Workgroup -> (kv head g, sequence s, partition j). Partitions vary slowest
// so that every sequence's first partition is dispatched before any second.
struct WorkItem {
    int g, s, j;
};
__device__ __forceinline__ WorkItem work_item(const DecodeArgs& a) {
    const int bid = blockIdx.x;
    const int g = bid % a.num_kv_heads;
    const int r = bid / a.num_kv_heads;
    return {g, r % a.num_seqs, r / a.num_seqs};
}

}  // namespace pa
