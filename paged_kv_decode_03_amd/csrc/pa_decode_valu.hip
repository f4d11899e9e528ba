// Paged decode attention, VALU kernel: multi-head (G = 1) and G = 2 layouts,
// where the query heads sharing a kv head are too few to make a dense
// contraction worth the matrix cores.
//
// Method: "PagedAttention kernel ... gathers KV data from non-contiguous
// physical blocks in-kernel, no compaction copy" (Continuous-Batching-LLM-
// Inference-Engine README, feature list); the decoder reads the block table
// ("How vrajpatel105/paged-inference-engine works", Connections).
//
// Workgroup = (kv head g, sequence s, partition j), 4 waves. The partition's
// tokens are taken 16 at a time ("chunks"; a block of 16 or 32 tokens holds
// 1 or 2 chunks); wave w takes chunks w, w+4, ... Inside a wave, lane
// (tt = lane/4, qq = lane%4) owns token row tt of the chunk and the 16-byte
// pieces 4m+qq of that row, so each load instruction reads whole 64-byte runs
// of 16 rows. Each lane keeps its own online-softmax state over "its" rows
// (natural-log units) for its quarter of the head dims; the 16 row states of a
// wave are merged with lane shuffles at the end, the 4 wave states in LDS.
#include "pa_decode_common.hpp"

namespace pa {
namespace {

constexpr int NW = 4;

template <Dtype T>
constexpr int esize() { return T == F32 ? 4 : T == BF16 ? 2 : 1; }

// 16 bytes of cache/query data -> 16/esize floats (exact).
template <Dtype T>
__device__ __forceinline__ void unpack16(const uint4& w, float* f) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
    if constexpr (T == F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
    } else if constexpr (T == BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16lo(v[i]);
            f[2 * i + 1] = bf16hi(v[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int n = 0; n < 4; ++n) f[4 * i + n] = i8_at(v[i], n);
    }
}

template <int D, int G, Dtype QT, Dtype CT>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(DecodeArgs a) {
    constexpr int CE = esize<CT>();
    constexpr int EPC = 16 / CE;              // cache elements per 16-byte piece
    constexpr int NM = D * CE / 64;           // pieces per lane per row
    constexpr int ND = NM * EPC;              // dims per lane (= D / 4)
    static_assert(ND * 4 == D, "lane split");

    __shared__ WaveStates<NW, G, D> st;

    const WorkItem wi = work_item(a);
    const int g = wi.g, s = wi.s, j = wi.j;
    const int L = a.context_lens[s];
    const int P = a.partition_size > 0 ? a.partition_size : L;
    const int t0 = j * P;
    if (L == 0 || t0 >= L) {
        if (a.partition_size == 0) store_zeros<G, D>(a, s, g);
        return;
    }
    const int t1 = min(L, t0 + P);
    const int c0 = t0 >> 4, c1 = (t1 + 15) >> 4;

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int tt = lane >> 2, qq = lane & 3;

    // query rows of the G heads, in this lane's dims
    float qf[G][ND];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const char* qrow = (const char*)a.q +
                           (((int64_t)s * a.num_heads + g * G + h) * D) * esize<QT>();
#pragma unroll
        for (int m = 0; m < NM; ++m) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const int d = (4 * m + qq) * EPC + e;
                qf[h][m * EPC + e] = (QT == F32) ? ((const float*)qrow)[d]
                                                 : bf16lo(((const uint16_t*)qrow)[d]);
            }
        }
    }

    float mrun[G], lrun[G], acc[G][ND];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        mrun[h] = kNegInf;
        lrun[h] = 0.0f;
#pragma unroll
        for (int i = 0; i < ND; ++i) acc[h][i] = 0.0f;
    }

    const int shift = (a.block_size == 32) ? 1 : 0;   // chunks per block: 1 or 2
    const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    const int64_t head_stride = (int64_t)a.block_size * D;
    const int64_t block_stride = head_stride * a.num_kv_heads;
    const int row_off = tt * D * CE + 16 * qq;        // bytes inside a 16-token chunk

    struct Chunk {
        uint4 k[NM], v[NM];
        float ks, vs;
    };
    auto load = [&](int c) {
        Chunk ch;
        const int phys = bt[c >> shift];
        const int64_t off = phys * block_stride + g * head_stride + (int64_t)(c & shift) * 16 * D;
        const char* kp = (const char*)a.k_cache + off * CE + row_off;
        const char* vp = (const char*)a.v_cache + off * CE + row_off;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            ch.k[m] = ld16(kp + 64 * m);
            ch.v[m] = ld16(vp + 64 * m);
        }
        if constexpr (CT == I8) {
            ch.ks = a.k_scale[(int64_t)phys * a.num_kv_heads + g];
            ch.vs = a.v_scale[(int64_t)phys * a.num_kv_heads + g];
        } else {
            ch.ks = ch.vs = 1.0f;
        }
        return ch;
    };

    int c = c0 + wave;
    Chunk cur;
    if (c < c1) cur = load(c);
    for (; c < c1; c += NW) {
        Chunk nxt;
        if (c + NW < c1) nxt = load(c + NW);

        float kf[ND], vf[ND];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            unpack16<CT>(cur.k[m], &kf[m * EPC]);
            unpack16<CT>(cur.v[m], &vf[m * EPC]);
        }
        const bool valid = (c << 4) + tt < t1;
        const float xs = a.scale * cur.ks;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float dot = 0.0f;
#pragma unroll
            for (int i = 0; i < ND; ++i) dot = fmaf(qf[h][i], kf[i], dot);
            dot = quad_sum(dot);
            if (valid) {
                // x is rounded once and both the max and exp(x - max) use
                // that value, so the largest weight is exactly 1 (the build
                // turns off fma contraction, which would break this)
                const float x = dot * xs;
                const float mnew = fmaxf(mrun[h], x);
                const float alpha = __builtin_amdgcn_exp2f((mrun[h] - mnew) * kLog2e);
                const float p = __builtin_amdgcn_exp2f((x - mnew) * kLog2e);
                lrun[h] = lrun[h] * alpha + p;
                const float pv = p * cur.vs;
#pragma unroll
                for (int i = 0; i < ND; ++i) acc[h][i] = fmaf(pv, vf[i], acc[h][i] * alpha);
                mrun[h] = mnew;
            }
        }
        cur = nxt;
    }

    // merge the 16 row states of the wave (lanes differing in tt)
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int mask = 4; mask < 64; mask <<= 1) merge_xor<false>(mrun[h], lrun[h], acc[h], mask);
    }
    if (tt == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (qq == 0) {
                st.m[wave][h] = mrun[h];
                st.l[wave][h] = lrun[h];
            }
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int e = 0; e < EPC; ++e) st.acc[wave][h][(4 * m + qq) * EPC + e] = acc[h][m * EPC + e];
        }
    }
    __syncthreads();
    finish<NW, G, D, false>(st, a, s, g, j);
}

template <int D, int G, Dtype QT, Dtype CT>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
    const int64_t nwg = (int64_t)a.num_kv_heads * a.num_seqs * a.num_partitions;
    hipLaunchKernelGGL((decode_valu_kernel<D, G, QT, CT>), dim3((unsigned)nwg), dim3(NW * 64), 0,
                       st, a);
    return hipGetLastError();
}

template <int D, int G>
hipError_t by_dtype(const DecodeArgs& a, hipStream_t st) {
    if (a.q_dtype == F32 && a.cache == F32) return launch<D, G, F32, F32>(a, st);
    if (a.q_dtype == BF16 && a.cache == BF16) return launch<D, G, BF16, BF16>(a, st);
    if (a.q_dtype == F32 && a.cache == I8) return launch<D, G, F32, I8>(a, st);
    if (a.q_dtype == BF16 && a.cache == I8) return launch<D, G, BF16, I8>(a, st);
    return hipErrorNotSupported;
}

}  // namespace

bool valu_supports(const DecodeArgs& a) {
    const int G = a.num_heads / a.num_kv_heads;
    const bool dt = (a.q_dtype == F32 && a.cache == F32) || (a.q_dtype == BF16 && a.cache == BF16) ||
                    (a.cache == I8 && (a.q_dtype == F32 || a.q_dtype == BF16));
    return dt && (G == 1 || G == 2) && (a.head_dim == 64 || a.head_dim == 128) &&
           (a.block_size == 16 || a.block_size == 32);
}

hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t st) {
    if (!valu_supports(a)) return hipErrorNotSupported;
    const int G = a.num_heads / a.num_kv_heads;
    if (a.head_dim == 64) return G == 1 ? by_dtype<64, 1>(a, st) : by_dtype<64, 2>(a, st);
    return G == 1 ? by_dtype<128, 1>(a, st) : by_dtype<128, 2>(a, st);
}

}  // namespace pa
