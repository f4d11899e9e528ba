// Paged decode attention, MFMA core for grouped-query attention (G = 4, 8
// query heads per kv head; head_dim 128; bf16 queries; bf16 or int8 cache).
//
// Method: "PagedAttention kernel ... gathers KV data from non-contiguous
// physical blocks in-kernel, no compaction copy" (Continuous-Batching-LLM-
// Inference-Engine README, feature list); int8 storage ("How vrajpatel105/
// paged-inference-engine works", summary).
//
// The G query heads of one kv head share every K and V row, so per 16-token
// chunk QK^T is a [16 tokens x 128] x [128 x G] product and PV a
// [G x 16] x [16 x 128] product. Both run on the matrix cores in their
// 16-block 4x4 forms, which fit G = 4 exactly (G = 8 is two 4-head groups):
//
//  QK^T: v_mfma_f32_4x4x4_16b_bf16, 8 per chunk and head group. Lane
//    l = 16*tg + 4*qd + j4 feeds K row 4*j4 + tg (A operand) and query head j4
//    (B operand), both restricted to dim quarter qd; the four qd partial
//    logits are summed with two DPP row rotations. Lane l then holds the
//    logits of head j4 for tokens 4*i + tg (i = 0..3, one per register).
//  softmax: each 16-lane row tg keeps its own online state (base-2 units,
//    log2(e) folded into the scale) over its tokens, so the running max needs
//    no cross-lane reduction inside the loop; the reference max only moves
//    when it is exceeded by more than 8, so rescales are rare.
//  PV: v_mfma_f32_4x4x1_16b_f32, 32 per chunk and head group. The A operand
//    is V row 4*step + tg, dims 8*(l%16) + e, straight from a fully coalesced
//    16-byte load; the B operand is the lane's own probability register
//    `step`, already in place. V and P stay in fp32.
//  The 4 row states are merged with lane shuffles, the 4 wave states in LDS.
//
// No LDS is used in the main loop: K and V go from HBM straight to registers
// with 16-byte loads, and the next chunk's loads are issued before the current
// chunk is computed.
#include "pa_decode_common.hpp"

namespace pa {
namespace {

template <int G_, Dtype CT>
struct MfmaCore {
    static constexpr int G = G_;
    static constexpr int D = 128;
    static constexpr bool BASE2 = true;
    static constexpr int NHB = G / 4;           // 4-head groups
    static constexpr bool Q8 = (CT == I8);
    static constexpr int CE = Q8 ? 1 : 2;        // cache bytes per element
    static constexpr float kSlack = 8.0f;        // see step()

    struct State {
        float m[NHB], l[NHB];
        f32x4 acc[NHB][8];                       // acc[hb][e][i]: dim 8*(4*qd+i)+e
    };
    struct Chunk {
        uint4 k[4];        // bf16: pieces m = 0..3; int8: k[0], k[1] used
        uint4 v[4];        // bf16: one 16-byte load per step; int8: .x/.y of each
        float ks, vs;
    };

    const DecodeArgs& a;
    int lane, j4, qd, tg;
    int k_off, v_off;                            // byte offsets inside a chunk
    float sl2;
    int shift;
    int64_t head_stride, block_stride;
    // per segment
    const int32_t* bt;
    int g;
    uint4 qr[NHB][4];

    __device__ explicit MfmaCore(const DecodeArgs& args) : a(args) {
        lane = threadIdx.x & 63;
        j4 = lane & 3;
        qd = (lane >> 2) & 3;
        tg = lane >> 4;
        k_off = (4 * j4 + tg) * D * CE + 16 * qd;
        v_off = tg * D * CE + (lane & 15) * 8 * CE;
        sl2 = a.scale * kLog2e;
        shift = (a.block_size == 32) ? 1 : 0;
        head_stride = (int64_t)a.block_size * D;
        block_stride = head_stride * a.num_kv_heads;
    }

    // Query operands. bf16 cache: dims 8*(4m+qd) .. +7 for m = 0..3.
    // int8 cache: dims 16*(4(m>>1)+qd) + 8(m&1) .. +7.
    __device__ void begin_segment(int s, int g_) {
        g = g_;
        bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            const uint16_t* qrow =
                (const uint16_t*)a.q + ((int64_t)s * a.num_heads + g * G + hb * 4 + j4) * D;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                qr[hb][m] = Q8 ? ld16(qrow + 16 * (4 * (m >> 1) + qd) + 8 * (m & 1))
                               : ld16(qrow + 8 * (4 * m + qd));
        }
    }

    __device__ void init(State& S) const {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            S.m[hb] = kNegInf;
            S.l[hb] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) S.acc[hb][e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }

    __device__ Chunk load(int c) const {
        Chunk ch;
        const int phys = ld_const(bt, c >> shift);
        const int64_t off = phys * block_stride + g * head_stride + (int64_t)(c & shift) * CHUNK * D;
        const char* kp = (const char*)a.k_cache + off * CE + k_off;
        const char* vp = (const char*)a.v_cache + off * CE + v_off;
        if constexpr (Q8) {
            ch.k[0] = ld16(kp);
            ch.k[1] = ld16(kp + 64);
            ch.k[2] = ch.k[3] = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int step = 0; step < 4; ++step) {
                const uint2 w = ld8(vp + step * 4 * D);
                ch.v[step] = make_uint4(w.x, w.y, 0, 0);
            }
            ch.ks = ld_const(a.k_scale, (int64_t)phys * a.num_kv_heads + g);
            ch.vs = ld_const(a.v_scale, (int64_t)phys * a.num_kv_heads + g);
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) ch.k[m] = ld16(kp + 64 * m);
#pragma unroll
            for (int step = 0; step < 4; ++step) ch.v[step] = ld16(vp + step * 4 * D * CE);
            ch.ks = ch.vs = 1.0f;
        }
        return ch;
    }

    __device__ void step(State& S, const Chunk& cur, int c, int t1) const {
        const bool tail = ((c + 1) * CHUNK) > t1;

        // ---- logits: x[hb][i] for token 4*i + tg, head 4*hb + j4 --------------
        i16x4 ka[8];
        if constexpr (Q8) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const uint32_t w4[4] = {cur.k[m].x, cur.k[m].y, cur.k[m].z, cur.k[m].w};
#pragma unroll
                for (int hq = 0; hq < 4; ++hq)
                    ka[4 * m + hq] = as_i16x4(pack_bf16_trunc(i8_at(w4[hq], 0), i8_at(w4[hq], 1)),
                                              pack_bf16_trunc(i8_at(w4[hq], 2), i8_at(w4[hq], 3)));
            }
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                ka[2 * m] = as_i16x4(cur.k[m].x, cur.k[m].y);
                ka[2 * m + 1] = as_i16x4(cur.k[m].z, cur.k[m].w);
            }
        }
        const float xs = sl2 * cur.ks;
        float p[NHB][4];
        float alpha[NHB];
        bool rescale = false;
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                sacc = mfma4x4x4bf16(ka[2 * m], as_i16x4(qr[hb][m].x, qr[hb][m].y), sacc);
                sacc = mfma4x4x4bf16(ka[2 * m + 1], as_i16x4(qr[hb][m].z, qr[hb][m].w), sacc);
            }
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // x is rounded once; the max and exp2(x - max) see the same x
                x[i] = row_ror8_add(row_ror4_add(sacc[i])) * xs;
                if (tail && c * CHUNK + 4 * i + tg >= t1) x[i] = kNegInf;
            }
            // The reference max moves only when a logit exceeds it by more
            // than kSlack (log2 units): unnormalised weights stay <= 2^kSlack,
            // and the accumulator rescale below is skipped on most chunks.
            const float mblk = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            const float mnew = (mblk > S.m[hb] + kSlack) ? mblk : S.m[hb];
            const float muse = (mnew == kNegInf) ? 0.0f : mnew;
            alpha[hb] = __builtin_amdgcn_exp2f(S.m[hb] - muse);
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[hb][i] = __builtin_amdgcn_exp2f(x[i] - muse);
                psum += p[hb][i];
            }
            S.l[hb] = S.l[hb] * alpha[hb] + psum;
            S.m[hb] = mnew;
            rescale |= (alpha[hb] != 1.0f);
        }
        if (__any(rescale)) {
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
                for (int e = 0; e < 8; ++e) S.acc[hb][e] *= alpha[hb];
        }

        // ---- PV ----------------------------------------------------------------
#pragma unroll
        for (int step = 0; step < 4; ++step) {
            float vf[8];
            if constexpr (Q8) {
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    vf[n] = i8_at(cur.v[step].x, n);
                    vf[4 + n] = i8_at(cur.v[step].y, n);
                }
            } else {
                const uint32_t w4[4] = {cur.v[step].x, cur.v[step].y, cur.v[step].z,
                                        cur.v[step].w};
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    vf[2 * n] = bf16lo(w4[n]);
                    vf[2 * n + 1] = bf16hi(w4[n]);
                }
            }
            if (tail && c * CHUNK + 4 * step + tg >= t1) {
#pragma unroll
                for (int e = 0; e < 8; ++e) vf[e] = 0.0f;   // excluded rows may hold NaN
            }
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) {
                const float pb = p[hb][step] * cur.vs;
#pragma unroll
                for (int e = 0; e < 8; ++e) S.acc[hb][e] = mfma4x4x1f32(vf[e], pb, S.acc[hb][e]);
            }
        }
    }

    // merge the 4 row states of the wave and write the wave's state
    __device__ void to_lds(State& S, WaveStates<G, D>& st, int wave) const {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            float flat[32];
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i) flat[4 * e + i] = S.acc[hb][e][i];
            float m = S.m[hb], l = S.l[hb];
            merge_xor<true>(m, l, flat, 16);
            merge_xor<true>(m, l, flat, 32);
            if (tg == 0) {
                const int h = hb * 4 + j4;
                if (qd == 0) {
                    st.m[wave][h] = m;
                    st.l[wave][h] = l;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 8; ++e) st.acc[wave][h][8 * (4 * qd + i) + e] = flat[4 * e + i];
            }
        }
    }
};

// Register budget per lane: 168 (3 waves per SIMD) for G = 4, 256 (2 waves)
// for G = 8; enough resident waves to keep HBM busy with one chunk in flight.
template <int G>
constexpr int kWavesPerEU = G == 4 ? 3 : 2;

template <int G, Dtype CT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<G>)))
void mfma_partitions(DecodeArgs a) {
    decode_partitions<MfmaCore<G, CT>>(a);
}

template <int G, Dtype CT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<G>)))
void mfma_balanced(DecodeArgs a) {
    decode_balanced<MfmaCore<G, CT>>(a);
}

template <int G, Dtype CT>
hipError_t launch(const DecodeArgs& a, Schedule sch, hipStream_t st) {
    if (sch == Schedule::Balanced) {
        const void* fn = reinterpret_cast<const void*>(&mfma_balanced<G, CT>);
        const int grid = balanced_grid(fn, st);
        if (grid <= 0) return hipErrorLaunchFailure;
        hipLaunchKernelGGL((mfma_balanced<G, CT>), dim3(grid), dim3(NW * 64), 0, st, a);
    } else {
        const int64_t nwg = (int64_t)a.num_kv_heads * a.num_seqs * a.num_partitions;
        hipLaunchKernelGGL((mfma_partitions<G, CT>), dim3((unsigned)nwg), dim3(NW * 64), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

bool mfma_supports(const DecodeArgs& a) {
    const int G = a.num_heads / a.num_kv_heads;
    return (G == 4 || G == 8) && a.head_dim == 128 && a.q_dtype == BF16 &&
           (a.cache == BF16 || a.cache == I8) && (a.block_size == 16 || a.block_size == 32);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, Schedule sch, hipStream_t st) {
    if (!mfma_supports(a)) return hipErrorNotSupported;
    const int G = a.num_heads / a.num_kv_heads;
    if (a.cache == BF16) return G == 4 ? launch<4, BF16>(a, sch, st) : launch<8, BF16>(a, sch, st);
    return G == 4 ? launch<4, I8>(a, sch, st) : launch<8, I8>(a, sch, st);
}

}  // namespace pa
