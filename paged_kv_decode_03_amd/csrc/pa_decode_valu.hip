// Paged decode attention, VALU core: multi-head (G = 1) and G = 2 layouts,
// where the query heads sharing a kv head are too few to make a dense
// contraction worth the matrix cores.
//
// Method: "PagedAttention kernel ... gathers KV data from non-contiguous
// physical blocks in-kernel, no compaction copy" (Continuous-Batching-LLM-
// Inference-Engine README, feature list); the decoder reads the block table
// ("How vrajpatel105/paged-inference-engine works", Connections).
//
// Per 16-token chunk, lane (tt = lane/4, qq = lane%4) owns token row tt and
// the 16-byte pieces 4m+qq of that row, so each load instruction reads whole
// 64-byte runs of 16 rows. Dot products are fmaf with a quad DPP sum; each
// lane keeps its own online-softmax state (natural-log units) over "its" rows
// for its quarter of the head dims. The 16 row states of a wave are merged
// with lane shuffles; a wave's merged state is laid out [head][dim] through a
// per-wave LDS buffer, so that outputs, workspace partials and their combine
// are coalesced.
#include "pa_decode_common.hpp"

namespace pa {
namespace {

template <Dtype T>
constexpr int esize() { return T == F32 ? 4 : T == BF16 ? 2 : 1; }

// 16 bytes of cache data -> 16/esize floats (exact).
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

template <int D_, int G_, Dtype QT, Dtype CT>
struct ValuCore {
    static constexpr int G = G_;
    static constexpr int D = D_;
    static constexpr bool BASE2 = false;
    static constexpr bool PAIR = false;          // one sequence per segment
    static constexpr int CE = esize<CT>();
    static constexpr int EPC = 16 / CE;          // cache elements per 16-byte piece
    static constexpr int NM = D * CE / 64;       // pieces per lane per row
    static constexpr int ND = NM * EPC;          // dims per lane (= D / 4)
    static_assert(ND * 4 == D, "lane split");

    struct State {
        float m[G], l[G], acc[G][ND];
    };
    struct Chunk {
        uint4 k[NM], v[NM];
        float ks, vs;
    };

    const DecodeArgs& a;
    bool cow = false;    // neighbouring sequences share blocks: keep those cached (load)
    int lane, tt, qq;
    uint32_t row_off;                            // bytes inside a 16-token chunk
    int shift;
    int64_t head_stride, block_stride;
    float qf[G][ND];

    __device__ explicit ValuCore(const DecodeArgs& args) : a(args) {
        lane = threadIdx.x & 63;
        tt = lane >> 2;
        qq = lane & 3;
        row_off = tt * D * CE + 16 * qq;
        shift = (a.block_size == 32) ? 1 : 0;
        head_stride = (int64_t)a.block_size * D;
        block_stride = head_stride * a.num_kv_heads;
    }

    __device__ void begin_segment(int s, int g) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const char* qrow = (const char*)a.q +
                               (((int64_t)s * a.num_heads + g * G + h) * D) * esize<QT>();
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    const int d = (4 * m + qq) * EPC + e;
                    qf[h][m * EPC + e] = (QT == F32) ? ((const float*)qrow)[d]
                                                     : bf16lo(((const uint16_t*)qrow)[d]);
                }
        }
    }

    __device__ void init(State& S) const {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            S.m[h] = kNegInf;
            S.l[h] = 0.0f;
#pragma unroll
            for (int i = 0; i < ND; ++i) S.acc[h][i] = 0.0f;
        }
    }

    // Non-temporal loads (each tile is read once per launch), except blocks
    // that a neighbouring sequence shares in a copy-on-write batch (cow), and
    // fp32 caches (there the two load paths push the largest instance into
    // register spills).
    __device__ Chunk load(int s, int g, int c) const {
        Chunk ch;
        const int64_t ri = (int64_t)s * a.max_blocks_per_seq + (c >> shift);
        const int phys = ld_uniform(a.block_tables, ri);
        const int64_t off = phys * block_stride + g * head_stride + (int64_t)(c & shift) * CHUNK * D;
        const char* kp = at((const char*)a.k_cache + off * CE, row_off);
        const char* vp = at((const char*)a.v_cache + off * CE, row_off);
        auto tiles = [&](auto nt) {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                ch.k[m] = ld16p<nt()>(kp + 64 * m);
                ch.v[m] = ld16p<nt()>(vp + 64 * m);
            }
        };
        if constexpr (CT == F32)
            tiles(std::false_type{});
        else if (!cow || !block_shared(a, s, ri, phys))
            tiles(std::true_type{});
        else
            tiles(std::false_type{});
        if constexpr (CT == I8) {
            ch.ks = ld_uniform(a.k_scale, (int64_t)phys * a.num_kv_heads + g);
            ch.vs = ld_uniform(a.v_scale, (int64_t)phys * a.num_kv_heads + g);
        } else {
            ch.ks = ch.vs = 1.0f;
        }
        return ch;
    }

    __device__ void step(State& S, const Chunk& cur, int c, int t1) const {
        float kf[ND], vf[ND];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            unpack16<CT>(cur.k[m], &kf[m * EPC]);
            unpack16<CT>(cur.v[m], &vf[m * EPC]);
        }
        const bool valid = c * CHUNK + tt < t1;
        const float xs = a.scale * cur.ks;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float dot = 0.0f;
#pragma unroll
            for (int i = 0; i < ND; ++i) dot = fmaf(qf[h][i], kf[i], dot);
            dot = quad_sum(dot);
            if (valid) {
                // x is rounded once and both the max and exp(x - max) use that
                // value, so the largest weight is exactly 1
                const float x = dot * xs;
                const float mnew = fmaxf(S.m[h], x);
                const float alpha = __builtin_amdgcn_exp2f((S.m[h] - mnew) * kLog2e);
                const float p = __builtin_amdgcn_exp2f((x - mnew) * kLog2e);
                S.l[h] = S.l[h] * alpha + p;
                const float pv = p * cur.vs;
#pragma unroll
                for (int i = 0; i < ND; ++i) S.acc[h][i] = fmaf(pv, vf[i], S.acc[h][i] * alpha);
                S.m[h] = mnew;
            }
        }
    }

    // Merge the 16 row states (lanes differing in tt): every lane then holds
    // the wave's state for its dims.
    __device__ void merge_rows(State& S) const {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int mask = 4; mask < 64; mask <<= 1)
                merge_xor<false>(S.m[h], S.l[h], S.acc[h], mask);
        }
    }

    __device__ void to_lds(State& S, WaveStates<G, D>& st, int wave) const {
        merge_rows(S);
        if (tt == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if (qq == 0) {
                    st.m[wave][h] = S.m[h];
                    st.l[wave][h] = S.l[h];
                }
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int e = 0; e < EPC; ++e)
                        st.acc[wave][h][(4 * m + qq) * EPC + e] = S.acc[h][m * EPC + e];
            }
        }
    }

    // The merged state's acc (divided by l if `normalise`) as [head][dim] in
    // this wave's LDS buffer, readable by every lane of the wave on return.
    __device__ const float* stage(const State& S, bool normalise) const {
        __shared__ float buf[NW][G * D];
        float* b = buf[uniform(threadIdx.x >> 6)];
        __builtin_amdgcn_wave_barrier();         // earlier reads of b are done
        if (tt == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int e = 0; e < EPC; ++e) {
                        const float x = S.acc[h][m * EPC + e];
                        b[h * D + (4 * m + qq) * EPC + e] = normalise ? x / S.l[h] : x;
                    }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        return b;
    }

    // heads g*G .. g*G+G-1 of sequence s are contiguous in out
    __device__ void store_final(const State& S, int s, int g) const {
        const float* b = stage(S, true);
        const int64_t base = ((int64_t)s * a.num_heads + g * G) * D;
        for (int i = lane; i < G * D; i += 64) store_out(a.out, base + i, b[i], a.q_dtype);
    }

    // Workspace slot: the unnormalised accumulator [head][dim] (G*D floats in
    // tmp_out), m (natural units) and l of head h at h in tmp_max / tmp_sum.
    __device__ void store_slot(const State& S, int64_t slot) const {
        const float* b = stage(S, false);
        float* acc = a.tmp_out + slot * (G * D);
        for (int i = lane; i < G * D; i += 64) ws_store<true>(acc + i, b[i]);
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                ws_store<true>(a.tmp_max + slot * G + h, S.m[h]);
                ws_store<true>(a.tmp_sum + slot * G + h, S.l[h]);
            }
        }
    }

    // Log-sum-exp of the partials of pieces first .. first+n-1 of (s, g) into
    // out; piece first + k left its partial in slot 2 (first + k) + (k == 0).
    __device__ void combine(long long first, int n, int s, int g) const {
        const int64_t base = ((int64_t)s * a.num_heads + g * G) * D;
        auto slot = [&](int k) -> int64_t { return 2 * (first + k) + (k == 0 ? 1 : 0); };
        for (int i = lane; i < G * D; i += 64) {
            const int h = i / D;
            float M = kNegInf;
            for (int k = 0; k < n; ++k) M = fmaxf(M, ws_load_coherent(a.tmp_max + slot(k) * G + h));
            float lsum = 0.0f, o = 0.0f;
            for (int k = 0; k < n; ++k) {
                const float W = rel_weight<false>(ws_load_coherent(a.tmp_max + slot(k) * G + h), M);
                lsum += W * ws_load_coherent(a.tmp_sum + slot(k) * G + h);
                o += W * ws_load_coherent(a.tmp_out + slot(k) * (G * D) + i);
            }
            store_out(a.out, base + i, o / lsum, a.q_dtype);
        }
    }
};

template <int D, int G, Dtype QT, Dtype CT>
__global__ __launch_bounds__(NW * 64) void valu_partitions(DecodeArgs a) {
    decode_partitions<ValuCore<D, G, QT, CT>>(a);
}

template <int D, int G, Dtype QT, Dtype CT>
__global__ __launch_bounds__(NW * 64) void valu_balanced(DecodeArgs a) {
    decode_balanced<ValuCore<D, G, QT, CT>>(a);
}

template <int D, int G, Dtype QT, Dtype CT>
hipError_t launch(const DecodeArgs& a, Schedule sch, hipStream_t st) {
    if (sch == Schedule::Balanced) {
        const void* fn = reinterpret_cast<const void*>(&valu_balanced<D, G, QT, CT>);
        const int grid = balanced_grid(fn, NW * 64, st);
        if (grid <= 0) return hipErrorLaunchFailure;
        hipLaunchKernelGGL((valu_balanced<D, G, QT, CT>), dim3(grid), dim3(NW * 64), 0, st, a);
    } else {
        const int64_t nwg = (int64_t)a.num_kv_heads * a.num_seqs * a.num_partitions;
        hipLaunchKernelGGL((valu_partitions<D, G, QT, CT>), dim3((unsigned)nwg), dim3(NW * 64), 0,
                           st, a);
    }
    return hipGetLastError();
}

// Waves of the balanced grid of each instance with head_dim D and group G.
template <int D, int G>
int waves_of(hipStream_t st) {
    const void* fns[4] = {reinterpret_cast<const void*>(&valu_balanced<D, G, F32, F32>),
                          reinterpret_cast<const void*>(&valu_balanced<D, G, BF16, BF16>),
                          reinterpret_cast<const void*>(&valu_balanced<D, G, F32, I8>),
                          reinterpret_cast<const void*>(&valu_balanced<D, G, BF16, I8>)};
    int m = 0;
    for (const void* fn : fns) {
        const int grid = balanced_grid(fn, NW * 64, st);
        if (grid <= 0) return -1;
        m = grid * NW > m ? grid * NW : m;
    }
    return m;
}

template <int D, int G>
hipError_t by_dtype(const DecodeArgs& a, Schedule sch, hipStream_t st) {
    if (a.q_dtype == F32 && a.cache == F32) return launch<D, G, F32, F32>(a, sch, st);
    if (a.q_dtype == BF16 && a.cache == BF16) return launch<D, G, BF16, BF16>(a, sch, st);
    if (a.q_dtype == F32 && a.cache == I8) return launch<D, G, F32, I8>(a, sch, st);
    if (a.q_dtype == BF16 && a.cache == I8) return launch<D, G, BF16, I8>(a, sch, st);
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

int balanced_waves_valu(int head_dim, int G, hipStream_t st) {
    if (head_dim == 64) return G == 1 ? waves_of<64, 1>(st) : G == 2 ? waves_of<64, 2>(st) : 0;
    if (head_dim == 128) return G == 1 ? waves_of<128, 1>(st) : G == 2 ? waves_of<128, 2>(st) : 0;
    return 0;
}

hipError_t launch_decode_valu(const DecodeArgs& a, Schedule sch, hipStream_t st) {
    if (!valu_supports(a)) return hipErrorNotSupported;
    const int G = a.num_heads / a.num_kv_heads;
    if (a.head_dim == 64) return G == 1 ? by_dtype<64, 1>(a, sch, st) : by_dtype<64, 2>(a, sch, st);
    return G == 1 ? by_dtype<128, 1>(a, sch, st) : by_dtype<128, 2>(a, sch, st);
}

}  // namespace pa
