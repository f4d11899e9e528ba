// Pieces shared by the decode kernels: online-softmax state merging, the two
// work drivers (fixed partitions; work-balanced pieces) and the epilogues.
//
// A softmax state over a set of tokens is (m, l, acc): m the largest logit, l
// the sum of exp(x_t - m), acc[d] the sum of exp(x_t - m) v_t[d]. Two states
// over disjoint token sets merge exactly into the state of their union:
//   M = max(m1, m2), l = l1 e^{m1-M} + l2 e^{m2-M}, acc likewise.
// A core keeps m either in natural units (VALU core) or in base-2 units with
// log2(e) folded into the logits (MFMA core); Core::BASE2 says which. Stored
// partials are always in natural units.
//
// A "core" supplies the per-chunk work for one (sequence, kv head) segment:
//   begin_segment(s, g)        load the G query rows of the segment
//   init(State&)               empty state
//   Chunk load(c)              issue the loads of 16-token chunk c
//   step(State&, chunk, c, t1) consume it (tokens >= t1 excluded)
//   to_lds(State&, st, wave)   merge the wave's lane states, write st[wave]
#pragma once

#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int NW = 4;        // waves per workgroup
constexpr int CHUNK = 16;    // tokens per chunk

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
template <int G, int D>
struct WaveStates {
    float m[NW][G];
    float l[NW][G];
    float acc[NW][G][D];
};

// Combined state of the NW waves for (head h, dim d): the normalised output,
// the max in natural units and the sum.
template <int G, int D, bool BASE2>
__device__ __forceinline__ void combine_waves(const WaveStates<G, D>& st, int h, int d, float& val,
                                              float& m_nat, float& lsum) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, st.m[w][h]);
    float o = 0.0f;
    lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float W = rel_weight<BASE2>(st.m[w][h], M);
        lsum += W * st.l[w][h];
        o += W * st.acc[w][h][d];
    }
    val = o / lsum;
    m_nat = BASE2 ? M * kLn2 : M;
}

// Final output of (s, g)'s G heads from the wave states.
template <int G, int D, bool BASE2>
__device__ __forceinline__ void store_final(const WaveStates<G, D>& st, const DecodeArgs& a, int s,
                                            int g) {
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D, d = idx - h * D;
        float val, m, l;
        combine_waves<G, D, BASE2>(st, h, d, val, m, l);
        store_out(a.out, ((int64_t)s * a.num_heads + g * G + h) * D + d, val, a.q_dtype);
    }
}

// Workspace accesses. COHERENT ones are agent-scope relaxed atomics: on
// gfx950 they bypass the per-XCD L2 (sc1), so a partial stored by one
// workgroup is read back intact by a workgroup on another XCD without any
// cache-wide write-back or invalidate (which an agent-scope fence costs).
template <bool COHERENT>
__device__ __forceinline__ void ws_store(float* p, float v) {
    if constexpr (COHERENT)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}
__device__ __forceinline__ float ws_load_coherent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Partial (normalised output, natural max, sum) of (s, g)'s G heads into
// workspace slot k of nslots.
template <int G, int D, bool BASE2, bool COHERENT>
__device__ __forceinline__ void store_partial(const WaveStates<G, D>& st, const DecodeArgs& a,
                                              int s, int g, int k, int nslots) {
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D, d = idx - h * D;
        float val, m, l;
        combine_waves<G, D, BASE2>(st, h, d, val, m, l);
        const int64_t sh = (int64_t)s * a.num_heads + g * G + h;
        ws_store<COHERENT>(&a.tmp_out[(sh * nslots + k) * D + d], val);
        if (d == 0) {
            ws_store<COHERENT>(&a.tmp_max[sh * nslots + k], m);
            ws_store<COHERENT>(&a.tmp_sum[sh * nslots + k], l);
        }
    }
}

// Most pieces one context can be cut into (the balanced driver sizes ranges
// so that this holds): the LDS weight table of combine_slots (2 * G * this
// many floats) then fits in the wave-state space (NW * G * D floats).
template <int D>
constexpr int kMaxPieces = NW * D / 2;

// Log-sum-exp combination of workspace slots 0..n-1 (n <= kMaxPieces<D>) of
// (s, g)'s G heads into out, with coherent loads (the slots were written by
// other workgroups). No load waits on another: lane k of wave h % NW reads
// slot k's max and sum, the weights W_k = l_k e^{m_k - M} go through LDS
// (wts: 2 * G * kMaxPieces<D> floats), and each output dim then issues its n
// slot loads back to back.
template <int G, int D>
__device__ __forceinline__ void combine_slots(const DecodeArgs& a, int s, int g, int n, int nslots,
                                              float* wts) {
    constexpr int KP = kMaxPieces<D>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float* wm = wts;                          // [G][KP]: m, then W
    float* wl = wts + G * KP;                 // [G][KP]: l
    for (int h = wave; h < G; h += NW) {
        const int64_t sh = (int64_t)s * a.num_heads + g * G + h;
        for (int k = lane; k < n; k += 64) {
            wm[h * KP + k] = ws_load_coherent(a.tmp_max + sh * nslots + k);
            wl[h * KP + k] = ws_load_coherent(a.tmp_sum + sh * nslots + k);
        }
        float M = kNegInf;
        for (int k = lane; k < n; k += 64) M = fmaxf(M, wm[h * KP + k]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        for (int k = lane; k < n; k += 64)
            wm[h * KP + k] =
                wl[h * KP + k] * __builtin_amdgcn_exp2f((wm[h * KP + k] - M) * kLog2e);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D, d = idx - h * D;
        const int64_t sh = (int64_t)s * a.num_heads + g * G + h;
        const float* op = a.tmp_out + sh * nslots * D + d;
        const float* w = wm + h * KP;
        float o = 0.0f, wsum = 0.0f;
        int k = 0;
        for (; k + 4 <= n; k += 4) {
            const float o0 = ws_load_coherent(op + (int64_t)(k + 0) * D);
            const float o1 = ws_load_coherent(op + (int64_t)(k + 1) * D);
            const float o2 = ws_load_coherent(op + (int64_t)(k + 2) * D);
            const float o3 = ws_load_coherent(op + (int64_t)(k + 3) * D);
            o += w[k] * o0 + w[k + 1] * o1 + w[k + 2] * o2 + w[k + 3] * o3;
            wsum += w[k] + w[k + 1] + w[k + 2] + w[k + 3];
        }
        for (; k < n; ++k) {
            o += w[k] * ws_load_coherent(op + (int64_t)k * D);
            wsum += w[k];
        }
        store_out(a.out, sh * D + d, o / wsum, a.q_dtype);
    }
}

// One pass over an empty context: the output is all zeros.
template <int G, int D>
__device__ __forceinline__ void store_zeros(const DecodeArgs& a, int s, int g) {
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D, d = idx - h * D;
        store_out(a.out, ((int64_t)s * a.num_heads + g * G + h) * D + d, 0.0f, a.q_dtype);
    }
}

// The NW waves of the workgroup take interleaved chunks of [c_begin, c_end)
// of the current segment (tokens >= t1 excluded); the merged state of each
// wave is left in st. Ends with a workgroup barrier.
template <class Core>
__device__ __forceinline__ void run_piece(Core& core, WaveStates<Core::G, Core::D>& st,
                                          int c_begin, int c_end, int t1) {
    const int wave = uniform(threadIdx.x >> 6);
    typename Core::State S;
    core.init(S);
    int c = c_begin + wave;
    // two chunk buffers used in turn (no register copies between iterations):
    // the loads of the next chunk are in flight while the current one computes
    typename Core::Chunk b0, b1;
    if (c < c_end) b0 = core.load(c);
    while (c < c_end) {
        if (c + NW < c_end) b1 = core.load(c + NW);
        core.step(S, b0, c, t1);
        c += NW;
        if (c >= c_end) break;
        if (c + NW < c_end) b0 = core.load(c + NW);
        core.step(S, b1, c, t1);
        c += NW;
    }
    core.to_lds(S, st, wave);
    __syncthreads();
}

// ---- driver 1: fixed partitions ---------------------------------------------
// Workgroup -> (kv head g, sequence s, partition j), partitions varying
// slowest. partition_size == 0: one pass over the whole context into out;
// otherwise the partial of partition j into slot j.
template <class Core>
__device__ __forceinline__ void decode_partitions(const DecodeArgs& a) {
    constexpr int G = Core::G, D = Core::D;
    __shared__ WaveStates<G, D> st;
    const int bid = blockIdx.x;
    const int g = bid % a.num_kv_heads;
    const int r = bid / a.num_kv_heads;
    const int s = r % a.num_seqs, j = r / a.num_seqs;
    const int L = ld_const(a.context_lens, s);
    const int P = a.partition_size > 0 ? a.partition_size : L;
    const int t0 = j * P;
    if (L == 0 || t0 >= L) {
        if (a.partition_size == 0) store_zeros<G, D>(a, s, g);
        return;
    }
    const int t1 = min(L, t0 + P);
    Core core(a);
    core.begin_segment(s, g);
    run_piece(core, st, t0 / CHUNK, (t1 + CHUNK - 1) / CHUNK, t1);
    if (a.partition_size > 0)
        store_partial<G, D, Core::BASE2, false>(st, a, s, g, j, a.num_partitions);
    else
        store_final<G, D, Core::BASE2>(st, a, s, g);
}

// ---- driver 2: work-balanced pieces --------------------------------------------
// All (sequence, kv head) segments are laid end to end as one list of
// T = Hkv * sum_s ceil(L_s / 16) chunks, sequence-major. Workgroup w takes the
// contiguous range [w*C, (w+1)*C), C = max(min_chunks, ceil(T / W)), so every
// workgroup streams the same number of chunks whatever the length mix. A
// segment wholly inside one range is finished in place; a segment cut by
// range ends leaves one partial per piece in the workspace, and the workgroup
// that completes its last piece (counted with an agent-scope atomic) combines
// them and resets the counter to 0.
//
// Logical range index: workgroups are dealt round-robin to the 8 XCDs, so the
// index is remapped to give each XCD a contiguous run of ranges (neighbouring
// sequences, e.g. those sharing prefix blocks, then share that XCD's L2).
struct BalancedShared {
    int part[NW * 64];
    int wave_tot[NW];
    long long total;
    int s0;
    long long base0;
    int last;
};

template <class Core>
__device__ __forceinline__ void decode_balanced(const DecodeArgs& a) {
    constexpr int G = Core::G, D = Core::D;
    __shared__ WaveStates<G, D> st;
    __shared__ BalancedShared sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = a.num_seqs, Hkv = a.num_kv_heads;
    const int W = gridDim.x;

    // logical range index (XCD-contiguous); a bijection when W % 8 == 0
    const int nx = 8;
    const int w = (W % nx) ? (int)blockIdx.x
                           : (int)(blockIdx.x % nx) * (W / nx) + (int)(blockIdx.x / nx);

    // 1. chunk counts per sequence: thread t sums its slice of sequences
    const int K = (S + NW * 64 - 1) / (NW * 64);
    const int sb = min(S, tid * K), se = min(S, sb + K);
    int my = 0;
    for (int s = sb; s < se; ++s) my += (ld_const(a.context_lens, s) + CHUNK - 1) / CHUNK;
    // inclusive scan over the workgroup
    int inc = my;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    if (lane == 63) sh.wave_tot[wave] = inc;
    __syncthreads();
    int wbase = 0;
    for (int v = 0; v < wave; ++v) wbase += sh.wave_tot[v];
    const int excl = wbase + inc - my;            // chunks of sequences before sb
    if (tid == NW * 64 - 1) sh.total = (long long)Hkv * (wbase + inc);
    if (w == 0) {
        // sequences with an empty context get zeros (no piece covers them)
        for (int s = sb; s < se; ++s)
            if (a.context_lens[s] == 0)
                for (int gg = 0; gg < Hkv; ++gg) {
                    for (int i = 0; i < G * D; ++i)
                        store_out(a.out, ((int64_t)s * a.num_heads + gg * G) * D + i, 0.0f,
                                  a.q_dtype);
                }
    }
    __syncthreads();
    const long long T = uniform64(sh.total);
    const long long minc = a.partition_size / CHUNK;
    long long C = (T + W - 1) / W;
    if (C < minc) C = minc;
    // at most kMaxPieces<D> pieces per context: pieces <= ceil(n / C) + 1
    constexpr int KP = kMaxPieces<D>;
    const long long maxn = (a.max_context_len + CHUNK - 1) / CHUNK;
    if (C < (maxn + KP - 3) / (KP - 2)) C = (maxn + KP - 3) / (KP - 2);
    if (C < 1) C = 1;
    const long long X0 = (long long)w * C;
    if (X0 >= T) return;                             // uniform across the workgroup
    const long long X1 = min(T, X0 + C);

    // 2. locate the sequence holding chunk X0: Hkv*P(s0) <= X0 < Hkv*P(s0+1)
    if ((long long)Hkv * excl <= X0 && X0 < (long long)Hkv * (excl + my)) {
        long long base = (long long)Hkv * excl;
        for (int s = sb; s < se; ++s) {
            const long long n = (long long)Hkv * ((a.context_lens[s] + CHUNK - 1) / CHUNK);
            if (X0 < base + n) {
                sh.s0 = s;
                sh.base0 = base;
                break;
            }
            base += n;
        }
    }
    __syncthreads();

    // 3. walk the segments of [X0, X1) (all wave-uniform: kept in SGPRs)
    Core core(a);
    int s = uniform(sh.s0);
    long long base = uniform64(sh.base0);            // first chunk of sequence s
    long long X = X0;
    int L = uniform(ld_const(a.context_lens, s));
    long long n = (L + CHUNK - 1) / CHUNK;
    int g = (int)((X - base) / n);
    while (X < X1) {
        if (n == 0) {                                // empty sequence: no segments
            ++s;
            L = uniform(ld_const(a.context_lens, s));
            n = (L + CHUNK - 1) / CHUNK;
            continue;
        }
        const long long A = base + g * n, B = A + n;
        const int cb = (int)(X - A), ce = (int)(min(X1, B) - A);
        core.begin_segment(s, g);
        run_piece(core, st, cb, ce, min(L, ce * CHUNK));
        if (A >= X0 && B <= X1) {
            store_final<G, D, Core::BASE2>(st, a, s, g);
        } else {
            const int first = (int)(A / C);
            const int pieces = (int)((B - 1) / C) - first + 1;
            store_partial<G, D, Core::BASE2, true>(st, a, s, g, w - first, a.num_partitions);
            // Every wave waits until its coherent stores have completed (the
            // workgroup barrier alone does not wait for them); then one atomic
            // publishes the piece, and the workgroup that brings the count to
            // `pieces` combines all of them with coherent loads.
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0)
                sh.last = atomicAdd(&a.counters[(int64_t)s * Hkv + g], 1) == pieces - 1;
            __syncthreads();
            if (sh.last) {
                // the wave states in st are no longer needed: their space holds the weights
                static_assert(sizeof(st.acc) >= 2 * G * KP * sizeof(float), "LDS");
                combine_slots<G, D>(a, s, g, pieces, a.num_partitions, &st.acc[0][0][0]);
                if (tid == 0) a.counters[(int64_t)s * Hkv + g] = 0;
            }
        }
        __syncthreads();                             // st is reused by the next piece
        X = min(X1, B);
        if (X == B && ++g == Hkv) {
            g = 0;
            base += Hkv * n;
            if (X < X1) {
                ++s;
                L = uniform(ld_const(a.context_lens, s));
                n = (L + CHUNK - 1) / CHUNK;
            }
        }
    }
}

}  // namespace pa
