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
//   Chunk load(s, g, c)        issue the loads of 16-token chunk c of (s, g)
//   step(State&, chunk, c, L)  consume it (tokens >= L excluded)
//   merge_rows(State&)         merge the wave's lane states: afterwards every
//                              lane holds the state of the whole wave
//   to_lds(State&, st, wave)   merge_rows, then write the wave's state to st
//   store_final(State&, s, g)  normalise a merged state and write out
//   store_slot(State&, slot)   a merged state into workspace slot `slot`, in
//                              the core's own layout, with coherent stores
//   combine(slot0, n, s, g)    log-sum-exp of slots slot0 .. slot0+n-1 into out
#pragma once

#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int NW = 4;        // waves per workgroup
constexpr int CHUNK = 16;    // tokens per chunk
constexpr int kFastShare = 160;   // see balanced_setup
constexpr int kFastShareCow = 152;   // the same, kv head major (copy-on-write) batches
constexpr int kChunkCost = 16;    // cost units per chunk (see balanced_setup)
constexpr int kSegCost = 32;      // cost units per segment (see balanced_setup)
constexpr int kSegCostG8 = 64;    // the same, 8 or more query heads per kv head


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

// The same merge with the partner in the other 16-lane row (MASK 16) or the
// other half-wave (MASK 32), exchanged by permlane swaps.
template <bool BASE2, int MASK, int N>
__device__ __forceinline__ void merge_rows_xor(float& m, float& l, float (&acc)[N]) {
    static_assert(MASK == 16 || MASK == 32, "cross-row masks only");
    auto other = [](float x) { return MASK == 16 ? lane_xor16(x) : lane_xor32(x); };
    const float mo = other(m);
    const float lo = other(l);
    const float M = fmaxf(m, mo);
    const float a = rel_weight<BASE2>(m, M);
    const float b = rel_weight<BASE2>(mo, M);
    l = l * a + lo * b;
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = acc[i] * a + other(acc[i]) * b;
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

// Whether logical block lb of sequence s (its block-table entry at index ri,
// holding phys) is also logical block lb of the previous or the next
// sequence: a block that neighbouring sequences share copy-on-write, and that
// other waves will read again. Only a cache hint rides on the answer, so
// entries past a neighbour's context (unused, of any value) do no harm.
__device__ __forceinline__ bool block_shared(const DecodeArgs& a, int s, int64_t ri, int phys) {
    const int64_t prev = s > 0 ? ri - a.max_blocks_per_seq : ri;
    const int64_t next = s + 1 < a.num_seqs ? ri + a.max_blocks_per_seq : ri;
    const int bp = ld_uniform(a.block_tables, prev), bn = ld_uniform(a.block_tables, next);
    return (prev != ri && bp == phys) || (next != ri && bn == phys);
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
__device__ __forceinline__ void run_piece(Core& core, WaveStates<Core::G, Core::D>& st, int s,
                                          int g, int c_begin, int c_end, int t1) {
    const int wave = uniform(threadIdx.x >> 6);
    typename Core::State S;
    core.init(S);
    int c = c_begin + wave;
    // two chunk buffers used in turn (no register copies between iterations):
    // the loads of the next chunk are in flight while the current one computes
    typename Core::Chunk b0, b1;
    if (c < c_end) b0 = core.load(s, g, c);
    while (c < c_end) {
        if (c + NW < c_end) b1 = core.load(s, g, c + NW);
        core.step(S, b0, c, t1);
        c += NW;
        if (c >= c_end) break;
        if (c + NW < c_end) b0 = core.load(s, g, c + NW);
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
    core.cow = first_block_shared(a.block_tables, a.max_blocks_per_seq, a.num_seqs, s);
    core.begin_segment(s, g);
    run_piece(core, st, s, g, t0 / CHUNK, (t1 + CHUNK - 1) / CHUNK, t1);
    if (a.partition_size > 0)
        store_partial<G, D, Core::BASE2, false>(st, a, s, g, j, a.num_partitions);
    else
        store_final<G, D, Core::BASE2>(st, a, s, g);
}

// ---- driver 2: work-balanced, wave by wave ---------------------------------------
// All (sequence, kv head) segments are laid end to end as one list of
// T = Hkv * sum_s ceil(L_s / 16) chunks, sequence-major. Every wave of the
// persistent grid takes one contiguous range of C = max(min_chunks,
// ceil(T / waves)) chunks, so all waves stream the same number of bytes
// whatever the length mix, and walks it on its own: no workgroup barrier after
// the set-up, and the loads of the next chunk -- in the same segment or the
// next one -- are in flight while the current chunk is computed.
// A segment wholly inside one range is finished in place. A segment cut by
// range ends leaves one partial per range that holds part of it, in the
// workspace slot 2j of range j when the segment started in an earlier range,
// 2j + 1 when it goes on past range j (a range cuts at most its first and its
// last segment, so the slots are distinct and number 4 per wave of the grid,
// whatever the context lengths). After its stores have completed, each
// piece's wave increments an agent-scope counter for the segment, and the wave
// that brings it to the number of pieces combines them in range order
// (coherent loads), writes out and resets the counter to 0. No wave ever waits
// for another.
//
// Workgroups are dealt round-robin to the 8 XCDs, so the workgroup index is
// remapped to give each XCD a contiguous run of ranges (neighbouring
// sequences, e.g. those sharing prefix blocks, then share that XCD's L2).
template <int NWG>                   // waves per workgroup
struct BalancedShared {
    int wave_tot[NWG], wave_shared[NWG];
    long long wave_cost[NWG];
    long long total, total_cost;
    int s0[NWG + 1], nu[NWG + 1], g0[NWG + 1];       // unit, its chunks, kv head
    int lu0[NWG + 1], lu1[NWG + 1];                  // its sequences' lengths (pair: both)
    long long base0[NWG + 1], cbase0[NWG + 1];
};

// Units of the segment list. For most cores a unit is one sequence. A core
// with PAIR set (the 16x16 core at 8 query heads per kv head, whose MFMA tile
// has 16 columns) takes two neighbouring sequences per unit, 2u in columns
// 0-7 and 2u + 1 (if any) in columns 8-15: first the ns leading chunks that
// lie on the same physical blocks in both block tables (copy-on-write
// prefixes), read and computed once for both, then the first sequence's own
// chunks [ns, n0), then the second's [ns, n1). A shared chunk holds no token
// of either sequence's last chunk (ns <= (L - 1) / 16 for both), so it is
// full for both and carries no new token. Segments are (unit, kv head).
constexpr int kMaxPairUnits = 2048;   // the pair table in LDS: 8 KB

// Position of one chunk in the segment list (all fields wave-uniform).
struct SegPos {
    int s, g, c;      // unit, kv head, chunk within the segment
    int L, n;         // context length of the unit's (first) sequence; the segment's chunks
    int L1, n0, ns;   // pair units: the second sequence's length, the first's chunks,
                      // the shared chunks (otherwise 0, n, 0)
    long long A;      // list index of chunk 0 of segment (s, g)
    long long Y;      // cost position where chunk 0 of segment (s, g) starts
};

template <bool PAIR>
__device__ __forceinline__ int num_units(const DecodeArgs& a) {
    return PAIR ? (a.num_seqs + 1) / 2 : a.num_seqs;
}

// Shared leading chunks of the pair (s0, s0 + 1) with lengths L0, L1 (both
// > 0), from the block tables: the run of equal entries, capped below both
// sequences' last chunk. Per-lane loads (set-up only).
__device__ __forceinline__ int pair_shared_chunks(const DecodeArgs& a, int s0, int L0, int L1) {
    const int cap = min((L0 - 1) / CHUNK, (L1 - 1) / CHUNK);
    if (cap <= 0) return 0;
    const int cpb = a.block_size / CHUNK;              // chunks per block (1 or 2)
    const int nb = (cap + cpb - 1) / cpb;              // blocks that may hold shared chunks
    const int32_t* t0 = a.block_tables + (int64_t)s0 * a.max_blocks_per_seq;
    const int32_t* t1 = t0 + a.max_blocks_per_seq;
    int b = 0;
    for (; b + 8 <= nb; b += 8) {                      // eight entries of each table at a time
        int eq = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) eq |= (t0[b + i] == t1[b + i]) ? 0 : (1 << i);
        if (eq) {
            b += __builtin_ctz(eq);
            return min(cap, b * cpb);
        }
    }
    while (b < nb && t0[b] == t1[b]) ++b;
    return min(cap, b * cpb);
}

// Fill p's unit fields for unit p.s. ns_tab: LDS byte address of the pair
// table (pair units' shared chunks, written by balanced_setup).
template <bool PAIR>
__device__ __forceinline__ void load_unit(const DecodeArgs& a, uint32_t ns_tab, SegPos& p) {
    if constexpr (PAIR) {
        const int s0 = 2 * p.s;
        p.L = ld_uniform(a.context_lens, s0);
        p.L1 = s0 + 1 < a.num_seqs ? ld_uniform(a.context_lens, s0 + 1) : 0;
        p.n0 = (p.L + CHUNK - 1) / CHUNK;
        p.ns = uniform((int)ds_read4_wait(ns_tab + 4 * p.s));
        p.n = p.n0 + (p.L1 + CHUNK - 1) / CHUNK - p.ns;
    } else {
        p.L = ld_uniform(a.context_lens, p.s);
        p.n = p.n0 = (p.L + CHUNK - 1) / CHUNK;
        p.L1 = p.ns = 0;
    }
}

// The chunk of a sequence that chunk p.c of segment (p.s, p.g) is: the
// sequence, its chunk index, its length (tokens >= t1 are masked), which
// columns it feeds (0 all, 1 the first sequence's, 2 the second's) and
// whether it is the sequence's last chunk (which holds its new token).
struct ChunkRef {
    int s, c, t1, who;
    bool last;
};
template <bool PAIR>
__device__ __forceinline__ ChunkRef chunk_ref(const SegPos& p) {
    if constexpr (!PAIR) {
        return {p.s, p.c, p.L, 0, p.c + 1 == p.n};
    } else {
        if (p.c < p.ns) return {2 * p.s, p.c, p.L, 0, false};
        if (p.c < p.n0) return {2 * p.s, p.c, p.L, 1, p.c + 1 == p.n0};
        return {2 * p.s + 1, p.c - p.n0 + p.ns, p.L1, 2, p.c + 1 == p.n};
    }
}

// hm: the segment list is kv head major; sc: a segment's fixed cost (see
// balanced_setup)
template <bool PAIR = false>
__device__ __forceinline__ SegPos next_pos(const DecodeArgs& a, SegPos p, bool hm, int sc,
                                           uint32_t ns_tab = 0) {
    if (p.c + 1 < p.n) {
        ++p.c;
        return p;
    }
    p.c = 0;
    p.Y += (long long)p.n * kChunkCost + sc;
    p.A += p.n;
    const int U = num_units<PAIR>(a);
    if (hm) {
        do {                               // units with no context have no segments
            if (++p.s == U) {
                p.s = 0;
                ++p.g;
            }
            load_unit<PAIR>(a, ns_tab, p);
        } while (p.n == 0);
        return p;
    }
    if (++p.g < a.num_kv_heads) return p;
    p.g = 0;
    do {
        ++p.s;
        load_unit<PAIR>(a, ns_tab, p);
    } while (p.n == 0);
    return p;
}

// The cut of the cost line (the chunk list weighted as balanced_setup says)
// into wave ranges. Workgroup w owns the contiguous run [w * span,
// (w + 1) * span), span = H * (Cf + Cs): its first H waves take Cf units each,
// the other H waves Cs <= Cf each. With H = 0 every range has Cs units.
struct Ranges {
    long long Cf, Cs;  // range lengths in cost units
    int H;
    __device__ long long span() const { return H ? H * (Cf + Cs) : Cs; }
    // first cost unit of range j (j = w * 2H + v; any j >= 0)
    __device__ long long start(long long j) const {
        if (!H) return j * Cs;
        const long long w = j / (2 * H);
        const int v = (int)(j - w * 2 * H);
        return w * span() + (v < H ? v * Cf : H * Cf + (v - H) * Cs);
    }
    // range holding cost unit X
    __device__ long long of(long long X) const {
        if (!H) return X / Cs;
        const long long w = X / span();
        const long long o = X - w * span();
        return w * 2 * H + (o < H * Cf ? o / Cf : H + (o - H * Cf) / Cs);
    }
};

// Where one wave's range starts; all fields wave-uniform.
struct WaveRange {
    long long X0, X1, wv;
    Ranges rg;
    SegPos cur;       // chunk X0
    bool hm;          // the segment list is kv head major
    int sc;           // a segment's fixed cost, cost units
};

// Set-up shared by the balanced drivers: chunk counts, their scan over the
// sequences, the range size C and the position of each wave's first chunk.
// Ends with a workgroup barrier; returns false for a wave with no work.
// PAIR: units are pairs of sequences; their shared chunks go to the LDS table
// ns_tab (int[kMaxPairUnits], unused otherwise).
template <int G, int D, int NWG, bool PAIR = false>
__device__ __forceinline__ bool balanced_setup(const DecodeArgs& a, BalancedShared<NWG>& sh,
                                               WaveRange& r, int* ns_tab = nullptr) {
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int S = a.num_seqs, Hkv = a.num_kv_heads;
    const int W = gridDim.x;

    // logical workgroup index (XCD-contiguous); a bijection when W % 8 == 0
    const int nx = 8;
    const int w = (W % nx) ? (int)blockIdx.x
                           : (int)(blockIdx.x % nx) * (W / nx) + (int)(blockIdx.x / nx);

    // Ranges are cut in cost units, kChunkCost to a chunk, so that the shares
    // are not rounded to whole chunks. A segment of n chunks costs
    // n kChunkCost + kSegCost, the kSegCost units standing for its fixed work
    // (query loads, merge and stores) and sitting before its first chunk. Two
    // chunks' worth was level with or faster than whole-chunk cuts with no
    // segment cost on every measured batch (1-3% on the mixed-length ones);
    // 24 and 48 units were 4-5% slower where all contexts have one length,
    // as the cuts then fall just off the segment boundaries. With eight query
    // heads to a kv head the fixed work is larger (twice the query rows and
    // partial states to merge): with the 4x4 core 96 units were 1-2% faster
    // on the mixed batch than 32, 128 and more slower again; with the 16x16
    // core (G = 8, bf16) 32 and 64 units were both 1.2% faster than 96, 0 level
    // with it. (kSegCost below stands for whichever applies.)
    // Segment order. Sequence major (the 8 kv heads of a sequence in a row):
    // chunk c of segment (s, g) spans the units from
    // P = Y_s Hkv + g (n_s kChunkCost + kSegCost) + kSegCost + c kChunkCost,
    // Y_s the cost of one kv head's segments of the sequences before s; a
    // block's kv-head tiles, contiguous in the pool, are then read by
    // neighbouring waves. Kv head major, chosen when at least a quarter of
    // the sequences start on the same physical block as the next one (copy-
    // on-write prefixes): P = g Yh + Y_s + kSegCost + c kChunkCost, Yh the cost
    // of one kv head's segments. Each XCD then takes about one kv head's share
    // of the list, so the shared prefix blocks that many sequences reread stay
    // in its L2 for one head (2 MB for the mixed batch's four 1024-token
    // prefixes) rather than for all heads (its whole 4 MB L2): 6% faster on
    // that batch, 1-2% slower on batches without sharing. (Every workgroup
    // takes the same decision from the same data.) A chunk belongs to the
    // range holding its last unit P + kChunkCost - 1.
    constexpr int CC = kChunkCost, SC = G >= 8 ? kSegCostG8 : kSegCost;

    // 1. chunk counts and costs per unit: thread t sums its slice of units
    // (and, for pair units, finds their shared chunks)
    const int U = num_units<PAIR>(a);
    const int K = (U + NWG * 64 - 1) / (NWG * 64);
    const int ub = min(U, tid * K), ue = min(U, ub + K);
    const int sb = PAIR ? min(S, 2 * ub) : ub, se = PAIR ? min(S, 2 * ue) : ue;   // its sequences
    // lengths of unit u's sequences (the second 0 without PAIR or past S)
    auto unit_lens = [&](int u, int& L0, int& L1) {
        if constexpr (PAIR) {
            L0 = ld_const(a.context_lens, 2 * u);
            L1 = 2 * u + 1 < S ? ld_const(a.context_lens, 2 * u + 1) : 0;
        } else {
            L0 = ld_const(a.context_lens, u);
            L1 = 0;
        }
    };
    // chunks of unit u (pair units: its shared chunks into the table)
    auto unit_chunks = [&](int u, bool fill, int L0, int L1) -> int {
        if constexpr (PAIR) {
            const int s0 = 2 * u;
            int ns;
            if (fill) {
                ns = (L0 > 0 && L1 > 0) ? pair_shared_chunks(a, s0, L0, L1) : 0;
                ns_tab[u] = ns;
            } else {
                ns = ns_tab[u];
            }
            return (L0 + CHUNK - 1) / CHUNK + (L1 + CHUNK - 1) / CHUNK - ns;
        } else {
            (void)fill;
            (void)L1;
            return (L0 + CHUNK - 1) / CHUNK;
        }
    };
    int my = 0;
    int shared = 0;                                  // s whose first block is s + 1's
    long long myc = 0;
    int n_ub = 0, L0_ub = 0, L1_ub = 0;             // the slice's first unit
    for (int u = ub; u < ue; ++u) {
        int L0, L1;
        unit_lens(u, L0, L1);
        const int n = unit_chunks(u, true, L0, L1);
        if (u == ub) {
            n_ub = n;
            L0_ub = L0;
            L1_ub = L1;
        }
        my += n;
        myc += n ? (long long)n * CC + SC : 0;
    }
    // (the locate below takes the first unit's lengths and count from here:
    // a slice is one unit up to 64 x NWG units, and a load per range start,
    // in turn, cost about as much as the rest of the set-up)
    auto slice_unit = [&](int u, int& L0, int& L1) {
        if (u == ub) {
            L0 = L0_ub;
            L1 = L1_ub;
            return n_ub;
        }
        unit_lens(u, L0, L1);
        return unit_chunks(u, false, L0, L1);
    };
    for (int s = sb; s < se; ++s) {
        // all four loads at once (entry 0 of a block-table row always exists)
        const int t = min(s + 1, S - 1);
        const int L = ld_const(a.context_lens, s), Ln = ld_const(a.context_lens, t);
        const int b = ld_const(a.block_tables, (int64_t)s * a.max_blocks_per_seq);
        const int bn = ld_const(a.block_tables, (int64_t)t * a.max_blocks_per_seq);
        if (t > s && L > a.block_size && Ln > a.block_size && b == bn) ++shared;
    }
    int inc = my;                                    // inclusive scans over the workgroup
    long long incc = myc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off);
        const long long yc = __shfl_up(incc, off);
        if (lane >= off) {
            inc += y;
            incc += yc;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) shared += __shfl_xor(shared, off);
    if (lane == 63) {
        sh.wave_tot[wave] = inc;
        sh.wave_cost[wave] = incc;
        sh.wave_shared[wave] = shared;
    }
    __syncthreads();
    int wbase = 0, nshared = 0;
    long long wbasec = 0;
    for (int v = 0; v < NWG; ++v) {
        if (v < wave) {
            wbase += sh.wave_tot[v];
            wbasec += sh.wave_cost[v];
        }
        nshared += sh.wave_shared[v];
    }
    const bool hm = uniform(nshared) * 4 >= S;       // kv head major (see above)
    const int excl = wbase + inc - my;               // chunks of units before ub
    const long long exclc = wbasec + incc - myc;     // their cost, per kv head
    if (tid == NWG * 64 - 1) {
        sh.total = (long long)Hkv * (wbase + inc);
        sh.total_cost = (long long)Hkv * (wbasec + incc);
    }
    if (w == 0) {
        // sequences with an empty context get zeros (no piece covers them)
        for (int s = sb; s < se; ++s)
            if (ld_const(a.context_lens, s) == 0)
                for (int i = 0; i < Hkv * G * D; ++i)
                    store_out(a.out, (int64_t)s * a.num_heads * D + i, 0.0f, a.q_dtype);
    }
    __syncthreads();
    const long long T = uniform64(sh.total);
    const long long Tc = uniform64(sh.total_cost);
    const long long Wv = (long long)W * NWG;
    const long long C = (Tc + Wv - 1) / Wv;          // mean range (cost units)
    const long long cmin = (long long)max(1, a.partition_size / CHUNK) * CC;
    // Age-weighted ranges. The first NWG/2 waves of an 8-wave workgroup are
    // dispatched first, one per SIMD, and the second half shares those SIMDs.
    // Under load the older wave of a SIMD wins the arbitration for memory
    // instruction issue: with equal ranges it finished 1.2-1.35x sooner, then
    // sat idle while the younger one ran alone. It gets a share kFastShare/256
    // of the pair's cost. (The CU's waves share one bandwidth, so this mostly
    // shortens the idle time rather than the launch: 0-4% faster measured.
    // Shares of 128, 144, 160, 176 and 192 measured in one process: 160 was
    // best or level on all four batches, 1.7% faster than 144 on the int8 one.)
    // In a copy-on-write batch many chunks come from the L2, where the older
    // wave's edge is smaller: on the mixed batch the older waves ended 24 us
    // after the younger ones (a speed ratio of 1.44 against the 1.67 the share
    // assumes), and kFastShareCow = 152 was 0.7% faster there and 2.0% with 32
    // query heads; 144 and 136 were slower.
    // Every range keeps at least the cost of a minimum piece, cmin.
    Ranges rg;
    if (NWG == 8) {
        rg.H = NWG / 2;
        rg.Cs = max(cmin, 2 * C * (256 - (hm ? kFastShareCow : kFastShare)) / 256);
        rg.Cf = max(rg.Cs, 2 * C - rg.Cs);
    } else {
        rg.H = 0;
        rg.Cs = rg.Cf = max(cmin, C);
    }

    // 2. locate the unit holding the cost position where each wave's range
    // starts (v = NWG: the next workgroup's first, where the last ends)
    const long long Th = T / Hkv, Tch = Tc / Hkv;    // one kv head's chunks and cost
    auto locate = [&](long long Y, int v) {
        if (hm) {
            if (Y >= Tc) return;
            const int g = (int)(Y / Tch);
            const long long Yr = Y - (long long)g * Tch;
            if (exclc <= Yr && Yr < exclc + myc) {
                long long base = excl, cbase = exclc;
                for (int u = ub; u < ue; ++u) {
                    int L0, L1;
                    const int n = slice_unit(u, L0, L1);
                    const long long cost = n ? (long long)n * CC + SC : 0;
                    if (Yr < cbase + cost) {
                        sh.s0[v] = u;
                        sh.nu[v] = n;
                        sh.lu0[v] = L0;
                        sh.lu1[v] = L1;
                        sh.g0[v] = g;
                        sh.base0[v] = (long long)g * Th + base;
                        sh.cbase0[v] = (long long)g * Tch + cbase;
                        break;
                    }
                    base += n;
                    cbase += cost;
                }
            }
            return;
        }
        if ((long long)Hkv * exclc <= Y && Y < (long long)Hkv * (exclc + myc)) {
            long long base = (long long)Hkv * excl, cbase = (long long)Hkv * exclc;
            for (int u = ub; u < ue; ++u) {
                int L0, L1;
                const int n = slice_unit(u, L0, L1);
                const long long cost = n ? (long long)Hkv * ((long long)n * CC + SC) : 0;
                if (Y < cbase + cost) {
                    sh.s0[v] = u;
                    sh.nu[v] = n;
                    sh.lu0[v] = L0;
                    sh.lu1[v] = L1;
                    sh.base0[v] = base;
                    sh.cbase0[v] = cbase;
                    break;
                }
                base += (long long)Hkv * n;
                cbase += cost;
            }
        }
    };
    for (int v = 0; v <= NWG; ++v) locate(rg.start((long long)w * NWG + v), v);
    __syncthreads();
    // chunk list index of the first chunk whose last unit is at or after Y
    auto chunk_at = [&](long long Y, int v, SegPos* p) -> long long {
        if (Y >= Tc) return T;
        const int u = uniform(sh.s0[v]), n = uniform(sh.nu[v]);
        const long long base = uniform64(sh.base0[v]), cbase = uniform64(sh.cbase0[v]);
        const long long sc = (long long)n * CC + SC;
        // head major: base / cbase already name segment (u, g0)
        const int g = hm ? uniform(sh.g0[v]) : (int)((Y - cbase) / sc);
        const long long gb = hm ? 0 : g;              // segments of u before (u, g)
        const long long off = (Y - cbase) - gb * sc;   // < sc, so c < n
        const int c = off < SC ? 0 : (int)((off - SC) / CC);
        if (p) {
            // the unit's fields as load_unit fills them, from the locate's
            // lengths in LDS rather than from memory
            p->s = u;
            p->L = uniform(sh.lu0[v]);
            if constexpr (PAIR) {
                p->L1 = uniform(sh.lu1[v]);
                p->n0 = (p->L + CHUNK - 1) / CHUNK;
                p->ns = uniform((int)ds_read4_wait(lds_addr(ns_tab) + 4 * u));
            } else {
                p->L1 = p->ns = 0;
                p->n0 = n;
            }
            p->n = n;
            p->g = g;
            p->c = c;
            p->A = base + gb * n;
            p->Y = cbase + gb * sc + SC;
        }
        return base + gb * n + c;
    };
    r.rg = rg;
    r.hm = hm;
    r.sc = SC;
    r.wv = (long long)w * NWG + wave;                 // this wave's range index
    const long long Y0 = rg.start(r.wv);
    if (Y0 >= Tc) return false;                      // uniform across the wave
    r.X0 = chunk_at(Y0, wave, &r.cur);
    r.X1 = chunk_at(min(Tc, rg.start(r.wv + 1)), wave + 1, nullptr);
    return r.X0 < r.X1;                              // a range inside a segment's fixed part is empty
}

// End of the piece of segment p held in St (this wave's chunks of it are all
// consumed). A segment wholly inside the range is written out; otherwise the
// piece is stored to its workspace slot and published -- now if it is the
// range's last (then after draining this wave's stores), or else held until
// then. Returns true if it issued global stores that are not yet waited for.
template <class Core>
struct PieceEnd {
    const DecodeArgs& a;
    const Core& core;
    const WaveRange& r;
    int64_t held_seg = -1;                           // a stored, unpublished piece
    long long held_first = 0;
    int held_pieces = 0;

    __device__ void publish(int64_t seg, long long first, int pieces) const {
        const int lane = threadIdx.x & 63;
        int prev = 0;
        if (lane == 0) prev = atomicAdd(&a.counters[seg], 1);
        prev = uniform(prev);
        if (prev == pieces - 1) {                    // every other piece is published
            const int Hkv = a.num_kv_heads;
            const int s = (int)(seg / Hkv), g = (int)(seg - (int64_t)s * Hkv);
            core.combine(first, pieces, s, g);
            if (lane == 0)
                __hip_atomic_store(&a.counters[seg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // `last`: p ends the range.
    __device__ void operator()(typename Core::State& St, const SegPos& p, bool last) {
        core.merge_rows(St);
        const long long B = p.A + p.n;
        if (p.A >= r.X0 && B <= r.X1) {
            core.store_final(St, p.s, p.g);
        } else {
            const long long first = r.rg.of(p.Y + kChunkCost - 1);
            const int pieces =
                (int)(r.rg.of(p.Y + (long long)p.n * kChunkCost - 1) - first) + 1;
            const int64_t seg = (int64_t)p.s * a.num_kv_heads + p.g;
            core.store_slot(St, 2 * r.wv + (p.A >= r.X0 ? 1 : 0));   // (see above)
            if (!last) {
                held_seg = seg;
                held_first = first;
                held_pieces = pieces;
                return;
            }
            __builtin_amdgcn_s_waitcnt(0);           // every store of this wave is complete
            if (held_seg >= 0) publish(held_seg, held_first, held_pieces);
            publish(seg, first, pieces);
            held_seg = -1;
            return;
        }
        if (last && held_seg >= 0) {
            __builtin_amdgcn_s_waitcnt(0);
            publish(held_seg, held_first, held_pieces);
            held_seg = -1;
        }
    }
};

// Register-path walk (cores without an LDS ring): the next chunk's loads go
// to registers while the current chunk is computed.
template <class Core>
__device__ __forceinline__ void decode_balanced(const DecodeArgs& a) {
    constexpr int G = Core::G, D = Core::D;
    __shared__ BalancedShared<NW> sh;
    WaveRange r;
    if (!balanced_setup<G, D, NW>(a, sh, r)) return;
    SegPos cur = r.cur;
    Core core(a);
    core.cow = r.hm;
    core.begin_segment(cur.s, cur.g);
    typename Core::State St;
    core.init(St);
    PieceEnd<Core> end{a, core, r};
    // chunks left in the range, in 32 bits: a 64-bit compare would need a VGPR
    // temporary, which may be one that an in-flight load still targets
    int left = (int)(r.X1 - r.X0);

    // One chunk: issue the loads of the next chunk into `nb` (at the range end
    // the current one again, so that every path has the same loads in flight
    // and the compiler's wait counts stay exact), compute `cb`, end a segment
    // that ends here. Returns false after the range's last chunk.
    auto one = [&](typename Core::Chunk& cb, typename Core::Chunk& nb) -> bool {
        const bool more = left > 1;
        const SegPos nxp = more ? next_pos(a, cur, r.hm, r.sc) : cur;
        nb = core.load(nxp.s, nxp.g, nxp.c);
        core.step(St, cb, cur.c, cur.L);
        if (more && nxp.c != 0) {                    // same segment
            --left;
            cur = nxp;
            return true;
        }
        end(St, cur, !more);
        if (!more) return false;
        core.begin_segment(nxp.s, nxp.g);
        core.init(St);
        --left;
        cur = nxp;
        return true;
    };
    typename Core::Chunk b0, b1;
    b0 = core.load(cur.s, cur.g, cur.c);
    while (one(b0, b1) && one(b1, b0)) {
    }
}

// LDS-ring walk: each wave keeps R chunks of its range in flight in its own
// LDS slots and computes from registers read out of the oldest.
//
// Every iteration issues the range's next chunk, if any, into the slot just
// read, so when chunk i is waited for, k = min(R - 1, n - 1 - i) chunks of at
// least DPC vector memory loads each have been issued after it, and the wait
// is vmcnt(k * DPC): loads complete in issue order, so with at most k * DPC
// instructions in flight the chunk's loads are done, whatever else (a new
// token's row loads, stores, which only leave the count earlier) was issued in
// between. Nothing is issued past the range end, so the last chunk's wait and
// the wave's final stores do not wait behind loads that are never used.
// Segment ends drain the wave instead: the query loads of the next segment are
// waited for there (so the compiler never sees them pending inside the loop),
// and so are the output stores, which may complete out of order with loads.
//
// wait_ring: wait until at most min(R - 1, later) * DPC vector memory
// instructions are in flight, `later` being the number of chunks issued after
// the one waited for.
template <int R, int DPC>
__device__ __forceinline__ void wait_ring(int later) {
    if (later >= R - 1) {
        wait_vmcnt<(R - 1) * DPC>();
    } else if constexpr (R > 2) {
        if (later == 2)
            wait_vmcnt<2 * DPC>();
        else if (later == 1)
            wait_vmcnt<DPC>();
        else
            wait_vmcnt<0>();
    } else {
        wait_vmcnt<0>();
    }
}

template <class Core, int NWG>
__device__ __forceinline__ void decode_balanced_ring(const DecodeArgs& a) {
    constexpr int G = Core::G, D = Core::D, R = Core::R, SLOT = Core::SLOT, DPC = Core::DPC;
    constexpr bool PAIR = Core::PAIR;
    __shared__ BalancedShared<NWG> sh;
    __shared__ int ns_tab[PAIR ? kMaxPairUnits : 1];
    __shared__ __attribute__((aligned(16))) char ring[NWG * R * SLOT];
    if (a.slot_mapping != nullptr && blockIdx.x == 0) {
        // new tokens of sequences with an empty context: no chunk carries them
        for (int s = threadIdx.x; s < a.num_seqs; s += blockDim.x)
            if (ld_const(a.context_lens, s) == 0)
                for (int g = 0; g < a.num_kv_heads; ++g)
                    for (int v = 0; v < D / 8; ++v)
                        Core::write_vector_at(a, s, g, v);
    }
    WaveRange r;
    if (!balanced_setup<G, D, NWG, PAIR>(a, sh, r, ns_tab)) return;
    const uint32_t nst = lds_addr(ns_tab);
    char* const mine = ring + uniform(threadIdx.x >> 6) * (R * SLOT);
    SegPos cur = r.cur;
    Core core(a);
    core.cow = r.hm;
    const int n = (int)(r.X1 - r.X0);                // chunks in the range (>= 1)
    SegPos ahead = cur;                              // next chunk to issue
    int issued = 0;
    // When the decode writes the new tokens: a sequence's last chunk holds its
    // new token of kv head g, and one wave consumes it. That wave loads the
    // token's rows with the chunk and, once both are in LDS, writes the token
    // into its cache slot and over the chunk's stale row (patch_new_token), so
    // the kernel never reads back what it stores.
    const bool writes = a.slot_mapping != nullptr;
    auto issue_next = [&](char* sp) {
        const ChunkRef q = chunk_ref<PAIR>(ahead);
        core.issue(sp, q.s, ahead.g, q.c, writes && q.last);
        if (++issued < n) ahead = next_pos<PAIR>(a, ahead, r.hm, r.sc, nst);
    };
#pragma unroll
    for (int k = 0; k < R; ++k)
        if (k < n) issue_next(mine + k * SLOT);
    core.begin_segment(cur.s, cur.g);
    wait_vmcnt<0>();
    typename Core::State St;
    core.init(St);
    PieceEnd<Core> end{a, core, r};
    int slot = 0;
    for (int i = 0;; ++i) {
        wait_ring<R, DPC>(n - 1 - i);                // chunk i is in its slot
        char* const sp = mine + slot * SLOT;
        const ChunkRef q = chunk_ref<PAIR>(cur);
        if (writes && q.last) core.patch_new_token(sp, cur.g, q.t1);
        const typename Core::Chunk ch = core.fetch(sp);   // the slot is free again
        if (issued < n) issue_next(sp);
        slot = (slot + 1 == R) ? 0 : slot + 1;
        if constexpr (PAIR)
            core.step(St, ch, q.c, q.t1, q.who);
        else
            core.step(St, ch, q.c, q.t1);
        const bool last = i + 1 == n;
        if (!last && cur.c + 1 < cur.n) {            // same segment
            ++cur.c;
            continue;
        }
        end(St, cur, last);
        if (last) break;
        cur = next_pos<PAIR>(a, cur, r.hm, r.sc, nst);
        core.begin_segment(cur.s, cur.g);
        wait_vmcnt<0>();
        core.init(St);
    }
    wait_vmcnt<0>();                                 // no load may land in LDS after the wave ends
}

}  // namespace pa
