// Several new query tokens per sequence over the paged KV cache: the target
// model scoring K drafted tokens in one pass (speculative decoding,
// Continuous-Batching-LLM-Inference-Engine README, feature list) and the
// prefill chunks that continuous batches mix with decode tokens ("How
// brave30/mini-inference-engine works", summary; Model Compute: prefill
// attention). The n new tokens of a sequence of L cached tokens are its last
// n; new token j sits at position L - n + j and attends to tokens 0 .. L-n+j.
//
// With several query rows per kv head the product is a real contraction, so it
// runs on 16x16x32 bf16 MFMAs:
//   S^T = K Q^T   A = K tile (16 tokens x 32 dims), B = Q^T (32 dims x 16 rows)
//   O^T += V^T P^T  A = V^T (16 dims x 32 tokens), B = P^T (32 tokens x 16 rows)
// A query row is a (new token, head of the group) pair, so the G heads that
// share a kv head share every K/V load. Computing S^T rather than S leaves
// each lane with one query row (lane % 16) and eight tokens, so the row max
// and sum need only the exchange between the four lanes of that row, and the
// S^T registers are already the P^T operand of the next MFMA: the k slots
// 8q..8q+7 of lane group q = lane / 16 stand for tokens 4q..4q+3 and
// 16+4q..16+4q+3 of the 32-token tile, and the V^T operand is read with the
// same pairing.
//
// Lane layout of v_mfma_f32_16x16x32_bf16: lane l holds A[l % 16][8q .. 8q+7],
// B[8q .. 8q+7][l % 16] and D[4q .. 4q+3][l % 16], q = l / 16.
// ds_read_b64_tr_b16 (LDS read with a transpose inside each 16-lane group):
// lane i of a group receives, as element k, element i % 4 of the 8 bytes that
// lane 4k + i / 4 of its group addressed. So V stays row-major in LDS, like
// K, and the V^T operand of lane (i, q) -- V[4q + k][d0 + i], k = 0..3 -- is
// one such read in which lane j of group q addresses row 4q + j / 4, columns
// d0 + 4 (j % 4) .. +3 (and a second one 16 rows further down).
//
// Workgroup: 4 waves for one (sequence, kv head, tile of query rows), as NR
// row groups x NT = 4 / NR token groups. A row group owns MB blocks of 16
// rows; a token group streams every NT-th 32-token KV tile through its own
// LDS buffer (K and V row-major), filled by the NR waves that consume it. Token groups merge their
// softmax states through LDS at the end. Few rows (the verify pass): NR = 1,
// and four waves split the context; many rows (prefill chunks): NR = 4, and
// each KV tile read from HBM feeds 128 rows.
#include "pa_device.hpp"
#include "pa_prefill.hpp"
#include "pa_write_row.hpp"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int PD = 128;               // head_dim
constexpr int TK = 32;                // tokens per KV tile
// K and V tile row stride in LDS (bytes): 72 dwords, 8 banks further per row,
// so the transposing V reads (4 rows x 32 bytes per 16-lane group) and the K
// operand reads (8 rows x 16 bytes per pass) hit distinct banks
constexpr int KSTR = PD * 2 + 32;
constexpr int KBYTES = TK * KSTR;
constexpr int TGBYTES = 2 * KBYTES;   // a token group's K and V tiles
constexpr float kLog2e = 1.4426950408889634f;
// The running output and sum are rescaled to a row's new max only once the
// max has grown by more than this (log2 units) over the max they refer to;
// until then the weights exp2(x - m) stay below 2^kLazy.
constexpr float kLazy = 8.0f;

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

typedef short i16x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ds_read_tr16(const char* p) {
    const i16x4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4v*)(p));
    return __builtin_bit_cast(uint2, r);
}

// Sixteen int8 codes -> sixteen bf16 (exact: |code| < 2^8).
__device__ __forceinline__ void i8_to_bf16(uint4 v, uint4& lo, uint4& hi) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        o[2 * k] = pack_bf16_trunc(i8_at(w[k], 0), i8_at(w[k], 1));
        o[2 * k + 1] = pack_bf16_trunc(i8_at(w[k], 2), i8_at(w[k], 3));
    }
    lo = make_uint4(o[0], o[1], o[2], o[3]);
    hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// Batches of at most this many sequences are placed by length (snake_place).
constexpr int kSnakeMax = 256;

// A workgroup's sequence, its first query row, its number of query rows and
// its context length.
struct SeqPlace {
    int s, q0, n, L;
};

// The sequence that takes place p of the XCD-contiguous sequence list when
// the places are dealt by length: the sequences ranked by context length
// (longest first, ties by index) go to the 8 XCDs' runs of the list in a
// snake (ranks 0-7 to XCDs 0-7, ranks 8-15 to XCDs 7-0, ...); within a run
// longest first, or (pair) the first half longest first and the second half
// shortest first. Every XCD then gets about the same share of the KV, with
// pair each CU a long and a short context, and the longest contexts start
// first. S = 8 runs of S / 8 places,
// S <= blockDim.x;
// all threads of the workgroup call it (it has barriers). The lengths and
// query starts are read once, into LDS (sh: 2 S + 2 ints, free again on
// return), and the sequence's own values are taken from there.
__device__ SeqPlace snake_place(const int32_t* lens, const int32_t* qsl, int S, int p, int* sh,
                                bool pair) {
    const int t = threadIdx.x;
    int* shq = sh + S;                                // S + 1 query starts
    if (t < S) sh[t] = lens[t];
    for (int i = t; i <= S; i += blockDim.x) shq[i] = qsl[i];
    __syncthreads();
    // pair (every workgroup resident at once): the run's second half in
    // reverse. The XCD's workgroups fill its CUs' first slots in run order,
    // then their second slots, so run positions j and j + per / 2 share a CU,
    // which then holds a long and a short context (Llama-shaped batch 63.4 ->
    // 60.8 us, verify 63.3 -> 59.8 us, against both halves longest first).
    // With more workgroups than slots the run stays longest first, which
    // starts the longest contexts first (the int8 batch, 128 sequences: 139.7
    // us longest first, 152.7 us paired).
    const int per = S / 8, x = p / per, j0 = p % per, half = per / 2;
    const int j = (!pair || j0 < half) ? j0 : per - 1 - (j0 - half);
    const int r = 8 * j + ((j & 1) ? 7 - x : x);
    if (t < S) {
        const int Lt = sh[t];
        int rank = 0;
        for (int u = 0; u < S; ++u) {
            const int Lu = sh[u];
            rank += (Lu > Lt) || (Lu == Lt && u < t);
        }
        if (rank == r) sh[2 * S + 1] = t;             // ranks are a permutation of 0..S-1
    }
    __syncthreads();
    SeqPlace sp;
    sp.s = sh[2 * S + 1];
    sp.q0 = shq[sp.s];
    sp.n = shq[sp.s + 1] - sp.q0;
    sp.L = sh[sp.s];
    __syncthreads();
    return sp;
}

// WR: the kernel also writes the new tokens (int8 caches: their codes under
// the (block, kv head) scales)
template <int NR, int MB, bool I8, int BS, bool WR>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
    constexpr int NT = 4 / NR;
    constexpr int RT = NR * MB * 16;                  // query rows per workgroup
    constexpr int TPT = NR * 64;                      // threads filling one token group's tile
    constexpr int EPP = I8 ? 16 : 8;                  // cache elements per 16-byte piece
    constexpr int PPR = PD / EPP;                     // pieces per token row
    constexpr int NLD = TK * PPR / TPT;               // pieces per thread per tile (K, and V)
    static_assert(TK * PPR % TPT == 0, "tile split");
    constexpr int ELT = I8 ? 1 : 2;
    // Tiles in flight in registers: two where a tile takes at most 2 pieces
    // per thread and pool (16 VGPRs: the 128-row instances, whose 4 waves
    // fill one tile together), one otherwise (a second would leave one wave
    // per SIMD). With two, each token group also has two LDS buffers used in
    // turn, and one barrier per tile suffices.
    constexpr int DEPTH = NLD <= 2 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) char lds[DEPTH * NT * TGBYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = wave % NR, tg = wave / NR;
    const int col = lane & 15, quad = lane >> 4;
    const int Hq = a.num_heads, Hkv = a.num_kv_heads;
    constexpr int B = BS;                             // block size (16 or 32)
    // workgroup -> (row tile, kv head, sequence). Consecutive workgroups go
    // to the 8 XCDs in turn; the logical index runs through each XCD's share
    // first, so the row tiles of one (sequence, kv head), which read the same
    // KV, share one XCD's L2, and so do the kv heads of a sequence, whose
    // tiles of a block are neighbours in the pool. (Spreading the kv heads
    // over the XCDs, which evens out the XCDs' shares of the KV, was 4-5%
    // slower on the 64-sequence batch, with or without rotating the heads.)
    // Split-K with one row tile: the logical index itself, with the partition
    // index rotated by the (sequence, kv head) index. The partitions of a
    // (sequence, kv head) then spread over the XCDs, and so do the first
    // partitions of the different sequences, which mixed lengths make the
    // busiest (copy-on-write batch, 1024-token partitions: 390 us with the
    // XCD-contiguous order, 280 us rotated, 878 us unrotated, where XCD j
    // took every partition j, j + 8, ...).
    const int W = gridDim.x, w0 = blockIdx.x;
    const bool spread = a.row_tiles == 1 && a.num_partitions > 1;
    const int w = (W % 8 || spread) ? w0 : (w0 % 8) * (W / 8) + w0 / 8;
    const int NP = a.num_partitions;                  // 1 without split-K
    const int rt = w % a.row_tiles, rest = w / a.row_tiles;
    const int sg = rest / NP, part = spread ? (rest + sg) % NP : rest % NP;
    const int g = sg % Hkv;
    // one row tile, no split: the sequences are placed by length (snake_place)
    static_assert((2 * kSnakeMax + 2) * 4 <= NT * TGBYTES, "placement scratch fits the LDS");
    SeqPlace sp;
    if (a.row_tiles == 1 && NP == 1 && W % 8 == 0 && a.num_seqs % 8 == 0 &&
        a.num_seqs <= kSnakeMax) {
        sp = snake_place(a.context_lens, a.query_start_loc, a.num_seqs, sg / Hkv,
                         reinterpret_cast<int*>(lds), a.one_round != 0);
    } else {
        sp.s = sg / Hkv;
        sp.q0 = ld_const(a.query_start_loc, sp.s);
        sp.n = ld_const(a.query_start_loc, sp.s + 1) - sp.q0;
        sp.L = ld_const(a.context_lens, sp.s);
    }
    // (the same in every lane: kept in scalar registers, which also makes
    // the tile loop's bounds and the block-table addresses scalar; chunked
    // prefill 304.1 -> 296.5 us)
    const int s = uniform(sp.s), q0 = uniform(sp.q0), n = uniform(sp.n), L = uniform(sp.L);
    const int G = Hq / Hkv;
    const int tiles = (n * G + RT - 1) / RT;
    if (rt >= tiles) return;
    const int tile = tiles - 1 - rt;                  // the tiles with the longest context first
    const int TQ = RT / G;                            // query tokens per tile (G divides 16)
    const int tok0 = tile * TQ;
    const int p_first = L - n + tok0;                 // position of the tile's first new token
    const int limit = p_first + min(TQ, n - tok0);    // the tile reads tokens [0, limit)
    // split-K: this workgroup takes the tokens [t_begin, min(t_begin + P, limit));
    // P is a multiple of the tile, so no tile straddles two partitions
    const int P = a.partition_size;
    const int t_begin = P > 0 ? part * P : 0;
    if (t_begin >= limit) return;
    const int kt0 = t_begin / TK;
    const int nkt = P > 0 ? (min(limit, t_begin + P) + TK - 1) / TK : (limit + TK - 1) / TK;
    const int nit = (nkt - kt0 + NT - 1) / NT;
    const float sl2 = a.scale * kLog2e;
    // bf16 caches: the logit scale is applied inside the exponent's fma and the
    // row max is taken over the unscaled products, which needs a factor >= 0; a
    // negative scale negates Q instead
    const bool negq = !I8 && sl2 < 0.0f;
    const float fq = negq ? -sl2 : sl2;
    const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    const int new0 = L - n;                           // position of the sequence's first new token

    if constexpr (WR) {
        // the new tokens of this tile's rows whose positions fall in this
        // partition go to their slots (every token exactly once over the grid)
        const int ntok = min(TQ, n - tok0);
        for (int idx = threadIdx.x; idx < ntok * (PD / 8); idx += 256) {
            const int j = tok0 + idx / (PD / 8), v = idx % (PD / 8);
            const int pos = new0 + j;
            if (P > 0 && (pos < t_begin || pos >= t_begin + P)) continue;
            constexpr Dtype CW = I8 ? Dtype::I8 : Dtype::BF16;
            write_vector<Dtype::BF16, CW>(a.key, a.value, a.k_cache_w, a.v_cache_w,
                                          a.slot_mapping, a.k_scale, a.v_scale, Hkv, PD, B,
                                          (int64_t)q0 + j, g, v);
        }
    }

    // query rows of this lane: Q^T operands and positions (-1: a padding row)
    int rpos[MB];
    bf16x8 qop[MB][4];
    int64_t orow[MB];                                 // element offset of the row in q / out
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int r = (rg * MB + mb) * 16 + col;
        const int j = r / G, h = r - j * G;
        const bool valid = tok0 + j < n;
        rpos[mb] = valid ? p_first + j : -1;
        orow[mb] = ((int64_t)(q0 + tok0 + j) * Hq + g * G + h) * PD;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (valid)
                v = ld16(reinterpret_cast<const uint16_t*>(a.q) + orow[mb] + 32 * ks + 8 * quad);
            if (negq) {
                v.x ^= 0x80008000u;
                v.y ^= 0x80008000u;
                v.z ^= 0x80008000u;
                v.w ^= 0x80008000u;
            }
            qop[mb][ks] = as_bf16x8(v);
        }
    }

    float m[MB], l[MB];
    f32x4 o[MB][8];
    // row sums of the bf16 weights by an MFMA against ones (the same weights
    // the P V product uses); every element holds the row's sum
    f32x4 lsum[MB];
    const bf16x8 ones = as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        m[mb] = -__builtin_huge_valf();
        l[mb] = 0.0f;
        lsum[mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[mb][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // this thread's pieces of a tile: piece p = ti + k TPT is token p / PPR,
    // elements (p % PPR) * EPP ..
    const int ti = rg * 64 + lane;
    uint4 kr[NLD], vr[NLD], kr2[NLD], vr2[NLD];
    // A piece's address: the (block, kv head) tile's base, a scalar, plus
    // the lane's offset inside the tile (a tile starts on a block boundary,
    // so token t of the tile is row t % B of its block).
    constexpr int64_t TILE_BYTES = (int64_t)B * PD * ELT;     // one (block, kv head) tile
    const int64_t blk_stride = (int64_t)Hkv * TILE_BYTES, head_off = (int64_t)g * TILE_BYTES;
    // tokens of one load instruction: all in the same 16-token half?
    constexpr int TOK_PER_LD = TPT / PPR;
    constexpr bool HALF_UNIFORM = TOK_PER_LD <= 16;
    // The tile's (at most two) block ids, as scalar loads (a vector load of
    // a block id would have to wait for every K/V load issued before it),
    // turned into the byte offsets of its (block, kv head) tiles. They are
    // fetched one tile ahead: under a saturated memory system even a cached
    // id takes long to come back, and waiting for it between a tile's arrival
    // and the next tile's loads would leave the wave with nothing in flight.
    // A half wholly past the context takes the other half's base (a block of
    // the sequence when the tile is computed at all; block 0 of the pool for
    // a spare tile past the context, which is loaded but never computed).
    // (kt is the same in every lane of the wave; saying so keeps the test and
    // the bases in scalar registers: 1-3% fewer VGPRs)
    // (int8: bid keeps the halves' block ids, -1 for a half wholly past the
    // context, for the scales)
    int bid[2] = {-1, -1};
    auto tile_bases = [&](int kt_, int64_t (&base)[2]) {
        const int kt = uniform(kt_);
        if constexpr (I8) {
            const int b0 = kt * TK < limit ? ld_uniform(bt, (kt * TK) / B) : -1;
            const int b1 = kt * TK + 16 < limit ? ld_uniform(bt, (kt * TK + 16) / B) : -1;
            base[0] = b0 >= 0 ? (int64_t)b0 * blk_stride + head_off : 0;
            base[1] = b1 >= 0 ? (int64_t)b1 * blk_stride + head_off : base[0];
            bid[0] = b0;
            bid[1] = b1;
        } else {
            base[0] = kt * TK < limit
                ? (int64_t)ld_uniform(bt, (kt * TK) / B) * blk_stride + head_off : 0;
            base[1] = kt * TK + 16 < limit
                ? (int64_t)ld_uniform(bt, (kt * TK + 16) / B) * blk_stride + head_off : base[0];
        }
    };
    // int8: the (block, kv head) scales of a tile's two halves (1 for a half
    // past the context), loaded when the tile's loads are issued, a tile
    // ahead of its compute: loaded at the start of the compute they held up
    // its first LDS reads, whose wait also waits for scalar loads
    struct Scales {
        float k0, k1, v0, v1;
    };
    auto fetch_scales = [&](Scales& sc) {
        sc.k0 = sc.k1 = sc.v0 = sc.v1 = 1.0f;
        {
            if (bid[0] >= 0) {
                sc.k0 = ld_uniform(a.k_scale, (int64_t)bid[0] * Hkv + g);
                sc.v0 = ld_uniform(a.v_scale, (int64_t)bid[0] * Hkv + g);
            }
            if (bid[1] >= 0) {
                sc.k1 = ld_uniform(a.k_scale, (int64_t)bid[1] * Hkv + g);
                sc.v1 = ld_uniform(a.v_scale, (int64_t)bid[1] * Hkv + g);
            }
        }
    };
    // A KV tile that no other workgroup of the launch reads is loaded
    // non-temporal: kept out of the L2's way, it leaves the room to lines that
    // are read again. That holds in the instances of at most 64 rows (one row
    // tile per sequence) unless the sequence starts on a block that a
    // neighbouring sequence shares copy-on-write. Llama-shaped decode 60.5 ->
    // 52.9 us, speculative verify 59.6 -> 52.2 us, 8 x 32768 split-K step
    // 188.8 -> 169.6 us. (The 128-row instance keeps cached loads: its row
    // tiles of a sequence read the same KV, and the second load path alone
    // slowed chunked prefill by 2%.)
    const bool stream = RT <= 64 &&
        !first_block_shared(a.block_tables, a.max_blocks_per_seq, a.num_seqs, s);
    // FRESH (WR, a tile that holds new tokens): negm and, int8, the scales
    // nks / nvs of the tile's two halves, for the new tokens' codes
    auto load_tile_p = [&](int kt, const int64_t (&base)[2], uint4 (&kr)[NLD], uint4 (&vr)[NLD],
                           uint32_t negm, const float (&nks)[2], const float (&nvs)[2], auto nt,
                           auto fresh_tag) {
        constexpr bool FRESH = decltype(fresh_tag)::value;
        // (the two bases as values: an index into `base` chosen per lane
        // would put the array in memory)
        const int64_t base0 = base[0], base1 = base[1];
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
            const int p = ti + k * TPT, t = p / PPR, e = (p % PPR) * EPP;
            // a token at or past `limit` reads the first token of its half's
            // block instead, a token of the context (so finite, whatever the
            // pool's unused blocks hold): every row masks it (x = -inf, weight 0)
            const bool in = kt * TK + t < limit;
            const uint32_t lo = (uint32_t)(((in ? t % B : 0) * PD + e) * ELT);
            const int64_t bb = HALF_UNIFORM ? ((k * TOK_PER_LD) / 16 ? base1 : base0)
                                            : (t < 16 ? base0 : base1);
            if constexpr (FRESH) {
                // a new token's row comes from key / value (its slot is being
                // written by this launch). A masked piece stands for the
                // tile's first token, kt TK (base 0): an older token or a new
                // one taken from key / value -- the first token of its own
                // half's block may be a new token whose slot this launch is
                // still writing. A tile wholly past the context (the last
                // iteration's spare waves) has jn >= n and reads block 0 of
                // the cache instead, like the other instances.
                const int tt = in ? t : 0;
                const int jn = kt * TK + tt - new0;
                const int64_t bf = in ? bb : base0;
                const char* kp = reinterpret_cast<const char*>(a.k_cache) + bf + lo;
                const char* vp = reinterpret_cast<const char*>(a.v_cache) + bf + lo;
                const bool fresh = jn >= 0 && jn < n && !((negm >> tt) & 1u);
                const int64_t src = (((int64_t)q0 + jn) * Hkv + g) * PD + e;
                const char* kn = reinterpret_cast<const char*>(a.key) + src * 2;
                const char* vn = reinterpret_cast<const char*>(a.value) + src * 2;
                if constexpr (I8) {
                    // the 16 codes the write stores: two 16-byte vectors of
                    // bf16 activations quantised with the half's scales (the
                    // block the write's slot names; the tables agree with the
                    // slots)
                    if (fresh) {
                        const float ks = tt < 16 ? nks[0] : nks[1];
                        const float vs = tt < 16 ? nvs[0] : nvs[1];
                        const uint2 k0 = codes_bf16x8(ld16(kn), ks), k1 = codes_bf16x8(ld16(kn + 16), ks);
                        const uint2 v0 = codes_bf16x8(ld16(vn), vs), v1 = codes_bf16x8(ld16(vn + 16), vs);
                        kr[k] = make_uint4(k0.x, k0.y, k1.x, k1.y);
                        vr[k] = make_uint4(v0.x, v0.y, v1.x, v1.y);
                    } else {
                        kr[k] = ld16p<nt()>(kp);
                        vr[k] = ld16p<nt()>(vp);
                    }
                } else {
                    kr[k] = ld16p<nt()>(fresh ? kn : kp);
                    vr[k] = ld16p<nt()>(fresh ? vn : vp);
                }
            } else {
                kr[k] = ld16p<nt()>(at(reinterpret_cast<const char*>(a.k_cache) + bb, lo));
                vr[k] = ld16p<nt()>(at(reinterpret_cast<const char*>(a.v_cache) + bb, lo));
            }
        }
    };
    auto load_tile = [&](int kt, const int64_t (&base)[2], uint4 (&kr)[NLD], uint4 (&vr)[NLD]) {
        using T1 = std::true_type;
        using T0 = std::false_type;
        const float one[2] = {1.0f, 1.0f};
        if constexpr (WR) {
            // A tile that holds new tokens (the same in every lane; the other
            // tiles take the plain loads). Bit t of negm is set when token
            // kt TK + t is a new token with a negative slot: it is not
            // written, so its position is read from the cache like any other.
            const int j0 = uniform(kt * TK - new0);   // new-token index of the tile's token 0
            if (j0 + TK > 0 && j0 < n) {
                uint32_t negm = 0;
                float nks[2] = {1.0f, 1.0f}, nvs[2] = {1.0f, 1.0f};
                // the slots' high words, eight scalar loads at a time (the
                // index clamped into the tile's new tokens), one wait each
                const int tb = max(0, -j0), te = min(TK, n - j0);
                const int32_t* shi = reinterpret_cast<const int32_t*>(a.slot_mapping) + 1;
                for (int t0 = tb; t0 < te; t0 += 8) {
                    int32_t hi[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        hi[u] = ld_uniform(shi, 2 * ((int64_t)q0 + j0 + min(t0 + u, te - 1)));
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (t0 + u < te && hi[u] < 0) negm |= 1u << (t0 + u);
                }
                if constexpr (I8) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int T = kt * TK + 16 * h;
                        if (T < limit) {
                            const int64_t b = ld_uniform(bt, T / B);
                            nks[h] = ld_uniform(a.k_scale, b * Hkv + g);
                            nvs[h] = ld_uniform(a.v_scale, b * Hkv + g);
                        }
                    }
                }
                if (RT <= 64 && stream)
                    load_tile_p(kt, base, kr, vr, negm, nks, nvs, T1{}, T1{});
                else
                    load_tile_p(kt, base, kr, vr, negm, nks, nvs, T0{}, T1{});
                return;
            }
        }
        if (RT <= 64 && stream)
            load_tile_p(kt, base, kr, vr, 0u, one, one, T1{}, T0{});
        else
            load_tile_p(kt, base, kr, vr, 0u, one, one, T0{}, T0{});
    };
    char* kl = lds + tg * TGBYTES;                    // the token group's buffer in use
    char* vl = kl + KBYTES;
    // this lane's address in the transposed V reads (see the file comment)
    const int vtr = (4 * quad + col / 4) * KSTR + 8 * (col % 4);
    auto store_tile = [&](const uint4 (&kr)[NLD], const uint4 (&vr)[NLD]) {
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
            const int p = ti + k * TPT, t = p / PPR, e = (p % PPR) * EPP;
            uint4 kv[2], vv[2];
            if (I8) {
                i8_to_bf16(kr[k], kv[0], kv[1]);
                i8_to_bf16(vr[k], vv[0], vv[1]);
            } else {
                kv[0] = kr[k];
                vv[0] = vr[k];
            }
#pragma unroll
            for (int hlf = 0; hlf < EPP / 8; ++hlf) {
                *reinterpret_cast<uint4*>(kl + t * KSTR + (e + 8 * hlf) * 2) = kv[hlf];
                *reinterpret_cast<uint4*>(vl + t * KSTR + (e + 8 * hlf) * 2) = vv[hlf];
            }
        }
    };

    // EDGE: some row of the tile must mask some token of this KV tile
    auto compute = [&](int kt, auto edge_tag, const Scales& sc) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        // int8: per-(block, kv head) scales of the two 16-token halves
        const float ksc[2] = {I8 ? sc.k0 : 1.0f, I8 ? sc.k1 : 1.0f};
        const float vsc[2] = {I8 ? sc.v0 : 1.0f, I8 ? sc.v1 : 1.0f};
        // S^T for every row block; each K operand is read right before its
        // MFMAs (all row blocks use it), which keeps few operands live
        f32x4 acc[MB][2];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) acc[mb][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // k slices outermost: the 2 MB accumulators take turns, so no MFMA
        // waits for the one before it. The wave raises its issue priority
        // for its runs of MFMAs (here and for P V): the other wave of the
        // SIMD, usually in its softmax, then issues its vector work in the
        // gaps, and the matrix cores idle less (chunked prefill 317.8 ->
        // 303.2 us; the QK^T run alone 313.0, the P V run alone 306.6 us;
        // priority 3 level with 1; the decode shapes level).
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const bf16x8 kop = as_bf16x8(*reinterpret_cast<const uint4*>(
                    kl + (tt * 16 + col) * KSTR + (32 * ks + 8 * quad) * 2));
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb][tt] = mfma16x16x32(kop, qop[mb][ks], acc[mb][tt]);
            }
        __builtin_amdgcn_s_setprio(0);
        bf16x8 pop[MB];
        if constexpr (!I8) {
            // every row block's max first, then one wave-uniform test for the
            // (rare) rescale of any of them, then the weights: no branch
            // separates the row blocks' exponentials and sums
            float mn[MB];
            bool grow = false;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                // max over the unscaled products (fq >= 0), masked ones excluded
                float mx = -__builtin_huge_valf();
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool msk = EDGE && kt * TK + tt * 16 + 4 * quad + i > rpos[mb];
                        mx = fmaxf(mx, msk ? -__builtin_huge_valf() : acc[mb][tt][i]);
                    }
                mx = fmaxf(mx, lane_xor16(mx));
                mx = fmaxf(mx, lane_xor32(mx));
                const float mxs = mx == -__builtin_huge_valf() ? mx : mx * fq;
                mn[mb] = fmaxf(m[mb], mxs);
                grow = grow || mn[mb] > m[mb] + kLazy;
            }
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    if (__builtin_amdgcn_ballot_w64(mn[mb] > m[mb] + kLazy) != 0) {   // wave-uniform
                        const float mu = mn[mb] == -__builtin_huge_valf() ? 0.0f : mn[mb];
                        const float alpha = __builtin_amdgcn_exp2f(m[mb] - mu);
                        m[mb] = mn[mb];
#pragma unroll
                        for (int i = 0; i < 4; ++i) lsum[mb][i] *= alpha;
#pragma unroll
                        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) o[mb][dt][i] *= alpha;
                    }
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const float nmu = m[mb] == -__builtin_huge_valf() ? 0.0f : -m[mb];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float pr = __builtin_amdgcn_exp2f(fmaf(acc[mb][tt][i], fq, nmu));
                        if (EDGE && kt * TK + tt * 16 + 4 * quad + i > rpos[mb]) pr = 0.0f;
                        pop[mb][4 * tt + i] = (__bf16)pr;
                    }
                lsum[mb] = mfma16x16x32(ones, pop[mb], lsum[mb]);
            }
        } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          {
            float x[2][4];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const float f = I8 ? sl2 * ksc[tt] : sl2;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[tt][i] = acc[mb][tt][i] * f;
                    if (EDGE && kt * TK + tt * 16 + 4 * quad + i > rpos[mb])
                        x[tt][i] = -__builtin_huge_valf();
                }
            }
            float mx = x[0][0];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[tt][i]);
            mx = fmaxf(mx, lane_xor16(mx));
            mx = fmaxf(mx, lane_xor32(mx));
            const float mn = fmaxf(m[mb], mx);
            if (__builtin_amdgcn_ballot_w64(mn > m[mb] + kLazy) != 0) {   // wave-uniform
                const float mu = mn == -__builtin_huge_valf() ? 0.0f : mn;
                const float alpha = __builtin_amdgcn_exp2f(m[mb] - mu);
                m[mb] = mn;
#pragma unroll
                for (int i = 0; i < 4; ++i) lsum[mb][i] *= alpha;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[mb][dt][i] *= alpha;
            }
            const float mu = m[mb] == -__builtin_huge_valf() ? 0.0f : m[mb];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pop[mb][4 * tt + i] = (__bf16)__builtin_amdgcn_exp2f(x[tt][i] - mu);
            lsum[mb] = mfma16x16x32(ones, pop[mb], lsum[mb]);
          }
        }
        }
        // O^T += V^T P^T, each V^T operand read right before its MFMAs. The k
        // slots 0-3 of a lane are tokens of the tile's first 16-token half and
        // slots 4-7 of its second, so on an int8 cache the product splits into
        // two 16x16x16 MFMAs, one per half (one block each), whose results are
        // scaled by that block's V scale in fp32.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const uint2 x0 = ds_read_tr16(vl + vtr + 32 * dt);
            const uint2 x1 = ds_read_tr16(vl + vtr + 16 * KSTR + 32 * dt);
            if constexpr (!I8) {
                const bf16x8 vop = as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y));
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) o[mb][dt] = mfma16x16x32(vop, pop[mb], o[mb][dt]);
            } else {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const i16x4v p0 = __builtin_bit_cast(i16x4v, __builtin_shufflevector(
                        pop[mb], pop[mb], 0, 1, 2, 3));
                    const i16x4v p1 = __builtin_bit_cast(i16x4v, __builtin_shufflevector(
                        pop[mb], pop[mb], 4, 5, 6, 7));
                    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
                    const f32x4 t0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        __builtin_bit_cast(i16x4v, x0), p0, zero, 0, 0, 0);
                    const f32x4 t1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        __builtin_bit_cast(i16x4v, x1), p1, zero, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        o[mb][dt][i] = fmaf(vsc[1], t1[i], fmaf(vsc[0], t0[i], o[mb][dt][i]));
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // One iteration: tile `it` (held in kr/vr) to LDS, tile it + 1 into
    // kr/vr, the block ids of tile it + 2 requested, then tile `it` computed
    // (the barrier counts are the same in every wave).
    // With one row group a token group is one wave, alone on its buffer: its
    // LDS accesses are performed in issue order, so no barrier is needed.
    // With two tiles in flight every iteration issues the loads of tile
    // it + 2, also past the last tile (such a tile reads in-bounds cache
    // memory, as spare tiles do, and is never computed): with the loads
    // unconditional the compiler's wait before storing a tile counts exactly
    // the other tile's loads as still in flight (conditional loads made it
    // wait for both).
    int64_t bnext[2] = {0, 0};
    Scales sc1{1.0f, 1.0f, 1.0f, 1.0f}, sc2{1.0f, 1.0f, 1.0f, 1.0f};   // kr/vr's and kr2/vr2's tiles
    if (DEPTH == 2 || nit > 0) {
        tile_bases(kt0 + tg, bnext);
        load_tile(kt0 + tg, bnext, kr, vr);
        if constexpr (I8) fetch_scales(sc1);
    }
    if (DEPTH == 2) {
        tile_bases(kt0 + tg + NT, bnext);
        load_tile(kt0 + tg + NT, bnext, kr2, vr2);
        if constexpr (I8) fetch_scales(sc2);
    }
    if (DEPTH == 2 || nit > DEPTH) tile_bases(kt0 + tg + DEPTH * NT, bnext);
    // Iteration it: its tile (in kr/vr) to LDS, tile it + DEPTH into the same
    // registers, the block ids of tile it + DEPTH + 1 requested, then tile it
    // computed.
    // With one LDS buffer the barrier before the store waits for the previous
    // tile's reads. With two, buffer b is written again two tiles later, after
    // the next tile's barrier, which every wave reaches only once it has
    // computed from b.
    auto iteration = [&](int it, uint4 (&kr)[NLD], uint4 (&vr)[NLD], Scales& sc, int buf) {
        const int kt = kt0 + it * NT + tg;
        kl = lds + (buf * NT + tg) * TGBYTES;
        vl = kl + KBYTES;
        if constexpr (NR > 1 && DEPTH == 1) __syncthreads();
        store_tile(kr, vr);
        const Scales cur = sc;                       // this tile's, before the next tile's
        if constexpr (NR > 1) __syncthreads();
        if (DEPTH == 2 || it + DEPTH < nit) {
            load_tile(kt + DEPTH * NT, bnext, kr, vr);
            if constexpr (I8) fetch_scales(sc);
            if (DEPTH == 2 || it + DEPTH + 1 < nit) tile_bases(kt + (DEPTH + 1) * NT, bnext);
        }
        if (kt < nkt) {
            if (kt * TK + TK - 1 > p_first)
                compute(kt, std::true_type{}, cur);
            else
                compute(kt, std::false_type{}, cur);
        }
    };
    if constexpr (DEPTH == 2) {
        // both halves unconditional inside the loop (see above), the odd
        // last tile after it
        int it = 0;
        for (; it + 1 < nit; it += 2) {
            iteration(it, kr, vr, sc1, 0);
            iteration(it + 1, kr2, vr2, sc2, 1);
        }
        if (it < nit) iteration(it, kr, vr, sc1, 0);
    } else {
        for (int it = 0; it < nit; ++it) iteration(it, kr, vr, sc1, 0);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) l[mb] = lsum[mb][0];   // already the whole row's sum

    if (NT > 1) {
        // token groups 1 .. NT-1 hand their states to token group 0 of their row group
        __syncthreads();
        float* st = reinterpret_cast<float*>(lds);
        constexpr int SLOT = MB * (8 * 64 * 4 + 2 * 64);   // floats per handed-over wave state
        static_assert((NT - 1) * NR * SLOT * 4 <= NT * TGBYTES, "merge states fit the tiles' LDS");
        if (tg > 0) {
            float* w = st + ((tg - 1) * NR + rg) * SLOT;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
                    *reinterpret_cast<f32x4*>(w + ((mb * 8 + dt) * 64 + lane) * 4) = o[mb][dt];
                w[MB * 8 * 64 * 4 + mb * 64 + lane] = m[mb];
                w[MB * 8 * 64 * 4 + (MB + mb) * 64 + lane] = l[mb];
            }
        }
        __syncthreads();
        if (tg > 0) return;
#pragma unroll
        for (int u = 1; u < NT; ++u) {
            const float* w = st + ((u - 1) * NR + rg) * SLOT;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const float m2 = w[MB * 8 * 64 * 4 + mb * 64 + lane];
                const float l2 = w[MB * 8 * 64 * 4 + (MB + mb) * 64 + lane];
                const float M = fmaxf(m[mb], m2);
                const float a1 = m[mb] == -__builtin_huge_valf() ? 0.0f : __builtin_amdgcn_exp2f(m[mb] - M);
                const float a2 = m2 == -__builtin_huge_valf() ? 0.0f : __builtin_amdgcn_exp2f(m2 - M);
                m[mb] = M;
                l[mb] = l[mb] * a1 + l2 * a2;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(w + ((mb * 8 + dt) * 64 + lane) * 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[mb][dt][i] = o[mb][dt][i] * a1 + v[i] * a2;
                }
            }
        }
    }

    if (P > 0) {
        // the partition's normalised output, its reference max in natural units
        // (within ln 2^kLazy below its largest logit) and its sum; rows that
        // see no token of the partition write nothing
        constexpr float kLn2 = 0.6931471805599453f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (rpos[mb] < t_begin) continue;
            const int64_t slot = orow[mb] / PD * NP + part;
            const float inv = 1.0f / l[mb];
            float* dst = a.tmp_out + slot * PD + 4 * quad;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const f32x4 v = {o[mb][dt][0] * inv, o[mb][dt][1] * inv, o[mb][dt][2] * inv,
                                 o[mb][dt][3] * inv};
                *reinterpret_cast<f32x4*>(dst + 16 * dt) = v;
            }
            if (quad == 0) {
                a.tmp_max[slot] = m[mb] * kLn2;
                a.tmp_sum[slot] = l[mb];
                // the reduce's length of this query token: its position + 1
                // (written once: kv head 0, the token's first head, partition 0)
                if (part == 0 && g == 0 && col % G == 0)
                    a.row_lens[orow[mb] / PD / Hq] = rpos[mb] + 1;
            }
        }
        return;
    }
    // out[row][d], d = 16 dt + 4 quad + i: four bf16 per store
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        if (rpos[mb] < 0) continue;
        const float inv = 1.0f / l[mb];
        uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + orow[mb] + 4 * quad;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const uint32_t w0 = f32_to_bf16(o[mb][dt][0] * inv) |
                                ((uint32_t)f32_to_bf16(o[mb][dt][1] * inv) << 16);
            const uint32_t w1 = f32_to_bf16(o[mb][dt][2] * inv) |
                                ((uint32_t)f32_to_bf16(o[mb][dt][3] * inv) << 16);
            *reinterpret_cast<uint2*>(dst + 16 * dt) = make_uint2(w0, w1);
        }
    }
}

template <int NR, int MB, bool I8, int BS, bool WR>
void launch_one(PrefillArgs a, dim3 grid, hipStream_t st) {
    const void* fn = reinterpret_cast<const void*>(&prefill_kernel<NR, MB, I8, BS, WR>);
    const int resident = balanced_grid(fn, 256, st);  // workgroups the device holds at once
    a.one_round = resident > 0 && (int64_t)grid.x <= resident;
    hipLaunchKernelGGL((prefill_kernel<NR, MB, I8, BS, WR>), grid, dim3(256), 0, st, a);
}

template <int NR, int MB, int BS>
void launch_bs(const PrefillArgs& a, dim3 grid, hipStream_t st) {
    if (a.cache == Dtype::I8 && a.key)
        launch_one<NR, MB, true, BS, true>(a, grid, st);
    else if (a.cache == Dtype::I8)
        launch_one<NR, MB, true, BS, false>(a, grid, st);
    else if (a.key)
        launch_one<NR, MB, false, BS, true>(a, grid, st);
    else
        launch_one<NR, MB, false, BS, false>(a, grid, st);
}

template <int NR, int MB>
hipError_t launch_shape(PrefillArgs a, int tiles, hipStream_t st) {
    const int64_t total = (int64_t)tiles * a.num_partitions * a.num_kv_heads * a.num_seqs;
    if (total > 0x7fffffff) return hipErrorInvalidValue;
    a.row_tiles = tiles;
    const dim3 grid((unsigned)total);
    if (a.block_size == 16)
        launch_bs<NR, MB, 16>(a, grid, st);
    else
        launch_bs<NR, MB, 32>(a, grid, st);
    return hipGetLastError();
}

}  // namespace

bool prefill_supports(const PrefillArgs& a) {
    const int G = a.num_kv_heads > 0 ? a.num_heads / a.num_kv_heads : 0;
    return a.head_dim == PD && (a.block_size == 16 || a.block_size == 32) &&
           a.q_dtype == Dtype::BF16 && (a.cache == Dtype::BF16 || a.cache == Dtype::I8) &&
           G >= 1 && G <= 16 && 16 % G == 0;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
    if (!prefill_supports(a)) return hipErrorNotSupported;
    if (a.num_seqs == 0 || a.max_query_len == 0) return hipSuccess;
    const int64_t rows = (int64_t)a.max_query_len * (a.num_heads / a.num_kv_heads);
    if (rows <= 16) return launch_shape<1, 1>(a, 1, st);
    // 17-64 rows: 2 row groups x 2 token groups. (One row group of two row
    // blocks, for up to 32 rows, was level without the fused write and 2-3%
    // slower with it, whose instance then needed more than 256 registers:
    // one wave per SIMD.)
    if (rows <= 64) return launch_shape<2, 2>(a, 1, st);
    return launch_shape<4, 2>(a, (int)((rows + 127) / 128), st);
}

}  // namespace pa
