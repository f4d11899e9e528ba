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
//  PV, bf16 cache: v_mfma_f32_4x4x4_16b_bf16, 8 per chunk and head group.
//    Block (tg, qd) sums over the 4 tokens 4*k + tg of row group tg: the A
//    operand of lane l is one dim (8*(l%16) + e) of those 4 V rows, taken
//    from the lane's own 16-byte row loads by byte permutes; the B operand is
//    the lane's 4 probabilities, rounded to bf16 (the row sum l adds the
//    rounded values, so the output is an exact convex combination of the
//    weights used).
//  PV, int8 cache: v_mfma_f32_4x4x1_16b_f32, 32 per chunk and head group, on
//    the codes and p * v_scale in fp32. The A operand is V row 4*step + tg,
//    dims 8*(l%16) + e; the B operand is the lane's own probability register
//    `step`, already in place.
//  The 4 row states are merged with lane shuffles. Afterwards lane
//  (tg, qd, j4) owns dims 8*(4*qd + tg) + e, e = 0..7, of head j4: the final
//  output, a workspace partial and the combine of partials all use that
//  assignment, so each is one coalesced 16-byte (or 8 x 4-byte) access per lane.
//
// The partition driver loads K and V from HBM straight to registers with
// 16-byte loads (load), the next chunk's issued before the current one is
// computed; the balanced driver streams them through a per-wave LDS ring
// filled by direct loads (issue / fetch).
#include "pa_decode_common.hpp"
#include "pa_write_row.hpp"

namespace pa {
namespace {

template <int G_, Dtype CT>
struct MfmaCore {
    static constexpr int G = G_;
    static constexpr int D = 128;
    static constexpr bool BASE2 = true;
    static constexpr bool PAIR = false;          // one sequence per segment
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
    bool cow = false;    // neighbouring sequences share blocks: keep those cached (issue, load)
    int lane, j4, qd, tg;
    uint32_t k_off, v_off;                       // byte offsets inside a chunk
    float sl2;
    int shift;
    int64_t head_stride, block_stride;
    uint4 qr[NHB][4];                            // query operands of the segment

    // ---- LDS ring: chunks move HBM -> LDS by direct loads, LDS -> registers
    // by ds_read, so the chunks in flight hold no VGPRs -----------------------
    static constexpr int KT = 16 * D * CE;       // bytes of one 16-token K (or V) tile
    static constexpr int NDK = KT / 1024;        // 1 KB load instructions per tile
    static constexpr int NEW = 2 * KT + (Q8 ? 16 : 0);   // K, V, the int8 scales, then a new
    static constexpr int SLOT = NEW + 4 * D + 16;        // token's bf16 K and V rows and slot
    static constexpr int DPC = 2 * NDK + (Q8 ? 2 : 0);   // vector memory instructions per chunk
    static constexpr int R = Q8 ? 4 : 2;         // ring slots per wave
    // The K tile is stored with its 16-byte pieces permuted inside each row, so
    // that the loads read whole rows (bf16: a quarter-wave reads one 256-byte
    // row; int8: two 128-byte rows) and the ds_reads that assemble the MFMA
    // operands hit distinct LDS banks in every group of 8 or 16 lanes. V is
    // stored as it is (its operand reads are already contiguous).
    // bf16 cache: the piece (16 bytes, dims 8*pc ..) of its row that lane
    // 16*q + t moves in load i.
    static __device__ int kpiece(int t, int i) {
        return (t & 1) | (((t >> 3) & 1) << 1) | ((((t >> 1) & 1) ^ (i & 1)) << 2) |
               ((((t >> 2) & 1) ^ (i >> 1)) << 3);
    }
    uint32_t kdma[NDK];    // source byte offset in the K tile, per load instruction
    uint32_t krd[NDK];     // LDS byte offset of the lane's K piece, per piece group
    uint32_t vrd;          // LDS byte offset of the lane's V piece for step 0

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
#pragma unroll
        for (int i = 0; i < NDK; ++i) {
            if constexpr (Q8) {
                // load i, lane 8*rr + t: row 8i + 4(rr&1) + rr/2, piece t^4i^2(rr&1)
                const int rr = lane >> 3, t = lane & 7;
                kdma[i] = (8 * i + 4 * (rr & 1) + (rr >> 1)) * 128 + 16 * (t ^ (4 * i) ^ (2 * (rr & 1)));
                // piece group i: row 4*j4 + tg, piece qd + 4i
                const int pc = qd + 4 * i;
                krd[i] = 1024 * (j4 >> 1) +
                         16 * (8 * (2 * tg + (j4 & 1)) + (pc ^ (4 * (j4 >> 1)) ^ (2 * (j4 & 1))));
            } else {
                // load i, lane 16*q + t: row 4i + q; piece bits (t0, t3, t1^i0, t2^i1)
                const int q = lane >> 4, t = lane & 15;
                kdma[i] = (4 * i + q) * 256 + 16 * kpiece(t, i);
                // piece group i: row 4*j4 + tg, piece qd + 4i
                const int tt = (qd & 1) | (((j4 & 1) ^ (i & 1)) << 1) | ((((j4 >> 1) & 1) ^ (i >> 1)) << 2) |
                               ((qd >> 1) << 3);
                krd[i] = 1024 * j4 + 16 * (16 * tg + tt);
            }
        }
        vrd = Q8 ? 128 * tg + 8 * (lane & 15) : 16 * lane;
    }

    // Start the loads of chunk c of segment (s, g) into ring slot `slot`
    // (DPC vector memory instructions; two more with `fresh`, which also load
    // sequence s's new K and V rows of kv head g from key / value, and its
    // slot_mapping entry). Tiles are loaded non-temporal: every (sequence, kv
    // head) tile is read once per launch, and kept out of the L2's way it
    // leaves the room to lines that are read again (int8 batch 130.5 -> 123.5
    // us; the mixed batch without shared prefixes 325 -> 294 us). In a batch
    // with copy-on-write sharing (cow) a block that a neighbouring sequence
    // shares is the exception: the other sequences of its group read it again,
    // from the L2 (mixed batch with four 64-sequence groups: HBM traffic 1.30x
    // -> 1.04x the algorithmic bytes, 213.0 -> 205.3 us).
    __device__ void issue(char* slot, int s, int g, int c, bool fresh) const {
        if (fresh) {
            if (lane < 32) {                     // lanes 0..15: K, 16..31: V, 16 bytes each
                const char* src = (const char*)(lane < 16 ? a.key : a.value);
                dma16(src + (((int64_t)s * a.num_kv_heads + g) * D + 8 * (lane & 15)) * 2,
                      slot + NEW);
            }
            if (lane < 2) dma4((const char*)(a.slot_mapping + s) + 4 * lane, slot + NEW + 4 * D);
        }
        const int64_t ri = (int64_t)s * a.max_blocks_per_seq + (c >> shift);
        const int phys = ld_uniform(a.block_tables, ri);
        const int64_t off = phys * block_stride + g * head_stride + (int64_t)(c & shift) * CHUNK * D;
        const char* kt = (const char*)a.k_cache + off * CE;
        const char* vt = (const char*)a.v_cache + off * CE;
        auto tiles = [&](auto nt) {
#pragma unroll
            for (int i = 0; i < NDK; ++i) dma16p<nt()>(at(kt, kdma[i]), slot + 1024 * i);
#pragma unroll
            for (int i = 0; i < NDK; ++i)
                dma16p<nt()>(at(vt + 1024 * i, 16u * lane), slot + KT + 1024 * i);
        };
        if (!cow || !block_shared(a, s, ri, phys))
            tiles(std::true_type{});
        else
            tiles(std::false_type{});
        if constexpr (Q8) {
            if (lane == 0) {
                dma4(a.k_scale + (int64_t)phys * a.num_kv_heads + g, slot + 2 * KT);
                dma4(a.v_scale + (int64_t)phys * a.num_kv_heads + g, slot + 2 * KT + 4);
            }
        }
    }

    static __device__ void write_vector_at(const DecodeArgs& a, int s, int g, int v) {
        write_vector<BF16, CT>(a.key, a.value, const_cast<void*>(a.k_cache),
                               const_cast<void*>(a.v_cache), a.slot_mapping, a.k_scale, a.v_scale,
                               a.num_kv_heads, D, a.block_size, s, g, v);
    }

    // Ring slot `slot` holds the last chunk of segment (s, g), loaded with
    // `fresh`: the chunk as the cache held it, and sequence s's new K and V
    // rows and slot. Its new token (position L - 1) is written here: into the
    // cache slot, and into the chunk in LDS, where each lane overwrites the
    // bytes of that row which its own loads of the chunk brought in. Both take
    // the bytes the write takes (a copy, or int8 codes), so the chunk is the one
    // a load after the write would give. The slot is the one of position L - 1,
    // in the chunk's block, whose int8 scales are already in the slot. A
    // negative slot writes nothing.
    __device__ void patch_new_token(char* slot, int g, int L) const {
        const uint32_t b = lds_addr(slot), nb = b + NEW;
        u32x2 sv = ds_read8<4 * D>(nb);
        u32x2 sc = ds_read8<Q8 ? 2 * KT : 0>(b);
        lds_wait(sv, sc);
        const int64_t sl = uniform64((long long)(((uint64_t)sv.y << 32) | sv.x));
        if (sl < 0) return;
        const int o = (L - 1) & (CHUNK - 1);     // the token's row in the chunk
        const int64_t blk = sl >> (4 + shift), off = sl & (a.block_size - 1);
        const int64_t row = ((blk * a.num_kv_heads + g) * a.block_size + off) * D;
        if constexpr (!Q8) {
            if (lane < 32) {                     // lanes 0..15: K, 16..31: V, 16 bytes each
                u32x4 w = ds_read16(nb + 16 * lane);
                lds_wait(w);
                char* dst = (char*)(lane < 16 ? a.k_cache : a.v_cache) + (row + 8 * (lane & 15)) * 2;
                *reinterpret_cast<uint4*>(dst) = make_uint4(w.x, w.y, w.z, w.w);
            }
            // load o/4 moves row o: K piece kpiece(t, o/4) and V piece t, lanes 16*(o%4) + t
            if ((lane >> 4) == (o & 3)) {
                const int i = o >> 2, t = lane & 15;
                u32x4 kw = ds_read16(nb + 16 * kpiece(t, i));
                u32x4 vw = ds_read16(nb + 2 * D + 16 * t);
                lds_wait(kw, vw);
                ds_write16(b + 1024 * i + 16 * lane, kw);
                ds_write16(b + KT + 1024 * i + 16 * lane, vw);
            }
        } else {
            // Every lane quantises 4 values once: lane l takes bytes 8*(l/32) ..
            // of 16-byte vector l%32 of the rows (K for l%32 < 16, else V), dims
            // e .. e+3 with e = 8*(l%16) + 4*(l/32). It stores the 4 codes into
            // the cache row, and into LDS over the rows already read: K codes at
            // nb + e, V codes at nb + D + e.
            const int v = lane & 31, half = lane >> 5;
            const bool isk = v < 16;
            const int e = 8 * (v & 15) + 4 * half;
            u32x2 w = ds_read8(nb + 16 * v + 8 * half);
            lds_wait(w);
            const uint32_t code = codes4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y),
                                         __uint_as_float(isk ? sc.x : sc.y));
            *reinterpret_cast<uint32_t*>((int8_t*)(isk ? a.k_cache : a.v_cache) + row + e) = code;
            ds_write4(nb + (isk ? 0 : D) + e, code);
            // load o/8 moves row o. K: lanes 8*rr + t, rr = 2*(o%4) + (o/4)%2,
            // piece t ^ 4*(o/8) ^ 2*(rr%2); V: lanes 8*(o%8) + t, piece t. A
            // piece is 16 codes, dims 16*piece .. +15.
            const int i = o >> 3, t = lane & 7;
            const int rr = 2 * (o & 3) + ((o >> 2) & 1);
            if ((lane >> 3) == rr) {
                u32x4 c = ds_read16(nb + 16 * (t ^ (4 * i) ^ (2 * (rr & 1))));
                lds_wait(c);
                ds_write16(b + 1024 * i + 16 * lane, c);
            }
            if ((lane >> 3) == (o & 7)) {
                u32x4 c = ds_read16(nb + D + 16 * t);
                lds_wait(c);
                ds_write16(b + KT + 1024 * i + 16 * lane, c);
            }
        }
    }

    // The chunk in ring slot `slot` (its loads complete) as MFMA operands.
    __device__ Chunk fetch(const char* slot) const {
        Chunk ch;
        const uint32_t b = lds_addr(slot);
        const uint32_t vb = b + KT + vrd;
        if constexpr (Q8) {
            u32x4 k0 = ds_read16(b + krd[0]), k1 = ds_read16(b + krd[1]);
            u32x2 v0 = ds_read8<0>(vb), v1 = ds_read8<512>(vb), v2 = ds_read8<1024>(vb),
                  v3 = ds_read8<1536>(vb);
            u32x2 sc = ds_read8<2 * KT>(b);
            lds_wait(k0, k1, v0, v1, v2, v3, sc);
            ch.k[0] = make_uint4(k0.x, k0.y, k0.z, k0.w);
            ch.k[1] = make_uint4(k1.x, k1.y, k1.z, k1.w);
            ch.k[2] = ch.k[3] = make_uint4(0, 0, 0, 0);
            ch.v[0] = make_uint4(v0.x, v0.y, 0, 0);
            ch.v[1] = make_uint4(v1.x, v1.y, 0, 0);
            ch.v[2] = make_uint4(v2.x, v2.y, 0, 0);
            ch.v[3] = make_uint4(v3.x, v3.y, 0, 0);
            ch.ks = __uint_as_float(sc.x);
            ch.vs = __uint_as_float(sc.y);
        } else {
            u32x4 k0 = ds_read16(b + krd[0]), k1 = ds_read16(b + krd[1]), k2 = ds_read16(b + krd[2]),
                  k3 = ds_read16(b + krd[3]);
            u32x4 v0 = ds_read16<0>(vb), v1 = ds_read16<1024>(vb), v2 = ds_read16<2048>(vb),
                  v3 = ds_read16<3072>(vb);
            lds_wait(k0, k1, k2, k3, v0, v1, v2, v3);
            ch.k[0] = make_uint4(k0.x, k0.y, k0.z, k0.w);
            ch.k[1] = make_uint4(k1.x, k1.y, k1.z, k1.w);
            ch.k[2] = make_uint4(k2.x, k2.y, k2.z, k2.w);
            ch.k[3] = make_uint4(k3.x, k3.y, k3.z, k3.w);
            ch.v[0] = make_uint4(v0.x, v0.y, v0.z, v0.w);
            ch.v[1] = make_uint4(v1.x, v1.y, v1.z, v1.w);
            ch.v[2] = make_uint4(v2.x, v2.y, v2.z, v2.w);
            ch.v[3] = make_uint4(v3.x, v3.y, v3.z, v3.w);
            ch.ks = ch.vs = 1.0f;
        }
        return ch;
    }

    // Query operands. bf16 cache: dims 8*(4m+qd) .. +7 for m = 0..3.
    // int8 cache: dims 16*(4(m>>1)+qd) + 8(m&1) .. +7.
    __device__ void begin_segment(int s, int g) {
        const uint16_t* q0 = (const uint16_t*)a.q + ((int64_t)s * a.num_heads + g * G) * D;
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int d = Q8 ? 16 * (4 * (m >> 1) + qd) + 8 * (m & 1) : 8 * (4 * m + qd);
                qr[hb][m] = ld16(at(q0, 2 * ((hb * 4 + j4) * D + d)));
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

    // (cache policy as in issue)
    __device__ Chunk load(int s, int g, int c) const {
        Chunk ch;
        const int64_t ri = (int64_t)s * a.max_blocks_per_seq + (c >> shift);
        const int phys = ld_uniform(a.block_tables, ri);
        const int64_t off = phys * block_stride + g * head_stride + (int64_t)(c & shift) * CHUNK * D;
        const char* kp = at((const char*)a.k_cache + off * CE, k_off);
        const char* vp = at((const char*)a.v_cache + off * CE, v_off);
        auto tiles = [&](auto nt) {
            if constexpr (Q8) {
                ch.k[0] = ld16p<nt()>(kp);
                ch.k[1] = ld16p<nt()>(kp + 64);
                ch.k[2] = ch.k[3] = make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int step = 0; step < 4; ++step) {
                    const uint2 w = ld8p<nt()>(vp + step * 4 * D);
                    ch.v[step] = make_uint4(w.x, w.y, 0, 0);
                }
            } else {
#pragma unroll
                for (int m = 0; m < 4; ++m) ch.k[m] = ld16p<nt()>(kp + 64 * m);
#pragma unroll
                for (int step = 0; step < 4; ++step) ch.v[step] = ld16p<nt()>(vp + step * 4 * D * CE);
            }
        };
        if (!cow || !block_shared(a, s, ri, phys))
            tiles(std::true_type{});
        else
            tiles(std::false_type{});
        if constexpr (Q8) {
            ch.ks = ld_uniform(a.k_scale, (int64_t)phys * a.num_kv_heads + g);
            ch.vs = ld_uniform(a.v_scale, (int64_t)phys * a.num_kv_heads + g);
        } else {
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
        uint32_t pk[NHB][2];                     // bf16 cache: p rounded, packed
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
            for (int i = 0; i < 4; ++i) p[hb][i] = __builtin_amdgcn_exp2f(x[i] - muse);
            if constexpr (Q8) {
                psum = (p[hb][0] + p[hb][1]) + (p[hb][2] + p[hb][3]);
            } else {
                // the weights PV uses, and their sum, are the bf16-rounded ones
                pk[hb][0] = pack_bf16_rne(p[hb][0], p[hb][1]);
                pk[hb][1] = pack_bf16_rne(p[hb][2], p[hb][3]);
                psum = (bf16lo(pk[hb][0]) + bf16hi(pk[hb][0])) +
                       (bf16lo(pk[hb][1]) + bf16hi(pk[hb][1]));
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
        if constexpr (!Q8) {
            // bf16 cache: one 4x4x4 bf16 product per dim e covers the row
            // group's 4 tokens. A operand of lane (tg, qd, j4): dim
            // 8*(4*qd + j4) + e of V rows 4k + tg, k = 0..3 (the lane's own
            // loads, transposed by byte permutes); B: its 4 weights, k = 0..3.
            // Rows past the context may hold NaN: their words are zeroed.
            uint32_t w[4][4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool z = tail && c * CHUNK + 4 * k + tg >= t1;
                w[k][0] = z ? 0u : cur.v[k].x;
                w[k][1] = z ? 0u : cur.v[k].y;
                w[k][2] = z ? 0u : cur.v[k].z;
                w[k][3] = z ? 0u : cur.v[k].w;
            }
            i16x4 va[8];
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                va[2 * n] = as_i16x4(lo_halves(w[0][n], w[1][n]), lo_halves(w[2][n], w[3][n]));
                va[2 * n + 1] = as_i16x4(hi_halves(w[0][n], w[1][n]), hi_halves(w[2][n], w[3][n]));
            }
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) {
                const i16x4 pb = as_i16x4(pk[hb][0], pk[hb][1]);
#pragma unroll
                for (int e = 0; e < 8; ++e) S.acc[hb][e] = mfma4x4x4bf16(va[e], pb, S.acc[hb][e]);
            }
            return;
        }
        // int8 cache: fp32 4x4x1 products, the codes and p * v_scale in fp32
#pragma unroll
        for (int step = 0; step < 4; ++step) {
            float vf[8];
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                vf[n] = i8_at(cur.v[step].x, n);
                vf[4 + n] = i8_at(cur.v[step].y, n);
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

    // Merge the 4 row states (lanes differing in tg): every lane then holds
    // the wave's state of head 4*hb + j4 for its dim quarter qd.
    __device__ void merge_rows(State& S) const {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            float flat[32];
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i) flat[4 * e + i] = S.acc[hb][e][i];
            merge_rows_xor<true, 16>(S.m[hb], S.l[hb], flat);
            merge_rows_xor<true, 32>(S.m[hb], S.l[hb], flat);
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i) S.acc[hb][e][i] = flat[4 * e + i];
        }
    }

    // Merge the row states and write the wave's state (partition driver). The
    // merge goes through LDS permutes here: with the register budget of three
    // waves per SIMD, the permlane form makes the allocator spill in the loop.
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

    // This lane's 8 accumulator values (dims 8*(4*qd + tg) + e) of head group hb.
    __device__ void own(const State& S, int hb, float (&v)[8]) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const f32x4 x = S.acc[hb][e];
            v[e] = tg == 0 ? x[0] : tg == 1 ? x[1] : tg == 2 ? x[2] : x[3];
        }
    }

    __device__ void store8(int s, int g, int hb, const float (&v)[8]) const {
        uint4 w;
        w.x = f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        w.y = f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        w.z = f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
        w.w = f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
        uint16_t* o0 = (uint16_t*)a.out + ((int64_t)s * a.num_heads + g * G) * D;
        *reinterpret_cast<uint4*>(at(o0, 2 * ((hb * 4 + j4) * D + 8 * (4 * qd + tg)))) = w;
    }

    // out = acc / l after merge_rows.
    __device__ void store_final(const State& S, int s, int g) const {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            float v[8];
            own(S, hb, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = v[e] / S.l[hb];
            store8(s, g, hb, v);
        }
    }

    // Workspace slot (G*D floats in tmp_out, G in tmp_max / tmp_sum): lane L's
    // 8 unnormalised accumulator values of head group hb at (hb*64 + L)*8, and
    // m (base 2) and l of head h at h.
    __device__ void store_slot(const State& S, int64_t slot) const {
        const __amdgpu_buffer_rsrc_t rs = ws_rsrc(a.tmp_out + slot * (G * D), G * D * 4);
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            float v[8];
            own(S, hb, v);
            const uint32_t off = (hb * 64 + lane) * 32;
            ws_store16(rs, off, v[0], v[1], v[2], v[3]);
            ws_store16(rs, off + 16, v[4], v[5], v[6], v[7]);
            if (lane < 4) {
                ws_store<true>(at(a.tmp_max + slot * G, 4 * (hb * 4 + j4)), S.m[hb]);
                ws_store<true>(at(a.tmp_sum + slot * G, 4 * (hb * 4 + j4)), S.l[hb]);
            }
        }
    }

    // Log-sum-exp of the partials of pieces first .. first+n-1 of (s, g) into
    // out (piece first + k left its partial in slot 2 (first + k) + (k == 0)):
    // the partials are read kBatch at a time with a running maximum (earlier
    // sums are rescaled when it moves), so their loads overlap.
    static constexpr int kBatch = 8;
    __device__ void combine(long long first, int n, int s, int g) const {
        const int64_t slot0 = 2 * first;
        const __amdgpu_buffer_rsrc_t rs = ws_rsrc(a.tmp_out + slot0 * (G * D), (uint32_t)(2 * n) * (G * D * 4));
        const __amdgpu_buffer_rsrc_t rm = ws_rsrc(a.tmp_max + slot0 * G, (uint32_t)(2 * n) * (G * 4));
        const __amdgpu_buffer_rsrc_t rl = ws_rsrc(a.tmp_sum + slot0 * G, (uint32_t)(2 * n) * (G * 4));
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            const uint32_t hoff = 4 * (hb * 4 + j4);
            const uint32_t aoff = (hb * 64 + lane) * 32;
            float M = kNegInf, lsum = 0.0f, o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = 0.0f;
            for (int k0 = 0; k0 < n; k0 += kBatch) {
                float mk[kBatch], lk[kBatch];
                u32x4_t a0[kBatch], a1[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const uint32_t k = (uint32_t)min(k0 + j, n - 1);
                    const uint32_t sl = 2 * k + (k == 0 ? 1u : 0u);
                    mk[j] = ws_load4(rm, sl * (G * 4) + hoff);
                    lk[j] = ws_load4(rl, sl * (G * 4) + hoff);
                    a0[j] = ws_load16(rs, sl * (G * D * 4) + aoff);
                    a1[j] = ws_load16(rs, sl * (G * D * 4) + aoff + 16);
                }
                float Mb = M;
#pragma unroll
                for (int j = 0; j < kBatch; ++j)
                    if (k0 + j < n) Mb = fmaxf(Mb, mk[j]);
                const float sc = rel_weight<true>(M, Mb);
                lsum *= sc;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] *= sc;
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const float W = (k0 + j < n) ? rel_weight<true>(mk[j], Mb) : 0.0f;
                    lsum += W * lk[j];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        o[e] += W * __uint_as_float(a0[j][e]);
                        o[4 + e] += W * __uint_as_float(a1[j][e]);
                    }
                }
                M = Mb;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = o[e] / lsum;
            store8(s, g, hb, o);
        }
    }
};

// ---- 16x16 core: bf16 cache, balanced ring driver -----------------------------
// The G query heads of a kv head as the columns of 16x16 MFMA tiles (G <= 16;
// columns G..15 carry zero queries and their results are dropped). Lane
// l = 16*qg + n:
//  QK^T: S^T = K Q^T on v_mfma_f32_16x16x32_bf16, 4 per chunk: A = K row n,
//    dims 32*kk + 8*qg .. +7 (one 16-byte LDS read), B = query head n, the same
//    dims. The lane receives the logits of head n for tokens 4*qg + i.
//  softmax: one running max per head, common to the 4 lanes holding its
//    tokens (a max over lanes n, n^16, n^32, n^48 per chunk), lazy as in
//    MfmaCore; each lane sums its own tokens' weights into l.
//  PV: O^T += V^T P^T on v_mfma_f32_16x16x16_bf16, 8 per chunk (16 dims each):
//    A = dims 16*j + n of V rows 4*qg .. +3 (one transposing LDS read), B = the
//    lane's own 4 weights rounded to bf16, already in place. The lane then
//    holds dims 16*j + 4*qg + i of head n, summed over all 16 tokens.
// Per chunk and wave this is 12 MFMAs and about 40 other VALU instructions,
// whatever G (MfmaCore at G = 8: 32 MFMAs and about 180).
//
// LDS layout of a ring slot (K tile, V tile, then a new token's rows): row r of
// the K tile holds its 16-byte piece p at position p ^ r, row r of the V tile
// at position p ^ 2*(r % 8), so the K operand reads (16 rows, one piece each)
// and the transposing V reads (rows 4*qg .. +3, 32 bytes each) spread over the
// banks. The direct loads write 16 bytes per lane at consecutive addresses, so
// the permutation is applied to the global addresses the lanes read.
//
// PAIR (G = 8): the segments are pairs of sequences (see the units of the
// balanced driver): column n is head n % G of sequence 2s + n / G, so the 16
// columns are all in use. A chunk that only one of the two sequences holds
// feeds only its columns (step's `who`); the other columns see it masked.
template <int G_, bool PAIR_ = false>
struct Mfma16Core {
    static constexpr int G = G_;
    static constexpr bool PAIR = PAIR_;
    static constexpr int GC = PAIR ? 2 * G : G;      // columns in use
    static constexpr int D = 128;
    static constexpr bool BASE2 = true;
    static constexpr float kSlack = 8.0f;
    static_assert(GC <= 16, "one 16-column tile of query heads");

    struct State {
        float m, l;
        f32x4 acc[8];                            // acc[j][i]: dim 16*j + 4*qg + i, head n
    };
    struct Chunk {
        uint4 k[4];                              // K operands, kk = 0..3
        u32x2 v[8];                              // V^T operands, j = 0..7
    };

    static constexpr int KT = 16 * D * 2;        // bytes of one 16-token K (or V) tile
    static constexpr int NDK = KT / 1024;        // 1 KB load instructions per tile
    static constexpr int NEW = 2 * KT;           // then a new token's K and V rows, and its slot
    static constexpr int SLOT = NEW + 4 * D + 16;
    static constexpr int DPC = 2 * NDK;          // vector memory instructions per chunk
    static constexpr int R = 2;                  // ring slots per wave

    const DecodeArgs& a;
    bool cow = false;    // as MfmaCore::cow
    int lane, n, qg;
    float sl2;
    int shift;
    int64_t head_stride, block_stride;
    uint4 qr[4];                                 // query operands of the segment
    uint32_t kdma[NDK], vdma[NDK];               // source byte offsets in a tile, per load
    uint32_t krd[4];                             // LDS byte offsets of the K operands
    uint32_t vrd[8];                             // LDS byte offsets of the V^T operands

    __device__ explicit Mfma16Core(const DecodeArgs& args) : a(args) {
        lane = threadIdx.x & 63;
        n = lane & 15;
        qg = lane >> 4;
        sl2 = a.scale * kLog2e;
        shift = (a.block_size == 32) ? 1 : 0;
        head_stride = (int64_t)a.block_size * D;
        block_stride = head_stride * a.num_kv_heads;
#pragma unroll
        for (int i = 0; i < NDK; ++i) {
            // load i, lane 16*q + t lands at row 4i + q, position t
            const int r = 4 * i + qg;
            kdma[i] = r * 256 + 16 * (n ^ r);
            vdma[i] = r * 256 + 16 * (n ^ (2 * (r & 7)));
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) krd[kk] = 256 * n + 16 * ((4 * kk + qg) ^ n);
        // transposing read j: lane 4*k4 + q of the 16-lane group qg addresses
        // V row 4*qg + k4, dims 16*j + 4*q .. +3 (8 bytes)
        const int r = 4 * qg + (n >> 2), q = n & 3;
#pragma unroll
        for (int j = 0; j < 8; ++j) vrd[j] = KT + 256 * r + 32 * (j ^ (r & 7)) + 8 * q;
    }

    __device__ void issue(char* slot, int s, int g, int c, bool fresh) const {
        if (fresh) {
            if (lane < 32) {                     // lanes 0..15: K, 16..31: V, 16 bytes each
                const char* src = (const char*)(lane < 16 ? a.key : a.value);
                dma16(src + (((int64_t)s * a.num_kv_heads + g) * D + 8 * (lane & 15)) * 2,
                      slot + NEW);
            }
            if (lane < 2) dma4((const char*)(a.slot_mapping + s) + 4 * lane, slot + NEW + 4 * D);
        }
        const int64_t ri = (int64_t)s * a.max_blocks_per_seq + (c >> shift);
        const int phys = ld_uniform(a.block_tables, ri);
        const int64_t off = phys * block_stride + g * head_stride + (int64_t)(c & shift) * CHUNK * D;
        const char* kt = (const char*)a.k_cache + off * 2;
        const char* vt = (const char*)a.v_cache + off * 2;
        auto tiles = [&](auto nt) {
#pragma unroll
            for (int i = 0; i < NDK; ++i) dma16p<nt()>(at(kt, kdma[i]), slot + 1024 * i);
#pragma unroll
            for (int i = 0; i < NDK; ++i) dma16p<nt()>(at(vt, vdma[i]), slot + KT + 1024 * i);
        };
        if (!cow || !block_shared(a, s, ri, phys))
            tiles(std::true_type{});
        else
            tiles(std::false_type{});
    }

    static __device__ void write_vector_at(const DecodeArgs& a, int s, int g, int v) {
        write_vector<BF16, BF16>(a.key, a.value, const_cast<void*>(a.k_cache),
                                 const_cast<void*>(a.v_cache), a.slot_mapping, a.k_scale,
                                 a.v_scale, a.num_kv_heads, D, a.block_size, s, g, v);
    }

    // As MfmaCore::patch_new_token, for this layout: the new token's row o of
    // the chunk was brought in by lanes 16*(o%4) + t of load o/4 (position t),
    // which overwrite it with the new row's pieces t ^ o (K) and t ^ 2*(o%8) (V).
    __device__ void patch_new_token(char* slot, int g, int L) const {
        const uint32_t b = lds_addr(slot), nb = b + NEW;
        u32x2 sv = ds_read8<4 * D>(nb);
        lds_wait(sv);
        const int64_t sl = uniform64((long long)(((uint64_t)sv.y << 32) | sv.x));
        if (sl < 0) return;
        const int o = (L - 1) & (CHUNK - 1);
        const int64_t blk = sl >> (4 + shift), off = sl & (a.block_size - 1);
        const int64_t row = ((blk * a.num_kv_heads + g) * a.block_size + off) * D;
        if (lane < 32) {
            u32x4 w = ds_read16(nb + 16 * lane);
            lds_wait(w);
            char* dst = (char*)(lane < 16 ? a.k_cache : a.v_cache) + (row + 8 * (lane & 15)) * 2;
            *reinterpret_cast<uint4*>(dst) = make_uint4(w.x, w.y, w.z, w.w);
        }
        if (qg == (o & 3)) {
            u32x4 kw = ds_read16(nb + 16 * (n ^ o));
            u32x4 vw = ds_read16(nb + 2 * D + 16 * (n ^ (2 * (o & 7))));
            lds_wait(kw, vw);
            ds_write16(b + 1024 * (o >> 2) + 16 * lane, kw);
            ds_write16(b + KT + 1024 * (o >> 2) + 16 * lane, vw);
        }
    }

    __device__ Chunk fetch(const char* slot) const {
        Chunk ch;
        const uint32_t b = lds_addr(slot);
        u32x4 k0 = ds_read16(b + krd[0]), k1 = ds_read16(b + krd[1]), k2 = ds_read16(b + krd[2]),
              k3 = ds_read16(b + krd[3]);
        u32x2 v0 = ds_read8_tr(b + vrd[0]), v1 = ds_read8_tr(b + vrd[1]),
              v2 = ds_read8_tr(b + vrd[2]), v3 = ds_read8_tr(b + vrd[3]),
              v4 = ds_read8_tr(b + vrd[4]), v5 = ds_read8_tr(b + vrd[5]),
              v6 = ds_read8_tr(b + vrd[6]), v7 = ds_read8_tr(b + vrd[7]);
        lds_wait(k0, k1, k2, k3, v0, v1, v2, v3, v4, v5, v6, v7);
        ch.k[0] = make_uint4(k0.x, k0.y, k0.z, k0.w);
        ch.k[1] = make_uint4(k1.x, k1.y, k1.z, k1.w);
        ch.k[2] = make_uint4(k2.x, k2.y, k2.z, k2.w);
        ch.k[3] = make_uint4(k3.x, k3.y, k3.z, k3.w);
        ch.v[0] = v0; ch.v[1] = v1; ch.v[2] = v2; ch.v[3] = v3;
        ch.v[4] = v4; ch.v[5] = v5; ch.v[6] = v6; ch.v[7] = v7;
        return ch;
    }

    // Row of q / out that column n of segment (s, g) holds, counted in heads
    // from row (first sequence of the segment, head g G): n, or for pair
    // units (n / G) Hq + n % G.
    __device__ uint32_t col_row() const {
        return PAIR ? (uint32_t)((n / G) * a.num_heads + n % G) : (uint32_t)n;
    }
    __device__ int64_t first_row(int s, int g) const {
        return ((int64_t)(PAIR ? 2 * s : s) * a.num_heads + g * G) * D;
    }

    // The query of column n (zero for a column with no head: n >= G, or the
    // missing second sequence of the last pair unit; the load is then
    // clamped to the segment's first row), dims 32*kk + 8*qg .. +7.
    __device__ void begin_segment(int s, int g) {
        const uint16_t* q0 = (const uint16_t*)a.q + first_row(s, g);
        const bool live = PAIR ? 2 * s + n / G < a.num_seqs : n < G;
        const uint32_t row = live ? col_row() : 0u;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const uint4 w = ld16(at(q0, 2 * (row * D + 32 * kk + 8 * qg)));
            qr[kk] = live ? w : make_uint4(0, 0, 0, 0);
        }
    }

    __device__ void init(State& S) const {
        S.m = kNegInf;
        S.l = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) S.acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // who (pair units): 0 the chunk feeds every column, 1 only the first
    // sequence's, 2 only the second's; the others see its tokens masked.
    __device__ void step(State& S, const Chunk& cur, int c, int t1, int who = 0) const {
        const bool tail = ((c + 1) * CHUNK) > t1;
        const bool off = PAIR && who != 0 && ((who == 1) == (n >= G));
        f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
        // the MFMA runs at raised issue priority, as in the multi-query
        // kernel (mixed copy-on-write batch 199.1 -> 198.1 us)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, cur.k[kk]), __builtin_bit_cast(bf16x8_t, qr[kk]), sacc,
                0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // x is rounded once; the max and exp2(x - max) see the same x
            x[i] = sacc[i] * sl2;
            if (off || (tail && c * CHUNK + 4 * qg + i >= t1)) x[i] = kNegInf;
        }
        float mloc = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mloc = fmaxf(mloc, lane_xor16(mloc));
        mloc = fmaxf(mloc, lane_xor32(mloc));
        const float mnew = (mloc > S.m + kSlack) ? mloc : S.m;
        const float muse = (mnew == kNegInf) ? 0.0f : mnew;
        // an empty state (no token yet: acc and l are 0) needs no rescale
        const float alpha = S.m == kNegInf ? 1.0f : __builtin_amdgcn_exp2f(S.m - muse);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - muse);
        // the weights PV uses, and their sum, are the bf16-rounded ones
        const uint32_t pk0 = pack_bf16_rne(p[0], p[1]), pk1 = pack_bf16_rne(p[2], p[3]);
        const float psum = (bf16lo(pk0) + bf16hi(pk0)) + (bf16lo(pk1) + bf16hi(pk1));
        S.l = S.l * alpha + psum;
        S.m = mnew;
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int j = 0; j < 8; ++j) S.acc[j] *= alpha;
        }
        // rows past the context may hold NaN: their bf16 halves are zeroed
        uint32_t m01 = 0xffffffffu, m23 = 0xffffffffu;
        if (tail) {
            const int t0 = c * CHUNK + 4 * qg;
            m01 = (t0 < t1 ? 0x0000ffffu : 0u) | (t0 + 1 < t1 ? 0xffff0000u : 0u);
            m23 = (t0 + 2 < t1 ? 0x0000ffffu : 0u) | (t0 + 3 < t1 ? 0xffff0000u : 0u);
        }
        const i16x4 pb = as_i16x4(pk0, pk1);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            S.acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                as_i16x4(cur.v[j].x & m01, cur.v[j].y & m23), pb, S.acc[j], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
    }

    // The 4 lanes of head n share m; their token sums add up.
    __device__ void merge_rows(State& S) const {
        S.l += lane_xor16(S.l);
        S.l += lane_xor32(S.l);
    }

    // The lane's 4 values of dims 16*j + 4*qg .. +3 of column n as bf16.
    __device__ void store4(int s, int g, int j, float v0, float v1, float v2, float v3) const {
        uint16_t* o0 = (uint16_t*)a.out + first_row(s, g);
        const uint2 w = make_uint2(f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16),
                                   f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16));
        *reinterpret_cast<uint2*>(at(o0, 2 * (col_row() * D + 16 * j + 4 * qg))) = w;
    }

    // (pair units: a column that saw no token belongs to a sequence with an
    // empty context, whose zeros are written elsewhere, or to none at all)
    __device__ void store_final(const State& S, int s, int g) const {
        if (n >= GC || (PAIR && !(S.l > 0.0f))) return;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            store4(s, g, j, S.acc[j][0] / S.l, S.acc[j][1] / S.l, S.acc[j][2] / S.l,
                   S.acc[j][3] / S.l);
    }

    // Workspace slot: tmp_out [GC][D] (unnormalised), tmp_max / tmp_sum [GC]
    // (m base 2, l), all with coherent stores.
    __device__ void store_slot(const State& S, int64_t slot) const {
        if (n >= GC) return;
        const __amdgpu_buffer_rsrc_t rs = ws_rsrc(a.tmp_out + slot * (GC * D), GC * D * 4);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            ws_store16(rs, 4 * (n * D + 16 * j + 4 * qg), S.acc[j][0], S.acc[j][1], S.acc[j][2],
                       S.acc[j][3]);
        if (qg == 0) {
            ws_store<true>(at(a.tmp_max + slot * GC, 4 * n), S.m);
            ws_store<true>(at(a.tmp_sum + slot * GC, 4 * n), S.l);
        }
    }

    // Log-sum-exp of the partials of pieces first .. first+np-1 of (s, g) into
    // out (piece first + k left its partial in slot 2 (first + k) + (k == 0)),
    // kBatch pieces at a time with a running maximum.
    static constexpr int kBatch = 2;
    __device__ void combine(long long first, int np, int s, int g) const {
        if (n >= GC) return;
        const int64_t slot0 = 2 * first;
        const __amdgpu_buffer_rsrc_t rs = ws_rsrc(a.tmp_out + slot0 * (GC * D), (uint32_t)(2 * np) * (GC * D * 4));
        const __amdgpu_buffer_rsrc_t rm = ws_rsrc(a.tmp_max + slot0 * GC, (uint32_t)(2 * np) * (GC * 4));
        const __amdgpu_buffer_rsrc_t rl = ws_rsrc(a.tmp_sum + slot0 * GC, (uint32_t)(2 * np) * (GC * 4));
        float M = kNegInf, lsum = 0.0f;
        f32x4 o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int k0 = 0; k0 < np; k0 += kBatch) {
            float mk[kBatch], lk[kBatch];
            u32x4_t x[kBatch][8];
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                const uint32_t k = (uint32_t)min(k0 + jj, np - 1);
                const uint32_t sl = 2 * k + (k == 0 ? 1u : 0u);
                mk[jj] = ws_load4(rm, 4 * (sl * GC + n));
                lk[jj] = ws_load4(rl, 4 * (sl * GC + n));
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    x[jj][j] = ws_load16(rs, 4 * (sl * (GC * D) + n * D + 16 * j + 4 * qg));
            }
            float Mb = M;
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj)
                if (k0 + jj < np) Mb = fmaxf(Mb, mk[jj]);
            const float sc = rel_weight<true>(M, Mb);
            lsum *= sc;
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] *= sc;
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                const float W = (k0 + jj < np) ? rel_weight<true>(mk[jj], Mb) : 0.0f;
                lsum += W * lk[jj];
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[j][i] += W * __uint_as_float(x[jj][j][i]);
            }
            M = Mb;
        }
        if (PAIR && !(lsum > 0.0f)) return;          // (as in store_final)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            store4(s, g, j, o[j][0] / lsum, o[j][1] / lsum, o[j][2] / lsum, o[j][3] / lsum);
    }
};

// Register budget per lane of the register-path kernel: 168 (3 waves per SIMD)
// for G = 4, 256 (2 waves) for G = 8; enough resident waves to keep HBM busy
// with one chunk in flight. The ring kernel is held to 2 waves per SIMD by its
// LDS ring (136-145 KB per 8-wave workgroup) and may use 256.
template <int G>
constexpr int kWavesPerEU = G == 4 ? 3 : 2;

template <int G, Dtype CT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<G>)))
void mfma_partitions(DecodeArgs a) {
    decode_partitions<MfmaCore<G, CT>>(a);
}

// The ring kernel runs one workgroup of 8 waves per CU (2 per SIMD, the LDS
// ring filling most of the CU's LDS): two 4-wave workgroups on one CU were
// measured to stream unevenly, the second one slower.
constexpr int NWR = 8;

// G = 8 with a bf16 cache runs the 16x16 core, the other instances MfmaCore.
// Measured in one process (balanced fused step, pieces >= 128 tokens): the
// mixed copy-on-write batch (G 8) 202.5 -> 197.3 us; at G = 4 the 16x16 core,
// three quarters of whose MFMA columns are then idle, was slower (8 x 32768
// batch 186.2 -> 195.1 us, Llama-shaped batch 67.3 -> 72.9 us).
// PAIR: the 16x16 core takes pairs of sequences (used up to 2 kMaxPairUnits
// sequences, the size of its LDS table).
template <int G, Dtype CT, bool PAIR>
using RingCore = typename std::conditional<CT == BF16 && G == 8, Mfma16Core<G, PAIR>,
                                           MfmaCore<G, CT>>::type;

template <int G, Dtype CT, bool PAIR = false>
__global__ __launch_bounds__(NWR * 64) __attribute__((amdgpu_waves_per_eu(2)))
void mfma_balanced(DecodeArgs a) {
    decode_balanced_ring<RingCore<G, CT, PAIR>, NWR>(a);
}

template <int G, Dtype CT, bool PAIR>
hipError_t launch_balanced(const DecodeArgs& a, hipStream_t st) {
    const void* fn = reinterpret_cast<const void*>(&mfma_balanced<G, CT, PAIR>);
    const int grid = balanced_grid(fn, NWR * 64, st);
    if (grid <= 0) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((mfma_balanced<G, CT, PAIR>), dim3(grid), dim3(NWR * 64), 0, st, a);
    return hipSuccess;
}

template <int G, Dtype CT>
hipError_t launch(const DecodeArgs& a, Schedule sch, hipStream_t st) {
    if (sch == Schedule::Balanced) {
        constexpr bool kPairs = CT == BF16 && G == 8;
        const hipError_t e = kPairs && (a.num_seqs + 1) / 2 <= kMaxPairUnits
                                 ? launch_balanced<G, CT, kPairs>(a, st)
                                 : launch_balanced<G, CT, false>(a, st);
        if (e != hipSuccess) return e;
    } else {
        const int64_t nwg = (int64_t)a.num_kv_heads * a.num_seqs * a.num_partitions;
        hipLaunchKernelGGL((mfma_partitions<G, CT>), dim3((unsigned)nwg), dim3(NW * 64), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

int balanced_waves_mfma(int head_dim, int G, hipStream_t st) {
    if (head_dim != 128 || (G != 4 && G != 8)) return 0;
    const void* fns[3] = {G == 4 ? reinterpret_cast<const void*>(&mfma_balanced<4, BF16>)
                                 : reinterpret_cast<const void*>(&mfma_balanced<8, BF16>),
                          G == 4 ? reinterpret_cast<const void*>(&mfma_balanced<4, I8>)
                                 : reinterpret_cast<const void*>(&mfma_balanced<8, I8>),
                          G == 4 ? reinterpret_cast<const void*>(&mfma_balanced<4, BF16>)
                                 : reinterpret_cast<const void*>(&mfma_balanced<8, BF16, true>)};
    int m = 0;
    for (const void* fn : fns) {
        const int grid = balanced_grid(fn, NWR * 64, st);
        if (grid <= 0) return -1;
        m = grid * NWR > m ? grid * NWR : m;
    }
    return m;
}

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
