// Device-side helpers shared by the gfx950 kernels of libpa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// ---- bf16 <-> fp32 -------------------------------------------------------

// Low / high bf16 of a packed pair, widened exactly.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((b >> 16) | 0x40u);
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

// Two fp32 -> packed bf16 pair, each rounded to nearest even.
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Low halves (resp. high halves) of two packed bf16 pairs: x's in the low
// half of the result, y's in the high half.
__device__ __forceinline__ uint32_t lo_halves(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// Two small exact integers held as fp32 -> packed bf16 pair (upper halves).
__device__ __forceinline__ uint32_t pack_bf16_trunc(float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// int8 byte n of w, sign-extended and converted exactly to fp32.
__device__ __forceinline__ float i8_at(uint32_t w, int n) {
    return (float)(int32_t)(int8_t)(uint8_t)(w >> (8 * n));
}

// ---- cross-lane reductions inside 16-lane rows (DPP) ----------------------

// v + the value 4 (resp. 8) lanes round the 16-lane row; applied twice it sums
// the four lanes {l, l^4, l^8, l^12} of a row.
__device__ __forceinline__ float row_ror4_add(float v) {
    return v + __builtin_amdgcn_update_dpp(0.0f, v, 0x124, 0xf, 0xf, false);
}
__device__ __forceinline__ float row_ror8_add(float v) {
    return v + __builtin_amdgcn_update_dpp(0.0f, v, 0x128, 0xf, 0xf, false);
}
// Sum over the 4 lanes of a quad (lanes 4k .. 4k+3): quad_perm [1,0,3,2] then [2,3,0,1].
__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0xb1, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4e, 0xf, 0xf, false);
    return v;
}

// ---- cross-row exchange (gfx950 permlane swaps, no LDS round trip) --------

// The value held by lane (lane ^ 16), resp. (lane ^ 32). The swap instructions
// exchange the odd 16-lane rows of their first operand with the even rows of
// the second (resp. the upper half of the first with the lower half of the
// second); with both operands x, each result holds every lane's partner in
// half of the lanes.
__device__ __forceinline__ float lane_xor16(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor32(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float((__lane_id() & 32) ? r[0] : r[1]);
}

// ---- MFMA ---------------------------------------------------------------

// 16 independent 4x4x4 bf16 products, fp32 accumulate.
// Block b = lane / 4. A_b[i][k]: lane 4b+i holds k = 0..3; B_b[k][j]: lane
// 4b+j holds k = 0..3; D_b[i][j]: lane 4b+j, register i.
__device__ __forceinline__ f32x4 mfma4x4x4bf16(i16x4 a, i16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
}
// 16 independent 4x4x1 fp32 outer products: A_b[i] at lane 4b+i, B_b[j] at
// lane 4b+j, D_b[i][j] at lane 4b+j, register i.
__device__ __forceinline__ f32x4 mfma4x4x1f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// Four packed bf16 (two dwords) as an MFMA operand.
__device__ __forceinline__ i16x4 as_i16x4(uint32_t lo, uint32_t hi) {
    return __builtin_bit_cast(i16x4, make_uint2(lo, hi));
}

// ---- memory --------------------------------------------------------------

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

// base + off, where base is wave-uniform and off a per-lane byte offset below
// 4 GiB: the address form of global memory instructions with a scalar base and
// a 32-bit lane offset. The empty asm keeps the compiler from folding the
// offset into a per-lane 64-bit pointer that it would then hold in two VGPRs
// for the whole kernel.
template <typename T>
__device__ __forceinline__ T* at(T* base, uint32_t off) {
    asm volatile("" : "+v"(off));
    typedef typename std::conditional<std::is_const<T>::value, const char, char>::type byte;
    return reinterpret_cast<T*>(reinterpret_cast<byte*>(base) + off);
}

// Read-only index data (block tables, lengths, scales): loads through the
// constant address space, which the kernel never writes, become scalar loads
// (s_load, into SGPRs) when the index is wave-uniform.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
    typedef const __attribute__((address_space(4))) T* const_ptr;
    return ((const_ptr)p)[i];   // an address-space cast (C-style cast required)
}

// Wave-uniform value (lets the compiler keep it in an SGPR).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uniform64(long long v) {
    const unsigned long long u = (unsigned long long)v;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

// p[i] for a wave-uniform i, as a scalar load: the address itself is made
// uniform, so the load cannot become a vector load whose wait would also wait
// for every vector load in flight.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p, int64_t i) {
    const long long addr = uniform64((long long)(p + i));
    return ld_const(reinterpret_cast<const T*>(addr), 0);
}

// ---- device-coherent workspace accesses ------------------------------------
// Buffer loads/stores with the sc1 cache policy: like agent-scope relaxed
// atomics they are coherent across the XCDs' separate L2 caches, but they move
// 16 bytes per lane. The resource covers [base, base + bytes); accesses outside
// it read 0 and write nothing.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kSC1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t ws_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSC1);
}
__device__ __forceinline__ float ws_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSC1));
}
__device__ __forceinline__ void ws_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, float a, float b, float c,
                                           float d) {
    const u32x4_t v = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kSC1);
}

// ---- direct global -> LDS loads ------------------------------------------
// global_load_lds_dwordx4: every lane reads 16 bytes at its own global address
// and the wave writes them to LDS at lds + 16 * lane (lds is wave-uniform). The
// transfer completes asynchronously and is counted by vmcnt like any other
// vector load; nothing but s_waitcnt tells when the data is in LDS.

typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte loads; with NT the non-temporal hint, for data that no other wave
// of the launch reads again (as for dma16p)
template <bool NT>
__device__ __forceinline__ uint4 ld16p(const void* p) {
    if constexpr (NT) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *reinterpret_cast<const uint4*>(p);
    }
}

__device__ __forceinline__ void dma16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
// The same with the non-temporal hint (NT): the L2 keeps the line for as
// short a time as it can, leaving its room to lines that are read again.
template <bool NT>
__device__ __forceinline__ void dma16p(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, NT ? 2 : 0);
}
// 4 bytes; with only lane 0 active they land at lds itself
__device__ __forceinline__ void dma4(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}

template <bool NT>
__device__ __forceinline__ uint2 ld8p(const void* p) {
    if constexpr (NT) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        return make_uint2(v.x, v.y);
    } else {
        return *reinterpret_cast<const uint2*>(p);
    }
}

// Whether sequence s starts on the same physical block as the previous or the
// next sequence (rows of mbps entries in bt): a member of a group sharing
// prefix blocks copy-on-write, whose blocks other workgroups read as well.
// Only a cache hint rides on the answer, so a neighbour's unused entry (of any
// value) does no harm.
__device__ __forceinline__ bool first_block_shared(const int32_t* bt, int64_t mbps, int S, int s) {
    const int64_t prev = s > 0 ? (int64_t)(s - 1) * mbps : -1;
    const int64_t next = s + 1 < S ? (int64_t)(s + 1) * mbps : -1;
    const int b = ld_uniform(bt, (int64_t)s * mbps);
    const int bp = ld_uniform(bt, prev >= 0 ? prev : (int64_t)s * mbps);
    const int bn = ld_uniform(bt, next >= 0 ? next : (int64_t)s * mbps);
    return (prev >= 0 && bp == b) || (next >= 0 && bn == b);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// LDS reads and writes written as inline asm: the compiler cannot tell which
// LDS bytes a pending global->LDS load writes, and would otherwise wait for
// every vector load in flight before each LDS access. The caller orders them
// with wait_vmcnt before and lds_wait after (a wave's LDS accesses are
// performed in issue order, so a read sees the same wave's earlier writes).
template <int OFF = 0>
__device__ __forceinline__ u32x4 ds_read16(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return v;
}
template <int OFF = 0>
__device__ __forceinline__ u32x2 ds_read8(uint32_t addr) {
    u32x2 v;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return v;
}
template <int OFF = 0>
__device__ __forceinline__ void ds_write16(uint32_t addr, u32x4 v) {
    asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF) : "memory");
}
// 4 bytes, waited for in the same asm block (for a lone read of a small table
// while global->LDS loads are in flight)
__device__ __forceinline__ uint32_t ds_read4_wait(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ void ds_write4(uint32_t addr, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives as its
// element k (of four 16-bit elements) element i % 4 of the 8 bytes addressed
// by lane 4k + i/4.
template <int OFF = 0>
__device__ __forceinline__ u32x2 ds_read8_tr(uint32_t addr) {
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return v;
}
// Wait for the LDS reads above; the operands tie their results to this point so
// that no use is scheduled before it.
__device__ __forceinline__ void lds_wait(u32x4& a) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a) : : "memory");
}
__device__ __forceinline__ void lds_wait(u32x4& a, u32x4& b) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b) : : "memory");
}
__device__ __forceinline__ void lds_wait(u32x2& a) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a) : : "memory");
}
__device__ __forceinline__ void lds_wait(u32x2& a, u32x2& b) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b) : : "memory");
}
__device__ __forceinline__ void lds_wait(u32x4& a, u32x4& b, u32x4& c, u32x4& d, u32x2& e, u32x2& f,
                                         u32x2& g, u32x2& h, u32x2& i, u32x2& j, u32x2& k,
                                         u32x2& l) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h),
                   "+v"(i), "+v"(j), "+v"(k), "+v"(l)
                 :
                 : "memory");
}
__device__ __forceinline__ void lds_wait(u32x4& a, u32x4& b, u32x4& c, u32x4& d, u32x4& e, u32x4& f,
                                         u32x4& g, u32x4& h) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h)
                 :
                 : "memory");
}
__device__ __forceinline__ void lds_wait(u32x4& a, u32x4& b, u32x2& c, u32x2& d, u32x2& e, u32x2& f,
                                         u32x2& g) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g)
                 :
                 : "memory");
}

// s_waitcnt vmcnt(N): at most N vector memory instructions still in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

}  // namespace pa
