// dr_lds.h -- device helpers of the matrix-core scans for gfx950: LDS
// access through the LDS address space, the 16x16x32 matrix-core op on raw
// 16-byte fragments, the transposing LDS read, global->LDS copies written as
// inline assembly (untracked by the compiler, waited for by count), the XOR
// swizzle of 64-row operand tiles and the bf16 hi + lo split of fp32 values.
#pragma once

#include <hip/hip_runtime.h>

#include "dr_device.h"

namespace dr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
// LDS addresses are kept in the LDS address space end to end: no generic
// pointers, so no null checks on conversion, and the compiler keeps exact
// knowledge of which LDS object every access touches.
typedef __attribute__((address_space(3))) char lchar;

// LDS load / store of a 2-, 4-, 8- or 16-byte value through plain integer
// (vector) types, reinterpreted to T.
template <int N>
struct LdsWord;
template <>
struct LdsWord<2> { typedef unsigned short type; };
template <>
struct LdsWord<4> { typedef unsigned type; };
template <>
struct LdsWord<8> { typedef unsigned type __attribute__((ext_vector_type(2))); };
template <>
struct LdsWord<16> { typedef unsigned type __attribute__((ext_vector_type(4))); };

template <class T>
__device__ __forceinline__ T lds_ld(const lchar* p) {
    typedef typename LdsWord<sizeof(T)>::type W;
    const W x = *reinterpret_cast<const __attribute__((address_space(3))) W*>(p);
    return __builtin_bit_cast(T, x);
}
template <class T>
__device__ __forceinline__ void lds_st(lchar* p, const T& v) {
    typedef typename LdsWord<sizeof(T)>::type W;
    *reinterpret_cast<__attribute__((address_space(3))) W*>(p) = __builtin_bit_cast(W, v);
}

// 16x16x32 matrix-core op on raw 16-byte fragments, bf16 or fp16 elements.
template <bool BF>
__device__ __forceinline__ f32x4 mfma_raw(const uint4& a, const uint4& b, const f32x4& c) {
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 lds16(const lchar* p) { return lds_ld<uint4>(p); }

// Transposed LDS read of four 16-bit values.  Within each group of 16 lanes,
// lane i receives element (i mod 4) of the 8-byte rows addressed by lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4, in that order.
__device__ __forceinline__ uint2 lds_tr4(const lchar* p) {
    s16x4 v = {0, 0, 0, 0};
#if defined(__HIP_DEVICE_COMPILE__)
    v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
#endif
    return __builtin_bit_cast(uint2, v);
}

// 16 bytes from global memory into LDS at lds_base + 16 * lane (lds_base
// must be the same for the whole wave; it goes to M0).  Written as inline
// assembly so that the compiler does not track these copies: it would
// otherwise assume any LDS access may alias a copy in flight and wait for
// all of them before every LDS read.  The copies have no register results;
// their completion is waited for explicitly, by count (vmcnt_imm).  M0 is
// saved and restored around the copy.
__device__ __forceinline__ void dma16(const void* g, lchar* lds_base) {
    const unsigned m = __builtin_amdgcn_readfirstlane((unsigned)(size_t)lds_base);
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(m)
        : "memory");
}

// One dword from global memory into LDS at lds_base + 4 * lane (as dma16).
__device__ __forceinline__ void dma4(const void* g, lchar* lds_base) {
    const unsigned m = __builtin_amdgcn_readfirstlane((unsigned)(size_t)lds_base);
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
        "global_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(m)
        : "memory");
}

// 16 bytes from base + voff (base the same for the whole wave, voff per
// lane) into LDS at lds_base + 16 * lane: the scalar-base addressing form,
// with no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16s(const char* base, unsigned voff, lchar* lds_base) {
    const unsigned m = __builtin_amdgcn_readfirstlane((unsigned)(size_t)lds_base);
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(m)
        : "memory");
}

// A pointer known to be the same in every lane, kept in scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
    const unsigned long long u = (unsigned long long)p;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
    return reinterpret_cast<const char*>(((unsigned long long)hi << 32) | lo);
}

// Swizzle of 16-byte pieces in a 64-row tile with RB bytes per row: piece p
// of row r is stored at piece p ^ swz(r).  256-byte rows: 16 consecutive rows
// land on 16 distinct bank groups; 128-byte rows: two rows share the 64
// banks, so pairs of rows get distinct swizzles.
template <int RB>
__device__ __forceinline__ int swz(int r) {
    return RB == 256 ? (r & 15) : ((r >> 1) & 7);
}

template <int RB>
__device__ __forceinline__ const lchar* tile_at(const lchar* tile, int r, int piece) {
    return tile + r * RB + 16 * (piece ^ swz<RB>(r));
}

// Four fp32 values as NPL 16-bit terms (bf16 hi/lo pair, or one fp16) at
// consecutive LDS halfs of each plane (plane stride in bytes).
template <bool BF, int NPL>
__device__ __forceinline__ void st4_terms(lchar* dst, int plane, const f32x4& v) {
    if constexpr (BF) {
        bf16x4 hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float x = v[j];
            asm volatile("" : "+v"(x));   // one rounding for both uses of hi
            const __bf16 h = (__bf16)x;
            hi[j] = h;
            lo[j] = (__bf16)(x - (float)h);
        }
        lds_st(dst, hi);
        if constexpr (NPL == 2) lds_st(dst + plane, lo);
    } else {
        half4 hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) hi[j] = (half_t)v[j];
        lds_st(dst, hi);
    }
}

// s_waitcnt immediate: wait until at most n vector-memory operations of this
// wave are outstanding (export and LDS counters not waited for).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

}  // namespace dr
