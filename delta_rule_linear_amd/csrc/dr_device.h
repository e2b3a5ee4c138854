// dr_device.h -- gfx950 device helpers shared by the delta-rule kernels:
// vector types, the 16x16x32 fp16 matrix-core op, operand fragments in one or
// two fp16 terms, and bf16/fp32 conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int CH = 64;     // tokens per chunk
constexpr int WAVE = 64;   // wavefront width

// ---------------------------------------------------------------------------
// Matrix core: D(16x16, fp32) += A(16x32, fp16) * B(32x16, fp16).
// Lane l holds A row (l & 15) and B column (l & 15), eight k-values each at
// k = 8 * (l >> 4) + [0, 8); it holds D rows 4 * (l >> 4) + [0, 4) of column
// (l & 15).  (A and B use the same lane-to-k map, so the k order inside the
// instruction never matters.)
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16(const half8& a, const half8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// An operand fragment carried as P fp16 terms: P == 1 is a plain fp16 value,
// P == 2 is hi + lo with hi = fp16(x), lo = fp16(x - hi) (about 22 significant
// bits).  Products drop lo * lo.
template <int P>
struct Frag {
    half8 t[P];
};

template <int PA, int PB>
__device__ __forceinline__ f32x4 mma(const Frag<PA>& a, const Frag<PB>& b, f32x4 c) {
#pragma unroll
    for (int i = 0; i < PA; ++i)
#pragma unroll
        for (int j = 0; j < PB; ++j)
            if (i + j < 2) c = mfma16(a.t[i], b.t[j], c);
    return c;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp32 matrix core, 16 x 16 x 4: lane l holds A[l % 16][l / 16] and
// B[l / 16][l % 16]; the accumulator layout is that of the 16x16x32 ops
// (lane l holds C[4 (l / 16) + j][l % 16]).
__device__ __forceinline__ f32x4 mfma_f32x4(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Two-term fp16 split x ~ hi + lo.  x is pinned in a register first: otherwise
// the compiler may fold x's producing multiply into one of the two conversions
// (a fused multiply-convert rounds the exact product, a plain convert the fp32
// product; the two differ by one fp16 ulp on near-ties) and then hi + lo is
// off by that ulp.
__device__ __forceinline__ void split2(float x, half_t& hi, half_t& lo) {
    asm volatile("" : "+v"(x));
    hi = (half_t)x;
    lo = (half_t)(x - (float)hi);
}

// Split eight fp32 values into P fp16 terms.
template <int P>
__device__ __forceinline__ Frag<P> split8(const float* x) {
    Frag<P> f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if constexpr (P == 2) {
            half_t hi, lo;
            split2(x[j], hi, lo);
            f.t[0][j] = hi;
            f.t[1][j] = lo;
        } else {
            f.t[0][j] = (half_t)x[j];
        }
    }
    return f;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& r, float* x) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(w[j] << 16);
        x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
}

// Eight consecutive input values (bf16 or fp32) at element offset `off`,
// converted to fp32; `ok == false` gives zeros without touching memory.
template <bool F32IN>
__device__ __forceinline__ void load8(const void* base, size_t off, bool ok, float* x) {
    if (!ok) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = 0.f;
        return;
    }
    if constexpr (F32IN) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
        float4 a = p[0], b = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
        uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
        unpack_bf16x8(r, x);
    }
}

// Load an fp16 operand fragment stored as P planes (plane stride in halfs).
template <int P>
__device__ __forceinline__ Frag<P> load_frag_h(const half_t* base, size_t off, size_t plane) {
    Frag<P> f;
#pragma unroll
    for (int p = 0; p < P; ++p) f.t[p] = *reinterpret_cast<const half8*>(base + off + p * plane);
    return f;
}

// Raw-input fragment: eight values of an input row, in P fp16 terms.
template <bool F32IN, int P>
__device__ __forceinline__ Frag<P> load_frag_in(const void* base, size_t off, bool ok) {
    float x[8];
    load8<F32IN>(base, off, ok, x);
    return split8<P>(x);
}

// Write four fp32 values as P fp16 terms at consecutive LDS halfs.
template <int P>
__device__ __forceinline__ void st4_lds(half_t* dst, size_t plane, const f32x4& v) {
    half4 hi, lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (P == 2) {
            half_t h, o;
            split2(v[j], h, o);
            hi[j] = h;
            lo[j] = o;
        } else {
            hi[j] = (half_t)v[j];
        }
    }
    *reinterpret_cast<half4*>(dst) = hi;
    if constexpr (P == 2) *reinterpret_cast<half4*>(dst + plane) = lo;
}

// Eight consecutive raw input values as loaded (bf16 bits or fp32), so a load
// can be issued early and converted later without a dependent wait.
template <bool F32IN>
struct Raw8 {
    uint4 x;
};
template <>
struct Raw8<true> {
    float4 a, b;
};

// Unconditional load of eight input values at element offset `off` (the caller
// keeps `off` in bounds, e.g. by clamping a masked row to a valid one).
template <bool F32IN>
__device__ __forceinline__ Raw8<F32IN> ld_raw8(const void* base, size_t off) {
    Raw8<F32IN> r;
    if constexpr (F32IN) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
        r.a = p[0];
        r.b = p[1];
    } else {
        r.x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    }
    return r;
}

// N (4 or 8) consecutive raw input values as loaded (bf16 bits or fp32 bits).
template <bool F32IN, int N>
struct RawN {
    uint32_t w[F32IN ? N : N / 2];
};

template <bool F32IN, int N>
__device__ __forceinline__ RawN<F32IN, N> ld_rawn(const void* base, size_t off) {
    RawN<F32IN, N> r;
    constexpr int W = F32IN ? N : N / 2;   // dwords
    const char* p = static_cast<const char*>(base) + off * (F32IN ? 4 : 2);
    if constexpr (W % 4 == 0) {
#pragma unroll
        for (int v = 0; v < W / 4; ++v) {
            const uint4 u = reinterpret_cast<const uint4*>(p)[v];
            r.w[4 * v] = u.x; r.w[4 * v + 1] = u.y; r.w[4 * v + 2] = u.z; r.w[4 * v + 3] = u.w;
        }
    } else {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        r.w[0] = u.x; r.w[1] = u.y;
    }
    return r;
}

template <bool F32IN, int N>
__device__ __forceinline__ void cvt_rawn(const RawN<F32IN, N>& r, float* x) {
#pragma unroll
    for (int j = 0; j < (F32IN ? N : N / 2); ++j) {
        if constexpr (F32IN) {
            x[j] = __uint_as_float(r.w[j]);
        } else {
            x[2 * j] = __uint_as_float(r.w[j] << 16);
            x[2 * j + 1] = __uint_as_float(r.w[j] & 0xffff0000u);
        }
    }
}

// Workgroup barrier over LDS only: wait for this wave's own LDS accesses,
// then s_barrier.  Global memory operations in flight (loads issued ahead,
// global->LDS copies) are not waited for, unlike __syncthreads.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Raw values to fp32, zeroed when !ok.
template <bool F32IN>
__device__ __forceinline__ void cvt_raw8(const Raw8<F32IN>& r, bool ok, float* x) {
    if constexpr (F32IN) {
        x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
        x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
    } else {
        unpack_bf16x8(r.x, x);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = ok ? x[j] : 0.f;
}

template <bool F32IN, int P>
__device__ __forceinline__ Frag<P> raw_to_frag(const Raw8<F32IN>& r, bool ok) {
    float x[8];
    cvt_raw8<F32IN>(r, ok, x);
    return split8<P>(x);
}

// One input value (bf16 or fp32) as fp32.
template <bool F32IN>
__device__ __forceinline__ float load1(const void* base, size_t off) {
    if constexpr (F32IN) return static_cast<const float*>(base)[off];
    else return bf16_to_f32(static_cast<const uint16_t*>(base)[off]);
}

// A strength as given, or the sigmoid of the given logit (input preparation).
__device__ __forceinline__ float strength(float x, int logit) {
    return logit ? 1.f / (1.f + expf(-x)) : x;
}

// Sum of x over aligned groups of N <= 32 consecutive lanes, in every lane of
// the group.  Within 16 lanes the butterfly runs on DPP moves (VALU speed, no
// LDS round trip): quad permutations pair lanes at distance 1 and 2, the
// half-row mirror pairs the two quads of 8 lanes, the row mirror the two
// halves of 16; the step across 16 lanes is one ds_swizzle in bit-mask mode
// (source lane (lane & 31) ^ 16).  No lane-address registers are held.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false);
    return x + __builtin_bit_cast(float, y);
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N >= 1 && N <= 32 && (N & (N - 1)) == 0, "group of 1..32 lanes, a power of two");
    if constexpr (N >= 2) x = dpp_add<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    if constexpr (N >= 4) x = dpp_add<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    if constexpr (N >= 8) x = dpp_add<0x141>(x);   // row_half_mirror
    if constexpr (N >= 16) x = dpp_add<0x140>(x);  // row_mirror
    if constexpr (N >= 32) {
        const int y = __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (16 << 10));
        x += __builtin_bit_cast(float, y);
    }
    return x;
}

// 1 / |x|_2 from a sum of squares, 0 for the zero vector.
__device__ __forceinline__ float inv_norm(float ssq) {
    return ssq > 0.f ? 1.f / sqrtf(ssq) : 0.f;
}

// Store one fp32 value as P fp16 terms: base[off + idx] (hi) and
// base[off + plane + idx] (lo).
template <int P>
__device__ __forceinline__ void store_split(half_t* base, size_t off, size_t plane, size_t idx,
                                            float x) {
    if constexpr (P == 2) {
        half_t hi, lo;
        split2(x, hi, lo);
        base[off + idx] = hi;
        base[off + plane + idx] = lo;
    } else {
        base[off + idx] = (half_t)x;
    }
}

// Store N (4 or 8) consecutive fp32 values as P fp16 terms at base[off + idx ..]
// (hi) and base[off + plane + idx ..] (lo), as one vector store per plane.
template <int P, int N>
__device__ __forceinline__ void store_split_n(half_t* base, size_t off, size_t plane, size_t idx, const float* x) {
    typedef half_t hvec __attribute__((ext_vector_type(N)));
    hvec hi, lo;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        if constexpr (P == 2) {
            half_t h, o;
            split2(x[j], h, o);
            hi[j] = h;
            lo[j] = o;
        } else {
            hi[j] = (half_t)x[j];
        }
    }
    *reinterpret_cast<hvec*>(base + off + idx) = hi;
    if constexpr (P == 2) *reinterpret_cast<hvec*>(base + off + plane + idx) = lo;
}

// N (4 or 8) consecutive input values (bf16 or fp32) as fp32.
template <bool F32IN, int N>
__device__ __forceinline__ void load_n(const void* base, size_t off, float* x) {
    if constexpr (F32IN) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
#pragma unroll
        for (int v = 0; v < N / 4; ++v) {
            const float4 f = p[v];
            x[4 * v] = f.x; x[4 * v + 1] = f.y; x[4 * v + 2] = f.z; x[4 * v + 3] = f.w;
        }
    } else {
        const uint16_t* h = static_cast<const uint16_t*>(base) + off;
        if constexpr (N == 8) {
            unpack_bf16x8(*reinterpret_cast<const uint4*>(h), x);
        } else {
            const uint2 u = *reinterpret_cast<const uint2*>(h);
            x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xffff0000u);
            x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xffff0000u);
        }
    }
}

// N (4 or 8) consecutive fp32 values.
template <int N>
__device__ __forceinline__ void load_f32_n(const float* p, float* x) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int v = 0; v < N / 4; ++v) {
        const float4 f = q[v];
        x[4 * v] = f.x; x[4 * v + 1] = f.y; x[4 * v + 2] = f.z; x[4 * v + 3] = f.w;
    }
}

// Strengths (beta or beta_v) of row `row`, channels ch0 .. ch0 + N - 1: one
// value per channel ([rows][dk]), or, with per_token, one value per token
// ([rows]) that every channel shares.
template <int N>
__device__ __forceinline__ void load_strength_n(const float* base, bool per_token, size_t row, int dk, int ch0,
                                                float* x) {
    if (per_token) {
        const float b = base[row];
#pragma unroll
        for (int j = 0; j < N; ++j) x[j] = b;
    } else {
        load_f32_n<N>(base + row * dk + ch0, x);
    }
}
__device__ __forceinline__ float strength_at(const float* base, bool per_token, size_t row, int dk, int col) {
    return per_token ? base[row] : base[row * dk + col];
}

// Store sixteen fp32 values as P fp16 terms at base[idx .. idx + 16) of each
// plane (16-byte aligned).
template <int P>
__device__ __forceinline__ void store_row16(half_t* base, size_t plane, size_t idx, const float* x) {
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
        half8 hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (P == 2) {
                half_t h, o;
                split2(x[8 * h8 + j], h, o);
                hi[j] = h;
                lo[j] = o;
            } else {
                hi[j] = (half_t)x[8 * h8 + j];
            }
        }
        *reinterpret_cast<half8*>(base + idx + 8 * h8) = hi;
        if constexpr (P == 2) *reinterpret_cast<half8*>(base + plane + idx + 8 * h8) = lo;
    }
}

}  // namespace dr
