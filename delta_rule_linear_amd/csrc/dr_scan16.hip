// dr_scan16.hip -- the inter-chunk state scan for bf16 inputs on gfx950.
//
// Same algebra as the scan in dr_chunk.hip (per chunk, with T^ and P from the
// prep kernel):  X = Ks S,  R = V - g X,  U = T^ R,  O = g Q S + P U,
// S <- g63 S + Kl^T (l U);  written for low instruction count:
//
//  * Operand types.  With a scalar beta and no channel gate, Ks = Kl = k and
//    Qs = q are the raw bf16 inputs: they feed bf16 matrix-core ops directly,
//    with the fp32 state S and l U carried as bf16 hi + lo pairs (16
//    significant bits).  With a channel-wise gate or beta the gated operands
//    come from the workspace in fp16 and S, U are single fp16 terms.  T^ R and
//    P U are fp16 ops in both cases.
//  * Kl^T fragments are read from a row-major LDS copy of the chunk's Kl with
//    the transposing LDS read (ds_read_b64_tr_b16), so no element-wise
//    transposition or conversion happens in registers.
//  * No masking: rows past a sequence's end load a valid clamped row; their
//    U is exactly zero (beta or the prep kernel's zero rows make it so), so
//    they contribute nothing to S, and their O is never stored.
//
// One workgroup of four waves per (sequence, 16-column tile of S).  Wave w owns
// chunk rows 16w..16w+15 for X, Y, R, U, O and state rows [DK/4 w, DK/4 (w+1))
// for the state update.  Three barriers per chunk.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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

__device__ __forceinline__ uint4 lds16(const half_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Transposed 4 x 16-bit LDS read (see the lane map in the kernel comment).
__device__ __forceinline__ uint2 lds_tr4(const half_t* p) {
    s16x4 v = {0, 0, 0, 0};
#if defined(__HIP_DEVICE_COMPILE__)
    v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
#endif
    return __builtin_bit_cast(uint2, v);
}

// Four fp32 values as NPL 16-bit terms (bf16 hi/lo pair, or one fp16) written
// to consecutive LDS halfs of each plane.
template <bool BF, int NPL>
__device__ __forceinline__ void st4_terms(half_t* dst, int plane, const f32x4& v) {
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
        *reinterpret_cast<bf16x4*>(dst) = hi;
        if constexpr (NPL == 2) *reinterpret_cast<bf16x4*>(dst + plane) = lo;
    } else {
        half4 hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) hi[j] = (half_t)v[j];
        *reinterpret_cast<half4*>(dst) = hi;
    }
}

template <int DK, bool RAW>
struct S16Smem {
    static constexpr int NPL = RAW ? 2 : 1;   // terms of S and of l U
    static constexpr int SP = DK + 8;         // pitch of S^T rows (halfs)
    static constexpr int RP = CH + 8;         // pitch of token-major rows
    static constexpr int KP = DK + 16;        // pitch of the Kl tile rows
    static constexpr int kS = 0;                       // [NPL][16][SP]   S^T
    static constexpr int kR = kS + NPL * 16 * SP;      // [16][RP]        R^T (fp16)
    static constexpr int kU = kR + 16 * RP;            // [16][RP]        U^T (fp16)
    static constexpr int kUl = kU + 16 * RP;           // [NPL][16][RP]   (l U)^T
    static constexpr int kK = kUl + NPL * 16 * RP;     // [64][KP]        Kl, row-major
    static constexpr int HALFS = kK + CH * KP;
};

// Operands of one chunk, prefetched a chunk ahead as raw 16-byte pieces.
template <int DK>
struct S16Regs {
    uint4 ks[DK / 32];        // A fragments of Ks, rows 16w + (l & 15)
    uint4 qs[DK / 32];        // A fragments of Qs
    uint4 th[2], pm[2];       // A fragments of T^ and P
    uint4 kt[DK / 32];        // this thread's piece of the Kl tile
    uint16_t v[4];            // V tile (bf16 bits, or fp16 bits of vt), accumulator layout
    float gam[4], lam[4];     // scalar-gate row factors
    float g63[DK / 64 * 4];   // state decay of this lane's state rows
};

template <int DK, bool RAW, bool CGATE, bool CBETA>
__device__ __forceinline__ void s16_fetch(const ChunkArgs& a, S16Regs<DK>& g, int seq, int c, int n0,
                                          int w, int l, int tid) {
    const int t0 = c * CH;
    const int Lc = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const size_t cs = (size_t)seq * a.NC + c;
    const size_t obase = cs * (size_t)(CH * DK);     // [64][DK] workspace operand of this chunk
    const int ra = 16 * w + (l & 15);
    const int rac = ra < Lc ? ra : 0;                // clamped row for raw inputs
    const uint16_t* k16 = static_cast<const uint16_t*>(a.k);
    const uint16_t* q16 = static_cast<const uint16_t*>(a.q);
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
        const int k0 = 32 * s + 8 * (l >> 4);
        if constexpr (RAW) {
            g.ks[s] = *reinterpret_cast<const uint4*>(k16 + (tok0 + rac) * DK + k0);
            g.qs[s] = *reinterpret_cast<const uint4*>(q16 + (tok0 + rac) * DK + k0);
        } else {
            g.ks[s] = *reinterpret_cast<const uint4*>(a.wsKs + obase + ra * DK + k0);
            g.qs[s] = *reinterpret_cast<const uint4*>(a.wsQ + obase + ra * DK + k0);
        }
    }
    const size_t tbase = cs * (size_t)(CH * CH);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int k0 = 32 * s + 8 * (l >> 4);
        g.th[s] = *reinterpret_cast<const uint4*>(a.wsT + tbase + ra * CH + k0);
        g.pm[s] = *reinterpret_cast<const uint4*>(a.wsP + tbase + ra * CH + k0);
    }
    {
        const int r = tid >> 2, c0 = (tid & 3) * (DK / 4);
        const int rc = r < Lc ? r : 0;
#pragma unroll
        for (int i = 0; i < DK / 32; ++i) {
            if constexpr (RAW) {
                g.kt[i] = *reinterpret_cast<const uint4*>(k16 + (tok0 + rc) * DK + c0 + 8 * i);
            } else {
                const half_t* src = (CGATE ? a.wsKl : a.wsKs) + obase + r * DK + c0 + 8 * i;
                g.kt[i] = *reinterpret_cast<const uint4*>(src);
            }
        }
    }
    const int col = n0 + (l & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 16 * w + 4 * (l >> 4) + j;
        if constexpr (CBETA) {
            g.v[j] = reinterpret_cast<const uint16_t*>(a.wsV)[obase + r * DK + col];
        } else {
            const int rc = r < Lc ? r : 0;
            g.v[j] = static_cast<const uint16_t*>(a.v)[(tok0 + rc) * a.Dv + col];
        }
        if constexpr (!CGATE) {
            g.gam[j] = a.wsG[cs * kGW + r];
            g.lam[j] = a.wsG[cs * kGW + 64 + r];
        }
    }
    if constexpr (!CGATE) {
        const float d = a.wsG[cs * kGW + 63];
#pragma unroll
        for (int j = 0; j < DK / 64 * 4; ++j) g.g63[j] = d;
    } else {
#pragma unroll
        for (int t = 0; t < DK / 64; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                g.g63[t * 4 + j] = a.wsG[cs * kGW + 16 * (w * (DK / 64) + t) + 4 * (l >> 4) + j];
    }
}

template <int DK, bool RAW, bool CGATE, bool CBETA>
__device__ __forceinline__ void s16_chunk(const ChunkArgs& a, const S16Regs<DK>& cur, f32x4 (&S)[DK / 64],
                                          half_t* smem, int seq, int c, int col, int w, int l, int tid) {
    using SM = S16Smem<DK, RAW>;
    constexpr int NPL = SM::NPL;
    constexpr int NTS = DK / 64;
    // raw bf16 operands use bf16 ops; workspace operands are fp16
    constexpr bool BF = RAW;
    half_t* sS = smem + SM::kS;
    half_t* sR = smem + SM::kR;
    half_t* sU = smem + SM::kU;
    half_t* sUl = smem + SM::kUl;
    half_t* sK = smem + SM::kK;
    const int i16 = l & 15, g = l >> 4;
    const int t0 = c * CH;
    const int Lc = min(CH, a.L - t0);

    // Kl tile for this chunk's state update (read after the next two barriers)
    {
        const int r = tid >> 2, c0 = (tid & 3) * (DK / 4);
#pragma unroll
        for (int i = 0; i < DK / 32; ++i) *reinterpret_cast<uint4*>(sK + r * SM::KP + c0 + 8 * i) = cur.kt[i];
    }

    // X = Ks S and Y = Qs S (rows 16w..16w+15)
    f32x4 X = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
#pragma unroll
        for (int p = 0; p < NPL; ++p) {
            const uint4 sf = lds16(sS + p * 16 * SM::SP + i16 * SM::SP + 32 * s + 8 * g);
            X = mfma_raw<BF>(cur.ks[s], sf, X);
            Y = mfma_raw<BF>(cur.qs[s], sf, Y);
        }
    }
    // R = V - g X
    f32x4 Rv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float vv;
        if constexpr (CBETA) vv = (float)__builtin_bit_cast(half_t, cur.v[j]);
        else vv = bf16_to_f32(cur.v[j]);
        Rv[j] = vv - (CGATE ? 1.f : cur.gam[j]) * X[j];
    }
    st4_terms<false, 1>(sR + i16 * SM::RP + 16 * w + 4 * g, 0, Rv);
    __syncthreads();

    // U = T^ R
    f32x4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s)
        U = mfma_raw<false>(cur.th[s], lds16(sR + i16 * SM::RP + 32 * s + 8 * g), U);
    st4_terms<false, 1>(sU + i16 * SM::RP + 16 * w + 4 * g, 0, U);
    {
        f32x4 Ul;
#pragma unroll
        for (int j = 0; j < 4; ++j) Ul[j] = CGATE ? U[j] : cur.lam[j] * U[j];
        st4_terms<BF, NPL>(sUl + i16 * SM::RP + 16 * w + 4 * g, 16 * SM::RP, Ul);
    }
    __syncthreads();

    // O = g Y + P U
    f32x4 O;
#pragma unroll
    for (int j = 0; j < 4; ++j) O[j] = (CGATE ? 1.f : cur.gam[j]) * Y[j];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        O = mfma_raw<false>(cur.pm[s], lds16(sU + i16 * SM::RP + 32 * s + 8 * g), O);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 16 * w + 4 * g + j;
        if (r < Lc) {
            const size_t oi = ((size_t)seq * a.L + t0 + r) * a.Dv + col;
            if (a.out_bf16) static_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(O[j]);
            else static_cast<float*>(a.o)[oi] = O[j];
        }
    }

    // S = g63 S + Kl^T (l U).  The A fragment (state row rt + (l & 15), tokens
    // 32 s + 8 g + 0..7) comes from two transposed reads: within each group
    // of 16 lanes, lane q points at token 32 s + 8 g + (q >> 2) (+4) and key
    // column rt + 4 (q & 3); lane i then holds column rt + i of four tokens.
#pragma unroll
    for (int t = 0; t < NTS; ++t) {
        const int rt = 16 * (w * NTS + t);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const half_t* kp = sK + (32 * s + 8 * g + (i16 >> 2)) * SM::KP + rt + 4 * (i16 & 3);
            const uint2 lo4 = lds_tr4(kp);
            const uint2 hi4 = lds_tr4(kp + 4 * SM::KP);
            const uint4 ka = {lo4.x, lo4.y, hi4.x, hi4.y};
#pragma unroll
            for (int p = 0; p < NPL; ++p)
                acc = mfma_raw<BF>(ka, lds16(sUl + p * 16 * SM::RP + i16 * SM::RP + 32 * s + 8 * g), acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) S[t][j] = cur.g63[t * 4 + j] * S[t][j] + acc[j];
        st4_terms<BF, NPL>(sS + i16 * SM::SP + rt + 4 * g, 16 * SM::SP, S[t]);
    }
    __syncthreads();
}

template <int DK, bool RAW, bool CGATE, bool CBETA>
__global__ __launch_bounds__(256) void scan16_kernel(ChunkArgs a) {
    using SM = S16Smem<DK, RAW>;
    constexpr int NTS = DK / 64;
    __shared__ __attribute__((aligned(16))) half_t smem[SM::HALFS];

    // all column tiles of one sequence on one XCD (workgroups are dealt
    // round-robin to the 8 XCDs), so they share the chunk operands in L2
    const int NT = a.Dv / 16;
    const int bid = blockIdx.x;
    const int seq = (bid / (8 * NT)) * 8 + (bid & 7);
    const int tile = (bid >> 3) % NT;
    if (seq >= a.nseq) return;
    const int n0 = tile * 16;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int col = n0 + (l & 15);

    f32x4 S[NTS];
#pragma unroll
    for (int t = 0; t < NTS; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * (w * NTS + t) + 4 * (l >> 4) + j;
            S[t][j] = a.S0 ? a.S0[((size_t)seq * DK + row) * a.Dv + col] : 0.f;
        }
        st4_terms<RAW, SM::NPL>(smem + SM::kS + (l & 15) * SM::SP + 16 * (w * NTS + t) + 4 * (l >> 4),
                                16 * SM::SP, S[t]);
    }

    // Three register sets in rotation: chunk c is consumed while the loads of
    // chunks c + 1 and c + 2 are in flight.  Fetches past the end re-read the
    // last chunk, so every fetch is unconditional (no control-flow join makes
    // the compiler wait on a newer set).
    S16Regs<DK> r0, r1, r2;
    const int last = a.NC - 1;
    s16_fetch<DK, RAW, CGATE, CBETA>(a, r0, seq, 0, n0, w, l, tid);
    s16_fetch<DK, RAW, CGATE, CBETA>(a, r1, seq, min(1, last), n0, w, l, tid);
    __syncthreads();
    for (int c = 0; c < a.NC; c += 3) {
        s16_fetch<DK, RAW, CGATE, CBETA>(a, r2, seq, min(c + 2, last), n0, w, l, tid);
        __builtin_amdgcn_sched_barrier(0);   // keep every prefetch load at the top
        s16_chunk<DK, RAW, CGATE, CBETA>(a, r0, S, smem, seq, c, col, w, l, tid);
        if (c + 1 > last) break;
        s16_fetch<DK, RAW, CGATE, CBETA>(a, r0, seq, min(c + 3, last), n0, w, l, tid);
        __builtin_amdgcn_sched_barrier(0);
        s16_chunk<DK, RAW, CGATE, CBETA>(a, r1, S, smem, seq, c + 1, col, w, l, tid);
        if (c + 2 > last) break;
        s16_fetch<DK, RAW, CGATE, CBETA>(a, r1, seq, min(c + 4, last), n0, w, l, tid);
        __builtin_amdgcn_sched_barrier(0);
        s16_chunk<DK, RAW, CGATE, CBETA>(a, r2, S, smem, seq, c + 2, col, w, l, tid);
    }

    if (a.S_final) {
#pragma unroll
        for (int t = 0; t < NTS; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * (w * NTS + t) + 4 * (l >> 4) + j;
                a.S_final[((size_t)seq * DK + row) * a.Dv + col] = S[t][j];
            }
    }
}

template <int DK, bool CGATE, bool CBETA>
static hipError_t launch_s16(const ChunkArgs& a, hipStream_t st) {
    constexpr bool RAW = !CGATE && !CBETA;
    const int NT = a.Dv / 16;
    const int groups = (a.nseq + 7) / 8;
    hipLaunchKernelGGL((scan16_kernel<DK, RAW, CGATE, CBETA>), dim3(groups * 8 * NT), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_scan16(const ChunkArgs& a, int Dk, bool cgate, bool cbeta, hipStream_t st) {
    if (Dk == 64) {
        if (cgate) return cbeta ? launch_s16<64, true, true>(a, st) : launch_s16<64, true, false>(a, st);
        return cbeta ? launch_s16<64, false, true>(a, st) : launch_s16<64, false, false>(a, st);
    }
    if (cgate) return cbeta ? launch_s16<128, true, true>(a, st) : launch_s16<128, true, false>(a, st);
    return cbeta ? launch_s16<128, false, true>(a, st) : launch_s16<128, false, false>(a, st);
}

}  // namespace dr
