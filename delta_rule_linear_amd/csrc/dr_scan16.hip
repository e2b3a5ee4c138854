// dr_scan16.hip -- the inter-chunk state scan for bf16 inputs on gfx950.
//
// Same algebra as the scan in dr_chunk.hip (per chunk, with T^ and P from the
// prep kernel):  X = Ks S,  R = V - g X,  U = T^ R,  O = g Q S + P U,
// S <- g63 S + Kl^T (l U).  Built around the data movement:
//
//  * Each chunk's operand tiles (Kl, Ks, Q, T^, P, the V tile, gate factors)
//    are copied once per workgroup straight into LDS with 16-byte global->LDS
//    loads, fully coalesced, one chunk ahead into a double buffer.  Rows of a
//    tile are stored with their 16-byte pieces XOR-swizzled by row, so the
//    fragment reads below are free of bank conflicts.
//  * Operand types.  With a scalar beta and no channel gate, Ks = Kl = k and
//    Q = q are the raw bf16 inputs: they feed bf16 matrix-core ops directly,
//    with the fp32 state S and l U carried as bf16 hi + lo pairs (16
//    significant bits).  With a channel-wise gate or beta the gated operands
//    come from the workspace in fp16 and S, U are single fp16 terms.  T^ R and
//    P U are fp16 ops in both cases.
//  * Kl^T fragments come from the row-major Kl tile through the transposing
//    LDS read (ds_read_b64_tr_b16): no transposition in registers.
//  * No masking: rows past a sequence's end load a valid clamped row; their
//    U is exactly zero (beta or the prep kernel's zero rows make it so), so
//    they contribute nothing to S, and their O is never stored.
//  * Barriers are raw s_barrier with an explicit LDS-only wait, so the
//    copies for the next chunk stay in flight across them; the copies are
//    waited for once, before the chunk's last barrier.
//
// One workgroup of four waves per (sequence, 16-column tile of S).  Wave w owns
// chunk rows 16w..16w+15 for X, Y, R, U, O and state rows [DK/4 w, DK/4 (w+1))
// for the state update.

#include <hip/hip_runtime.h>

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

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

__device__ __forceinline__ uint4 lds16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// Transposed LDS read of four 16-bit values.  Within each group of 16 lanes,
// lane i receives element (i mod 4) of the 8-byte rows addressed by lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4, in that order.
__device__ __forceinline__ uint2 lds_tr4(const char* p) {
    s16x4 v = {0, 0, 0, 0};
#if defined(__HIP_DEVICE_COMPILE__)
    v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
#endif
    return __builtin_bit_cast(uint2, v);
}

// 16 bytes from global memory into LDS at lds_base + 16 * lane (lds_base
// must be the same for the whole wave).
__device__ __forceinline__ void dma16(const void* g, char* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 16, 0, 0);
#endif
}

// Workgroup barrier over LDS only: wait for this wave's own LDS accesses,
// then s_barrier.  Global->LDS copies in flight are not waited for.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait for every vector-memory operation of this wave, including the
// global->LDS copies.
__device__ __forceinline__ void vmem_wait_all() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    asm volatile("" ::: "memory");
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
__device__ __forceinline__ const char* tile_at(const char* tile, int r, int piece) {
    return tile + r * RB + 16 * (piece ^ swz<RB>(r));
}

// Copy a [64][RB]-byte tile of 16-bit values (row r at src + r * pitch
// elements; rows >= valid read row 0) into swizzled LDS; the four waves
// share it, 1 KiB per instruction.
template <int RB>
__device__ __forceinline__ void dma_tile(const uint16_t* src, size_t pitch, int valid, char* tile, int w, int l) {
    constexpr int PPR = RB / 16;      // pieces per row
    constexpr int RPI = 64 / PPR;     // rows per 1 KiB instruction
    constexpr int NI = 64 / RPI / 4;  // instructions per wave
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int blk = w * NI + j;
        const int r = blk * RPI + l / PPR;
        const int rc = r < valid ? r : 0;
        const int lp = (l % PPR) ^ swz<RB>(r);
        dma16(src + (size_t)rc * pitch + 8 * lp, tile + blk * 1024);
    }
}

// Four fp32 values as NPL 16-bit terms (bf16 hi/lo pair, or one fp16) at
// consecutive LDS halfs of each plane (plane stride in bytes).
template <bool BF, int NPL>
__device__ __forceinline__ void st4_terms(char* dst, int plane, const f32x4& v) {
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

// LDS plan (bytes).  Two operand buffers, each
//   [Kl 64 x RB][Ks 64 x RB, channel gate only][Q 64 x RB][T^ 64 x 128][P 64 x 128]
//   [V 64 x 32][gate factors 512]
// then the working area [S^T NPL x 16 x SP][R^T 16 x RP][U^T 16 x RP][(lU)^T NPL x 16 x RP].
template <int DK, bool RAW, bool CGATE>
struct SD {
    static constexpr int NPL = RAW ? 2 : 1;
    static constexpr int RB = DK * 2;               // bytes per K / Q row
    static constexpr int KL = 0;
    static constexpr int KS = CGATE ? KL + 64 * RB : KL;   // Ks == Kl unless the gate is per channel
    static constexpr int QT = KS + 64 * RB;
    static constexpr int TT = QT + 64 * RB;
    static constexpr int PT = TT + 64 * 128;
    static constexpr int VT = PT + 64 * 128;
    static constexpr int GT = VT + 64 * 32;
    static constexpr int BUF = GT + 512;
    static constexpr int SP = (DK + 8) * 2;          // bytes per S^T row
    static constexpr int RP = (CH + 8) * 2;          // bytes per token-major row
    static constexpr int WS = 2 * BUF;
    static constexpr int WR = WS + NPL * 16 * SP;
    static constexpr int WU = WR + 16 * RP;
    static constexpr int WUL = WU + 16 * RP;
    static constexpr int TOTAL = WUL + NPL * 16 * RP;
};

// Issue the copies of chunk c's operands into buffer `buf`.
template <int DK, bool RAW, bool CGATE, bool CBETA>
__device__ __forceinline__ void s16_dma(const ChunkArgs& a, char* buf, int seq, int c, int n0, int w, int l) {
    using L = SD<DK, RAW, CGATE>;
    const int t0 = c * CH;
    const int Lc = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const size_t cs = (size_t)seq * a.NC + c;
    const size_t obase = cs * (size_t)(CH * DK);
    if constexpr (RAW) {
        dma_tile<L::RB>(static_cast<const uint16_t*>(a.k) + tok0 * DK, DK, Lc, buf + L::KL, w, l);
        dma_tile<L::RB>(static_cast<const uint16_t*>(a.q) + tok0 * DK, DK, Lc, buf + L::QT, w, l);
    } else {
        const half_t* kl = CGATE ? a.wsKl : a.wsKs;
        dma_tile<L::RB>(reinterpret_cast<const uint16_t*>(kl) + obase, DK, CH, buf + L::KL, w, l);
        if constexpr (CGATE)
            dma_tile<L::RB>(reinterpret_cast<const uint16_t*>(a.wsKs) + obase, DK, CH, buf + L::KS, w, l);
        dma_tile<L::RB>(reinterpret_cast<const uint16_t*>(a.wsQ) + obase, DK, CH, buf + L::QT, w, l);
    }
    const size_t tbase = cs * (size_t)(CH * CH);
    dma_tile<128>(reinterpret_cast<const uint16_t*>(a.wsT) + tbase, CH, CH, buf + L::TT, w, l);
    dma_tile<128>(reinterpret_cast<const uint16_t*>(a.wsP) + tbase, CH, CH, buf + L::PT, w, l);
    if (w < 2) {   // V tile: 64 rows x 16 columns, two 16-byte pieces per row
        const int r = 32 * w + (l >> 1), piece = l & 1;
        if constexpr (CBETA) {
            dma16(reinterpret_cast<const uint16_t*>(a.wsV) + obase + r * DK + n0 + 8 * piece, buf + L::VT + w * 1024);
        } else {
            const int rc = r < Lc ? r : 0;
            dma16(static_cast<const uint16_t*>(a.v) + (tok0 + rc) * a.Dv + n0 + 8 * piece, buf + L::VT + w * 1024);
        }
    } else if (w == 2) {   // gate factors: gamma[64] and lambda[64], or the state decay [DK]
        constexpr int NG = CGATE ? DK / 4 : 32;
        if (l < NG) dma16(a.wsG + cs * kGW + 4 * l, buf + L::GT);
    }
}

// How many chunks ahead the L2 is warmed (see s16_warm).
#ifndef DR_SCAN_PFD
#define DR_SCAN_PFD 3
#endif

// Warm L2 with chunk cc's operands: each workgroup of a sequence touches one
// dword in a 1/NT share of the chunk's 128-byte operand lines (two per
// thread), so the lines are already on their way from HBM when the copies
// into LDS ask for them.  The caller keeps the loaded values until its
// end-of-chunk wait for all vector memory, so no extra wait is ever taken.
template <int DK, bool RAW, bool CGATE, bool CBETA>
__device__ __forceinline__ void s16_warm(const ChunkArgs& a, int seq, int cc, int li, float& w0, float& w1) {
    const int t0 = cc * CH;
    const int Lc = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const size_t cs = (size_t)seq * a.NC + cc;
    const size_t ob = cs * (size_t)(CH * DK) * 2;   // byte offset of a workspace operand tile
    const int nraw = (Lc * DK * 2 + 127) >> 7;
    const char* p0 = nullptr;
    const char* p1 = nullptr;
    int x0 = li, x1 = li + 256 * (a.Dv / 16);
    auto region = [&](const void* base, int n) {
        if (!p0 && x0 >= 0 && x0 < n) p0 = static_cast<const char*>(base) + 128 * x0;
        if (!p1 && x1 >= 0 && x1 < n) p1 = static_cast<const char*>(base) + 128 * x1;
        x0 -= n;
        x1 -= n;
    };
    if constexpr (RAW) {
        region(static_cast<const char*>(a.k) + tok0 * DK * 2, nraw);
        region(static_cast<const char*>(a.q) + tok0 * DK * 2, nraw);
    } else {
        region(reinterpret_cast<const char*>(CGATE ? a.wsKl : a.wsKs) + ob, DK);
        if constexpr (CGATE) region(reinterpret_cast<const char*>(a.wsKs) + ob, DK);
        region(reinterpret_cast<const char*>(a.wsQ) + ob, DK);
    }
    region(a.wsT + cs * (CH * CH), CH * CH * 2 / 128);
    region(a.wsP + cs * (CH * CH), CH * CH * 2 / 128);
    if constexpr (CBETA) region(reinterpret_cast<const char*>(a.wsV) + ob, DK);
    else region(static_cast<const char*>(a.v) + tok0 * a.Dv * 2, (Lc * a.Dv * 2 + 127) >> 7);
    region(a.wsG + cs * kGW, kGW * 4 / 128);
    w0 = p0 ? *reinterpret_cast<const float*>(p0) : 0.f;
    w1 = p1 ? *reinterpret_cast<const float*>(p1) : 0.f;
}

template <int DK, bool RAW, bool CGATE, bool CBETA>
__global__ __launch_bounds__(256) void scan16_kernel(ChunkArgs a) {
    using L = SD<DK, RAW, CGATE>;
    constexpr int NPL = L::NPL;
    constexpr int NTS = DK / 64;   // 16-row state tiles per wave
    constexpr bool BF = RAW;       // raw bf16 operands use bf16 ops, workspace ones fp16
    // Separate LDS objects for the two operand buffers and the working area:
    // the compiler then sees that the copies into one buffer cannot alias the
    // reads of the other, and does not wait for the copies before every LDS
    // access.
    __shared__ __attribute__((aligned(16))) char lds_buf0[L::BUF];
    __shared__ __attribute__((aligned(16))) char lds_buf1[L::BUF];
    __shared__ __attribute__((aligned(16))) char lds_work[L::TOTAL - L::WS];

    // all column tiles of one sequence on one XCD (workgroups are dealt
    // round-robin to the 8 XCDs), so they share the chunk operands in L2
    const int NT = a.Dv / 16;
    const int bid = blockIdx.x;
    const int seq = (bid / (8 * NT)) * 8 + (bid & 7);
    const int tile = (bid >> 3) % NT;
    if (seq >= a.nseq) return;
    const int n0 = tile * 16;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int i16 = l & 15, g = l >> 4;
    const int col = n0 + i16;
    const int ra = 16 * w + i16;
    char* sS = lds_work;
    char* sR = lds_work + (L::WR - L::WS);
    char* sU = lds_work + (L::WU - L::WS);
    char* sUl = lds_work + (L::WUL - L::WS);

    f32x4 S[NTS];
#pragma unroll
    for (int t = 0; t < NTS; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * (w * NTS + t) + 4 * g + j;
            S[t][j] = a.S0 ? a.S0[((size_t)seq * DK + row) * a.Dv + col] : 0.f;
        }
        st4_terms<BF, NPL>(sS + i16 * L::SP + 2 * (16 * (w * NTS + t) + 4 * g), 16 * L::SP, S[t]);
    }
    s16_dma<DK, RAW, CGATE, CBETA>(a, lds_buf0, seq, 0, n0, w, l);
    vmem_wait_all();
    lds_barrier();

    f32x4 Oprev = {0.f, 0.f, 0.f, 0.f};
    int oprev_t0 = -1, oprev_Lc = 0;
    auto store_o = [&]() {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * w + 4 * g + j;
            if (r < oprev_Lc) {
                const size_t oi = ((size_t)seq * a.L + oprev_t0 + r) * a.Dv + col;
                if (a.out_bf16) static_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(Oprev[j]);
                else static_cast<float*>(a.o)[oi] = Oprev[j];
            }
        }
    };

    // one chunk: operands in `buf`, copies of the next chunk into `nbuf`
    auto chunk = [&](const int c, const char* buf, char* nbuf) {
        const int t0 = c * CH;
        const int Lc = min(CH, a.L - t0);
        // copies for the next chunk into the other buffer (last read in the
        // previous chunk, before its final barrier)
        if (c + 1 < a.NC) s16_dma<DK, RAW, CGATE, CBETA>(a, nbuf, seq, c + 1, n0, w, l);
        float warm0 = 0.f, warm1 = 0.f;
        if (DR_SCAN_PFD > 1 && c + DR_SCAN_PFD < a.NC)
            s16_warm<DK, RAW, CGATE, CBETA>(a, seq, c + DR_SCAN_PFD, tile + NT * tid, warm0, warm1);

        // X = Ks S and Y = Q S (rows 16w..16w+15)
        f32x4 X = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            const uint4 kf = lds16(tile_at<L::RB>(buf + L::KS, ra, 4 * s + g));
            const uint4 qf = lds16(tile_at<L::RB>(buf + L::QT, ra, 4 * s + g));
#pragma unroll
            for (int p = 0; p < NPL; ++p) {
                const uint4 sf = lds16(sS + p * 16 * L::SP + i16 * L::SP + 2 * (32 * s + 8 * g));
                X = mfma_raw<BF>(kf, sf, X);
                Y = mfma_raw<BF>(qf, sf, Y);
            }
        }
        // the previous chunk's output, deferred so that its store is not
        // waited for at the end of the chunk it was computed in
        if (oprev_t0 >= 0) store_o();
        // R = V - g X
        const float* gt = reinterpret_cast<const float*>(buf + L::GT);
        f32x4 Rv, gam, lam;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * w + 4 * g + j;
            const uint16_t vb = *reinterpret_cast<const uint16_t*>(buf + L::VT + r * 32 + 2 * i16);
            const float vv = CBETA ? (float)__builtin_bit_cast(half_t, vb) : bf16_to_f32(vb);
            gam[j] = CGATE ? 1.f : gt[r];
            lam[j] = CGATE ? 1.f : gt[64 + r];
            Rv[j] = vv - gam[j] * X[j];
        }
        st4_terms<false, 1>(sR + i16 * L::RP + 2 * (16 * w + 4 * g), 0, Rv);
        lds_barrier();

        // U = T^ R
        f32x4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s)
            U = mfma_raw<false>(lds16(tile_at<128>(buf + L::TT, ra, 4 * s + g)),
                                lds16(sR + i16 * L::RP + 2 * (32 * s + 8 * g)), U);
        st4_terms<false, 1>(sU + i16 * L::RP + 2 * (16 * w + 4 * g), 0, U);
        {
            f32x4 Ul;
#pragma unroll
            for (int j = 0; j < 4; ++j) Ul[j] = lam[j] * U[j];
            st4_terms<BF, NPL>(sUl + i16 * L::RP + 2 * (16 * w + 4 * g), 16 * L::RP, Ul);
        }
        lds_barrier();

        // O = g Y + P U (stored during the next chunk)
        f32x4 O;
#pragma unroll
        for (int j = 0; j < 4; ++j) O[j] = gam[j] * Y[j];
#pragma unroll
        for (int s = 0; s < 2; ++s)
            O = mfma_raw<false>(lds16(tile_at<128>(buf + L::PT, ra, 4 * s + g)),
                                lds16(sU + i16 * L::RP + 2 * (32 * s + 8 * g)), O);
        Oprev = O;
        oprev_t0 = t0;
        oprev_Lc = Lc;

        // S = g63 S + Kl^T (l U).  A fragment (state row rt + i16, tokens
        // 32 s + 8 g + 0..7) from two transposed reads: lane q of each
        // 16-lane group points at token 32 s + 8 g + (q >> 2) (+4) and key
        // column rt + 4 (q & 3); lane i then holds column rt + i.
#pragma unroll
        for (int t = 0; t < NTS; ++t) {
            const int rt = 16 * (w * NTS + t);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int tok = 32 * s + 8 * g + (i16 >> 2);
                const int d = rt + 4 * (i16 & 3);
                const uint2 lo4 = lds_tr4(tile_at<L::RB>(buf + L::KL, tok, d >> 3) + 2 * (d & 7));
                const uint2 hi4 = lds_tr4(tile_at<L::RB>(buf + L::KL, tok + 4, d >> 3) + 2 * (d & 7));
                const uint4 ka = {lo4.x, lo4.y, hi4.x, hi4.y};
#pragma unroll
                for (int p = 0; p < NPL; ++p)
                    acc = mfma_raw<BF>(ka, lds16(sUl + p * 16 * L::RP + i16 * L::RP + 2 * (32 * s + 8 * g)), acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float d63 = CGATE ? gt[rt + 4 * g + j] : gt[63];
                S[t][j] = d63 * S[t][j] + acc[j];
            }
            st4_terms<BF, NPL>(sS + i16 * L::SP + 2 * (rt + 4 * g), 16 * L::SP, S[t]);
        }
        vmem_wait_all();   // the next chunk's copies have landed
        asm volatile("" ::"v"(warm0), "v"(warm1));
        lds_barrier();
    };
    for (int c = 0; c < a.NC; c += 2) {
        chunk(c, lds_buf0, lds_buf1);
        if (c + 1 < a.NC) chunk(c + 1, lds_buf1, lds_buf0);
    }
    if (oprev_t0 >= 0) store_o();

    if (a.S_final) {
#pragma unroll
        for (int t = 0; t < NTS; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * (w * NTS + t) + 4 * g + j;
                a.S_final[((size_t)seq * DK + row) * a.Dv + col] = S[t][j];
            }
    }
}

template <int DK, bool CGATE, bool CBETA>
static hipError_t launch_s16(const ChunkArgs& a, hipStream_t st) {
    constexpr bool RAW = !CGATE && !CBETA;
    using L = SD<DK, RAW, CGATE>;
    static_assert(L::TOTAL <= 160 * 1024, "LDS plan exceeds 160 KiB");
    auto kern = scan16_kernel<DK, RAW, CGATE, CBETA>;
    const int NT = a.Dv / 16;
    const int groups = (a.nseq + 7) / 8;
    hipLaunchKernelGGL(kern, dim3(groups * 8 * NT), dim3(256), 0, st, a);
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
