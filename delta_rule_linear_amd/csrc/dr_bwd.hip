// dr_bwd.hip -- gradients of the chunked forward: the kernels for a scalar gate
// (or none) first, then their channel-gate variants, then the passes that take
// a channel-wise beta (or separate strengths) through the same kernels with
// unit strength.  fp32 arithmetic on the matrix cores (state-sized products of
// the per-chunk kernel as two fp16 terms).
//
// The pages print no backward; this is the reverse-mode derivative of the
// chunk algebra of the forward (DeltaNet page, chunkwise form and its
// hardware notes; FG2-GDN page, section 2 for the gated recurrence).  Per
// chunk of 64 tokens with start state S, cumulative log-decay g_r, gamma_r =
// e^{g_r}, lambda_r = e^{g_63 - g_r}, E_ri = e^{g_r - g_i}:
//   A = strict lower of Diag(beta) K K^T o E,   T = (I + A)^-1,
//   P = lower (diagonal included) of Q K^T o E,
//   R = V - Gamma K S,   U = T Diag(beta) R,
//   O = Gamma Q S + P U,   S' = gamma_63 S + K^T Lambda U.
// With H the gradient of the loss with respect to S' (the next chunk's start
// state, dS_final after the last chunk):
//   dU = P^T dO + Lambda K H,   dR = Diag(beta) T^T dU  (= dV),
//   dS = gamma_63 H + Q^T Gamma dO - K^T Gamma dR,
//   dP = dO U^T,   dT^ = dU R^T,   dA = -T^T (dT^ Diag(beta)) T^T,
// and dq, dk, dbeta, dg follow from the products above; d log alpha is the
// reverse cumulative sum of dg within the chunk.
//
// Four kernels (per gate kind):
//   prep   one workgroup per chunk: g, A's factor K K^T o E, P, T
//   fscan  one per (sequence, 16 state columns): the start state of every
//          chunk, R and U (sequential over chunks)
//   rscan  one per (sequence, 16 state columns), chunks in reverse: H per
//          chunk, dU, dV, and dS0
//   post   one per chunk: dq, dk, dbeta, d log alpha
// Tokens past the end of a sequence enter the last chunk as zeros (q, k, v,
// dO, beta and log alpha), which leaves every real token's terms unchanged.

#include <algorithm>

#include "dr_internal.h"
#include "dr_lds.h"

namespace dr {
namespace {

constexpr int NTH = 256;
constexpr int PT = CH + 1;   // LDS pitch of 64-wide fp32 rows

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Rows [0, 64) x [0, DK) of q or k for the chunk starting at token t0 into
// LDS (pitch DK + 1), as fp32, zeros past the end.
template <int DK, bool F32IN>
__device__ __forceinline__ void load_rows(float* dst, const void* src, size_t tok0, int valid, int tid) {
    constexpr int KP = DK + 1;
    for (int e = tid; e < CH * DK / 8; e += NTH) {
        const int r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
        float x[8];
        load8<F32IN>(src, (tok0 + r) * DK + c8, r < valid, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[r * KP + c8 + j] = x[j];
    }
}

// A 64 x 64 fp32 workspace matrix into LDS (pitch 65).
__device__ __forceinline__ void load_mat(float* dst, const float* src, int tid) {
    for (int e = tid; e < CH * CH / 4; e += NTH) {
        const float4 x = reinterpret_cast<const float4*>(src)[e];
        const int r = e >> 4, c = (e & 15) * 4;
        dst[r * PT + c] = x.x;
        dst[r * PT + c + 1] = x.y;
        dst[r * PT + c + 2] = x.z;
        dst[r * PT + c + 3] = x.w;
    }
}

// Register prefetch of a chunk's q or k rows: raw values (bf16 bits or fp32),
// loaded one chunk ahead and converted when stored to LDS.  Rows past the end
// load row 0 (in bounds) and are zeroed on the store.
template <int DK, bool F32IN, int NT = NTH>
struct RowsPre {
    static constexpr int N = CH * DK / 8 / NT;
    Raw8<F32IN> x[N];
};

template <int DK, bool F32IN, int NT>
__device__ __forceinline__ void pre_rows(RowsPre<DK, F32IN, NT>& p, const void* src, size_t tok0, int valid,
                                         int tid) {
#pragma unroll
    for (int n = 0; n < RowsPre<DK, F32IN, NT>::N; ++n) {
        const int e = tid + n * NT;
        const int r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
        p.x[n] = ld_raw8<F32IN>(src, (tok0 + (r < valid ? r : 0)) * DK + c8);
    }
}

template <int DK, bool F32IN, int NT>
__device__ __forceinline__ void put_rows(const RowsPre<DK, F32IN, NT>& p, float* dst, int valid, int tid) {
    constexpr int KP = DK + 1;
#pragma unroll
    for (int n = 0; n < RowsPre<DK, F32IN, NT>::N; ++n) {
        const int e = tid + n * NT;
        const int r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
        float x[8];
        cvt_raw8<F32IN>(p.x[n], r < valid, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[r * KP + c8 + j] = x[j];
    }
}

// Register prefetch of a 64 x 64 fp32 workspace matrix.
template <int NT = NTH>
struct MatPre {
    float4 x[CH * CH / 4 / NT];
};

template <int NT>
__device__ __forceinline__ void pre_mat(MatPre<NT>& p, const float* src, int tid) {
#pragma unroll
    for (int n = 0; n < CH * CH / 4 / NT; ++n) p.x[n] = reinterpret_cast<const float4*>(src)[tid + n * NT];
}

template <int NT>
__device__ __forceinline__ void put_mat(const MatPre<NT>& p, float* dst, int tid) {
#pragma unroll
    for (int n = 0; n < CH * CH / 4 / NT; ++n) {
        const int e = tid + n * NT, r = e >> 4, c = (e & 15) * 4;
        dst[r * PT + c] = p.x[n].x;
        dst[r * PT + c + 1] = p.x[n].y;
        dst[r * PT + c + 2] = p.x[n].z;
        dst[r * PT + c + 3] = p.x[n].w;
    }
}

// Column tiles of one sequence on one XCD (workgroups are dealt round-robin
// to the 8 XCDs), so they share the chunk's operands in L2.
__device__ __forceinline__ void scan_tile(const BwdArgs& a, int& seq, int& tile) {
    const int NT = a.Dv / 16, bid = blockIdx.x;
    seq = (bid / (8 * NT)) * 8 + (bid & 7);
    tile = (bid >> 3) % NT;
}

// T = (I + A)^-1 for the strictly lower 64 x 64 A in LDS (pitch PT), written to
// sT and to Tg (64 x 64, zeros above the diagonal).  Four waves.  Diagonal
// 16 x 16 blocks by forward substitution (wave w inverts block w, lane j < 16
// owns column j); off-diagonal blocks one block row R at a time:
//   T_RI = -T_RR sum_{m in [16 I, 16 R)} A[16 R + .][m] T[m][16 I + .]
__device__ __forceinline__ void tri_inverse(const float* sA, float* sT, float (*sX)[16 * 17], float* Tg, int tid) {
    const int w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    if (l < 16) {
        const int base = 16 * w, j = l;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) s += sA[(base + r) * PT + base + i] * t[i];
            t[r] = r == j ? 1.f : (r < j ? 0.f : -s);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(base + r) * PT + base + j] = t[r];
    }
    lds_barrier();
    for (int R = 1; R < 4; ++R) {
        if (w < R) {
            const int I = w;
            f32x4 X = zero4();
            for (int s = 4 * I; s < 4 * R; ++s) {
                const int m = 4 * s + g;
                X = mfma_f32x4(sA[(16 * R + i16) * PT + m], sT[m * PT + 16 * I + i16], X);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) sX[w][(4 * g + j) * 17 + i16] = X[j];
        }
        lds_barrier();
        if (w < R) {
            const int I = w;
            f32x4 Y = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int m = 4 * s + g;
                Y = mfma_f32x4(sT[(16 * R + i16) * PT + 16 * R + m], sX[w][m * 17 + i16], Y);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) sT[(16 * R + 4 * g + j) * PT + 16 * I + i16] = -Y[j];
        }
        lds_barrier();
    }
    for (int e = tid; e < CH * CH; e += NTH) {
        const int r = e >> 6, i = e & 63;
        Tg[e] = i <= r ? sT[r * PT + i] : 0.f;
    }
}

// x as a bf16 pair, x = hi + lo to 16 significant bits (bit patterns)
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
    asm volatile("" : "+v"(x));   // one rounding for both uses of h
    const __bf16 h = (__bf16)x;
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, (__bf16)(x - (float)h));
}

// The matrix-core scans' operands of chunk slot cs (layout at kBF in
// dr_internal.h): T^ = T Diag(beta) in packed lower blocks and P^T in packed
// upper blocks, each as hi and lo planes, then gamma and lambda.  T and P are
// fp32 in LDS (pitch PT, lower blocks valid, zero above the diagonal).
__device__ void pack_scan_operands(const BwdArgs& a, const float* sT, const float* sPm, const float* sg,
                                   const float* sb, size_t cs, int tid) {
    char* base = a.wF + cs * (size_t)kBF;
    // two matrices of 10 blocks x 16 rows x 2 halves of 8 values
    for (int e = tid; e < 2 * 320; e += NTH) {
        const int mat = e / 320, pc = e - 320 * mat;
        const int b = pc >> 5, rr = (pc >> 1) & 15, hh = pc & 1;
        const int R = b >= 6 ? 3 : b >= 3 ? 2 : b >= 1 ? 1 : 0;   // lower block (R, I) at index b
        const int I = b - R * (R + 1) / 2;
        const int ch = hh ^ ((rr >> 3) & 1);                        // column half held by this piece
        uint16_t hi[8], lo[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            float x;
            if (mat == 0) {
                const int r = 16 * R + rr, c = 16 * I + 8 * ch + q;
                x = c <= r ? sT[r * PT + c] * sb[c] : 0.f;
            } else {
                // element (r, c) of the transpose, upper block (3 - R, 3 - I)
                const int r = 16 * (3 - R) + rr, c = 16 * (3 - I) + 8 * ch + q;
                x = r > c ? 0.f : sPm[c * PT + r];
            }
            split_bf16(x, hi[q], lo[q]);
        }
        const size_t at = (size_t)mat * 2 * kTriBytes + (size_t)b * 512 + rr * 32 + 16 * hh;
        uint4 vh, vl;
        vh.x = hi[0] | ((unsigned)hi[1] << 16); vh.y = hi[2] | ((unsigned)hi[3] << 16);
        vh.z = hi[4] | ((unsigned)hi[5] << 16); vh.w = hi[6] | ((unsigned)hi[7] << 16);
        vl.x = lo[0] | ((unsigned)lo[1] << 16); vl.y = lo[2] | ((unsigned)lo[3] << 16);
        vl.z = lo[4] | ((unsigned)lo[5] << 16); vl.w = lo[6] | ((unsigned)lo[7] << 16);
        *reinterpret_cast<uint4*>(base + at) = vh;
        *reinterpret_cast<uint4*>(base + at + kTriBytes) = vl;
    }
    if (tid < CH) {
        float* gr = reinterpret_cast<float*>(base + kBfGate);
        gr[tid] = expf(sg[tid]);                    // gamma_r
        gr[CH + tid] = expf(sg[CH - 1] - sg[tid]);  // lambda_r
    }
}

// --------------------------------------------------------------------- prep
template <int DK, bool F32IN>
__global__ __launch_bounds__(NTH) void bwd_prep_kernel(BwdArgs a) {
    constexpr int KP = DK + 1;
    static_assert(2 * CH * PT <= 2 * CH * KP, "A and T fit where q and k were");
    // the k and q rows (fp32 for fp32 inputs; the raw bf16 tiles for bf16
    // inputs), then (once the products are in registers) A and T, and (bf16
    // inputs) P beside them when it fits
    constexpr bool PFIT = 3 * CH * PT <= 2 * CH * KP;
    __shared__ float sKQ[2 * CH * KP];
    __shared__ float sPx[!F32IN && !PFIT ? CH * PT : 1];
    __shared__ float sX[4][16 * 17];
    __shared__ float sg[CH], sb[CH];
    float* sK = sKQ;
    float* sQ = sKQ + CH * KP;
    float* sA = sKQ;
    float* sT = sKQ + CH * PT;
    float* sPm = PFIT ? sKQ + 2 * CH * PT : sPx;
    const bool fast = !F32IN && a.wF != nullptr;
    const int cs = blockIdx.x;
    const int seq = cs / a.NC, c = cs - seq * a.NC;
    const int t0 = c * CH, valid = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const size_t mo = (size_t)cs * CH * CH;

    // bf16 inputs: the raw k and q rows as bf16 tiles (16-byte pieces
    // XOR-swizzled by row), the matrix-core operands of the products below;
    // fp32 inputs: fp32 rows
    constexpr int RB = 2 * DK;
    lchar* tK = (lchar*)sKQ;
    lchar* tQ = tK + CH * RB;
    if constexpr (F32IN) {
        load_rows<DK, F32IN>(sK, a.k, tok0, valid, tid);
        load_rows<DK, F32IN>(sQ, a.q, tok0, valid, tid);
    } else {
        static_assert(2 * CH * RB <= (int)sizeof(float) * 2 * CH * KP, "the bf16 tiles fit");
        const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + tok0 * DK);
        const uint4* qs = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + tok0 * DK);
        const uint4 z = {0u, 0u, 0u, 0u};
        for (int e = tid; e < CH * (DK / 8); e += NTH) {
            const int r = e / (DK / 8), pc = e % (DK / 8);
            const int at = r * RB + 16 * (pc ^ swz<RB>(r));
            lds_st(tK + at, r < valid ? ks[e] : z);
            lds_st(tQ + at, r < valid ? qs[e] : z);
        }
    }
    if (tid < CH) {
        const bool ok = tid < valid;
        sb[tid] = ok ? a.beta[tok0 + tid] : 0.f;
        float x = (ok && a.has_gate) ? a.log_alpha[tok0 + tid] : 0.f;
        // inclusive prefix sum over the 64 lanes of wave 0
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(x, o);
            if (l >= o) x += y;
        }
        sg[tid] = x;
        a.wG[(size_t)cs * CH + tid] = x;
    }
    lds_barrier();

    // lower blocks (R = w, I <= R) of K K^T and Q K^T, kept in registers until
    // every wave is done with the q and k rows; E applied per element
    {
        const int R = w;
        f32x4 aK[4], aQ[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            aK[I] = aQ[I] = zero4();
            if (I <= R) {
                if constexpr (F32IN) {
                    for (int s = 0; s < DK / 4; ++s) {
                        const int m = 4 * s + g;
                        const float kb = sK[(16 * I + i16) * KP + m];
                        aK[I] = mfma_f32x4(sK[(16 * R + i16) * KP + m], kb, aK[I]);
                        aQ[I] = mfma_f32x4(sQ[(16 * R + i16) * KP + m], kb, aQ[I]);
                    }
                } else {
                    // bf16 x bf16 products are exact in fp32: the 16 x 16 x 32
                    // ops on the raw tiles (rows 16 R + i16 and 16 I + i16,
                    // columns 32 s + 8 g .. + 7), same output fragments
#pragma unroll
                    for (int s = 0; s < DK / 32; ++s) {
                        const uint4 kb = lds16(tile_at<RB>(tK, 16 * I + i16, 4 * s + g));
                        aK[I] = mfma_raw<true>(lds16(tile_at<RB>(tK, 16 * R + i16, 4 * s + g)), kb, aK[I]);
                        aQ[I] = mfma_raw<true>(lds16(tile_at<RB>(tQ, 16 * R + i16, 4 * s + g)), kb, aQ[I]);
                    }
                }
            }
        }
        lds_barrier();
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * g + j, i = 16 * I + i16;
                const float e = i <= r ? __builtin_amdgcn_exp2f((sg[r] - sg[i]) * 1.4426950408889634f) : 0.f;
                const float araw = i < r ? aK[I][j] * e : 0.f;
                sA[r * PT + i] = sb[r] * araw;
                const float pv = i <= r ? aQ[I][j] * e : 0.f;
                if (fast) {
                    if (I <= R) sPm[r * PT + i] = pv;
                } else {
                    a.wA[mo + r * CH + i] = araw;
                    a.wP[mo + r * CH + i] = pv;
                }
            }
        }
    }
    lds_barrier();

    tri_inverse(sA, sT, sX, a.wT + mo, tid);
    if (fast) pack_scan_operands(a, sT, sPm, sg, sb, (size_t)cs, tid);
}

// ------------------------------------------------------- forward state scan
// Eight waves per workgroup: wave w takes the 16 rows 16 (w & 3) .. of X = K S
// over half (w >> 2) of its contraction (the upper half's partial sums pass
// through LDS), waves 0-3 form R and U, and wave w updates state rows
// 16 w .. .  The next chunk's operands are loaded into registers while the
// current one is computed; the barriers are LDS-only, so neither those loads
// nor the workspace stores are waited for inside the loop.
constexpr int SNT = 512;

template <int DK, bool F32IN>
__global__ __launch_bounds__(SNT) void bwd_fscan_kernel(BwdArgs a) {
    constexpr int KP = DK + 1, NKS = DK / 8;
    __shared__ float sK[CH * KP];
    __shared__ float sT[CH * PT];
    __shared__ float sS[DK * 17];
    __shared__ float sR[CH * 17];   // upper-half partial X, then R
    __shared__ float sU[CH * 17];
    __shared__ float sg[CH], sb[CH];
    int seq, tile;
    scan_tile(a, seq, tile);
    if (seq >= a.nseq) return;
    const int n0 = 16 * tile, Dv = a.Dv;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const int R = w & 3, h = w >> 2;

    RowsPre<DK, F32IN, SNT> pk;
    MatPre<SNT> pt;
    float pg = 0.f, pb = 0.f, pv[4] = {0.f, 0.f, 0.f, 0.f};
    auto prefetch = [&](int c) {
        const size_t cs = (size_t)seq * a.NC + c;
        const int t0 = c * CH, valid = min(CH, a.L - t0);
        const size_t tok0 = (size_t)seq * a.L + t0;
        pre_rows<DK, F32IN, SNT>(pk, a.k, tok0, valid, tid);
        pre_mat(pt, a.wT + cs * CH * CH, tid);
        if (tid < CH) {
            pg = a.wG[cs * CH + tid];
            pb = a.beta[tok0 + (tid < valid ? tid : 0)];
        }
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                pv[j] = load1<F32IN>(a.v, (tok0 + (row < valid ? row : 0)) * Dv + n0 + i16);
            }
        }
    };

    for (int e = tid; e < DK * 16; e += SNT) {
        const int d = e >> 4, cc = e & 15;
        sS[d * 17 + cc] = a.S0 ? a.S0[((size_t)seq * DK + d) * Dv + n0 + cc] : 0.f;
    }
    prefetch(0);
    for (int c = 0; c < a.NC; ++c) {
        const size_t cs = (size_t)seq * a.NC + c;
        const int t0 = c * CH, valid = min(CH, a.L - t0);
        lds_barrier();
        put_rows<DK, F32IN, SNT>(pk, sK, valid, tid);
        put_mat(pt, sT, tid);
        if (tid < CH) {
            sg[tid] = pg;
            sb[tid] = tid < valid ? pb : 0.f;
        }
        float vv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) vv[j] = 16 * R + 4 * g + j < valid ? pv[j] : 0.f;
        for (int e = tid; e < DK * 16; e += SNT) {
            const int d = e >> 4, cc = e & 15;
            a.wS[(cs * DK + d) * Dv + n0 + cc] = sS[d * 17 + cc];
        }
        lds_barrier();
        if (c + 1 < a.NC) prefetch(c + 1);
        // X = K S over this wave's half of the contraction
        f32x4 X = zero4();
#pragma unroll
        for (int s2 = 0; s2 < NKS; ++s2) {
            const int s = h * NKS + s2;
            const int m = 4 * s + g;
            X = mfma_f32x4(sK[(16 * R + i16) * KP + m], sS[m * 17 + i16], X);
        }
        if (h == 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sR[(16 * R + 4 * g + j) * 17 + i16] = X[j];
        }
        lds_barrier();
        if (h == 0) {
            // R = V - Gamma X (each lane reads its own partial sums, then overwrites them)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                const float r = vv[j] - expf(sg[row]) * (X[j] + sR[row * 17 + i16]);
                sR[row * 17 + i16] = r;
                a.wR[(cs * CH + row) * Dv + n0 + i16] = r;
            }
        }
        lds_barrier();
        const float g63 = sg[CH - 1];
        if (h == 0) {
            // U = T Diag(beta) R
            f32x4 U = zero4();
            // the factor's row 16 R + i16 is zero past the diagonal: all 16 k-steps
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                U = mfma_f32x4(sT[(16 * R + i16) * PT + m] * sb[m], sR[m * 17 + i16], U);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                a.wU[(cs * CH + row) * Dv + n0 + i16] = U[j];
                sU[row * 17 + i16] = expf(g63 - sg[row]) * U[j];
            }
        }
        lds_barrier();
        // S <- gamma_63 S + K^T Lambda U  (state rows 16 w ..)
        if (w < DK / 16) {
            const float gam63 = expf(g63);
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                acc = mfma_f32x4(sK[m * KP + 16 * w + i16], sU[m * 17 + i16], acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = 16 * w + 4 * g + j;
                sS[d * 17 + i16] = gam63 * sS[d * 17 + i16] + acc[j];
            }
        }
    }
}

// ------------------------------------------------------ reverse adjoint scan
// Eight waves, prefetched one chunk ahead (backwards) like the forward scan:
// Z = K H split over the contraction's halves, the upper-half waves also
// forming P^T dO; waves 0-3 then finish dU and dV; wave w updates H's rows
// 16 w .. .
template <int DK, bool F32IN>
__global__ __launch_bounds__(SNT) void bwd_rscan_kernel(BwdArgs a) {
    constexpr int KP = DK + 1, NKS = DK / 8;
    __shared__ float sK[CH * KP];
    __shared__ float sQ[CH * KP];
    __shared__ float sT[CH * PT];
    __shared__ float sP[CH * PT];
    __shared__ float sH[DK * 17];
    __shared__ float sO[CH * 17];   // dO, then Gamma dO
    __shared__ float sD[CH * 17];   // upper-half partial dU, then dU, then Gamma dR
    __shared__ float sgam[CH], slam[CH], sb[CH];
    int seq, tile;
    scan_tile(a, seq, tile);
    if (seq >= a.nseq) return;
    const int n0 = 16 * tile, Dv = a.Dv;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const int R = w & 3, h = w >> 2;

    RowsPre<DK, F32IN, SNT> pk, pq;
    MatPre<SNT> pt, pp;
    float pg = 0.f, pg63 = 0.f, pb = 0.f, po[4] = {0.f, 0.f, 0.f, 0.f};
    auto prefetch = [&](int c) {
        const size_t cs = (size_t)seq * a.NC + c;
        const int t0 = c * CH, valid = min(CH, a.L - t0);
        const size_t tok0 = (size_t)seq * a.L + t0;
        pre_rows<DK, F32IN, SNT>(pk, a.k, tok0, valid, tid);
        pre_rows<DK, F32IN, SNT>(pq, a.q, tok0, valid, tid);
        pre_mat(pt, a.wT + cs * CH * CH, tid);
        pre_mat(pp, a.wP + cs * CH * CH, tid);
        if (tid < CH) {
            pg = a.wG[cs * CH + tid];
            pg63 = a.wG[cs * CH + CH - 1];
            pb = a.beta[tok0 + (tid < valid ? tid : 0)];
        }
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                po[j] = a.dO[(tok0 + (row < valid ? row : 0)) * Dv + n0 + i16];
            }
        }
    };

    for (int e = tid; e < DK * 16; e += SNT) {
        const int d = e >> 4, cc = e & 15;
        sH[d * 17 + cc] = a.dS_final ? a.dS_final[((size_t)seq * DK + d) * Dv + n0 + cc] : 0.f;
    }
    prefetch(a.NC - 1);
    for (int c = a.NC - 1; c >= 0; --c) {
        const size_t cs = (size_t)seq * a.NC + c;
        const int t0 = c * CH, valid = min(CH, a.L - t0);
        const size_t tok0 = (size_t)seq * a.L + t0;
        lds_barrier();
        put_rows<DK, F32IN, SNT>(pk, sK, valid, tid);
        put_rows<DK, F32IN, SNT>(pq, sQ, valid, tid);
        put_mat(pt, sT, tid);
        put_mat(pp, sP, tid);
        if (tid < CH) {
            sgam[tid] = expf(pg);
            slam[tid] = expf(pg63 - pg);
            sb[tid] = tid < valid ? pb : 0.f;
        }
        float od[4] = {0.f, 0.f, 0.f, 0.f};
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                od[j] = row < valid ? po[j] : 0.f;
                sO[row * 17 + i16] = od[j];
            }
        }
        for (int e = tid; e < DK * 16; e += SNT) {
            const int d = e >> 4, cc = e & 15;
            a.wH[(cs * DK + d) * Dv + n0 + cc] = sH[d * 17 + cc];
        }
        lds_barrier();
        if (c > 0) prefetch(c - 1);
        // dU = P^T dO + Lambda K H  (rows 16 R ..): K H over this wave's half
        // of the contraction; the upper half also takes P^T dO
        f32x4 Z = zero4();
#pragma unroll
        for (int s2 = 0; s2 < NKS; ++s2) {
            const int s = h * NKS + s2;
            const int m = 4 * s + g;
            Z = mfma_f32x4(sK[(16 * R + i16) * KP + m], sH[m * 17 + i16], Z);
        }
        if (h == 1) {
            f32x4 Y = zero4();
            // the factor's column 16 R + i16 is zero above the diagonal: all 16 k-steps
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                Y = mfma_f32x4(sP[m * PT + 16 * R + i16], sO[m * 17 + i16], Y);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                sD[row * 17 + i16] = slam[row] * Z[j] + Y[j];
            }
        }
        lds_barrier();
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                const float du = slam[row] * Z[j] + sD[row * 17 + i16];
                sD[row * 17 + i16] = du;
                a.wdU[(cs * CH + row) * Dv + n0 + i16] = du;
            }
        }
        lds_barrier();
        // dR = Diag(beta) T^T dU
        f32x4 Rr = zero4();
        if (h == 0) {
            // the factor's column 16 R + i16 is zero above the diagonal: all 16 k-steps
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                Rr = mfma_f32x4(sT[m * PT + 16 * R + i16], sD[m * 17 + i16], Rr);
            }
        }
        const float gam63 = sgam[CH - 1];
        lds_barrier();
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                const float dr = sb[row] * Rr[j];
                if (row < valid) a.dv[(tok0 + row) * Dv + n0 + i16] = dr;
                sD[row * 17 + i16] = sgam[row] * dr;
                sO[row * 17 + i16] = sgam[row] * od[j];
            }
        }
        lds_barrier();
        // H <- gamma_63 H + Q^T Gamma dO - K^T Gamma dR  (state rows 16 w ..)
        if (w < DK / 16) {
            f32x4 hq = zero4(), hk = zero4();
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                hq = mfma_f32x4(sQ[m * KP + 16 * w + i16], sO[m * 17 + i16], hq);
                hk = mfma_f32x4(sK[m * KP + 16 * w + i16], sD[m * 17 + i16], hk);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = 16 * w + 4 * g + j;
                sH[d * 17 + i16] = gam63 * sH[d * 17 + i16] + (hq[j] - hk[j]);
            }
        }
    }
    lds_barrier();
    if (a.dS0) {
        for (int e = tid; e < DK * 16; e += SNT) {
            const int d = e >> 4, cc = e & 15;
            a.dS0[((size_t)seq * DK + d) * Dv + n0 + cc] = sH[d * 17 + cc];
        }
    }
}

// -------------------------------------------------- per-chunk gradient terms
// Eight waves: wave w takes the 16 rows 16 (w & 3) .. of every product and
// half (w >> 2) of its columns.  The state-sized operands stream through LDS
// in slabs of 32 state columns, each prefetched into registers while the
// previous slab is multiplied; the last slab's turn prefetches q, k, T, P
// and K K^T o E for the 64 x 64 part.
constexpr int PNT = 512;

template <int DK>
struct PostLds {
    static constexpr int KP = DK + 1;
    static constexpr int VS = 32;          // state columns per slab
    // slab planes: (S, H: DK rows; dO, dV, R, U, dU: 64 rows) x 32 columns x
    // (hi, lo) fp16, in floats
    static constexpr int SLAB = (2 * DK + 5 * CH) * VS;
    static constexpr int QK = 2 * CH * KP;
    static constexpr int R1 = SLAB > QK ? SLAB : QK;
};

// A slab operand in LDS: rows of 32 state columns as two fp16 planes, hi and
// lo (x ~ hi + lo, about 22 significant bits).  Row r keeps its four
// eight-column groups in the order grp ^ ((r >> 2) & 3), so that the 16 lanes
// that read one group of 16 consecutive rows fall on distinct banks.
__device__ __forceinline__ int slab_off(int r, int grp) { return r * 32 + 8 * (grp ^ ((r >> 2) & 3)); }

typedef half_t half4_t __attribute__((ext_vector_type(4)));

// Four consecutive columns c4 .. c4 + 3 (c4 a multiple of 4) of row r.
__device__ __forceinline__ void put_split4(half_t* hi, half_t* lo, int r, int c4, const float4& v) {
    const int off = slab_off(r, c4 >> 3) + (c4 & 7);
    half4_t h, l;
    half_t a, b;
    split2(v.x, a, b); h[0] = a; l[0] = b;
    split2(v.y, a, b); h[1] = a; l[1] = b;
    split2(v.z, a, b); h[2] = a; l[2] = b;
    split2(v.w, a, b); h[3] = a; l[3] = b;
    *reinterpret_cast<half4_t*>(hi + off) = h;
    *reinterpret_cast<half4_t*>(lo + off) = l;
}

// The matrix-core fragment of row r, column group grp (eight columns).
__device__ __forceinline__ Frag<2> slab_frag(const half_t* hi, const half_t* lo, int r, int grp) {
    const int off = slab_off(r, grp);
    Frag<2> f;
    f.t[0] = *reinterpret_cast<const half8*>(hi + off);
    f.t[1] = *reinterpret_cast<const half8*>(lo + off);
    return f;
}

// Sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the same column of an
// accumulator block).
// x summed over the wave's 64 lanes by shuffles (a fixed order), written to
// part[wave] by lane 0
__device__ __forceinline__ void wave_partial(float x, float* part) {
    x = group_sum<32>(x);
    x += __shfl_xor(x, 32);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
}

__device__ __forceinline__ float col4_sum(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ void st4(float* p, const float4& v) {
    p[0] = v.x; p[1] = v.y; p[2] = v.z; p[3] = v.w;
}

// Register prefetch of a chunk's [64][DK] fp32 workspace plane, stored to LDS
// rows of pitch DK + 1.
template <int DK, int NT>
struct PlanePre {
    float4 x[CH * DK / 4 / NT];
};

template <int DK, int NT>
__device__ __forceinline__ void pre_plane(PlanePre<DK, NT>& p, const float* src, int tid) {
#pragma unroll
    for (int n = 0; n < CH * DK / 4 / NT; ++n) p.x[n] = reinterpret_cast<const float4*>(src)[tid + n * NT];
}

template <int DK, int NT>
__device__ __forceinline__ void put_plane(const PlanePre<DK, NT>& p, float* dst, int tid) {
    constexpr int KP = DK + 1;
#pragma unroll
    for (int n = 0; n < CH * DK / 4 / NT; ++n) {
        const int e = tid + n * NT, r = e / (DK / 4), c = (e % (DK / 4)) * 4;
        dst[r * KP + c] = p.x[n].x;
        dst[r * KP + c + 1] = p.x[n].y;
        dst[r * KP + c + 2] = p.x[n].z;
        dst[r * KP + c + 3] = p.x[n].w;
    }
}

// The state-sized products of the per-chunk gradient kernel, over slabs of VS
// state columns on the fp16 matrix cores with two-term operands (three
// products per pair, lo * lo dropped):
//   z1 = dO S^T, z2 = dR S^T, z3 = U H^T   (rows 16 R .., column blocks D0 ..)
//   acc = dO U^T (hf 0) or dU R^T (hf 1)   (rows 16 R .., column blocks I <= R)
// and <H, S>: summed into shs[0], or per state row into shs[d] (CG).  The
// last slab's turn prefetches T, P, K K^T (and, for bf16 inputs without a
// channel gate, the q and k rows; with one, the gated Kc and Q^ rows) for the
// 64 x 64 part.
template <int DK, bool F32IN, bool CG>
__device__ __forceinline__ void post_state_products(const BwdArgs& a, int cs, int valid, size_t tok0, float* s1,
                                                    f32x4 (&z1)[DK / 32], f32x4 (&z2)[DK / 32], f32x4 (&z3)[DK / 32],
                                                    f32x4 (&acc)[4], float* shs, RowsPre<DK, F32IN, PNT>& pk,
                                                    RowsPre<DK, F32IN, PNT>& pq, MatPre<PNT>& pt, MatPre<PNT>& pp,
                                                    MatPre<PNT>& pa, PlanePre<DK, PNT>* pkc = nullptr,
                                                    PlanePre<DK, PNT>* pqh = nullptr) {
    using Lp = PostLds<DK>;
    constexpr int VS = Lp::VS, NDH = DK / 32;
    constexpr int NS = DK * VS / 4 / PNT;   // float4 of S (and of H) per thread and slab
    static_assert(CH * VS / 4 == PNT, "one float4 of each 64-row slab per thread");
    const int Dv = a.Dv;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const int R = w & 3, hf = w >> 2, D0 = hf * NDH;
    const size_t mo = (size_t)cs * CH * CH;
    // ---- slab prefetch registers
    float4 ps[NS], ph[NS], po, pd, pr, pu, pdu;
    auto pre_slab = [&](int v0) {
        const int vw = min(VS, Dv - v0);   // 16 or 32
        const float4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const int e = tid + n * PNT, d = e / (VS / 4), c4 = (e % (VS / 4)) * 4;
            ps[n] = ph[n] = z;
            if (c4 < vw) {
                const size_t off = ((size_t)cs * DK + d) * Dv + v0 + c4;
                ps[n] = *reinterpret_cast<const float4*>(a.wS + off);
                ph[n] = *reinterpret_cast<const float4*>(a.wH + off);
            }
        }
        const int r = tid / (VS / 4), c4 = (tid % (VS / 4)) * 4;
        po = pd = pr = pu = pdu = z;
        if (c4 < vw) {
            const size_t wo = ((size_t)cs * CH + r) * Dv + v0 + c4;
            pr = *reinterpret_cast<const float4*>(a.wR + wo);
            pu = *reinterpret_cast<const float4*>(a.wU + wo);
            pdu = *reinterpret_cast<const float4*>(a.wdU + wo);
            const size_t io = (tok0 + (r < valid ? r : 0)) * Dv + v0 + c4;
            po = *reinterpret_cast<const float4*>(a.dO + io);
            pd = *reinterpret_cast<const float4*>(a.dv + io);
        }
    };
    // ---- state terms over slabs of VS state columns, on the fp16 matrix cores
    // with two-term operands (three products per pair, lo * lo dropped):
    //   z1 = dO S^T, z2 = dR S^T, z3 = U H^T   (rows 16 R .., column blocks D0 ..)
    //   acc = dO U^T (hf 0) or dU R^T (hf 1)   (rows 16 R .., column blocks I <= R)
#pragma unroll
    for (int D = 0; D < NDH; ++D) z1[D] = z2[D] = z3[D] = zero4();
#pragma unroll
    for (int I = 0; I < 4; ++I) acc[I] = zero4();
    float hs = 0.f;
    float hsr[NS] = {};   // CG: <H, S> of this thread's state row in each of its NS pieces, over the slabs
    half_t* sSh = reinterpret_cast<half_t*>(s1);
    half_t* sSl = sSh + DK * VS;
    half_t* sHh = sSl + DK * VS;
    half_t* sHl = sHh + DK * VS;
    half_t* sOh = sHl + DK * VS;
    half_t* sOl = sOh + CH * VS;
    half_t* sRh = sOl + CH * VS;
    half_t* sRl = sRh + CH * VS;
    half_t* sUh = sRl + CH * VS;
    half_t* sUl = sUh + CH * VS;
    half_t* sdUh = sUl + CH * VS;
    half_t* sdUl = sdUh + CH * VS;
    half_t* sdRh = sdUl + CH * VS;
    half_t* sdRl = sdRh + CH * VS;
    pre_slab(0);
    for (int v0 = 0; v0 < Dv; v0 += VS) {
        lds_barrier();
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const int e = tid + n * PNT, d = e / (VS / 4), c4 = (e % (VS / 4)) * 4;
            const float hsn = ps[n].x * ph[n].x + ps[n].y * ph[n].y + ps[n].z * ph[n].z + ps[n].w * ph[n].w;
            if constexpr (CG) hsr[n] += hsn;
            else hs += hsn;
            put_split4(sSh, sSl, d, c4, ps[n]);
            put_split4(sHh, sHl, d, c4, ph[n]);
        }
        {
            const int r = tid / (VS / 4), c4 = (tid % (VS / 4)) * 4;
            const float4 z = {0.f, 0.f, 0.f, 0.f};
            put_split4(sOh, sOl, r, c4, r < valid ? po : z);
            put_split4(sdRh, sdRl, r, c4, r < valid ? pd : z);
            put_split4(sRh, sRl, r, c4, pr);
            put_split4(sUh, sUl, r, c4, pu);
            put_split4(sdUh, sdUl, r, c4, pdu);
        }
        lds_barrier();
        if (v0 + VS < Dv) {
            pre_slab(v0 + VS);
        } else {
            if constexpr (!F32IN && !CG) {   // fp32 rows would not fit the register budget
                pre_rows<DK, F32IN, PNT>(pk, a.k, tok0, valid, tid);
                pre_rows<DK, F32IN, PNT>(pq, a.q, tok0, valid, tid);
            }
            pre_mat(pt, a.wT + mo, tid);
            pre_mat(pp, a.wP + mo, tid);
            pre_mat(pa, a.wA + mo, tid);
            if constexpr (CG) {   // the gated Kc and Q^ rows
                pre_plane(*pkc, a.wKc + (size_t)cs * CH * DK, tid);
                pre_plane(*pqh, a.wQh + (size_t)cs * CH * DK, tid);
            }
        }
        const int ra = 16 * R + i16;
        const Frag<2> fo = slab_frag(sOh, sOl, ra, g);
        const Frag<2> fr = slab_frag(sdRh, sdRl, ra, g);
        const Frag<2> fu = slab_frag(sUh, sUl, ra, g);
#pragma unroll
        for (int D = 0; D < NDH; ++D) {
            const Frag<2> fs = slab_frag(sSh, sSl, 16 * (D0 + D) + i16, g);
            const Frag<2> fh = slab_frag(sHh, sHl, 16 * (D0 + D) + i16, g);
            z1[D] = mma<2, 2>(fo, fs, z1[D]);
            z2[D] = mma<2, 2>(fr, fs, z2[D]);
            z3[D] = mma<2, 2>(fu, fh, z3[D]);
        }
        if (hf == 0) {
#pragma unroll
            for (int I = 0; I < 4; ++I)
                if (I <= R) acc[I] = mma<2, 2>(fo, slab_frag(sUh, sUl, 16 * I + i16, g), acc[I]);
        } else {
            const Frag<2> fdu = slab_frag(sdUh, sdUl, ra, g);
#pragma unroll
            for (int I = 0; I < 4; ++I)
                if (I <= R) acc[I] = mma<2, 2>(fdu, slab_frag(sRh, sRl, 16 * I + i16, g), acc[I]);
        }
    }
    if constexpr (CG) {
        // the VS / 4 consecutive lanes of a state row summed by shuffles (a
        // fixed order), written once per row
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const float x = group_sum<VS / 4>(hsr[n]);
            if (tid % (VS / 4) == 0) shs[(tid + n * PNT) / (VS / 4)] = x;
        }
    } else {
        wave_partial(hs, shs);
    }
}

// Where piece `piece` of row r of a swizzled tile is written (as tile_at).
template <int RB>
__device__ __forceinline__ lchar* tile_st(lchar* tile, int r, int piece) {
    return tile + r * RB + 16 * (piece ^ swz<RB>(r));
}

// bf16 hi + lo pair of a 16-byte fragment (eight values)
struct BF2 {
    uint4 h, l;
};

// c += a b for split a and b: hi hi + hi lo + lo hi
__device__ __forceinline__ f32x4 mma3(const BF2& a, const BF2& b, f32x4 c) {
    c = mfma_raw<true>(a.h, b.h, c);
    c = mfma_raw<true>(a.h, b.l, c);
    return mfma_raw<true>(a.l, b.h, c);
}

// Four consecutive fp32 values (columns c4 .. c4 + 3 of row r) into a bf16 hi
// and lo slab plane pair (the slab_off layout, byte planes).
__device__ __forceinline__ void put_split4_bf(lchar* hi, lchar* lo, int r, int c4, const float4& v) {
    const int off = 2 * (slab_off(r, c4 >> 3) + (c4 & 7));
    uint16_t h[4], o[4];
    split_bf16(v.x, h[0], o[0]);
    split_bf16(v.y, h[1], o[1]);
    split_bf16(v.z, h[2], o[2]);
    split_bf16(v.w, h[3], o[3]);
    uint2 vh, vl;
    vh.x = h[0] | ((unsigned)h[1] << 16); vh.y = h[2] | ((unsigned)h[3] << 16);
    vl.x = o[0] | ((unsigned)o[1] << 16); vl.y = o[2] | ((unsigned)o[3] << 16);
    lds_st(hi + off, vh);
    lds_st(lo + off, vl);
}

// One value into a bf16 hi and lo slab plane pair.
__device__ __forceinline__ void put_split1_bf(lchar* hi, lchar* lo, int r, int c, float x) {
    const int off = 2 * (slab_off(r, c >> 3) + (c & 7));
    uint16_t h, o;
    split_bf16(x, h, o);
    lds_st(hi + off, h);
    lds_st(lo + off, o);
}

// Row fragment of a slab plane pair: row r, columns 8 grp .. +7.
__device__ __forceinline__ BF2 slab_row(const lchar* hi, const lchar* lo, int r, int grp) {
    const int off = 2 * slab_off(r, grp);
    return {lds16(hi + off), lds16(lo + off)};
}

// Column fragment of one slab plane (the B operand of a contraction over its
// rows): lane (i16, g) receives column c0 + i16 at rows 32 s + 8 g .. +7,
// through the transposing LDS read.
__device__ __forceinline__ uint4 slab_col(const lchar* pl, int c0, int s, int i16, int g) {
    const int r = 32 * s + 8 * g + (i16 >> 2);
    const int c = c0 + 4 * (i16 & 3);
    const uint2 lo4 = lds_tr4(pl + 2 * (slab_off(r, c >> 3) + (c & 7)));
    const uint2 hi4 = lds_tr4(pl + 2 * (slab_off(r + 4, c >> 3) + (c & 7)));
    return {lo4.x, lo4.y, hi4.x, hi4.y};
}

// The per-chunk kernel's state products for bf16 inputs without a channel
// gate.  R and U are not read back: per slab of VS state columns they are
// formed here, R = V - Gamma K S (rows past the end zero) and U = T^ R, with k
// exact and S, R, T^ as bf16 hi + lo; then
//   z1 = dO S^T, z2 = dR S^T, z3 = U H^T   (rows 16 R .., column blocks D0 ..)
//   acc = dO U^T (hf 0) or dU R^T (hf 1)   (rows 16 R .., column blocks I <= R)
// and <H, S> into shs[0], every slab operand a bf16 hi + lo pair.  The chunk's
// k tile and T^ (packed lower, hi and lo) arrive with the first slab, into
// tKs and tTs; the slab planes are in `slab`.  The last slab's turn prefetches
// T, the packed P^T (hi and lo: pieces tid < 320 into ppk) and the q rows for
// the 64 x 64 part (the k rows stay in tKs).
template <int DK>
__device__ __forceinline__ void post_slabs_rc(const BwdArgs& a, int cs, size_t ss, int valid, size_t tok0, lchar* slab,
                                              lchar* tKs, lchar* tTs, const float* sgam,
                                              f32x4 (&z1)[DK / 32], f32x4 (&z2)[DK / 32], f32x4 (&z3)[DK / 32],
                                              f32x4 (&acc)[4], float* shs, RowsPre<DK, false, PNT>& pq,
                                              MatPre<PNT>& pt, uint4 (&ppk)[2]) {
    constexpr int VS = PostLds<DK>::VS, NDH = DK / 32, RB = 2 * DK;
    constexpr int NS = DK * VS / 4 / PNT;   // float4 of S (and of H) per thread and slab
    static_assert(CH * VS / 4 == PNT, "one float4 of each 64-row slab per thread");
    constexpr int PS = DK * VS * 2, PT6 = CH * VS * 2;   // bytes of an S / H plane and of a 64-row plane
    const int Dv = a.Dv;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const int R = w & 3, hf = w >> 2, D0 = hf * NDH;
    const size_t mo = (size_t)cs * CH * CH;
    lchar* sSh = slab;
    lchar* sSl = sSh + PS;
    lchar* sHh = sSl + PS;
    lchar* sHl = sHh + PS;
    lchar* sOh = sHl + PS;
    lchar* sOl = sOh + PT6;
    lchar* sRh = sOl + PT6;
    lchar* sRl = sRh + PT6;
    lchar* sUh = sRl + PT6;
    lchar* sUl = sUh + PT6;
    lchar* sdUh = sUl + PT6;
    lchar* sdUl = sdUh + PT6;
    lchar* sdRh = sdUl + PT6;
    lchar* sdRl = sdRh + PT6;
    // this wave's block of R and U: rows 16 R .., slab columns 16 hf ..
    const int rrow = 16 * R + 4 * g;
    // ---- prefetch registers: S, H, dO, dR, dU of a slab, V at this lane's R
    // entries, and with the first slab the k tile and T^
    float4 ps[NS], ph[NS], po, pd, pdu;
    uint16_t pv[4];
    uint4 kt[2], tt[2];
    auto pre_slab = [&](int v0) {
        const int vw = min(VS, Dv - v0);   // 16 or 32
        const float4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const int e = tid + n * PNT, d = e / (VS / 4), c4 = (e % (VS / 4)) * 4;
            ps[n] = ph[n] = z;
            if (c4 < vw) {
                const size_t off = (ss * DK + d) * Dv + v0 + c4;
                ps[n] = *reinterpret_cast<const float4*>(a.wS + off);
                ph[n] = *reinterpret_cast<const float4*>(a.wH + off);
            }
        }
        const int r = tid / (VS / 4), c4 = (tid % (VS / 4)) * 4;
        po = pd = pdu = z;
        if (c4 < vw) {
            pdu = *reinterpret_cast<const float4*>(a.wdU + (ss * CH + r) * Dv + v0 + c4);
            const size_t io = (tok0 + (r < valid ? r : 0)) * Dv + v0 + c4;
            po = *reinterpret_cast<const float4*>(a.dO + io);
            pd = *reinterpret_cast<const float4*>(a.dv + io);
        }
        const int vc = 16 * hf + i16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = rrow + j;
            pv[j] = vc < vw ? static_cast<const uint16_t*>(a.v)[(tok0 + (rr < valid ? rr : 0)) * Dv + v0 + vc] : 0;
        }
    };
#pragma unroll
    for (int D = 0; D < NDH; ++D) z1[D] = z2[D] = z3[D] = zero4();
#pragma unroll
    for (int I = 0; I < 4; ++I) acc[I] = zero4();
    float hs = 0.f;
    {
        // the k tile (64 x DK bf16) and T^ (two 5 KiB planes), 16 bytes per piece
        const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + tok0 * DK);
        const uint4* ts = reinterpret_cast<const uint4*>(a.wF + (size_t)cs * kBF);
        const uint4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int e = tid + n * PNT;                    // piece: row e / (DK / 8), 16 bytes
            const int r = e / (DK / 8);
            kt[n] = e < CH * DK / 8 ? ks[(size_t)(r < valid ? r : 0) * (DK / 8) + e % (DK / 8)] : z;
            tt[n] = e < 2 * kTriBytes / 16 ? ts[e] : z;
        }
    }
    pre_slab(0);
    for (int v0 = 0; v0 < Dv; v0 += VS) {
        const int vw = min(VS, Dv - v0);
        lds_barrier();
        if (v0 == 0) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int e = tid + n * PNT;
                if (e < CH * DK / 8) {
                    const int r = e / (DK / 8), pc = e % (DK / 8);
                    const uint4 z = {0u, 0u, 0u, 0u};
                    lds_st(tile_st<RB>(tKs, r, pc), r < valid ? kt[n] : z);
                }
                if (e < 2 * kTriBytes / 16) lds_st(tTs + 16 * e, tt[n]);
            }
        }
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const int e = tid + n * PNT, d = e / (VS / 4), c4 = (e % (VS / 4)) * 4;
            hs += ps[n].x * ph[n].x + ps[n].y * ph[n].y + ps[n].z * ph[n].z + ps[n].w * ph[n].w;
            put_split4_bf(sSh, sSl, d, c4, ps[n]);
            put_split4_bf(sHh, sHl, d, c4, ph[n]);
        }
        float vv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) vv[j] = bf16_to_f32(pv[j]);
        {
            const int r = tid / (VS / 4), c4 = (tid % (VS / 4)) * 4;
            const float4 z = {0.f, 0.f, 0.f, 0.f};
            put_split4_bf(sOh, sOl, r, c4, r < valid ? po : z);
            put_split4_bf(sdRh, sdRl, r, c4, r < valid ? pd : z);
            put_split4_bf(sdUh, sdUl, r, c4, pdu);
        }
        lds_barrier();
        if (v0 + VS < Dv) {
            pre_slab(v0 + VS);
        } else {
            pre_rows<DK, false, PNT>(pq, a.q, tok0, valid, tid);
            pre_mat(pt, a.wT + mo, tid);
            if (tid < kTriBytes / 16) {
                const uint4* pk2 = reinterpret_cast<const uint4*>(a.wF + (size_t)cs * kBF + kBfPt);
                ppk[0] = pk2[tid];
                ppk[1] = pk2[kTriBytes / 16 + tid];
            }
        }
        // R = V - Gamma K S: this wave's block (rows 16 R .., columns 16 hf ..)
        {
            f32x4 X = zero4();
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                const uint4 kf = lds16(tile_at<RB>(tKs, 16 * R + i16, 4 * s + g));
                X = mfma_raw<true>(kf, slab_col(sSh, 16 * hf, s, i16, g), X);
                X = mfma_raw<true>(kf, slab_col(sSl, 16 * hf, s, i16, g), X);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = rrow + j, c = 16 * hf + i16;
                const float rv = r < valid && c < vw ? vv[j] - sgam[r] * X[j] : 0.f;
                put_split1_bf(sRh, sRl, r, c, rv);
            }
        }
        lds_barrier();
        // U = T^ R
        {
            f32x4 U = zero4();
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int I = 2 * s + (g >> 1);
                const int Ic = I <= R ? I : R;
                const int off = tri_block(R, Ic) * 512 + i16 * 32 + 16 * ((g & 1) ^ ((i16 >> 3) & 1));
                const uint32_t m = I <= R ? ~0u : 0u;
                uint4 th = lds16(tTs + off), tl = lds16(tTs + kTriBytes + off);
                th.x &= m; th.y &= m; th.z &= m; th.w &= m;
                tl.x &= m; tl.y &= m; tl.z &= m; tl.w &= m;
                const BF2 rb = {slab_col(sRh, 16 * hf, s, i16, g), slab_col(sRl, 16 * hf, s, i16, g)};
                U = mma3({th, tl}, rb, U);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) put_split1_bf(sUh, sUl, rrow + j, 16 * hf + i16, U[j]);
        }
        lds_barrier();
        const int ra = 16 * R + i16;
        const BF2 fo = slab_row(sOh, sOl, ra, g);
        const BF2 fr = slab_row(sdRh, sdRl, ra, g);
        const BF2 fu = slab_row(sUh, sUl, ra, g);
#pragma unroll
        for (int D = 0; D < NDH; ++D) {
            const BF2 fs = slab_row(sSh, sSl, 16 * (D0 + D) + i16, g);
            const BF2 fh = slab_row(sHh, sHl, 16 * (D0 + D) + i16, g);
            z1[D] = mma3(fo, fs, z1[D]);
            z2[D] = mma3(fr, fs, z2[D]);
            z3[D] = mma3(fu, fh, z3[D]);
        }
        if (hf == 0) {
#pragma unroll
            for (int I = 0; I < 4; ++I)
                if (I <= R) acc[I] = mma3(fo, slab_row(sUh, sUl, 16 * I + i16, g), acc[I]);
        } else {
            const BF2 fdu = slab_row(sdUh, sdUl, ra, g);
#pragma unroll
            for (int I = 0; I < 4; ++I)
                if (I <= R) acc[I] = mma3(fdu, slab_row(sRh, sRl, 16 * I + i16, g), acc[I]);
        }
    }
    wave_partial(hs, shs);
}

// bf16 rows prefetched by pre_rows into a swizzled [64][2 DK]-byte tile (rows
// at or past `valid` zeroed), the layout of the matrix-core scans' tiles.
template <int DK, int NT>
__device__ __forceinline__ void put_rows_tile(const RowsPre<DK, false, NT>& p, lchar* tile, int valid, int tid) {
#pragma unroll
    for (int n = 0; n < RowsPre<DK, false, NT>::N; ++n) {
        const int e = tid + n * NT;
        const int r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
        const uint4 z = {0u, 0u, 0u, 0u};
        lds_st(tile_st<2 * DK>(tile, r, c8 >> 3), r < valid ? p.x[n].x : z);
    }
}

// Element (r, col) of such a tile.
template <int DK>
__device__ __forceinline__ float tile_val(const lchar* tile, int r, int col) {
    return bf16_to_f32(lds_ld<uint16_t>(tile_at<2 * DK>(tile, r, col >> 3) + 2 * (col & 7)));
}

// The K^T-style fragment of a row-major 16-bit tile (RB bytes per row):
// lane (i16, g) receives column c0 + i16 at rows 32 s + 8 g .. +7, i.e. the A
// operand of (tile^T) rows c0 .. or the B operand of tile columns c0 ..
template <int RB>
__device__ __forceinline__ uint4 tr_frag(const lchar* tile, int c0, int s, int i16, int g) {
    const int tok = 32 * s + 8 * g + (i16 >> 2);
    const int d = c0 + 4 * (i16 & 3);
    const uint2 lo4 = lds_tr4(tile_at<RB>(tile, tok, d >> 3) + 2 * (d & 7));
    const uint2 hi4 = lds_tr4(tile_at<RB>(tile, tok + 4, d >> 3) + 2 * (d & 7));
    return {lo4.x, lo4.y, hi4.x, hi4.y};
}

template <int DK, bool F32IN>
__global__ __launch_bounds__(PNT) void bwd_post_kernel(BwdArgs a) {
    using Lp = PostLds<DK>;
    constexpr int KP = Lp::KP, ND = DK / 16, NDH = ND / 2;
    // bf16 inputs: the q and k rows as bf16 tiles, then N and M as bf16 hi + lo tiles
    constexpr int RB = 2 * DK, TB = CH * RB, MB = CH * 128;
    static_assert(F32IN || 2 * TB + 4 * MB <= (int)sizeof(float) * Lp::R1, "tiles fit the slab area");
    __shared__ __attribute__((aligned(16))) float s1[Lp::R1];
    // bf16 inputs: sM0 and sM1 hold the k tile and T^ during the slabs
    __shared__ __attribute__((aligned(16))) float sM0[CH * PT];   // T
    __shared__ __attribute__((aligned(16))) float sM1[CH * PT];   // P, then M = Diag(beta) (dA o E)
    __shared__ float sM2[CH * PT];   // K K^T o E (strict lower)
    __shared__ float sM3[CH * PT];   // N = dP o E
    __shared__ float sM4[CH * PT];   // dT^ Diag(beta), then T^T of it
    __shared__ float sg[CH], sgam[CH], slam[CH], sb[CH];
    __shared__ float shs[PNT / 64];   // <H, S>: one partial per wave
    // chunk c0 + (bid mod cN) of sequence bid / cN; S_c, H_c and dU in slot ss
    const int seq = blockIdx.x / a.cN, c = a.c0 + (blockIdx.x - seq * a.cN);
    const int cs = seq * a.NC + c;
    const size_t ss = (size_t)seq * a.sC + c % a.sC;
    const int t0 = c * CH, valid = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const int Dv = a.Dv;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const int R = w & 3, hf = w >> 2, D0 = hf * NDH;
    const size_t mo = (size_t)cs * CH * CH;

    if (tid < CH) {
        const float* gp = a.wG + (size_t)cs * CH;
        const float gv = gp[tid], g63 = gp[CH - 1];
        sg[tid] = gv;
        sgam[tid] = expf(gv);
        slam[tid] = expf(g63 - gv);
        sb[tid] = tid < valid ? a.beta[tok0 + tid] : 0.f;
    }

    RowsPre<DK, F32IN, PNT> pk, pq;
    MatPre<PNT> pt, pp, pa;
    uint4 ppk[2] = {};   // bf16 inputs: the packed P^T (hi, lo), pieces tid < 320
    f32x4 z1[NDH], z2[NDH], z3[NDH], acc[4];
    if constexpr (F32IN) {
        // one slot per chunk on this path (sC == NC, so ss == cs)
        post_state_products<DK, F32IN, false>(a, cs, valid, tok0, s1, z1, z2, z3, acc, shs, pk, pq, pt, pp, pa);
    } else {
        static_assert(F32IN || CH * 2 * DK <= (int)sizeof(float) * CH * PT, "the k tile fits sM0");
        static_assert(F32IN || 2 * kTriBytes <= (int)sizeof(float) * CH * PT, "T^ fits sM1");
        post_slabs_rc<DK>(a, cs, ss, valid, tok0, (lchar*)s1, (lchar*)sM0, (lchar*)sM1, sgam, z1, z2, z3, acc, shs, pq,
                          pt, ppk);
    }
    lds_barrier();

    // ---- q, k rows and the 64 x 64 matrices
    float* sK = s1;
    float* sQ = s1 + CH * KP;
    lchar* tK = (lchar*)s1;
    lchar* tQ = tK + TB;
    if constexpr (F32IN) {
        for (int e = tid; e < CH * DK / 8; e += PNT) {
            const int r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
            float x[8];
            load8<F32IN>(a.k, (tok0 + r) * DK + c8, r < valid, x);
#pragma unroll
            for (int j = 0; j < 8; ++j) sK[r * KP + c8 + j] = x[j];
            load8<F32IN>(a.q, (tok0 + r) * DK + c8, r < valid, x);
#pragma unroll
            for (int j = 0; j < 8; ++j) sQ[r * KP + c8 + j] = x[j];
        }
    } else {
        // the k tile from where the slabs used it (sM0, in the same layout),
        // before T takes that space
        for (int e = tid; e < TB / 16; e += PNT) lds_st(tK + 16 * e, lds16((const lchar*)sM0 + 16 * e));
        put_rows_tile<DK, PNT>(pq, tQ, valid, tid);
        lds_barrier();
    }
    put_mat(pt, sM0, tid);
    if constexpr (F32IN) {
        put_mat(pp, sM1, tid);
        put_mat(pa, sM2, tid);
    } else {
        // P from the packed P^T (hi + lo): piece tid of each plane holds row
        // rr of upper block (3 - Rb, 3 - Ib), columns 8 ch .. +7, i.e. P at
        // those columns' rows and that row's column; zero above P's diagonal
        // blocks
        if (tid < kTriBytes / 16) {
            const int b = tid >> 5, rr = (tid >> 1) & 15, hh = tid & 1;
            const int Rb = b >= 6 ? 3 : b >= 3 ? 2 : b >= 1 ? 1 : 0, Ib = b - Rb * (Rb + 1) / 2;
            const int ch = hh ^ ((rr >> 3) & 1);
            const int pr = 16 * (3 - Rb) + rr, pc0 = 16 * (3 - Ib) + 8 * ch;   // P^T row, first column
            const uint32_t hw[4] = {ppk[0].x, ppk[0].y, ppk[0].z, ppk[0].w};
            const uint32_t lw[4] = {ppk[1].x, ppk[1].y, ppk[1].z, ppk[1].w};
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float x = bf16_to_f32((uint16_t)(hw[q >> 1] >> (16 * (q & 1)))) +
                                bf16_to_f32((uint16_t)(lw[q >> 1] >> (16 * (q & 1))));
                sM1[(pc0 + q) * PT + pr] = x;
            }
        }
        for (int e = tid; e < 6 * 256; e += PNT) {   // the six blocks above the diagonal
            const int ub = e >> 8, rb = ub >= 5 ? 2 : ub >= 3 ? 1 : 0;   // (0,1..3) (1,2..3) (2,3)
            const int ib = rb == 0 ? ub + 1 : rb == 1 ? ub - 1 : 3;
            sM1[(16 * rb + ((e >> 4) & 15)) * PT + 16 * ib + (e & 15)] = 0.f;
        }
        // K K^T o E, strictly lower, from the k tile: row block R, column
        // blocks 2 hf, 2 hf + 1 (zero above the diagonal blocks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int I = 2 * hf + h;
            f32x4 ak = zero4();
            if (I <= R) {
#pragma unroll
                for (int s = 0; s < DK / 32; ++s)
                    ak = mfma_raw<true>(lds16(tile_at<RB>(tK, 16 * R + i16, 4 * s + g)),
                                        lds16(tile_at<RB>(tK, 16 * I + i16, 4 * s + g)), ak);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * g + j, i = 16 * I + i16;
                const float ee = __builtin_amdgcn_exp2f((sg[r] - sg[i]) * 1.4426950408889634f);
                sM2[r * PT + i] = I <= R && i < r ? ak[j] * ee : 0.f;
            }
        }
    }
    lds_barrier();

    const int rb = 16 * R + 4 * g;   // this lane's first accumulator row
    float rowg[4] = {0.f, 0.f, 0.f, 0.f}, rowb[4] = {0.f, 0.f, 0.f, 0.f};
    float colg[4] = {0.f, 0.f, 0.f, 0.f}, colb[4] = {0.f, 0.f, 0.f, 0.f};
    float g63part = 0.f;
    // state terms: dq = Gamma z1, dk = -Gamma z2 + Lambda z3
    f32x4 dq[NDH], dk[NDH];
#pragma unroll
    for (int D = 0; D < NDH; ++D) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = rb + j, col = 16 * (D0 + D) + i16;
            const float qv = F32IN ? sQ[r * KP + col] : tile_val<DK>(tQ, r, col);
            const float kv = F32IN ? sK[r * KP + col] : tile_val<DK>(tK, r, col);
            const float x1 = sgam[r] * z1[D][j];
            const float x2 = -sgam[r] * z2[D][j];
            const float x3 = slam[r] * z3[D][j];
            dq[D][j] = x1;
            dk[D][j] = x2 + x3;
            rowg[j] += qv * x1 + kv * x2 - kv * x3;
            g63part += kv * x3;
        }
    }
    // hf 0: dP -> N = dP o E (lower) and the sums of dP o P;
    // hf 1: dT^ -> dT = dT^ Diag(beta), and dbeta's column sums of dT^ o T
#pragma unroll
    for (int I = 0; I < 4; ++I) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = rb + j, i = 16 * I + i16;
            const bool lo = i <= r;
            const float x = lo ? acc[I][j] : 0.f;
            if (hf == 0) {
                const float pd_ = x * sM1[r * PT + i];
                rowg[j] += pd_;
                colg[I] -= pd_;
                sM3[r * PT + i] = lo ? x * __builtin_amdgcn_exp2f((sg[r] - sg[i]) * 1.4426950408889634f) : 0.f;
            } else {
                colb[I] += x * sM0[r * PT + i];
                sM4[r * PT + i] = x * sb[i];
            }
        }
    }
    lds_barrier();
    // Y = T^T dT  (rows 16 R .., column blocks 2 hf, 2 hf + 1).  T holds exact
    // zeros above its diagonal (T[m][a] = 0 for m < a), so the contraction runs
    // over all 64 rows m with a fixed trip count: every operand read is issued
    // ahead of the products instead of one LDS round trip per k-step.
    f32x4 y[2] = {zero4(), zero4()};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const int m = 4 * s + g;
        const float tv = sM0[m * PT + 16 * R + i16];
#pragma unroll
        for (int h = 0; h < 2; ++h) y[h] = mfma_f32x4(tv, sM4[m * PT + 16 * (2 * hf + h) + i16], y[h]);
    }
    lds_barrier();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) sM4[(rb + j) * PT + 16 * (2 * hf + h) + i16] = y[h][j];
    lds_barrier();
    // dA = -Y T^T on the strict lower part, then M = Diag(beta) (dA o E) into
    // sM1 (P is no longer read).  T[c][m] = 0 for m > c: the contraction runs
    // over all 64 m with a fixed trip count, as for Y.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int I = 2 * hf + h;
        f32x4 da = zero4();
        if (I <= R) {
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                da = mfma_f32x4(sM4[(16 * R + i16) * PT + m], sM0[(16 * I + i16) * PT + m], da);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = rb + j, cc = 16 * I + i16;
            const bool lo = cc < r;
            const float dav = lo ? -da[j] : 0.f;
            const float adr = dav * sM2[r * PT + cc];
            rowb[j] += adr;
            const float ad = sb[r] * adr;
            rowg[j] += ad;
            colg[I] -= ad;
            sM1[r * PT + cc] = lo ? dav * sb[r] * __builtin_amdgcn_exp2f((sg[r] - sg[cc]) * 1.4426950408889634f) : 0.f;
        }
    }
    lds_barrier();
    // dq += N K;  dk += M K + N^T Q + M^T K
    if constexpr (!F32IN) {
        // on the bf16 matrix cores: N and M as hi + lo tiles (N at tN, M at
        // tN + 2 MB), q and k exact; the products over all 64 tokens (N and M
        // vanish outside their triangles)
        lchar* tN = tQ + TB;
        for (int e = tid; e < 2 * CH * 8; e += PNT) {
            const int mat = e >> 9, r = (e >> 3) & 63, pc = e & 7;
            const float* src = (mat ? sM1 : sM3) + r * PT + 8 * pc;
            uint16_t hi[8], lo[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) split_bf16(src[q], hi[q], lo[q]);
            uint4 vh, vl;
            vh.x = hi[0] | ((unsigned)hi[1] << 16); vh.y = hi[2] | ((unsigned)hi[3] << 16);
            vh.z = hi[4] | ((unsigned)hi[5] << 16); vh.w = hi[6] | ((unsigned)hi[7] << 16);
            vl.x = lo[0] | ((unsigned)lo[1] << 16); vl.y = lo[2] | ((unsigned)lo[3] << 16);
            vl.z = lo[4] | ((unsigned)lo[5] << 16); vl.w = lo[6] | ((unsigned)lo[7] << 16);
            lchar* t = tN + mat * 2 * MB;
            lds_st(tile_st<128>(t, r, pc), vh);
            lds_st(tile_st<128>(t + MB, r, pc), vl);
        }
        lds_barrier();
        uint4 nf[2][2], mf[2][2], ntf[2][2], mtf[2][2];   // [s][hi, lo]
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                nf[s][p] = lds16(tile_at<128>(tN + p * MB, 16 * R + i16, 4 * s + g));
                mf[s][p] = lds16(tile_at<128>(tN + 2 * MB + p * MB, 16 * R + i16, 4 * s + g));
                ntf[s][p] = tr_frag<128>(tN + p * MB, 16 * R, s, i16, g);
                mtf[s][p] = tr_frag<128>(tN + 2 * MB + p * MB, 16 * R, s, i16, g);
            }
#pragma unroll
        for (int D = 0; D < NDH; ++D) {
            const int c0 = 16 * (D0 + D);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const uint4 kb = tr_frag<RB>(tK, c0, s, i16, g);
                const uint4 qb = tr_frag<RB>(tQ, c0, s, i16, g);
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    dq[D] = mfma_raw<true>(nf[s][p], kb, dq[D]);
                    dk[D] = mfma_raw<true>(mf[s][p], kb, dk[D]);
                    dk[D] = mfma_raw<true>(ntf[s][p], qb, dk[D]);
                    dk[D] = mfma_raw<true>(mtf[s][p], kb, dk[D]);
                }
            }
        }
    } else {
#pragma unroll
        for (int D = 0; D < NDH; ++D) {
            const int cb = 16 * (D0 + D) + i16;
            for (int s = 0; s < 4 * (R + 1); ++s) {
                const int m = 4 * s + g;
                const float kb = sK[m * KP + cb];
                dq[D] = mfma_f32x4(sM3[(16 * R + i16) * PT + m], kb, dq[D]);
                dk[D] = mfma_f32x4(sM1[(16 * R + i16) * PT + m], kb, dk[D]);
            }
            for (int s = 4 * R; s < 16; ++s) {
                const int m = 4 * s + g;
                dk[D] = mfma_f32x4(sM3[m * PT + 16 * R + i16], sQ[m * KP + cb], dk[D]);
                dk[D] = mfma_f32x4(sM1[m * PT + 16 * R + i16], sK[m * KP + cb], dk[D]);
            }
        }
    }
    // ---- reductions of the gate and strength terms, in a fixed order (so
    // that the gradients do not depend on the order the waves finish in):
    // each wave's row and column partials go to their own slots of sM2
    // (K K^T o E, no longer read), then lane l of wave 0 adds those of
    // token l.  Rows: [2 halves][64] for dg, then for dbeta; columns: [8
    // waves][64] for each; then the 8 waves' parts of the last row's sum.
    float* prg = sM2;
    float* prb = prg + 2 * CH;
    float* pcg = prb + 2 * CH;
    float* pcb = pcg + 8 * CH;
    float* p63 = pcb + 8 * CH;
    static_assert(PNT == 512 && 20 * CH + 8 <= CH * PT, "the partials fit sM2");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float xg = group_sum<16>(rowg[j]);
        const float xb = group_sum<16>(rowb[j]);
        if (i16 == 0) {
            prg[hf * CH + rb + j] = xg;
            prb[hf * CH + rb + j] = xb;
        }
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const float xg = col4_sum(colg[I]);
        const float xb = col4_sum(colb[I]);
        if (g == 0) {
            pcg[w * CH + 16 * I + i16] = xg;
            pcb[w * CH + 16 * I + i16] = xb;
        }
    }
    {
        float x = group_sum<32>(g63part);
        x += __shfl_xor(x, 32);
        if (l == 0) p63[w] = x;
    }
    lds_barrier();
    if (w == 0) {
        float x = prg[l] + prg[CH + l], xb = prb[l] + prb[CH + l];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            x += pcg[v * CH + l];
            xb += pcb[v * CH + l];
        }
        if (l == CH - 1) {
            float h = 0.f;
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                x += p63[v];
                h += shs[v];
            }
            x += expf(sg[CH - 1]) * h;
        }
        // d log alpha_t = sum over r >= t of dg_r (suffix sum over the lanes)
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y2 = __shfl_down(x, o);
            if (l + o < 64) x += y2;
        }
        if (l < valid) {
            if (a.dlog_alpha) a.dlog_alpha[tok0 + l] = x;
            a.dbeta[tok0 + l] = xb;
        }
    }
#pragma unroll
    for (int D = 0; D < NDH; ++D) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = rb + j;
            if (r < valid) {
                a.dq[(tok0 + r) * DK + 16 * (D0 + D) + i16] = dq[D][j];
                a.dk[(tok0 + r) * DK + 16 * (D0 + D) + i16] = dk[D][j];
            }
        }
    }
}

// ======================================================= channel gate
// With a per-channel decay the chunk algebra keeps its form on gated operands
// (G the per-channel cumulative log decay within the chunk, G_63 its last row):
//   Q^ = Q o e^G, K^ = K o e^G, Kc = K o e^-G, K~ = K o e^(G_63 - G),
//   A = strict lower of Diag(beta) K^ Kc^T,  P = lower of Q^ Kc^T,
//   R = V - K^ S,  U = T Diag(beta) R,  O = Q^ S + P U,
//   S' = Diag(e^G_63) S + K~^T U.
// Backward: dU = P^T dO + K~ H, dR = Diag(beta) T^T dU, dS = Diag(e^G_63) H +
// Q^^T dO - K^^T dR; dQ^ = dO S^T + N Kc, dK^ = -dR S^T + M Kc,
// dKc = N^T Q^ + M^T K^, dK~ = U H^T (N = lower dP, M = Diag(beta) dA), and
// per element dq = dQ^ e^G, dk = dK^ e^G + dKc e^-G + dK~ e^(G_63 - G),
// dG = dQ^ Q^ + dK^ K^ - dKc Kc - dK~ K~, plus at the last row the sums of
// dK~ K~ over the chunk and e^G_63 <H_c, S_c>; d log alpha is dG's reverse
// cumulative sum per channel.
//
// Strong decays.  e^-G overflows fp32 once a channel's decay over the chunk,
// G_63, falls below about -88.  A chunk in which some channel's G_63 is below
// kShiftBelow takes shifted operands for its 64 x 64 products instead: with
// the per-channel reference G_m = G_63 / 2, the products run on
// Q o e^(G - G_m), K o e^(G - G_m) and Kc o e^(G_m) = K o e^(G_m - G), every
// factor within e^(|G_63| / 2), and the per-element step applies e^(G - G_m)
// or e^(G_m - G) to their terms (the state-sized terms keep e^G).  That holds
// a chunk's decay down to about -170 in every channel (an average log alpha of
// about -2.7 per token).  The other chunks keep the unshifted arithmetic.

// A [64][DK] fp32 workspace plane straight into LDS rows of pitch DK + 1.
template <int DK, int NT>
__device__ __forceinline__ void load_plane(float* dst, const float* src, int tid) {
    constexpr int KP = DK + 1;
    for (int e = tid; e < CH * DK / 4; e += NT) {
        const float4 x = reinterpret_cast<const float4*>(src)[e];
        const int r = e / (DK / 4), c = (e % (DK / 4)) * 4;
        dst[r * KP + c] = x.x;
        dst[r * KP + c + 1] = x.y;
        dst[r * KP + c + 2] = x.z;
        dst[r * KP + c + 3] = x.w;
    }
}

constexpr float kShiftBelow = -60.f;

template <int DK, bool F32IN>
__global__ __launch_bounds__(NTH) void bwd_prep_cg_kernel(BwdArgs a) {
    constexpr int KP = DK + 1;
    static_assert(2 * CH * PT <= 3 * CH * KP, "A and T fit where the operands were");
    __shared__ float sOp[3 * CH * KP];   // K^, Kc, Q^; then A and T
    __shared__ float sG[CH * KP];        // log alpha, then its cumulative sums
    __shared__ float sX[4][16 * 17];
    __shared__ float sb[CH];
    __shared__ int s_shift;
    float* sKh = sOp;
    float* sKc = sOp + CH * KP;
    float* sQh = sOp + 2 * CH * KP;
    float* sA = sOp;
    float* sT = sOp + CH * PT;
    const int cs = blockIdx.x;
    const int seq = cs / a.NC, c = cs - seq * a.NC;
    const int t0 = c * CH, valid = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const size_t mo = (size_t)cs * CH * CH, po = (size_t)cs * CH * DK;

    if (tid < CH) sb[tid] = tid < valid ? a.beta[tok0 + tid] : 0.f;
    if (tid == 0) s_shift = 0;
    // log alpha rows into LDS (zeros past the end: no decay), then each
    // channel's cumulative sum in place
    for (int e = tid; e < CH * DK / 4; e += NTH) {
        const int r = e / (DK / 4), c4 = (e % (DK / 4)) * 4;
        float4 x = {0.f, 0.f, 0.f, 0.f};
        if (r < valid && a.gmode == 2) x = *reinterpret_cast<const float4*>(a.log_alpha + (tok0 + r) * DK + c4);
        if (r < valid && a.gmode == 1) x.x = x.y = x.z = x.w = a.log_alpha[tok0 + r];
        sG[r * KP + c4] = x.x;
        sG[r * KP + c4 + 1] = x.y;
        sG[r * KP + c4 + 2] = x.z;
        sG[r * KP + c4 + 3] = x.w;
    }
    lds_barrier();
    // each channel's 64 values into registers first (independent reads), the
    // running sum there, then back
    for (int ch = tid; ch < DK; ch += NTH) {
        float v[CH];
#pragma unroll
        for (int r = 0; r < CH; ++r) v[r] = sG[r * KP + ch];
        float G = 0.f;
#pragma unroll
        for (int r = 0; r < CH; ++r) {
            G += v[r];
            sG[r * KP + ch] = G;
        }
        if (G < kShiftBelow) s_shift = 1;
    }
    lds_barrier();
    const bool shift = s_shift != 0;   // workgroup-uniform
    // the gated operands, eight channels of one row per thread and step (rows
    // past the end: zero operands); with shift the 64 x 64 products take them
    // relative to G_m = G_63 / 2 (Kc's workspace plane too)
    for (int e = tid; e < CH * DK / 8; e += NTH) {
        const int r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
        float kx[8], qx[8], gq[8], gh[8], gc[8], gt[8], gg[8], wx[8];
        load8<F32IN>(a.k, (tok0 + r) * DK + c8, r < valid, kx);
        load8<F32IN>(a.q, (tok0 + r) * DK + c8, r < valid, qx);
        if (a.ks) load8<true>(a.ks, (tok0 + r) * DK + c8, r < valid, wx);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float G = sG[r * KP + c8 + j], G63 = sG[(CH - 1) * KP + c8 + j];
            const float Gm = shift ? 0.5f * G63 : 0.f;
            // e^x as the hardware 2^(x log2 e)
            auto ex = [](float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); };
            const float eg = ex(G), emg = ex(Gm - G);
            const float wk = a.ks ? wx[j] * kx[j] : kx[j];   // the write key
            gg[j] = G;
            gq[j] = qx[j] * eg;
            gh[j] = kx[j] * eg;
            gc[j] = wk * emg;
            gt[j] = wk * ex(G63 - G);
            const float es = shift ? ex(G - Gm) : eg;
            sQh[r * KP + c8 + j] = qx[j] * es;
            sKh[r * KP + c8 + j] = kx[j] * es;
            sKc[r * KP + c8 + j] = gc[j];
        }
        const size_t at = po + (size_t)r * DK + c8;
        float* const dst[5] = {a.wG + at, a.wQh + at, a.wKh + at, a.wKc + at, a.wKt + at};
        const float* const src[5] = {gg, gq, gh, gc, gt};
#pragma unroll
        for (int t = 0; t < 5; ++t) {
            reinterpret_cast<float4*>(dst[t])[0] = make_float4(src[t][0], src[t][1], src[t][2], src[t][3]);
            reinterpret_cast<float4*>(dst[t])[1] = make_float4(src[t][4], src[t][5], src[t][6], src[t][7]);
        }
    }
    lds_barrier();
    // lower blocks (R = w, I <= R) of K^ Kc^T and Q^ Kc^T, in registers until
    // every wave is done with the operands
    {
        const int R = w;
        f32x4 aK[4], aQ[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            aK[I] = aQ[I] = zero4();
            if (I <= R) {
                for (int s = 0; s < DK / 4; ++s) {
                    const int m = 4 * s + g;
                    const float kb = sKc[(16 * I + i16) * KP + m];
                    aK[I] = mfma_f32x4(sKh[(16 * R + i16) * KP + m], kb, aK[I]);
                    aQ[I] = mfma_f32x4(sQh[(16 * R + i16) * KP + m], kb, aQ[I]);
                }
            }
        }
        lds_barrier();
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * g + j, i = 16 * I + i16;
                const float araw = i < r ? aK[I][j] : 0.f;
                sA[r * PT + i] = sb[r] * araw;
                a.wA[mo + r * CH + i] = araw;
                a.wP[mo + r * CH + i] = i <= r ? aQ[I][j] : 0.f;
            }
        }
    }
    lds_barrier();
    tri_inverse(sA, sT, sX, a.wT + mo, tid);
}

// bf16 inputs: the same outputs from one workgroup per chunk with the rows in
// the 16x16x32 operand layout (as in the forward's channel-gate preparation):
// wave w owns rows 16 w .. 16 w + 15, lane (i16, g) row 16 w + i16 at
// channels 32 s + 8 g .. + 7, so a row's inputs stay in its lane.  The gate's
// prefix over a block's 16 rows runs across a DPP row; one thread per channel
// combines the four blocks into per-block constants (E_b: G at the end of
// block b, E_{-1} = 0, T_b = E_b - E_{b-1}).  Per element two exponentials
// inside the row's own block, y = e^{G_r - E_{w-1}} and z = e^{E_w - G_r}:
//   e^G = e^{E_{w-1}} y,  e^{G_63 - G} = e^{G_63 - E_w} z,
//   e^{G_m - G} = e^{G_m - E_w} z,  e^{G - G_m} = e^{E_{w-1} - G_m} y
// (G_m = 0, or G_63 / 2 for a shifted chunk).  The 64 x 64 products run on
// bf16 ops with hi + lo operands (16 significant bits each, three ops per
// product); the column side of blocks 0..2 goes through LDS, the diagonal
// pair takes both sides from registers.
template <int DK>
struct BPC16 {
    static constexpr int RB = DK * 2;             // bytes per bf16 row
    static constexpr int KC = 0;                  // column side, blocks 0..2: hi [48][RB], then lo
    static constexpr int GS = 0;                  // in-block gate sums [4][DK], read before the tiles are written
    static constexpr int CT = 2 * 48 * RB;        // constants [CB_ROWS][DK]
    static constexpr int CTE = CT + 24 * DK * 4;
    static constexpr int SA = 0;                  // A, T and the solve's scratch once the products are formed
    static constexpr int ST = SA + CH * PT * 4;
    static constexpr int SX = ST + CH * PT * 4;
    static constexpr int SXE = SX + 4 * 16 * 17 * 4;
    static constexpr int SB = SXE > CTE ? SXE : CTE;
    static constexpr int FL = SB + CH * 4;
    static constexpr int TOTAL = FL + 16;
    static_assert(4 * DK * 4 <= CT, "the gate sums fit under the tiles");
};
// constant rows (+ block b): T_b, E_{b-1}, e^{E_{b-1}}, e^{G_63 - E_b},
// e^{G_m - E_b}, e^{E_{b-1} - G_m}
enum { CB_T = 0, CB_EP = 4, CB_C1 = 8, CB_C2 = 12, CB_C3 = 16, CB_C4 = 20 };

// Lane i of each 16-lane row receives lane i - N of that row, 0 for i < N.
template <int N>
__device__ __forceinline__ float dpp_row_shr(float x) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, false));
}

// Eight floats from 16-byte aligned shared memory.
__device__ __forceinline__ void ld8f(const float* p, float* x) {
    const float4 u = reinterpret_cast<const float4*>(p)[0];
    const float4 v = reinterpret_cast<const float4*>(p)[1];
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
}

template <int DK>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(3, 8))) void bwd_prep_cg16_kernel(BwdArgs a) {
    using L = BPC16<DK>;
    constexpr int NS = DK / 32;
    constexpr float kL2E = 1.4426950408889634f;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    lchar* sKc = (lchar*)(smem + L::KC);
    float* sGS = reinterpret_cast<float*>(smem + L::GS);
    float* sCT = reinterpret_cast<float*>(smem + L::CT);
    float* sA = reinterpret_cast<float*>(smem + L::SA);
    float* sT = reinterpret_cast<float*>(smem + L::ST);
    float(*sX)[16 * 17] = reinterpret_cast<float(*)[16 * 17]>(smem + L::SX);
    float* sb = reinterpret_cast<float*>(smem + L::SB);
    int* sflag = reinterpret_cast<int*>(smem + L::FL);

    const int cs = blockIdx.x;
    const int seq = cs / a.NC, c = cs - seq * a.NC;
    const int t0 = c * CH, valid = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: its branches are scalar
    const int i16 = l & 15, g = l >> 4;
    const int r = 16 * w + i16;
    const bool live = r < valid;
    const size_t row = tok0 + (live ? r : 0);   // rows past the end load row 0 and are masked
    const size_t mo = (size_t)cs * CH * CH, po = (size_t)cs * CH * DK + (size_t)r * DK;
    auto ex = [](float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); };

    // ------------------------------------------------------------ loads
    uint4 kr[NS], qr[NS];
    float G[NS][8];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int c0 = 32 * s + 8 * g;
        kr[s] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + row * DK + c0);
        qr[s] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + row * DK + c0);
        if (a.gmode == 2) {
            load_f32_n<8>(a.log_alpha + row * DK + c0, G[s]);
        } else {
            const float x = a.gmode == 1 ? a.log_alpha[row] : 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) G[s][j] = x;
        }
    }
    if (!live) {
#pragma unroll
        for (int s = 0; s < NS; ++s) kr[s] = qr[s] = uint4{0u, 0u, 0u, 0u};
    }
    if (g == 0) sb[r] = live ? a.beta[row] : 0.f;
    if (tid == 0) sflag[0] = 0;

    // ------------------------------------ the gate's prefix inside the block
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float x = live ? G[s][j] : 0.f;
            x += dpp_row_shr<1>(x);
            x += dpp_row_shr<2>(x);
            x += dpp_row_shr<4>(x);
            x += dpp_row_shr<8>(x);
            G[s][j] = x;   // sum over rows 16 w .. r
        }
    if (i16 == 15) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            float* d = sGS + w * DK + 32 * s + 8 * g;
            reinterpret_cast<float4*>(d)[0] = make_float4(G[s][0], G[s][1], G[s][2], G[s][3]);
            reinterpret_cast<float4*>(d)[1] = make_float4(G[s][4], G[s][5], G[s][6], G[s][7]);
        }
    }
    lds_barrier();
    // one thread per channel: the block constants, and whether the chunk is
    // shifted (some channel's G_63 below kShiftBelow); then the constants
    // that depend on the shift
    float E[4] = {0.f, 0.f, 0.f, 0.f};
    if (tid < DK) {
        float run = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float t = sGS[b * DK + tid];
            run += t;
            E[b] = run;
            const float ep = b > 0 ? E[b - 1] : 0.f;
            sCT[(CB_T + b) * DK + tid] = t;
            sCT[(CB_EP + b) * DK + tid] = ep;
        }
        if (E[3] < kShiftBelow) atomicOr(sflag, 1);
    }
    lds_barrier();
    const bool shift = sflag[0] != 0;   // workgroup-uniform
    if (tid < DK) {
        const float gm = shift ? 0.5f * E[3] : 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float ep = b > 0 ? E[b - 1] : 0.f;
            sCT[(CB_C1 + b) * DK + tid] = ex(ep);
            sCT[(CB_C2 + b) * DK + tid] = ex(E[3] - E[b]);
            sCT[(CB_C3 + b) * DK + tid] = ex(gm - E[b]);
            sCT[(CB_C4 + b) * DK + tid] = ex(ep - gm);
        }
    }
    lds_barrier();

    // ----- planes, the column-side tiles and the diagonal pair (own rows);
    // the row side of the off-diagonal pairs (k e^{G - G_m}, q e^{G - G_m})
    // stays as bf16 hi + lo fragments
    uint4 fk[NS][2], fq[NS][2];
    f32x4 dA = zero4(), dP = zero4();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int c0 = 32 * s + 8 * g;
        // (a) the two exponentials and the five workspace planes
        float kx[8], qx[8], y[8], pc[8];
        {
            float tw[8], ep[8], c1[8], c2[8], c3[8], wk[8];
            ld8f(sCT + (CB_T + w) * DK + c0, tw);
            ld8f(sCT + (CB_EP + w) * DK + c0, ep);
            ld8f(sCT + (CB_C1 + w) * DK + c0, c1);
            ld8f(sCT + (CB_C2 + w) * DK + c0, c2);
            ld8f(sCT + (CB_C3 + w) * DK + c0, c3);
            unpack_bf16x8(kr[s], kx);
            unpack_bf16x8(qr[s], qx);
            if (a.ks) load_f32_n<8>(a.ks + row * DK + c0, wk);
            float pg[8], pq[8], ph[8], pt[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float gl = G[s][j];
                y[j] = ex(gl);
                const float z = ex(tw[j] - gl);
                const float eg = c1[j] * y[j];
                const float wz = (a.ks ? wk[j] * kx[j] : kx[j]) * z;   // the write key times z
                pg[j] = gl + ep[j];
                pq[j] = qx[j] * eg;
                ph[j] = kx[j] * eg;
                pc[j] = wz * c3[j];
                pt[j] = wz * c2[j];
            }
            float* const dst[5] = {a.wG + po + c0, a.wQh + po + c0, a.wKh + po + c0, a.wKc + po + c0,
                                   a.wKt + po + c0};
            const float* const src[5] = {pg, pq, ph, pc, pt};
#pragma unroll
            for (int t = 0; t < 5; ++t) {
                reinterpret_cast<float4*>(dst[t])[0] = make_float4(src[t][0], src[t][1], src[t][2], src[t][3]);
                reinterpret_cast<float4*>(dst[t])[1] = make_float4(src[t][4], src[t][5], src[t][6], src[t][7]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // (b) the row and column sides of the products as bf16 hi + lo
        uint16_t akh[8], akl[8], aqh[8], aql[8], bh[8], bl[8];
        {
            float c4[8];
            ld8f(sCT + (CB_C4 + w) * DK + c0, c4);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float es = y[j] * c4[j];   // e^{G - G_m}
                split_bf16(kx[j] * es, akh[j], akl[j]);
                split_bf16(qx[j] * es, aqh[j], aql[j]);
                split_bf16(pc[j], bh[j], bl[j]);
            }
        }
        auto pack = [](const uint16_t* x) {
            return uint4{x[0] | ((uint32_t)x[1] << 16), x[2] | ((uint32_t)x[3] << 16), x[4] | ((uint32_t)x[5] << 16),
                         x[6] | ((uint32_t)x[7] << 16)};
        };
        fk[s][0] = pack(akh);
        fk[s][1] = pack(akl);
        fq[s][0] = pack(aqh);
        fq[s][1] = pack(aql);
        const uint4 b0 = pack(bh), b1 = pack(bl);
        if (w < 3) {
            const int at = r * L::RB + 16 * ((4 * s + g) ^ swz<L::RB>(r));   // as tile_at
            lds_st(sKc + at, b0);
            lds_st(sKc + 48 * L::RB + at, b1);
        }
        dA = mfma_raw<true>(fk[s][0], b0, dA);
        dA = mfma_raw<true>(fk[s][0], b1, dA);
        dA = mfma_raw<true>(fk[s][1], b0, dA);
        dP = mfma_raw<true>(fq[s][0], b0, dP);
        dP = mfma_raw<true>(fq[s][0], b1, dP);
        dP = mfma_raw<true>(fq[s][1], b0, dP);
        __builtin_amdgcn_sched_barrier(0);   // one slice of channels at a time: fewer live registers
    }
    lds_barrier();   // the column-side tiles are complete

    // ------------------------- off-diagonal pairs (w, I), I < w, on bf16 ops
    f32x4 oA[3], oP[3];
#pragma unroll
    for (int I = 0; I < 3; ++I) oA[I] = oP[I] = zero4();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int I = 0; I < 3; ++I) {
            if (I < w) {   // wave-uniform
                const uint4 b0 = lds16(tile_at<L::RB>(sKc, 16 * I + i16, 4 * s + g));
                const uint4 b1 = lds16(tile_at<L::RB>(sKc + 48 * L::RB, 16 * I + i16, 4 * s + g));
                oA[I] = mfma_raw<true>(fk[s][0], b0, oA[I]);
                oA[I] = mfma_raw<true>(fk[s][0], b1, oA[I]);
                oA[I] = mfma_raw<true>(fk[s][1], b0, oA[I]);
                oP[I] = mfma_raw<true>(fq[s][0], b0, oP[I]);
                oP[I] = mfma_raw<true>(fq[s][0], b1, oP[I]);
                oP[I] = mfma_raw<true>(fq[s][1], b0, oP[I]);
            }
        }
    }
    lds_barrier();   // every product is formed: A, T and the scratch take the tiles' place

    // K^ Kc^T (strict lower, without beta) and Q^ Kc^T (lower) of block row w
    // to the workspace, zeros above the diagonal blocks; beta-scaled A to LDS
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const f32x4 cA = I == w ? dA : I == 0 ? oA[0] : I == 1 ? oA[1] : oA[2];
        const f32x4 cP = I == w ? dP : I == 0 ? oP[0] : I == 1 ? oP[1] : oP[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = 16 * w + 4 * g + j, ii = 16 * I + i16;
            const float araw = I <= w && ii < rr ? cA[j] : 0.f;
            sA[rr * PT + ii] = sb[rr] * araw;
            a.wA[mo + rr * CH + ii] = araw;
            a.wP[mo + rr * CH + ii] = I <= w && ii <= rr ? cP[j] : 0.f;
        }
    }
    lds_barrier();
    tri_inverse(sA, sT, sX, a.wT + mo, tid);
}

template <int DK, bool F32IN>
__global__ __launch_bounds__(SNT) void bwd_fscan_cg_kernel(BwdArgs a) {
    constexpr int KP = DK + 1, NKS = DK / 8;
    __shared__ float sKh[CH * KP];
    __shared__ float sKt[CH * KP];
    __shared__ float sT[CH * PT];
    __shared__ float sS[DK * 17];
    __shared__ float sR[CH * 17];   // upper-half partial X, then R
    __shared__ float sU[CH * 17];
    __shared__ float sb[CH], sd63[DK];
    int seq, tile;
    scan_tile(a, seq, tile);
    if (seq >= a.nseq) return;
    const int n0 = 16 * tile, Dv = a.Dv;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const int R = w & 3, h = w >> 2;

    PlanePre<DK, SNT> pkh, pkt;
    MatPre<SNT> pt;
    float pb = 0.f, pd = 0.f, pv[4] = {0.f, 0.f, 0.f, 0.f};
    auto prefetch = [&](int c) {
        const size_t cs = (size_t)seq * a.NC + c;
        const int t0 = c * CH, valid = min(CH, a.L - t0);
        const size_t tok0 = (size_t)seq * a.L + t0;
        pre_plane(pkh, a.wKh + cs * CH * DK, tid);
        pre_plane(pkt, a.wKt + cs * CH * DK, tid);
        pre_mat(pt, a.wT + cs * CH * CH, tid);
        if (tid < CH) pb = a.beta[tok0 + (tid < valid ? tid : 0)];
        if (tid < DK) pd = a.wG[cs * CH * DK + (CH - 1) * DK + tid];
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                pv[j] = load1<F32IN>(a.v, (tok0 + (row < valid ? row : 0)) * Dv + n0 + i16);
            }
        }
    };

    for (int e = tid; e < DK * 16; e += SNT) {
        const int d = e >> 4, cc = e & 15;
        sS[d * 17 + cc] = a.S0 ? a.S0[((size_t)seq * DK + d) * Dv + n0 + cc] : 0.f;
    }
    prefetch(0);
    for (int c = 0; c < a.NC; ++c) {
        const size_t cs = (size_t)seq * a.NC + c;
        const int t0 = c * CH, valid = min(CH, a.L - t0);
        lds_barrier();
        put_plane(pkh, sKh, tid);
        put_plane(pkt, sKt, tid);
        put_mat(pt, sT, tid);
        if (tid < CH) sb[tid] = tid < valid ? pb : 0.f;
        if (tid < DK) sd63[tid] = expf(pd);
        float vv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) vv[j] = 16 * R + 4 * g + j < valid ? pv[j] : 0.f;
        for (int e = tid; e < DK * 16; e += SNT) {
            const int d = e >> 4, cc = e & 15;
            a.wS[(cs * DK + d) * Dv + n0 + cc] = sS[d * 17 + cc];
        }
        lds_barrier();
        if (c + 1 < a.NC) prefetch(c + 1);
        // X = K^ S over this wave's half of the contraction
        f32x4 X = zero4();
#pragma unroll
        for (int s2 = 0; s2 < NKS; ++s2) {
            const int s = h * NKS + s2;
            const int m = 4 * s + g;
            X = mfma_f32x4(sKh[(16 * R + i16) * KP + m], sS[m * 17 + i16], X);
        }
        if (h == 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sR[(16 * R + 4 * g + j) * 17 + i16] = X[j];
        }
        lds_barrier();
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                const float r = vv[j] - (X[j] + sR[row * 17 + i16]);
                sR[row * 17 + i16] = r;
                a.wR[(cs * CH + row) * Dv + n0 + i16] = r;
            }
        }
        lds_barrier();
        if (h == 0) {
            // U = T Diag(beta) R
            f32x4 U = zero4();
            // the factor's row 16 R + i16 is zero past the diagonal: all 16 k-steps
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                U = mfma_f32x4(sT[(16 * R + i16) * PT + m] * sb[m], sR[m * 17 + i16], U);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                a.wU[(cs * CH + row) * Dv + n0 + i16] = U[j];
                sU[row * 17 + i16] = U[j];
            }
        }
        lds_barrier();
        // S <- Diag(e^G_63) S + K~^T U  (state rows 16 w ..)
        if (w < DK / 16) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                acc = mfma_f32x4(sKt[m * KP + 16 * w + i16], sU[m * 17 + i16], acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = 16 * w + 4 * g + j;
                sS[d * 17 + i16] = sd63[d] * sS[d * 17 + i16] + acc[j];
            }
        }
    }
}

template <int DK>
__global__ __launch_bounds__(SNT) void bwd_rscan_cg_kernel(BwdArgs a) {
    constexpr int KP = DK + 1, NKS = DK / 8;
    __shared__ float sKt[CH * KP];
    __shared__ float sQh[CH * KP];
    __shared__ float sKh[CH * KP];
    __shared__ float sT[CH * PT];
    __shared__ float sP[CH * PT];
    __shared__ float sH[DK * 17];
    __shared__ float sO[CH * 17];   // dO
    __shared__ float sD[CH * 17];   // upper-half partial dU, then dU, then dR
    __shared__ float sb[CH], sd63[DK];
    int seq, tile;
    scan_tile(a, seq, tile);
    if (seq >= a.nseq) return;
    const int n0 = 16 * tile, Dv = a.Dv;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const int R = w & 3, h = w >> 2;

    PlanePre<DK, SNT> pkt, pqh, pkh;
    MatPre<SNT> pt, pp;
    float pb = 0.f, pd = 0.f, po[4] = {0.f, 0.f, 0.f, 0.f};
    auto prefetch = [&](int c) {
        const size_t cs = (size_t)seq * a.NC + c;
        const int t0 = c * CH, valid = min(CH, a.L - t0);
        const size_t tok0 = (size_t)seq * a.L + t0;
        pre_plane(pkt, a.wKt + cs * CH * DK, tid);
        pre_plane(pqh, a.wQh + cs * CH * DK, tid);
        pre_plane(pkh, a.wKh + cs * CH * DK, tid);
        pre_mat(pt, a.wT + cs * CH * CH, tid);
        pre_mat(pp, a.wP + cs * CH * CH, tid);
        if (tid < CH) pb = a.beta[tok0 + (tid < valid ? tid : 0)];
        if (tid < DK) pd = a.wG[cs * CH * DK + (CH - 1) * DK + tid];
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                po[j] = a.dO[(tok0 + (row < valid ? row : 0)) * Dv + n0 + i16];
            }
        }
    };

    for (int e = tid; e < DK * 16; e += SNT) {
        const int d = e >> 4, cc = e & 15;
        sH[d * 17 + cc] = a.dS_final ? a.dS_final[((size_t)seq * DK + d) * Dv + n0 + cc] : 0.f;
    }
    prefetch(a.NC - 1);
    for (int c = a.NC - 1; c >= 0; --c) {
        const size_t cs = (size_t)seq * a.NC + c;
        const int t0 = c * CH, valid = min(CH, a.L - t0);
        const size_t tok0 = (size_t)seq * a.L + t0;
        lds_barrier();
        put_plane(pkt, sKt, tid);
        put_plane(pqh, sQh, tid);
        put_plane(pkh, sKh, tid);
        put_mat(pt, sT, tid);
        put_mat(pp, sP, tid);
        if (tid < CH) sb[tid] = tid < valid ? pb : 0.f;
        if (tid < DK) sd63[tid] = expf(pd);
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                sO[row * 17 + i16] = row < valid ? po[j] : 0.f;
            }
        }
        for (int e = tid; e < DK * 16; e += SNT) {
            const int d = e >> 4, cc = e & 15;
            a.wH[(cs * DK + d) * Dv + n0 + cc] = sH[d * 17 + cc];
        }
        lds_barrier();
        if (c > 0) prefetch(c - 1);
        // dU = P^T dO + K~ H  (rows 16 R ..): K~ H over this wave's half of
        // the contraction; the upper half also takes P^T dO
        f32x4 Z = zero4();
#pragma unroll
        for (int s2 = 0; s2 < NKS; ++s2) {
            const int s = h * NKS + s2;
            const int m = 4 * s + g;
            Z = mfma_f32x4(sKt[(16 * R + i16) * KP + m], sH[m * 17 + i16], Z);
        }
        if (h == 1) {
            f32x4 Y = zero4();
            // the factor's column 16 R + i16 is zero above the diagonal: all 16 k-steps
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                Y = mfma_f32x4(sP[m * PT + 16 * R + i16], sO[m * 17 + i16], Y);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) sD[(16 * R + 4 * g + j) * 17 + i16] = Z[j] + Y[j];
        }
        lds_barrier();
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                const float du = Z[j] + sD[row * 17 + i16];
                sD[row * 17 + i16] = du;
                a.wdU[(cs * CH + row) * Dv + n0 + i16] = du;
            }
        }
        lds_barrier();
        // dR = Diag(beta) T^T dU
        f32x4 Rr = zero4();
        if (h == 0) {
            // the factor's column 16 R + i16 is zero above the diagonal: all 16 k-steps
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                Rr = mfma_f32x4(sT[m * PT + 16 * R + i16], sD[m * 17 + i16], Rr);
            }
        }
        lds_barrier();
        if (h == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * R + 4 * g + j;
                const float dr = sb[row] * Rr[j];
                if (row < valid) a.dv[(tok0 + row) * Dv + n0 + i16] = dr;
                sD[row * 17 + i16] = dr;
            }
        }
        lds_barrier();
        // H <- Diag(e^G_63) H + Q^^T dO - K^^T dR  (state rows 16 w ..)
        if (w < DK / 16) {
            f32x4 hq = zero4(), hk = zero4();
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                hq = mfma_f32x4(sQh[m * KP + 16 * w + i16], sO[m * 17 + i16], hq);
                hk = mfma_f32x4(sKh[m * KP + 16 * w + i16], sD[m * 17 + i16], hk);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = 16 * w + 4 * g + j;
                sH[d * 17 + i16] = sd63[d] * sH[d * 17 + i16] + (hq[j] - hk[j]);
            }
        }
    }
    lds_barrier();
    if (a.dS0) {
        for (int e = tid; e < DK * 16; e += SNT) {
            const int d = e >> 4, cc = e & 15;
            a.dS0[((size_t)seq * DK + d) * Dv + n0 + cc] = sH[d * 17 + cc];
        }
    }
}

template <int DK, bool F32IN>
__global__ __launch_bounds__(PNT) void bwd_post_cg_kernel(BwdArgs a) {
    using Lp = PostLds<DK>;
    constexpr int KP = Lp::KP, ND = DK / 16, NDH = ND / 2;
    __shared__ float s1[Lp::R1];
    __shared__ float sM0[CH * PT];   // T
    __shared__ float sM1[CH * PT];   // P (unused), then M = Diag(beta) dA
    __shared__ float sM2[CH * PT];   // K^ Kc^T (strict lower)
    __shared__ float sM3[CH * PT];   // N = lower dP
    __shared__ float sM4[CH * PT];   // dT^ Diag(beta), then T^T of it
    __shared__ float sb[CH], shs[DK];
    __shared__ int s_shift;
    const int cs = blockIdx.x;
    const int seq = cs / a.NC, c = cs - seq * a.NC;
    const int t0 = c * CH, valid = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const int R = w & 3, hf = w >> 2, D0 = hf * NDH;
    const size_t mo = (size_t)cs * CH * CH, pofs = (size_t)cs * CH * DK;

    if (tid < CH) sb[tid] = tid < valid ? a.beta[tok0 + tid] : 0.f;
    if (tid == 0) s_shift = 0;
    // shifted operands, as the preparation kernel chose them for this chunk
    // (rows of a chunk operand relative to G_m = G_63 / 2)
    auto shifted_rows = [&](float* dst, const void* src) {
        for (int e = tid; e < CH * DK; e += PNT) {
            const int r = e / DK, cc = e % DK;
            const float G = a.wG[pofs + (size_t)r * DK + cc], G63 = a.wG[pofs + (size_t)(CH - 1) * DK + cc];
            const float x = r < valid ? load1<F32IN>(src, (tok0 + r) * DK + cc) : 0.f;
            dst[r * KP + cc] = x * expf(G - 0.5f * G63);
        }
    };

    RowsPre<DK, F32IN, PNT> pk, pq;   // not used with a channel gate
    MatPre<PNT> pt, pp, pa;
    PlanePre<DK, PNT> pkc, pqh;
    f32x4 z1[NDH], z2[NDH], z3[NDH], acc[4];
    post_state_products<DK, F32IN, true>(a, cs, valid, tok0, s1, z1, z2, z3, acc, shs, pk, pq, pt, pp, pa, &pkc,
                                         &pqh);
    lds_barrier();

    // ---- Kc and Q^ rows, T and K^ Kc^T
    float* sKx = s1;             // Kc, later K^
    float* sQh = s1 + CH * KP;
    if (tid < DK && a.wG[pofs + (size_t)(CH - 1) * DK + tid] < kShiftBelow) s_shift = 1;
    put_plane(pkc, sKx, tid);
    put_plane(pqh, sQh, tid);
    put_mat(pt, sM0, tid);
    put_mat(pa, sM2, tid);
    lds_barrier();
    const bool shift = s_shift != 0;   // workgroup-uniform
    if (shift) {
        shifted_rows(sQh, a.q);
        lds_barrier();
    }

    const int rb = 16 * R + 4 * g;   // this lane's first accumulator row
    float rowb[4] = {0.f, 0.f, 0.f, 0.f}, colb[4] = {0.f, 0.f, 0.f, 0.f};
    // state terms: dQ^ = z1, dK^ = -z2, dK~ = z3; dKc from the 64 x 64 part.
    // With shift the 64 x 64 terms accumulate on their own; the state terms'
    // share of dq and dk (z1 e^G, -z2 e^G) is stored now and completed below
    // by the same lanes.
    f32x4 dqh[NDH], dkh[NDH], dkc[NDH], dkt[NDH];
#pragma unroll
    for (int D = 0; D < NDH; ++D) {
        dqh[D] = shift ? zero4() : z1[D];
        dkh[D] = shift ? zero4() : -z2[D];
        dkt[D] = z3[D];
        dkc[D] = zero4();
        if (shift) {
            const int col = 16 * (D0 + D) + i16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = rb + j;
                if (r < valid) {
                    const float eg = expf(a.wG[pofs + (size_t)r * DK + col]);
                    a.dq[(tok0 + r) * DK + col] = z1[D][j] * eg;
                    a.dk[(tok0 + r) * DK + col] = -z2[D][j] * eg;
                }
            }
        }
    }
    // hf 0: N = lower dP; hf 1: dT = dT^ Diag(beta) and dbeta's sums of dT^ o T
#pragma unroll
    for (int I = 0; I < 4; ++I) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = rb + j, i = 16 * I + i16;
            const bool lo = i <= r;
            const float x = lo ? acc[I][j] : 0.f;
            if (hf == 0) {
                sM3[r * PT + i] = x;
            } else {
                colb[I] += x * sM0[r * PT + i];
                sM4[r * PT + i] = x * sb[i];
            }
        }
    }
    lds_barrier();
    // Y = T^T dT  (rows 16 R .., column blocks 2 hf, 2 hf + 1)
    f32x4 y[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int I = 2 * hf + hh;
        y[hh] = zero4();
        // the factor's column 16 R + i16 is zero above the diagonal: all 16 k-steps
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int m = 4 * s + g;
            y[hh] = mfma_f32x4(sM0[m * PT + 16 * R + i16], sM4[m * PT + 16 * I + i16], y[hh]);
        }
    }
    lds_barrier();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int j = 0; j < 4; ++j) sM4[(rb + j) * PT + 16 * (2 * hf + hh) + i16] = y[hh][j];
    lds_barrier();
    // dA = -Y T^T on the strict lower part; M = Diag(beta) dA into sM1
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int I = 2 * hf + hh;
        f32x4 da = zero4();
        if (I <= R) {
            // T's row 16 I + i16 is zero past the diagonal: all 16 k-steps
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int m = 4 * s + g;
                da = mfma_f32x4(sM4[(16 * R + i16) * PT + m], sM0[(16 * I + i16) * PT + m], da);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = rb + j, cc = 16 * I + i16;
            const bool lo = cc < r;
            const float dav = lo ? -da[j] : 0.f;
            rowb[j] += dav * sM2[r * PT + cc];
            sM1[r * PT + cc] = dav * sb[r];
        }
    }
    lds_barrier();
    // dQ^ += N Kc;  dK^ += M Kc;  dKc = N^T Q^
#pragma unroll
    for (int D = 0; D < NDH; ++D) {
        const int cb = 16 * (D0 + D) + i16;
        // the factor's row 16 R + i16 is zero past the diagonal: all 16 k-steps
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int m = 4 * s + g;
            const float kb = sKx[m * KP + cb];
            dqh[D] = mfma_f32x4(sM3[(16 * R + i16) * PT + m], kb, dqh[D]);
            dkh[D] = mfma_f32x4(sM1[(16 * R + i16) * PT + m], kb, dkh[D]);
        }
        // the factor's column 16 R + i16 is zero above the diagonal: all 16 k-steps
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int m = 4 * s + g;
            dkc[D] = mfma_f32x4(sM3[m * PT + 16 * R + i16], sQh[m * KP + cb], dkc[D]);
        }
    }
    lds_barrier();
    if (shift) shifted_rows(sKx, a.k);   // K^, shifted, in place of Kc
    else load_plane<DK, PNT>(sKx, a.wKh + pofs, tid);   // K^ in place of Kc
    lds_barrier();
    // dKc += M^T K^
#pragma unroll
    for (int D = 0; D < NDH; ++D) {
        const int cb = 16 * (D0 + D) + i16;
        // the factor's column 16 R + i16 is zero above the diagonal: all 16 k-steps
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int m = 4 * s + g;
            dkc[D] = mfma_f32x4(sM1[m * PT + 16 * R + i16], sKx[m * KP + cb], dkc[D]);
        }
    }
    // ---- dbeta's row and column sums, in a fixed order: each wave's partials
    // to their own slots of sM2 (K^ Kc^T, no longer read), rows [2 halves][64]
    // then columns [8 waves][64], added up per token at the end
    float* prb = sM2;
    float* pcb = prb + 2 * CH;
    static_assert(PNT == 512 && 10 * CH <= CH * PT, "the partials fit sM2");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float xb = group_sum<16>(rowb[j]);
        if (i16 == 0) prb[hf * CH + rb + j] = xb;
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const float xb = col4_sum(colb[I]);
        if (g == 0) pcb[w * CH + 16 * I + i16] = xb;
    }
    lds_barrier();
    // ---- per element: dq, dk, and the two parts of dG,
    //   X = dQ^ Q^ + dK^ K^ - dKc Kc,  Y = dK~ K~  (dG = X - Y, plus the last row's sums)
    float* sXg = s1;
    float* sYg = s1 + CH * KP;
    if (shift) __threadfence_block();   // the partial dq, dk stores above, read back by the same lanes
    // e^x as the hardware 2^(x log2 e)
    auto ex = [](float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); };
#pragma unroll
    for (int D = 0; D < NDH; ++D) {
        const int col = 16 * (D0 + D) + i16;
        const float G63 = a.wG[pofs + (size_t)(CH - 1) * DK + col];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = rb + j;
            const size_t at = pofs + (size_t)r * DK + col;
            const float G = a.wG[at];
            const float xq = dqh[D][j], xh = dkh[D][j], xc = dkc[D][j], xt = dkt[D][j];
            const float et = ex(G63 - G);
            if (shift) {
                // every term relative to G_m: dq = z1 e^G + xq e^(G - G_m),
                // dk_read likewise, Kc's term e^(G_m - G); X and Y from the
                // inputs and the complete gradients
                const float Gm = 0.5f * G63, es = ex(G - Gm), ems = ex(Gm - G);
                const size_t e = (tok0 + r) * DK + col;
                const bool ok = r < valid;
                const float qv = ok ? load1<F32IN>(a.q, e) : 0.f, kv = ok ? load1<F32IN>(a.k, e) : 0.f;
                const float sv = (a.ks && ok) ? a.ks[e] : 1.f;
                const float dqt = (ok ? a.dq[e] : 0.f) + xq * es;
                const float dkr = (ok ? a.dk[e] : 0.f) + xh * es;
                const float dwc = xc * ems, dwt = xt * et, wv = sv * kv;
                sXg[r * KP + col] = dqt * qv + dkr * kv - dwc * wv;
                sYg[r * KP + col] = dwt * wv;
                if (ok) {
                    a.dq[e] = dqt;
                    a.dk[e] = dkr + sv * (dwc + dwt);
                    if (a.ks) a.dks[e] = kv * (dwc + dwt);
                }
                continue;
            }
            const float eg = ex(G), emg = ex(-G);
            sXg[r * KP + col] = xq * a.wQh[at] + xh * a.wKh[at] - xc * a.wKc[at];
            sYg[r * KP + col] = xt * a.wKt[at];
            if (r < valid) {
                const size_t e = (tok0 + r) * DK + col;
                const float dw = xc * emg + xt * et;   // gradient of the write key
                a.dq[e] = xq * eg;
                if (a.ks) {
                    a.dk[e] = xh * eg + a.ks[e] * dw;
                    a.dks[e] = load1<F32IN>(a.k, e) * dw;
                } else {
                    a.dk[e] = xh * eg + dw;
                }
            }
        }
    }
    lds_barrier();
    // d log alpha_rc = sum_{r' >= r} X + sum_{i < r} Y + e^G_63 <H_c, S_c>,
    // each channel's rows split into NP parts of RP rows, one thread per part
    constexpr int NP = PNT / DK, RP = CH / NP;
    static_assert(2 * NP * DK <= CH * PT, "part sums fit in sM3");
    const int ch = tid % DK, part = tid / DK;
    float px = 0.f, py = 0.f;
    for (int r = part * RP; r < (part + 1) * RP; ++r) {
        px += sXg[r * KP + ch];
        py += sYg[r * KP + ch];
    }
    float* sPx = sM3;   // N is no longer read
    float* sPy = sM3 + NP * DK;
    sPx[part * DK + ch] = px;
    sPy[part * DK + ch] = py;
    lds_barrier();
    float sufX = 0.f, before = 0.f;   // X below this part, Y above it
    for (int q = 0; q < NP; ++q) {
        if (q > part) sufX += sPx[q * DK + ch];
        if (q < part) before += sPy[q * DK + ch];
    }
    const float hsc = expf(a.wG[pofs + (size_t)(CH - 1) * DK + ch]) * shs[ch];
    float sy = 0.f;   // Y of this part from row r down
    for (int r = (part + 1) * RP - 1; r >= part * RP; --r) {
        sufX += sXg[r * KP + ch];
        sy += sYg[r * KP + ch];
        if (r < valid && a.dla_cg) a.dla_cg[(tok0 + r) * DK + ch] = sufX + before + (py - sy) + hsc;
    }
    if (w == 0 && l < valid) {
        float xb = prb[l] + prb[CH + l];
#pragma unroll
        for (int v = 0; v < 8; ++v) xb += pcb[v * CH + l];
        a.dbeta[tok0 + l] = xb;
    }
}

template <int DK, bool F32IN>
hipError_t launch_bwd_cg_t(const BwdArgs& a, hipStream_t st) {
    const unsigned nch = (unsigned)a.nseq * (unsigned)a.NC;
    const unsigned nscan = (unsigned)((a.nseq + 7) / 8) * 8u * (unsigned)(a.Dv / 16);
    hipError_t e;
    if constexpr (F32IN) {
        e = launch_k(kProfBwdPrep, bwd_prep_cg_kernel<DK, F32IN>, dim3(nch), dim3(NTH), 0, st, a);
    } else {
        constexpr int lds = BPC16<DK>::TOTAL;
        static_assert(lds <= 64 * 1024, "LDS plan of the channel-gate backward preparation");
        e = launch_k(kProfBwdPrep, bwd_prep_cg16_kernel<DK>, dim3(nch), dim3(NTH), lds, st, a);
    }
    if (e == hipSuccess)
        e = launch_k(kProfBwdFscan, bwd_fscan_cg_kernel<DK, F32IN>, dim3(nscan), dim3(SNT), 0, st, a);
    if (e == hipSuccess) e = launch_k(kProfBwdRscan, bwd_rscan_cg_kernel<DK>, dim3(nscan), dim3(SNT), 0, st, a);
    if (e == hipSuccess) e = launch_k(kProfBwdPost, bwd_post_cg_kernel<DK, F32IN>, dim3(nch), dim3(PNT), 0, st, a);
    return e;
}

// ============================================== channel-wise beta (FG2-GDN)
// With a channel-wise beta, kt = sqrt(beta) (.) k and vt = sqrt(beta) (.) v
// enter the recurrence as a key and a value of unit strength (with separate
// strengths, FG2-GDN+: beta_k on k, beta_v on v).  So the backward runs the
// kernels above on (q, kt, vt) with beta = 1, then maps the gradients of kt
// and vt back: dk = sqrt(beta_k) dkt, dv = sqrt(beta_v) dvt,
// dbeta_k = dkt k / (2 sqrt(beta_k)), dbeta_v = dvt v / (2 sqrt(beta_v)) per
// channel (strengths > 0), summed for one strength.

// q, kt = sqrt(beta_k) k, vt = sqrt(beta_v) v as fp32, and a unit strength per
// token (beta_v is beta_k itself for one strength)
// The per-token mapping passes: DK / 4 consecutive lanes take one token, four
// channels each (16-byte accesses for fp32 arrays, 8-byte for bf16), so a wave
// covers 64 / (DK / 4) tokens per step of its grid-stride loop.
template <bool F32IN>
__device__ __forceinline__ f32x4 ld4(const void* p, size_t i) {
    if constexpr (F32IN) {
        return *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
    } else {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
        return f32x4{bf16_to_f32((uint16_t)u.x), bf16_to_f32((uint16_t)(u.x >> 16)), bf16_to_f32((uint16_t)u.y),
                     bf16_to_f32((uint16_t)(u.y >> 16))};
    }
}
__device__ __forceinline__ f32x4 ldf4(const float* p, size_t i) { return *reinterpret_cast<const f32x4*>(p + i); }
__device__ __forceinline__ void stf4(float* p, size_t i, const f32x4& x) { *reinterpret_cast<f32x4*>(p + i) = x; }
__device__ __forceinline__ float sum4(const f32x4& x) { return (x[0] + x[1]) + (x[2] + x[3]); }
__device__ __forceinline__ f32x4 strength4(const f32x4& x, int logit) {
    return f32x4{strength(x[0], logit), strength(x[1], logit), strength(x[2], logit), strength(x[3], logit)};
}
__device__ __forceinline__ f32x4 sqrt4(const f32x4& x) {
    return f32x4{sqrtf(x[0]), sqrtf(x[1]), sqrtf(x[2]), sqrtf(x[3])};
}
// the four strengths of channels c4 .. c4 + 3 of token t (one value per token
// with per_token)
__device__ __forceinline__ f32x4 strengths_at(const float* base, int per_token, size_t t, int dk, int c4,
                                              int logit) {
    const f32x4 x = per_token ? f32x4{base[t], base[t], base[t], base[t]} : ldf4(base, t * dk + c4);
    return strength4(x, logit);
}

// What the recurrence sees, as fp32 copies (the mapping is described at
// launch_bwd_map_in in dr_internal.h).
template <int DK, bool F32IN>
__global__ __launch_bounds__(256) void bwd_map_in_kernel(BwdMap m) {
    constexpr int LPT = DK / 4, TPW = 64 / LPT;
    const int l = threadIdx.x & 63, c4 = 4 * (l % LPT);
    const size_t wv = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const size_t nw = ((size_t)gridDim.x * blockDim.x) >> 6;
    for (size_t t0 = wv * TPW; t0 < m.ntok; t0 += nw * TPW) {
        const size_t tl = t0 + l / LPT;
        const bool ok = tl < m.ntok;
        const size_t t = ok ? tl : t0;   // lanes past the end repeat token t0 and store nothing
        if (!m.copy) {
            if (ok && c4 == 0) m.b32[t] = strength(m.beta[t], m.logit);
            continue;
        }
        const f32x4 q = ld4<F32IN>(m.q, t * DK + c4), k = ld4<F32IN>(m.k, t * DK + c4);
        float rq = 1.f, rk = 1.f;
        if (m.l2) {
            rq = inv_norm(group_sum<LPT>(sum4(q * q)));
            rk = inv_norm(group_sum<LPT>(sum4(k * k)));
        }
        if (!ok) continue;
        if (m.l2 && c4 == 0) {
            m.rq[t] = rq;
            m.rk[t] = rk;
        }
        stf4(m.q32, t * DK + c4, q * rq);
        if (m.cbeta) {
            // Dv == DK on this route
            const f32x4 v = ld4<F32IN>(m.v, t * DK + c4);
            stf4(m.k32, t * DK + c4, sqrt4(strengths_at(m.beta, m.per_token, t, DK, c4, m.logit)) * (k * rk));
            stf4(m.v32, t * DK + c4, sqrt4(strengths_at(m.beta_v, m.per_token, t, DK, c4, m.logit)) * v);
            if (c4 == 0) m.b32[t] = 1.f;
        } else {
            stf4(m.k32, t * DK + c4, k * rk);
            for (int j4 = c4; j4 < m.Dv; j4 += 4 * LPT)
                stf4(m.v32, t * m.Dv + j4, ld4<F32IN>(m.v, t * m.Dv + j4));
            if (c4 == 0) m.b32[t] = strength(m.beta[t], m.logit);
        }
    }
}

// The gradients of the copies, on entry in dq, dk, dv (and dbeta for a scalar
// beta, with respect to the strength's value), mapped to those of the inputs
// in place.
template <int DK, bool F32IN>
__global__ __launch_bounds__(256) void bwd_map_out_kernel(BwdMap m, float* dq, float* dk, float* dv, float* dbeta,
                                                          float* dbeta_v) {
    constexpr int LPT = DK / 4, TPW = 64 / LPT;
    const int l = threadIdx.x & 63, c4 = 4 * (l % LPT);
    const size_t wv = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const size_t nw = ((size_t)gridDim.x * blockDim.x) >> 6;
    for (size_t t0 = wv * TPW; t0 < m.ntok; t0 += nw * TPW) {
        const size_t tl = t0 + l / LPT;
        const bool ok = tl < m.ntok;
        const size_t t = ok ? tl : t0;
        const size_t e = t * DK + c4;
        if (!m.cbeta) {
            // a scalar strength: its gradient (written by the kernels with
            // respect to the strength's value) through the sigmoid
            if (m.logit && ok && c4 == 0) {
                const float b = strength(m.beta[t], 1);
                dbeta[t] *= b * (1.f - b);
            }
            if (!m.l2) continue;
        }
        const float rq = m.l2 ? m.rq[t] : 1.f, rk = m.l2 ? m.rk[t] : 1.f;
        const f32x4 kh = ld4<F32IN>(m.k, e) * rk;
        const f32x4 dkt = ldf4(dk, e);
        f32x4 dkh = dkt, gk = f32x4{0.f, 0.f, 0.f, 0.f};
        if (m.cbeta) {
            const f32x4 bk = strengths_at(m.beta, m.per_token, t, DK, c4, m.logit), sbk = sqrt4(bk);
            dkh = sbk * dkt;
            gk = dkt * kh / (2.f * sbk);
            if (m.logit) gk = gk * bk * (1.f - bk);
        }
        if (m.l2) {
            const f32x4 qh = ld4<F32IN>(m.q, e) * rq;
            const f32x4 dqh = ldf4(dq, e);
            const float pq = group_sum<LPT>(sum4(qh * dqh));
            const float pk = group_sum<LPT>(sum4(kh * dkh));
            if (ok) {
                stf4(dq, e, rq * (dqh - qh * pq));
                stf4(dk, e, rk * (dkh - kh * pk));
            }
        } else if (ok) {
            stf4(dk, e, dkh);
        }
        if (!m.cbeta) continue;
        // the value side (Dv == DK on this route)
        const f32x4 dvt = ldf4(dv, e);
        const f32x4 bv = strengths_at(m.beta_v, m.per_token, t, DK, c4, m.logit), sbv = sqrt4(bv);
        f32x4 gv = dvt * ld4<F32IN>(m.v, e) / (2.f * sbv);
        if (m.logit) gv = gv * bv * (1.f - bv);
        if (ok) stf4(dv, e, sbv * dvt);
        if (m.per_token) {
            const float gks = group_sum<LPT>(sum4(gk)), gvs = group_sum<LPT>(sum4(gv));
            if (ok && c4 == 0) {
                if (m.sepv) {
                    dbeta[t] = gks;
                    dbeta_v[t] = gvs;
                } else {
                    dbeta[t] = gks + gvs;
                }
            }
        } else if (ok) {
            if (m.sepv) {
                stf4(dbeta, e, gk);
                stf4(dbeta_v, e, gv);
            } else {
                stf4(dbeta, e, gk + gv);
            }
        }
    }
}

template <int DK, bool F32IN>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
    const unsigned nch = (unsigned)a.nseq * (unsigned)a.NC;
    const unsigned nscan = (unsigned)((a.nseq + 7) / 8) * 8u * (unsigned)(a.Dv / 16);
    // bf16 inputs: the scans on the matrix cores (dr_bwd16.hip) when the prep
    // kernel writes their operands
    const bool mc = !F32IN && a.wF != nullptr;
    hipError_t e = launch_k(kProfBwdPrep, bwd_prep_kernel<DK, F32IN>, dim3(nch), dim3(NTH), 0, st, a);
    if (e != hipSuccess) return e;
    if (!mc || a.sC >= a.NC) {
        e = mc ? launch_bwd_fscan16(a, DK, st)
               : launch_k(kProfBwdFscan, bwd_fscan_kernel<DK, F32IN>, dim3(nscan), dim3(SNT), 0, st, a);
        if (e == hipSuccess)
            e = mc ? launch_bwd_rscan16(a, DK, st)
                   : launch_k(kProfBwdRscan, bwd_rscan_kernel<DK, F32IN>, dim3(nscan), dim3(SNT), 0, st, a);
        if (e == hipSuccess) e = launch_k(kProfBwdPost, bwd_post_kernel<DK, F32IN>, dim3(nch), dim3(PNT), 0, st, a);
        return e;
    }
    // Bounded workspace: segments of sC chunks.  A first forward pass over
    // every chunk leaves checkpoints of S at the segments' starts and the
    // last segment's S_c in the slots; then, last segment first, the forward
    // scan recomputes a segment's S_c from its checkpoint (not for the last
    // one), the reverse scan walks it from the gradient carried in from the
    // next segment (dS_final for the last one) and leaves the gradient at
    // its start in the carry (dS0 for the first one), and the per-chunk
    // kernel takes its chunks.
    const int nseg = (a.NC + a.sC - 1) / a.sC, last = (nseg - 1) * a.sC;
    const size_t sts = (size_t)a.nseq * DK * a.Dv;   // floats of one state per sequence
    BwdArgs f = a;
    f.ckEnd = last;
    e = launch_bwd_fscan16(f, DK, st);
    for (int sg = nseg - 1; sg >= 0 && e == hipSuccess; --sg) {
        BwdArgs s = a;
        s.wCk = nullptr;
        s.c0 = sg * a.sC;
        s.cN = std::min(a.sC, a.NC - s.c0);
        if (sg < nseg - 1) {
            s.S0 = sg == 0 ? a.S0 : a.wCk + (size_t)(sg - 1) * sts;
            e = launch_bwd_fscan16(s, DK, st);
        }
        s.dS_final = sg == nseg - 1 ? a.dS_final : a.wHc;
        s.dS0 = sg == 0 ? a.dS0 : a.wHc;
        if (e == hipSuccess) e = launch_bwd_rscan16(s, DK, st);
        if (e == hipSuccess)
            e = launch_k(kProfBwdPost, bwd_post_kernel<DK, F32IN>, dim3((unsigned)a.nseq * (unsigned)s.cN),
                         dim3(PNT), 0, st, s);
    }
    return e;
}

}  // namespace

// One wave per token: the sum of its DK per-channel values.
__global__ __launch_bounds__(256) void bwd_gate_sum_kernel(const float* dla_ch, float* dla, size_t ntok, int dk) {
    const int l = threadIdx.x & 63;
    const size_t wv = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const size_t nw = ((size_t)gridDim.x * blockDim.x) >> 6;
    for (size_t t = wv; t < ntok; t += nw) {
        float x = 0.f;
        for (int c = l; c < dk; c += 64) x += dla_ch[t * dk + c];
        x = group_sum<32>(x);
        x += __shfl_xor(x, 32);
        if (l == 0) dla[t] = x;
    }
}

hipError_t launch_bwd_gate_sum(const float* dla_ch, float* dla, size_t ntok, int dk, hipStream_t st) {
    if (ntok == 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<size_t>((ntok + 3) / 4, 4096);
    return launch_k(kProfNone, bwd_gate_sum_kernel, dim3(blocks), dim3(256), 0, st, dla_ch, dla, ntok, dk);
}

static unsigned map_blocks(const BwdMap& m) {
    const size_t per_block = 4 * (size_t)(256 / m.Dk);   // tokens per step of a 256-thread block
    return (unsigned)std::min<size_t>((m.ntok + per_block - 1) / per_block, 4096);
}

hipError_t launch_bwd_map_in(const BwdMap& m, hipStream_t st) {
    if (m.ntok == 0) return hipSuccess;
    const dim3 g(map_blocks(m)), b(256);
    if (m.Dk == 64)
        return m.f32in ? launch_k(kProfNone, bwd_map_in_kernel<64, true>, g, b, 0, st, m)
                       : launch_k(kProfNone, bwd_map_in_kernel<64, false>, g, b, 0, st, m);
    return m.f32in ? launch_k(kProfNone, bwd_map_in_kernel<128, true>, g, b, 0, st, m)
                   : launch_k(kProfNone, bwd_map_in_kernel<128, false>, g, b, 0, st, m);
}

hipError_t launch_bwd_map_out(const BwdMap& m, float* dq, float* dk, float* dv, float* dbeta, float* dbeta_v,
                              hipStream_t st) {
    if (m.ntok == 0) return hipSuccess;
    const dim3 g(map_blocks(m)), b(256);
    if (m.Dk == 64)
        return m.f32in ? launch_k(kProfNone, bwd_map_out_kernel<64, true>, g, b, 0, st, m, dq, dk, dv, dbeta, dbeta_v)
                       : launch_k(kProfNone, bwd_map_out_kernel<64, false>, g, b, 0, st, m, dq, dk, dv, dbeta,
                                  dbeta_v);
    return m.f32in ? launch_k(kProfNone, bwd_map_out_kernel<128, true>, g, b, 0, st, m, dq, dk, dv, dbeta, dbeta_v)
                   : launch_k(kProfNone, bwd_map_out_kernel<128, false>, g, b, 0, st, m, dq, dk, dv, dbeta, dbeta_v);
}

hipError_t launch_bwd(const BwdArgs& a, int Dk, bool f32in, hipStream_t st) {
    if (a.cgate) {
        if (Dk == 128) return f32in ? launch_bwd_cg_t<128, true>(a, st) : launch_bwd_cg_t<128, false>(a, st);
        return f32in ? launch_bwd_cg_t<64, true>(a, st) : launch_bwd_cg_t<64, false>(a, st);
    }
    if (Dk == 128) return f32in ? launch_bwd_t<128, true>(a, st) : launch_bwd_t<128, false>(a, st);
    return f32in ? launch_bwd_t<64, true>(a, st) : launch_bwd_t<64, false>(a, st);
}

}  // namespace dr
