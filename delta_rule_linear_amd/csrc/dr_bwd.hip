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

#include "dr_internal.h"

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

// --------------------------------------------------------------------- prep
template <int DK, bool F32IN>
__global__ __launch_bounds__(NTH) void bwd_prep_kernel(BwdArgs a) {
    constexpr int KP = DK + 1;
    static_assert(2 * CH * PT <= 2 * CH * KP, "A and T fit where q and k were");
    // q and k rows, then (once the products are in registers) A and T
    __shared__ float sKQ[2 * CH * KP];
    __shared__ float sX[4][16 * 17];
    __shared__ float sg[CH], sb[CH];
    float* sK = sKQ;
    float* sQ = sKQ + CH * KP;
    float* sA = sKQ;
    float* sT = sKQ + CH * PT;
    const int cs = blockIdx.x;
    const int seq = cs / a.NC, c = cs - seq * a.NC;
    const int t0 = c * CH, valid = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const size_t mo = (size_t)cs * CH * CH;

    load_rows<DK, F32IN>(sK, a.k, tok0, valid, tid);
    load_rows<DK, F32IN>(sQ, a.q, tok0, valid, tid);
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
                for (int s = 0; s < DK / 4; ++s) {
                    const int m = 4 * s + g;
                    const float kb = sK[(16 * I + i16) * KP + m];
                    aK[I] = mfma_f32x4(sK[(16 * R + i16) * KP + m], kb, aK[I]);
                    aQ[I] = mfma_f32x4(sQ[(16 * R + i16) * KP + m], kb, aQ[I]);
                }
            }
        }
        lds_barrier();
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * g + j, i = 16 * I + i16;
                const float e = i <= r ? expf(sg[r] - sg[i]) : 0.f;
                const float araw = i < r ? aK[I][j] * e : 0.f;
                sA[r * PT + i] = sb[r] * araw;
                a.wA[mo + r * CH + i] = araw;
                a.wP[mo + r * CH + i] = i <= r ? aQ[I][j] * e : 0.f;
            }
        }
    }
    lds_barrier();

    tri_inverse(sA, sT, sX, a.wT + mo, tid);
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
        for (int s = h * NKS; s < (h + 1) * NKS; ++s) {
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
            for (int s = 0; s < 4 * (R + 1); ++s) {
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
        for (int s = h * NKS; s < (h + 1) * NKS; ++s) {
            const int m = 4 * s + g;
            Z = mfma_f32x4(sK[(16 * R + i16) * KP + m], sH[m * 17 + i16], Z);
        }
        if (h == 1) {
            f32x4 Y = zero4();
            for (int s = 4 * R; s < 16; ++s) {
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
            for (int s = 4 * R; s < 16; ++s) {
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
            if constexpr (CG) atomicAdd(&shs[d], hsn);
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
    if constexpr (!CG) atomicAdd(&shs[0], hs);
}

template <int DK, bool F32IN>
__global__ __launch_bounds__(PNT) void bwd_post_kernel(BwdArgs a) {
    using Lp = PostLds<DK>;
    constexpr int KP = Lp::KP, ND = DK / 16, NDH = ND / 2;
    __shared__ float s1[Lp::R1];
    __shared__ float sM0[CH * PT];   // T
    __shared__ float sM1[CH * PT];   // P, then M = Diag(beta) (dA o E)
    __shared__ float sM2[CH * PT];   // K K^T o E (strict lower)
    __shared__ float sM3[CH * PT];   // N = dP o E
    __shared__ float sM4[CH * PT];   // dT^ Diag(beta), then T^T of it
    __shared__ float sg[CH], sgam[CH], slam[CH], sb[CH], sdg[CH], sdb[CH];
    __shared__ float shs;
    const int cs = blockIdx.x;
    const int seq = cs / a.NC, c = cs - seq * a.NC;
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
        sdg[tid] = 0.f;
        sdb[tid] = 0.f;
    }
    if (tid == 0) shs = 0.f;

    RowsPre<DK, F32IN, PNT> pk, pq;
    MatPre<PNT> pt, pp, pa;
    f32x4 z1[NDH], z2[NDH], z3[NDH], acc[4];
    post_state_products<DK, F32IN, false>(a, cs, valid, tok0, s1, z1, z2, z3, acc, &shs, pk, pq, pt, pp, pa);
    lds_barrier();

    // ---- q, k rows and the 64 x 64 matrices
    float* sK = s1;
    float* sQ = s1 + CH * KP;
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
        put_rows<DK, F32IN, PNT>(pk, sK, valid, tid);
        put_rows<DK, F32IN, PNT>(pq, sQ, valid, tid);
    }
    put_mat(pt, sM0, tid);
    put_mat(pp, sM1, tid);
    put_mat(pa, sM2, tid);
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
            const float qv = sQ[r * KP + col], kv = sK[r * KP + col];
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
                sM3[r * PT + i] = lo ? x * expf(sg[r] - sg[i]) : 0.f;
            } else {
                colb[I] += x * sM0[r * PT + i];
                sM4[r * PT + i] = x * sb[i];
            }
        }
    }
    lds_barrier();
    // Y = T^T dT  (rows 16 R .., column blocks 2 hf, 2 hf + 1; T[m][a] vanishes for m < a)
    f32x4 y[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int I = 2 * hf + h;
        y[h] = zero4();
        for (int s = 4 * R; s < 16; ++s) {
            const int m = 4 * s + g;
            y[h] = mfma_f32x4(sM0[m * PT + 16 * R + i16], sM4[m * PT + 16 * I + i16], y[h]);
        }
    }
    lds_barrier();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) sM4[(rb + j) * PT + 16 * (2 * hf + h) + i16] = y[h][j];
    lds_barrier();
    // dA = -Y T^T on the strict lower part, then M = Diag(beta) (dA o E) into
    // sM1 (P is no longer read)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int I = 2 * hf + h;
        f32x4 da = zero4();
        if (I <= R) {
            for (int s = 0; s < 4 * (I + 1); ++s) {
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
            sM1[r * PT + cc] = lo ? dav * sb[r] * expf(sg[r] - sg[cc]) : 0.f;
        }
    }
    lds_barrier();
    // dq += N K;  dk += M K + N^T Q + M^T K
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
    // ---- reductions of the gate and strength terms
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float xg = group_sum<16>(rowg[j]);
        const float xb = group_sum<16>(rowb[j]);
        if (i16 == 0) {
            atomicAdd(&sdg[rb + j], xg);
            atomicAdd(&sdb[rb + j], xb);
        }
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const float xg = col4_sum(colg[I]);
        const float xb = col4_sum(colb[I]);
        if (g == 0) {
            atomicAdd(&sdg[16 * I + i16], xg);
            atomicAdd(&sdb[16 * I + i16], xb);
        }
    }
    {
        float x = group_sum<32>(g63part);
        x += __shfl_xor(x, 32);
        if (l == 0) atomicAdd(&sdg[CH - 1], x);
    }
    lds_barrier();
    if (w == 0) {
        // d log alpha_t = sum over r >= t of dg_r (suffix sum over the lanes)
        float x = sdg[l];
        if (l == CH - 1) x += expf(sg[CH - 1]) * shs;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y2 = __shfl_down(x, o);
            if (l + o < 64) x += y2;
        }
        if (l < valid) {
            if (a.dlog_alpha) a.dlog_alpha[tok0 + l] = x;
            a.dbeta[tok0 + l] = sdb[l];
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
// cumulative sum per channel.  e^-G needs the within-chunk cumulative log
// decay of every channel to stay above about -88 (fp32 range).

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

template <int DK, bool F32IN>
__global__ __launch_bounds__(NTH) void bwd_prep_cg_kernel(BwdArgs a) {
    constexpr int KP = DK + 1;
    static_assert(2 * CH * PT <= 3 * CH * KP, "A and T fit where the operands were");
    __shared__ float sOp[3 * CH * KP];   // K^, Kc, Q^; then A and T
    __shared__ float sG[CH * KP];        // log alpha, then its cumulative sums
    __shared__ float sX[4][16 * 17];
    __shared__ float sb[CH];
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
    // log alpha rows into LDS (zeros past the end: no decay), then each
    // channel's cumulative sum in place
    for (int e = tid; e < CH * DK / 4; e += NTH) {
        const int r = e / (DK / 4), c4 = (e % (DK / 4)) * 4;
        float4 x = {0.f, 0.f, 0.f, 0.f};
        if (r < valid) x = *reinterpret_cast<const float4*>(a.log_alpha + (tok0 + r) * DK + c4);
        sG[r * KP + c4] = x.x;
        sG[r * KP + c4 + 1] = x.y;
        sG[r * KP + c4 + 2] = x.z;
        sG[r * KP + c4 + 3] = x.w;
    }
    lds_barrier();
    for (int ch = tid; ch < DK; ch += NTH) {
        float G = 0.f;
        for (int r = 0; r < CH; ++r) {
            G += sG[r * KP + ch];
            sG[r * KP + ch] = G;
        }
    }
    lds_barrier();
    // the gated operands, eight channels of one row per thread and step (rows
    // past the end: zero operands)
    for (int e = tid; e < CH * DK / 8; e += NTH) {
        const int r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
        float kx[8], qx[8], gq[8], gh[8], gc[8], gt[8], gg[8];
        load8<F32IN>(a.k, (tok0 + r) * DK + c8, r < valid, kx);
        load8<F32IN>(a.q, (tok0 + r) * DK + c8, r < valid, qx);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float G = sG[r * KP + c8 + j], G63 = sG[(CH - 1) * KP + c8 + j];
            const float eg = expf(G), emg = expf(-G);
            gg[j] = G;
            gq[j] = qx[j] * eg;
            gh[j] = kx[j] * eg;
            gc[j] = kx[j] * emg;
            gt[j] = kx[j] * expf(G63 - G);
            sQh[r * KP + c8 + j] = gq[j];
            sKh[r * KP + c8 + j] = gh[j];
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
        for (int s = h * NKS; s < (h + 1) * NKS; ++s) {
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
            for (int s = 0; s < 4 * (R + 1); ++s) {
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
        for (int s = h * NKS; s < (h + 1) * NKS; ++s) {
            const int m = 4 * s + g;
            Z = mfma_f32x4(sKt[(16 * R + i16) * KP + m], sH[m * 17 + i16], Z);
        }
        if (h == 1) {
            f32x4 Y = zero4();
            for (int s = 4 * R; s < 16; ++s) {
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
            for (int s = 4 * R; s < 16; ++s) {
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
    __shared__ float sb[CH], sdb[CH], shs[DK];
    const int cs = blockIdx.x;
    const int seq = cs / a.NC, c = cs - seq * a.NC;
    const int t0 = c * CH, valid = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, i16 = l & 15, g = l >> 4;
    const int R = w & 3, hf = w >> 2, D0 = hf * NDH;
    const size_t mo = (size_t)cs * CH * CH, pofs = (size_t)cs * CH * DK;

    if (tid < CH) {
        sb[tid] = tid < valid ? a.beta[tok0 + tid] : 0.f;
        sdb[tid] = 0.f;
    }
    if (tid < DK) shs[tid] = 0.f;

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
    put_plane(pkc, sKx, tid);
    put_plane(pqh, sQh, tid);
    put_mat(pt, sM0, tid);
    put_mat(pa, sM2, tid);
    lds_barrier();

    const int rb = 16 * R + 4 * g;   // this lane's first accumulator row
    float rowb[4] = {0.f, 0.f, 0.f, 0.f}, colb[4] = {0.f, 0.f, 0.f, 0.f};
    // state terms: dQ^ = z1, dK^ = -z2, dK~ = z3; dKc from the 64 x 64 part
    f32x4 dqh[NDH], dkh[NDH], dkc[NDH], dkt[NDH];
#pragma unroll
    for (int D = 0; D < NDH; ++D) {
        dqh[D] = z1[D];
        dkh[D] = -z2[D];
        dkt[D] = z3[D];
        dkc[D] = zero4();
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
        for (int s = 4 * R; s < 16; ++s) {
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
            for (int s = 0; s < 4 * (I + 1); ++s) {
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
        for (int s = 0; s < 4 * (R + 1); ++s) {
            const int m = 4 * s + g;
            const float kb = sKx[m * KP + cb];
            dqh[D] = mfma_f32x4(sM3[(16 * R + i16) * PT + m], kb, dqh[D]);
            dkh[D] = mfma_f32x4(sM1[(16 * R + i16) * PT + m], kb, dkh[D]);
        }
        for (int s = 4 * R; s < 16; ++s) {
            const int m = 4 * s + g;
            dkc[D] = mfma_f32x4(sM3[m * PT + 16 * R + i16], sQh[m * KP + cb], dkc[D]);
        }
    }
    lds_barrier();
    load_plane<DK, PNT>(sKx, a.wKh + pofs, tid);   // K^ in place of Kc
    lds_barrier();
    // dKc += M^T K^
#pragma unroll
    for (int D = 0; D < NDH; ++D) {
        const int cb = 16 * (D0 + D) + i16;
        for (int s = 4 * R; s < 16; ++s) {
            const int m = 4 * s + g;
            dkc[D] = mfma_f32x4(sM1[m * PT + 16 * R + i16], sKx[m * KP + cb], dkc[D]);
        }
    }
    // ---- dbeta's row and column sums
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float xb = group_sum<16>(rowb[j]);
        if (i16 == 0) atomicAdd(&sdb[rb + j], xb);
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const float xb = col4_sum(colb[I]);
        if (g == 0) atomicAdd(&sdb[16 * I + i16], xb);
    }
    lds_barrier();
    // ---- per element: dq, dk, and the two parts of dG,
    //   X = dQ^ Q^ + dK^ K^ - dKc Kc,  Y = dK~ K~  (dG = X - Y, plus the last row's sums)
    float* sXg = s1;
    float* sYg = s1 + CH * KP;
#pragma unroll
    for (int D = 0; D < NDH; ++D) {
        const int col = 16 * (D0 + D) + i16;
        const float G63 = a.wG[pofs + (size_t)(CH - 1) * DK + col];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = rb + j;
            const size_t at = pofs + (size_t)r * DK + col;
            const float G = a.wG[at];
            const float eg = expf(G), emg = expf(-G), et = expf(G63 - G);
            const float xq = dqh[D][j], xh = dkh[D][j], xc = dkc[D][j], xt = dkt[D][j];
            sXg[r * KP + col] = xq * a.wQh[at] + xh * a.wKh[at] - xc * a.wKc[at];
            sYg[r * KP + col] = xt * a.wKt[at];
            if (r < valid) {
                a.dq[(tok0 + r) * DK + col] = xq * eg;
                a.dk[(tok0 + r) * DK + col] = xh * eg + xc * emg + xt * et;
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
        if (r < valid) a.dlog_alpha[(tok0 + r) * DK + ch] = sufX + before + (py - sy) + hsc;
    }
    if (w == 0 && l < valid) a.dbeta[tok0 + l] = sdb[l];
}

template <int DK, bool F32IN>
hipError_t launch_bwd_cg_t(const BwdArgs& a, hipStream_t st) {
    const unsigned nch = (unsigned)a.nseq * (unsigned)a.NC;
    const unsigned nscan = (unsigned)((a.nseq + 7) / 8) * 8u * (unsigned)(a.Dv / 16);
    prof_mark(st, kProfBwdPrep);
    hipLaunchKernelGGL((bwd_prep_cg_kernel<DK, F32IN>), dim3(nch), dim3(NTH), 0, st, a);
    prof_mark(st, kProfBwdFscan);
    hipLaunchKernelGGL((bwd_fscan_cg_kernel<DK, F32IN>), dim3(nscan), dim3(SNT), 0, st, a);
    prof_mark(st, kProfBwdRscan);
    hipLaunchKernelGGL((bwd_rscan_cg_kernel<DK>), dim3(nscan), dim3(SNT), 0, st, a);
    prof_mark(st, kProfBwdPost);
    hipLaunchKernelGGL((bwd_post_cg_kernel<DK, F32IN>), dim3(nch), dim3(PNT), 0, st, a);
    prof_mark(st, kProfEnd);
    return hipGetLastError();
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
__global__ void bwd_cbeta_in_kernel(const void* q, const void* k, const void* v, const float* beta_k,
                                    const float* beta_v, int f32in, size_t n, size_t ntok, float* q32, float* k32,
                                    float* v32, float* ones) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const float qv = f32in ? load1<true>(q, i) : load1<false>(q, i);
        const float kv = f32in ? load1<true>(k, i) : load1<false>(k, i);
        const float vv = f32in ? load1<true>(v, i) : load1<false>(v, i);
        q32[i] = qv;
        k32[i] = sqrtf(beta_k[i]) * kv;
        v32[i] = sqrtf(beta_v[i]) * vv;
        if (i < ntok) ones[i] = 1.f;
    }
}

// dk, dv hold the gradients of kt and vt on entry, those of k and v on exit;
// with dbeta_v NULL (one strength) both strength terms go to dbeta_k
__global__ void bwd_cbeta_out_kernel(const void* k, const void* v, const float* beta_k, const float* beta_v,
                                     int f32in, size_t n, float* dk, float* dv, float* dbeta_k, float* dbeta_v) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const float sk = sqrtf(beta_k[i]), sv = sqrtf(beta_v[i]);
        const float kv = f32in ? load1<true>(k, i) : load1<false>(k, i);
        const float vv = f32in ? load1<true>(v, i) : load1<false>(v, i);
        const float dkt = dk[i], dvt = dv[i];
        const float gk = dkt * kv / (2.f * sk), gv = dvt * vv / (2.f * sv);
        if (dbeta_v) {
            dbeta_k[i] = gk;
            dbeta_v[i] = gv;
        } else {
            dbeta_k[i] = gk + gv;
        }
        dk[i] = sk * dkt;
        dv[i] = sv * dvt;
    }
}

template <int DK, bool F32IN>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
    const unsigned nch = (unsigned)a.nseq * (unsigned)a.NC;
    const unsigned nscan = (unsigned)((a.nseq + 7) / 8) * 8u * (unsigned)(a.Dv / 16);
    prof_mark(st, kProfBwdPrep);
    hipLaunchKernelGGL((bwd_prep_kernel<DK, F32IN>), dim3(nch), dim3(NTH), 0, st, a);
    prof_mark(st, kProfBwdFscan);
    hipLaunchKernelGGL((bwd_fscan_kernel<DK, F32IN>), dim3(nscan), dim3(SNT), 0, st, a);
    prof_mark(st, kProfBwdRscan);
    hipLaunchKernelGGL((bwd_rscan_kernel<DK, F32IN>), dim3(nscan), dim3(SNT), 0, st, a);
    prof_mark(st, kProfBwdPost);
    hipLaunchKernelGGL((bwd_post_kernel<DK, F32IN>), dim3(nch), dim3(PNT), 0, st, a);
    prof_mark(st, kProfEnd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_cbeta_in(const void* q, const void* k, const void* v, const float* beta_k,
                               const float* beta_v, bool f32in, size_t n, size_t ntok, float* q32, float* k32,
                               float* v32, float* ones, hipStream_t st) {
    hipLaunchKernelGGL(bwd_cbeta_in_kernel, dim3(2048), dim3(256), 0, st, q, k, v, beta_k, beta_v, (int)f32in, n,
                       ntok, q32, k32, v32, ones);
    return hipGetLastError();
}

hipError_t launch_bwd_cbeta_out(const void* k, const void* v, const float* beta_k, const float* beta_v, bool f32in,
                                size_t n, float* dk, float* dv, float* dbeta_k, float* dbeta_v, hipStream_t st) {
    hipLaunchKernelGGL(bwd_cbeta_out_kernel, dim3(2048), dim3(256), 0, st, k, v, beta_k, beta_v, (int)f32in, n, dk,
                       dv, dbeta_k, dbeta_v);
    return hipGetLastError();
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
