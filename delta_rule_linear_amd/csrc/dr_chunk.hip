// dr_chunk.hip -- chunked forward of the delta-rule recurrence on gfx950.
//
// Recurrence (FG2-GDN page, section 2, scaled key/value and state-update
// equations; DeltaNet page, step list, steps 3-6):
//   S_t = (I - kt kt^T) Diag(alpha_t) S_{t-1} + kt vt^T,  o_t = S_t^T q_t,
//   kt = sqrt(beta) (.) k, vt = sqrt(beta) (.) v,
// or vt = sqrt(beta_v) (.) v with a separate channel-wise write strength
// (FG2-GDN page, section "Erweiterung: FG2-GDN+"; beta stays on both kt).
//
// Chunk algebra (the chunkwise / WY form the DeltaNet page's step 7 and the
// FG2-GDN page's section 2 refer to, written out here for 64-token chunks).
// Inside a chunk with start state S, rows r = 0..63, cumulative log gate
// G_r = sum_{j<=r} log alpha_j (scalar or per key channel):
//   A_ri = sum_c kt_rc kt_ic e^{G_rc - G_ic}   (i < r),   T = (I + A)^-1
//   P_ri = sum_c q_rc  kt_ic e^{G_rc - G_ic}   (i <= r)
//   U    = T (Vt - (Kt (.) e^G) S)                      (the per-chunk "new values")
//   O    = (Q (.) e^G) S + P U
//   S'   = Diag(e^{G_63}) S + (Kt (.) e^{G_63 - G})^T U
// For a scalar beta the kernels use the equivalent "beta form": A carries beta
// on its rows, T^ = T Diag(beta), Kt -> k and Vt -> v (a diagonal similarity
// transform of the above, exact in exact arithmetic), so the raw bf16 inputs
// are matrix-core operands without any rounding.
//
// Kernels in this file:
//   prep  one workgroup per (chunk, head, batch): G, A and P on the matrix
//         cores, T = (I + A)^-1 by blocked forward substitution in fp32,
//         writes T^ and P, the gate factors, and for channel-wise gates /
//         betas the gated fp16 operands the scan needs.  Used for fp32 inputs
//         and for bf16 inputs with a scalar gate and a channel-wise beta;
//         other bf16 inputs use prep16_kernel (dr_prep16.hip, scalar gate and
//         beta) or prepcg16_kernel (dr_prepcg16.hip, channel-wise gate or
//         write-side key scales).
//   scan  (fp32 inputs) one workgroup per (sequence, 16-column tile of S):
//         walks the chunks in order holding its fp32 S tile in registers; per
//         chunk X = Ks S, R = V - g X, U = T^ R, O = g Q S + P U,
//         S = g63 S + Kl^T U.  Columns of S evolve independently (the
//         transition acts on the key side only), so tiles of one head never
//         exchange data.  bf16 inputs use scan16_kernel (dr_scan16.hip).
//
// Matrix-core operands here are fp16; fp32 inputs use two fp16 terms (hi +
// lo).  Accumulation and the state are fp32.

#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {

// ===========================================================================
// prep kernel
// ===========================================================================


// Largest |G_r - G_m| (m = block middle) for which a diagonal block's factors
// e^{G_r - G_m}, e^{G_m - G_i} stay in fp16's normal range.
constexpr float kDiagRange = 9.0f;

// Shared-memory plan of the prep kernel (in floats).
//   channel gate: [Kg | Ki | Qg | constants | A | P | g | beta | flags], with T
//                 and the blocked-solve scratch X reusing Kg/Ki/Qg once A and P exist;
//   scalar gate:  [A | P | T | X | g | beta | flags].
template <int DK, bool CGATE>
struct PrepSmem {
    static constexpr int KP = DK + 4;    // fp32 row pitch of the factor arrays
    static constexpr int NCST = 14;      // per-channel constants (channel gate)
    static constexpr int kKg = 0;
    static constexpr int kKi = kKg + (CGATE ? 64 * KP : 0);
    static constexpr int kQg = kKi + (CGATE ? 64 * KP : 0);
    static constexpr int kCst = kQg + (CGATE ? 64 * KP : 0);
    static constexpr int kA = kCst + (CGATE ? NCST * DK : 0);
    static constexpr int kP = kA + 64 * 65;
    static constexpr int kT = CGATE ? kKg : kP + 64 * 65;
    static constexpr int kX = kT + 64 * 65;
    static constexpr int kG = CGATE ? kP + 64 * 65 : kX + 3 * 16 * 17;
    static constexpr int kB = kG + 64;
    static constexpr int kNq = kB + 64;   // 1 / |q_r| (input preparation)
    static constexpr int kNk = kNq + 64;  // 1 / |k_r|
    static constexpr int kFlag = kNk + 64;
    static constexpr int FLOATS = kFlag + 4;
    static_assert(!CGATE || kX + 3 * 16 * 17 <= kCst, "T and X must fit inside Kg, Ki, Qg");
    static_assert(KP % 4 == 0 && kKi % 4 == 0 && kQg % 4 == 0 && kCst % 4 == 0 && DK % 4 == 0,
                  "factor rows are read as 16-byte vectors");
};

// Per-channel constants of the channel-gate prep (G is the cumulative log
// gate inside the chunk, blocks are 16 tokens, m = 16R + 8 a block middle):
//   CST_C + p   e^{G_{16R} - G_{16I+15}} for off-diagonal pair p = (R, I)
//   CST_IGM + R e^{G_{16R} - G_m}        diagonal row-factor rescale
//   CST_IIM + R e^{G_m - G_{16R+15}}     diagonal column-factor rescale
// Row factors are stored relative to the block start, column factors relative
// to the block end, so every factor of an off-diagonal pair is <= 1.
enum { CST_C = 0, CST_IGM = 6, CST_IIM = 10 };

// Eight floats from 16-byte aligned shared memory.
__device__ __forceinline__ void ld8_lds(const float* p, float* x) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Off-diagonal pair index of (R, I), R > I: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
__device__ __forceinline__ int offdiag_index(int R, int I) { return R * (R - 1) / 2 + I; }

// Threads of the prep workgroup: with a channel gate one per 4 tokens x 4
// channels (512 at d_k = 128: two waves per SIMD hide each other's
// latencies), otherwise 256.
template <int DK, bool CGATE>
constexpr int prep_threads() { return CGATE ? 4 * DK : 256; }

// One thread's raw inputs of a chunk for the channel-gate prep: tokens
// 4 tg .. 4 tg + 3, channels 4 cg .. 4 cg + 3 (cg = tid % (DK / 4),
// tg = tid / (DK / 4)).  Rows past the sequence's end load row 0 of the chunk
// and are masked at use.
// With a separate write strength (SEPV) v is not held here: v and beta_v are
// loaded at the start of the chunk's preparation instead.  KS marks the
// variant with write-side key scales, whose gate may be scalar or absent (it
// runs on this path with the gate broadcast to every channel).
template <int DK, bool F32IN, bool CBETA, bool SEPV = false, bool KS = false>
struct CgIn {
    static constexpr int CPT = 4;
    float la[4][CPT];               // log alpha
    RawN<F32IN, CPT> k[4], q[4];
    RawN<F32IN, CPT> v[CBETA && !SEPV ? 4 : 1];
    float be[CBETA ? 4 : 1][CPT];   // channel beta
    float bs;                       // scalar beta of token tid % 64
};

// Part PART of the loads (0: log alpha and k, 1: q and scalar beta, 2: channel
// beta and v, -1: all), so that a chunk's loads can be spread over the next
// chunk's phases instead of queueing behind one another.
template <int DK, bool F32IN, bool CBETA, bool SEPV, bool KS, int PART = -1>
__device__ __forceinline__ void cg_fetch(const ChunkArgs& a, CgIn<DK, F32IN, CBETA, SEPV, KS>& in, int job,
                                         int tid) {
    constexpr int CPT = 4;
    constexpr bool P0 = PART < 0 || PART == 0, P1 = PART < 0 || PART == 1, P2 = PART < 0 || PART == 2;
    const int seq = job / a.NC, c = job % a.NC;
    const int t0 = c * CH;
    const int Lc = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const int ch0 = (tid % (DK / 4)) * CPT, tg = tid / (DK / 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = 4 * tg + u;
        const size_t row = tok0 + (r < Lc ? r : 0);
        if constexpr (P0) {
            if constexpr (KS) {
                if (a.gate_mode == 2) {
                    load_f32_n<CPT>(a.log_alpha + row * DK + ch0, in.la[u]);
                } else {
                    const float x = a.gate_mode == 1 ? a.log_alpha[row] : 0.f;
#pragma unroll
                    for (int cc = 0; cc < CPT; ++cc) in.la[u][cc] = x;
                }
            } else {
                load_f32_n<CPT>(a.log_alpha + row * DK + ch0, in.la[u]);
            }
            in.k[u] = ld_rawn<F32IN, CPT>(a.k, row * DK + ch0);
        }
        if constexpr (P1) in.q[u] = ld_rawn<F32IN, CPT>(a.q, row * DK + ch0);
        if constexpr (CBETA && P2) {
            load_strength_n<CPT>(a.beta, a.beta_tok, row, DK, ch0, in.be[u]);
            if constexpr (!SEPV) in.v[u] = ld_rawn<F32IN, CPT>(a.v, row * a.Dv + ch0);
        }
    }
    if constexpr (!CBETA && P1) {
        const int r = tid & 63;
        in.bs = a.beta[tok0 + (r < Lc ? r : 0)];
    }
}

// The preparation of chunk c of sequence seq.  With a channel gate the
// chunk's raw inputs arrive in `in`; once they are consumed, the inputs of
// chunk `next_job` (>= 0) are loaded into it, so that those loads are in
// flight during this chunk's matrix work.
template <int DK, bool F32IN, bool CGATE, bool CBETA, bool SEPV, bool QKN, bool KS>
__device__ __forceinline__ void prep_chunk(const ChunkArgs& a, float* smem, const int seq, const int c,
                                           CgIn<DK, F32IN, CBETA, SEPV, KS>& in, const int next_job) {
    constexpr int P = F32IN ? 2 : 1;
    constexpr int NTH = prep_threads<DK, CGATE>();
    using SM = PrepSmem<DK, CGATE>;
    float(*sA)[65] = reinterpret_cast<float(*)[65]>(smem + SM::kA);
    float(*sP)[65] = reinterpret_cast<float(*)[65]>(smem + SM::kP);
    float(*sT)[65] = reinterpret_cast<float(*)[65]>(smem + SM::kT);
    float(*sX)[16][17] = reinterpret_cast<float(*)[16][17]>(smem + SM::kX);
    float* sg = smem + SM::kG;
    float* sb = smem + SM::kB;
    float* snq = smem + SM::kNq;
    float* snk = smem + SM::kNk;
    int* sflag = reinterpret_cast<int*>(smem + SM::kFlag);
    // the channel-gate preparation has no registers to spare: its input
    // normalisation is a separate variant (QKN), the others test the flag
    const bool qkn = CGATE ? QKN : a.qk_norm != 0;
    const int blg = a.beta_logit;

    const size_t cs = (size_t)seq * a.NC + c;
    const int t0 = c * CH;
    const int Lc = min(CH, a.L - t0);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const size_t tok0 = (size_t)seq * a.L + t0;
    const int Dv = a.Dv;

    if (tid < 4) sflag[tid] = 0;
    // flags are set with atomicOr by other waves below; in a loop over chunks
    // this barrier also orders the previous chunk's last reads before this
    // chunk's first writes
    lds_barrier();

    // ---------------------------------------------------------------- gates
    if constexpr (!CGATE) {
        // input preparation: 1/|q_r| and 1/|k_r|, four lanes per row
        if (qkn) {
            const int r = tid >> 2, qd = tid & 3;
            const int rc = r < Lc ? r : 0;
            float ssq = 0.f, ssk = 0.f;
#pragma unroll
            for (int i = 0; i < DK / 32; ++i) {
                const int k0 = 8 * (qd + 4 * i);
                float xk[8], xq[8];
                cvt_raw8<F32IN>(ld_raw8<F32IN>(a.k, (tok0 + rc) * DK + k0), true, xk);
                cvt_raw8<F32IN>(ld_raw8<F32IN>(a.q, (tok0 + rc) * DK + k0), true, xq);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    ssk += xk[j] * xk[j];
                    ssq += xq[j] * xq[j];
                }
            }
            ssk = group_sum<4>(ssk);
            ssq = group_sum<4>(ssq);
            if (qd == 0) {
                snk[r] = inv_norm(ssk);
                snq[r] = inv_norm(ssq);
            }
            lds_barrier();
        }
        if (w == 0) {
            const int lc = l < Lc ? l : 0;   // masked rows load a valid row, then drop it
            float g = a.has_gate ? a.log_alpha[tok0 + lc] : 0.f;
            g = l < Lc ? g : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                float y = __shfl_up(g, off);
                if (l >= off) g += y;
            }
            sg[l] = g;
            if constexpr (!CBETA) {
                const float bl = strength(a.beta[tok0 + lc], blg);
                sb[l] = l < Lc ? bl : 0.f;
            } else {
                sb[l] = 0.f;
            }
            const float g63 = __shfl(g, 63);
            const float gam = expf(g), lam = expf(g63 - g);
            a.wsG[cs * kGW + l] = gam;   // gamma_r = e^{G_r}
            if (!qkn) {
                a.wsG[cs * kGW + 64 + l] = lam;   // lambda_r = e^{G_63 - G_r}
            } else {
                // the raw key rows are scan operands without a channel beta;
                // with one, the workspace keys are normalised here.  The
                // fp32 scan reads raw query rows either way.
                const float nk = CBETA ? 1.f : snk[l];
                a.wsG[cs * kGW + 64 + l] = lam * nk;
                a.wsG[cs * kGW + 128 + l] = gam * nk;
                a.wsG[cs * kGW + 192 + l] = gam * snq[l];
            }
        }
        // channel beta with a scalar gate: the scan needs kt, vt (and q) in fp16
        if constexpr (CBETA) {
            for (int e = tid; e < CH * DK; e += 256) {
                const int r = e / DK, col = e % DK;
                const int rc = r < Lc ? r : 0;
                const float sbv = sqrtf(strength(strength_at(a.beta, a.beta_tok, tok0 + rc, DK, col), blg));
                const float sbw = sqrtf(strength(strength_at(a.beta_v, a.beta_tok, tok0 + rc, DK, col), blg));
                float kv = sbv * load1<F32IN>(a.k, (tok0 + rc) * DK + col);
                float vv = sbw * load1<F32IN>(a.v, (tok0 + rc) * Dv + col);
                float qv = load1<F32IN>(a.q, (tok0 + rc) * DK + col);
                if (qkn) {
                    kv *= snk[r];
                    qv *= snq[r];
                }
                kv = r < Lc ? kv : 0.f;
                vv = r < Lc ? vv : 0.f;
                qv = r < Lc ? qv : 0.f;
                store_split<P>(a.wsQ, cs * (size_t)(P * CH * DK), (size_t)CH * DK, r * DK + col, qv);
                store_split<P>(a.wsKs, cs * (size_t)(P * CH * DK), (size_t)CH * DK, r * DK + col, kv);
                store_split<P>(a.wsV, cs * (size_t)(P * CH * DK), (size_t)CH * DK, r * DK + col, vv);
            }
        }
    } else {
        float* sKg = smem + SM::kKg;
        float* sKi = smem + SM::kKi;
        float* sQg = smem + SM::kQg;
        float* cst = smem + SM::kCst;
        constexpr int KP = SM::KP;
        // scratch, free until A and P are formed: per token-group totals of
        // log alpha, and G at each block's start, middle, end and at token 63
        float* stot = smem + SM::kA;   // [16][DK]
        float* sbnd = smem + SM::kP;   // [13][DK]: 3 R + {0, 1, 2}, then 12: G_63
        constexpr float kL2E = 1.4426950408889634f;
        // thread = (channel group cg: CPT channels, token group tg: 4 tokens)
        constexpr int CPT = 4;
        const int cg = tid % (DK / 4), tg = tid / (DK / 4);
        const int ch0 = cg * CPT;
        const size_t pl = (size_t)CH * DK, base = cs * (size_t)(P * CH * DK);
        // with a separate write strength, v and beta_v are not among the
        // inputs held across chunks (no registers to spare there): they are
        // loaded here, and land during the gate prefix
        float bwv[SEPV ? 4 : 1][CPT];
        RawN<F32IN, CPT> vin[SEPV ? 4 : 1];
        if constexpr (SEPV) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const size_t row = tok0 + (4 * tg + u < Lc ? 4 * tg + u : 0);
                load_strength_n<CPT>(a.beta_v, a.beta_tok, row, DK, ch0, bwv[u]);
                vin[u] = ld_rawn<F32IN, CPT>(a.v, row * Dv + ch0);
            }
        }
        // write-side key scales, likewise loaded here
        float ksv[KS ? 4 : 1][CPT];
        if constexpr (KS) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const size_t row = tok0 + (4 * tg + u < Lc ? 4 * tg + u : 0);
                load_f32_n<CPT>(a.key_scale + row * DK + ch0, ksv[u]);
            }
        }
        float G[4][CPT];
        {
            float run[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) run[c] = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = 4 * tg + u;
                const float* x = in.la[u];
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    run[c] += (r < Lc) ? x[c] : 0.f;
                    G[u][c] = run[c];
                }
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) stot[tg * DK + ch0 + c] = run[c];
        }
        lds_barrier();
        if (tid < DK) {
            // one thread per channel: exclusive prefix of the 16 group totals, in place
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) x[t] = stot[t * DK + tid];
            float run = 0.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                stot[t * DK + tid] = run;
                run += x[t];
            }
        }
        lds_barrier();
        {
            const float4 o4 = *reinterpret_cast<const float4*>(stot + tg * DK + ch0);
            const float off[CPT] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = 4 * tg + u;
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    G[u][c] += off[c];
                    const int slot = (r & 15) == 0 ? 0 : (r & 15) == 8 ? 1 : (r & 15) == 15 ? 2 : -1;
                    if (slot >= 0) sbnd[(3 * (r >> 4) + slot) * DK + ch0 + c] = G[u][c];
                    if (r == 63) sbnd[12 * DK + ch0 + c] = G[u][c];
                }
            }
        }
        lds_barrier();
        // gated operands of this thread's 4 tokens x CPT channels:
        //   rowf_r = e^{G_r - G_{16R}},  colf_r = e^{G_{16R+15} - G_r}  (<= 1)
        // for the A / P products here, and Q e^{G}, Kt e^{G}, Kt e^{G_63 - G}
        // (and vt) for the scan
        // all four tokens of this thread lie in block R = tg / 4
        // e^{G_r} = e^{G_{16R}} rowf_r and e^{G_63 - G_r} = e^{G_63 - G_{16R+15}} colf_r:
        // two exponentials per element (G does not increase, so every factor is <= 1)
        const int R = tg >> 2;
        float gs2[CPT], ge2[CPT], egs[CPT], e63[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const float gs = sbnd[(3 * R) * DK + ch0 + c];
            const float ge = sbnd[(3 * R + 2) * DK + ch0 + c];
            const float g63 = sbnd[12 * DK + ch0 + c];
            gs2[c] = gs * kL2E;
            ge2[c] = ge * kL2E;
            egs[c] = __builtin_amdgcn_exp2f(gs2[c]);
            e63[c] = __builtin_amdgcn_exp2f((g63 - ge) * kL2E);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 4 * tg + u;
            const bool live = r < Lc;
            float kx[CPT], qx[CPT], vx[CPT];
            cvt_rawn<F32IN, CPT>(in.k[u], kx);
            cvt_rawn<F32IN, CPT>(in.q[u], qx);
            if (qkn) {
                // input preparation: the token's squared norms summed over
                // the DK / 4 lanes that hold its channels (DPP moves), then
                // unit vectors
                float ssk = 0.f, ssq = 0.f;
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    ssk += kx[cc] * kx[cc];
                    ssq += qx[cc] * qx[cc];
                }
                const float nk = inv_norm(group_sum<DK / 4>(ssk));
                const float nq = inv_norm(group_sum<DK / 4>(ssq));
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    kx[cc] *= nk;
                    qx[cc] *= nq;
                }
            }
            if constexpr (SEPV) cvt_rawn<F32IN, CPT>(vin[u], vx);
            else if constexpr (CBETA) cvt_rawn<F32IN, CPT>(in.v[u], vx);
            float okg[CPT], oki[CPT], oqg[CPT], wq[CPT], wks[CPT], wkl[CPT], wv[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const float sbv = CBETA ? sqrtf(strength(in.be[u][c], blg)) : 1.f;
                const float sbw = SEPV ? sqrtf(strength(bwv[u][c], blg)) : sbv;
                const float kt = live ? sbv * kx[c] : 0.f;
                const float qv = live ? qx[c] : 0.f;
                const float g2 = G[u][c] * kL2E;
                const float rowf = __builtin_amdgcn_exp2f(g2 - gs2[c]);
                const float colf = __builtin_amdgcn_exp2f(ge2[c] - g2);
                // the write-side key (column side of A and P, the state
                // update) takes the key scale; the read side keeps kt
                const float wk = KS ? kt * ksv[u][c] : kt;
                okg[c] = kt * rowf;
                oki[c] = wk * colf;
                oqg[c] = qv * rowf;
                const float eg = egs[c] * rowf;
                wq[c] = qv * eg;
                wks[c] = kt * eg;
                wkl[c] = wk * (e63[c] * colf);
                wv[c] = CBETA ? (live ? sbw * vx[c] : 0.f) : 0.f;
            }
#pragma unroll
            for (int c = 0; c < CPT; c += 4) {
                *reinterpret_cast<float4*>(sKg + r * KP + ch0 + c) = make_float4(okg[c], okg[c + 1], okg[c + 2], okg[c + 3]);
                *reinterpret_cast<float4*>(sKi + r * KP + ch0 + c) = make_float4(oki[c], oki[c + 1], oki[c + 2], oki[c + 3]);
                *reinterpret_cast<float4*>(sQg + r * KP + ch0 + c) = make_float4(oqg[c], oqg[c + 1], oqg[c + 2], oqg[c + 3]);
            }
            store_split_n<P, CPT>(a.wsQ, base, pl, r * DK + ch0, wq);
            store_split_n<P, CPT>(a.wsKs, base, pl, r * DK + ch0, wks);
            store_split_n<P, CPT>(a.wsKl, base, pl, r * DK + ch0, wkl);
            if constexpr (CBETA) store_split_n<P, CPT>(a.wsV, base, pl, r * DK + ch0, wv);
        }
        // per-channel constants, the range check of the diagonal blocks and
        // the state decay over the chunk (one thread per channel)
        if (tid < DK) {
            const int col = tid;
            int badbits = 0;
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                const float gs = sbnd[(3 * R) * DK + col];
                const float gm = sbnd[(3 * R + 1) * DK + col];
                const float ge = sbnd[(3 * R + 2) * DK + col];
                // the diagonal block's rescaled factors reach e^{|G_r - G_m|}
                if (!(gs - gm <= kDiagRange && gm - ge <= kDiagRange &&
                      gs - gm >= -kDiagRange && gm - ge >= -kDiagRange))
                    badbits |= 1 << R;
                cst[(CST_IGM + R) * DK + col] = expf(gs - gm);
                cst[(CST_IIM + R) * DK + col] = expf(gm - ge);
            }
#pragma unroll
            for (int R = 1; R < 4; ++R)
#pragma unroll
                for (int I = 0; I < R; ++I)
                    cst[(CST_C + offdiag_index(R, I)) * DK + col] =
                        expf(sbnd[(3 * R) * DK + col] - sbnd[(3 * I + 2) * DK + col]);
            a.wsG[cs * kGW + col] = expf(sbnd[12 * DK + col]);   // state decay over the chunk
            if (badbits) atomicOr(&sflag[0], badbits);
        }
        if constexpr (!CBETA) {
            if (w == 3) sb[l] = l < Lc ? strength(in.bs, blg) : 0.f;
        }
        if (next_job >= 0) cg_fetch<DK, F32IN, CBETA, SEPV, KS, 0>(a, in, next_job, tid);
    }
    lds_barrier();

    // ------------------------------------------------- A and P on the matrix cores
    // 10 lower block pairs (R, I).  A and P of a pair share the k_I fragments
    // and the decay factors; the pairs of a wave share the block row R, so its
    // k_R and q_R rows are read once per k-step.  Pairs per wave: with 8 waves
    // (3,0-1) (3,2-3) (2,0-1) (2,2) (1,0-1) (0,0); with 4 waves (3,0-2)
    // (2,0-2) (1,0-1) and (0,0) + (3,3).
    const int badmask = CGATE ? sflag[0] : 0;
    auto pair_group = [&](const int R, const int I0, const int NI) {
        const int ra = 16 * R + (l & 15);   // operand row (A side)
        const int rac = ra < Lc ? ra : 0;
        f32x4 accA[2], accP[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) accA[t] = accP[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 accA2 = {0.f, 0.f, 0.f, 0.f}, accP2 = accA2;   // third pair (4 waves only)
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            const int k0 = 32 * s + 8 * (l >> 4);
            // A side: the raw rows of block R
            float xk[8], xq[8];
            if constexpr (!CGATE) {
                cvt_raw8<F32IN>(ld_raw8<F32IN>(a.k, (tok0 + rac) * DK + k0), ra < Lc, xk);
                cvt_raw8<F32IN>(ld_raw8<F32IN>(a.q, (tok0 + rac) * DK + k0), ra < Lc, xq);
                if constexpr (CBETA) {
                    float ba[8];
                    load_strength_n<8>(a.beta, a.beta_tok, tok0 + rac, DK, k0, ba);
#pragma unroll
                    for (int j = 0; j < 8; ++j) xk[j] *= sqrtf(strength(ba[j], blg));
                }
            } else {
                ld8_lds(smem + SM::kKg + ra * SM::KP + k0, xk);
                ld8_lds(smem + SM::kQg + ra * SM::KP + k0, xq);
            }
            Frag<P> fk, fq;
            if constexpr (!CGATE) {
                fk = split8<P>(xk);
                fq = split8<P>(xq);
            }
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                if (t < NI) {   // wave-uniform
                    const int I = I0 + t;
                    if (CGATE && R == I && (badmask >> R) & 1) continue;   // exact path below
                    const int ca = 16 * I + (l & 15);   // operand row (B side)
                    float xb[8];
                    if constexpr (!CGATE) {
                        const int cac = ca < Lc ? ca : 0;
                        cvt_raw8<F32IN>(ld_raw8<F32IN>(a.k, (tok0 + cac) * DK + k0), ca < Lc, xb);
                        if constexpr (CBETA) {
                            float bb[8];
                            load_strength_n<8>(a.beta, a.beta_tok, tok0 + cac, DK, k0, bb);
#pragma unroll
                            for (int j = 0; j < 8; ++j) xb[j] *= sqrtf(strength(bb[j], blg));
                        }
                    } else {
                        const float* cst = smem + SM::kCst;
                        // rescale both factors to a reference point between
                        // the two blocks (off-diagonal: end of block I;
                        // diagonal: middle)
                        const int frow = (R == I) ? CST_IGM + R : CST_C + offdiag_index(R, I);
                        float fr[8], yk[8], yq[8];
                        ld8_lds(smem + SM::kKi + ca * SM::KP + k0, xb);
                        ld8_lds(cst + frow * DK + k0, fr);
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            yk[j] = xk[j] * fr[j];
                            yq[j] = xq[j] * fr[j];
                        }
                        if (R == I) {   // wave-uniform
                            float fc[8];
                            ld8_lds(cst + (CST_IIM + R) * DK + k0, fc);
#pragma unroll
                            for (int j = 0; j < 8; ++j) xb[j] *= fc[j];
                        }
                        fk = split8<P>(yk);
                        fq = split8<P>(yq);
                    }
                    const Frag<P> fb = split8<P>(xb);
                    if (t == 0) {
                        accA[0] = mma<P, P>(fk, fb, accA[0]);
                        accP[0] = mma<P, P>(fq, fb, accP[0]);
                    } else if (t == 1) {
                        accA[1] = mma<P, P>(fk, fb, accA[1]);
                        accP[1] = mma<P, P>(fq, fb, accP[1]);
                    } else {
                        accA2 = mma<P, P>(fk, fb, accA2);
                        accP2 = mma<P, P>(fq, fb, accP2);
                    }
                }
            }
        }
        // gate factors and masks; write the blocks to LDS
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            if (t < NI) {
                const int I = I0 + t;
                if (CGATE && R == I && (badmask >> R) & 1) continue;
                const f32x4 cA = t == 0 ? accA[0] : t == 1 ? accA[1] : accA2;
                const f32x4 cP = t == 0 ? accP[0] : t == 1 ? accP[1] : accP2;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * R + 4 * (l >> 4) + j;
                    const int i = 16 * I + (l & 15);
                    float dec = 1.f;
                    if constexpr (!CGATE) dec = (i <= r) ? expf(sg[r] - sg[i]) : 0.f;
                    float vp = cP[j] * dec;
                    float va = cA[j] * dec;
                    if constexpr (!CBETA) va *= sb[r];
                    if constexpr (!CGATE) {
                        // raw rows here: the normalisation as row and column factors
                        if (qkn) {
                            va *= snk[r] * snk[i];
                            vp *= snq[r] * snk[i];
                        }
                    }
                    sP[r][i] = (i <= r) ? vp : 0.f;
                    sA[r][i] = (i < r) ? va : 0.f;
                }
            }
        }
    };
    if constexpr (NTH / 64 == 8) {
        if (w == 0) pair_group(3, 0, 2);
        else if (w == 1) pair_group(3, 2, 2);
        else if (w == 2) pair_group(2, 0, 2);
        else if (w == 3) pair_group(2, 2, 1);
        else if (w == 4) pair_group(1, 0, 2);
        else if (w == 5) pair_group(0, 0, 1);
    } else {
        if (w == 0) pair_group(3, 0, 3);
        else if (w == 1) pair_group(2, 0, 3);
        else if (w == 2) pair_group(1, 0, 2);
        else {
            pair_group(0, 0, 1);
            pair_group(3, 3, 1);
        }
    }
    if constexpr (CGATE) {
        if (badmask) {
            lds_barrier();
            // exact path for diagonal blocks whose in-block decay exceeds the
            // fp16 factor range: sum_c kt_rc kt_ic e^{G_rc - G_ic}, the exponent
            // taken as the sum of log alpha over tokens i+1..r
            for (int R = 0; R < 4; ++R) {
                if (!((badmask >> R) & 1)) continue;
                if (tid >= 256) continue;
                const int r = 16 * R + (tid >> 4), i = 16 * R + (tid & 15);
                float accA = 0.f, accP = 0.f;
                // squared norms of the raw rows, for the input preparation
                // (summed here: this rare path keeps no factors of its own)
                float ssr = 0.f, ssi = 0.f, ssq = 0.f;
                if (i <= r && r < Lc) {
                    for (int col = 0; col < DK; ++col) {
                        float e = 0.f;
                        for (int t = i + 1; t <= r; ++t) {
                            if constexpr (KS) {
                                e += a.gate_mode == 2 ? a.log_alpha[(tok0 + t) * DK + col]
                                   : a.gate_mode == 1 ? a.log_alpha[tok0 + t] : 0.f;
                            } else {
                                e += a.log_alpha[(tok0 + t) * DK + col];
                            }
                        }
                        const float dec = expf(e);
                        float kr = load1<F32IN>(a.k, (tok0 + r) * DK + col);
                        float ki = load1<F32IN>(a.k, (tok0 + i) * DK + col);
                        const float qr = load1<F32IN>(a.q, (tok0 + r) * DK + col);
                        ssr += kr * kr;
                        ssi += ki * ki;
                        ssq += qr * qr;
                        if constexpr (CBETA) {
                            kr *= sqrtf(strength(strength_at(a.beta, a.beta_tok, tok0 + r, DK, col), blg));
                            ki *= sqrtf(strength(strength_at(a.beta, a.beta_tok, tok0 + i, DK, col), blg));
                        }
                        if constexpr (KS) ki *= a.key_scale[(tok0 + i) * DK + col];   // write side
                        accA += kr * ki * dec;
                        accP += qr * ki * dec;
                    }
                }
                if constexpr (!CBETA) accA *= sb[r];
                if (qkn) {
                    const float ni = inv_norm(ssi);
                    accA *= inv_norm(ssr) * ni;
                    accP *= inv_norm(ssq) * ni;
                }
                sA[r][i] = (i < r) ? accA : 0.f;
                sP[r][i] = (i <= r) ? accP : 0.f;
            }
        }
    }
    lds_barrier();

    // ------------------------------------------- T = (I + A)^-1, blocked, fp32
    if constexpr (CGATE) {
        if (next_job >= 0) cg_fetch<DK, F32IN, CBETA, SEPV, KS, 1>(a, in, next_job, tid);
    }
    // diagonal 16x16 blocks: wave w inverts block w, lane j < 16 owns column j
    if (w < 4 && l < 16) {
        const int base = 16 * w, j = l;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) s += sA[base + r][base + i] * t[i];
            t[r] = (r == j) ? 1.f : (r < j ? 0.f : -s);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[base + r][base + j] = t[r];
    }
    lds_barrier();
    if constexpr (CGATE) {
        if (next_job >= 0) cg_fetch<DK, F32IN, CBETA, SEPV, KS, 2>(a, in, next_job, tid);
    }
    // off-diagonal blocks, one block row R at a time on the fp32 matrix cores;
    // wave I < R computes
    //   X_RI = sum_{m in [16 I, 16 R)} A[16 R + .][m] T[m][16 I + .],  T_RI = -T_RR X_RI
    {
        const int i16 = l & 15, g = l >> 4;
        for (int R = 1; R < 4; ++R) {
            if (w < R) {
                const int I = w;
                // two accumulators (even / odd k-steps) halve the dependent chain
                f32x4 X0 = {0.f, 0.f, 0.f, 0.f}, X1 = X0;
                for (int s = 0; s < 4 * (R - I); s += 2) {
                    const int m = 16 * I + 4 * s + g;
                    X0 = mfma_f32x4(sA[16 * R + i16][m], sT[m][16 * I + i16], X0);
                    X1 = mfma_f32x4(sA[16 * R + i16][m + 4], sT[m + 4][16 * I + i16], X1);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) sX[w][4 * g + j][i16] = X0[j] + X1[j];
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's scratch is written
                __builtin_amdgcn_wave_barrier();
                asm volatile("" ::: "memory");
                f32x4 T0 = {0.f, 0.f, 0.f, 0.f}, T1 = T0;
#pragma unroll
                for (int s = 0; s < 4; s += 2) {
                    T0 = mfma_f32x4(sT[16 * R + i16][16 * R + 4 * s + g], sX[w][4 * s + g][i16], T0);
                    T1 = mfma_f32x4(sT[16 * R + i16][16 * R + 4 * s + 4 + g], sX[w][4 * s + 4 + g][i16], T1);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) sT[16 * R + 4 * g + j][16 * I + i16] = -(T0[j] + T1[j]);
            }
            lds_barrier();
        }
    }

    // --------------------------------------------------- outputs T^ and P
    if constexpr (P == 1) {
        // packed lower-block form (tri_off), one 8-column piece per thread and step
        for (int e = tid; e < 2 * 320; e += NTH) {
            const bool isP = e >= 320;
            const int x = isP ? e - 320 : e;
            const int blk = x >> 5, r = (x >> 1) & 15, hh = x & 1;
            const int R = blk < 1 ? 0 : blk < 3 ? 1 : blk < 6 ? 2 : 3;
            const int I = blk - R * (R + 1) / 2;
            const int row = 16 * R + r, c0 = 16 * I + 8 * hh;
            half8 hv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = c0 + j;
                float tt = 0.f;
                if (col <= row) {
                    tt = isP ? sP[row][col] : sT[row][col];
                    if (!isP && !CBETA) tt *= sb[col];
                }
                hv[j] = (half_t)tt;
            }
            half_t* dst = (isP ? a.wsP : a.wsT) + cs * (size_t)(CH * CH) + tri_off(row, c0);
            *reinterpret_cast<half8*>(dst) = hv;
        }
    } else if (tid < 256) {
        const int r = tid >> 2, i0 = 16 * (tid & 3);
        float tv[16], pv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int i = i0 + j;
            float tt = (i <= r) ? sT[r][i] : 0.f;
            if constexpr (!CBETA) tt *= sb[i];
            tv[j] = tt;
            pv[j] = (i <= r) ? sP[r][i] : 0.f;
        }
        const size_t base = cs * (size_t)(P * CH * CH);
        store_row16<P>(a.wsT + base, (size_t)CH * CH, r * CH + i0, tv);
        store_row16<P>(a.wsP + base, (size_t)CH * CH, r * CH + i0, pv);
    }
}

// One workgroup per chunk, or, with a channel gate, a persistent loop over
// chunks (job = chunk + NC * sequence) that loads the next chunk's inputs
// while it works on the current one.
template <int DK, bool F32IN, bool CGATE, bool CBETA, bool SEPV = false, bool QKN = false, bool KS = false>
__global__ __launch_bounds__((prep_threads<DK, CGATE>())) void prep_kernel(ChunkArgs a) {
    using SM = PrepSmem<DK, CGATE>;
    __shared__ __attribute__((aligned(16))) float smem[SM::FLOATS];
    CgIn<DK, F32IN, CBETA, SEPV, KS> in;
    if constexpr (CGATE) {
        // fp32 inputs would need twice the registers: they are loaded per chunk
        constexpr bool PREF = !F32IN;
        const int njobs = a.nseq * a.NC;
        int job = blockIdx.x;
        if (PREF && job < njobs) cg_fetch(a, in, job, threadIdx.x);
        for (; job < njobs; job += gridDim.x) {
            if (!PREF) cg_fetch(a, in, job, threadIdx.x);
            const int nj = job + gridDim.x;
            prep_chunk<DK, F32IN, CGATE, CBETA, SEPV, QKN, KS>(a, smem, job / a.NC, job % a.NC, in,
                                                           PREF && nj < njobs ? nj : -1);
        }
    } else {
        prep_chunk<DK, F32IN, CGATE, CBETA, SEPV, QKN, KS>(a, smem, blockIdx.z * a.H + blockIdx.y, blockIdx.x, in,
                                                       -1);
    }
}

// ===========================================================================
// scan kernel
// ===========================================================================

template <int DK, int P>
struct ScanSmem {
    static constexpr int SP = DK + 8;   // half pitch of S^T rows
    static constexpr int RP = CH + 8;   // half pitch of token-major rows
    static constexpr int kS = 0;                       // [P][16][SP]  S^T (B operand of K S)
    static constexpr int kR = kS + P * 16 * SP;        // [P][16][RP]  R^T
    static constexpr int kV = kR + P * 16 * RP;        // [P][16][RP]  U^T
    static constexpr int kVl = kV + P * 16 * RP;       // [P][16][RP]  (lambda U)^T
    static constexpr int kKT = kVl + P * 16 * RP;      // [P][DK][RP]  Kl^T
    static constexpr int HALFS = kKT + P * DK * RP;
};

// Per-chunk operands a thread prefetches one chunk ahead.  Loads are issued
// unconditionally (masked rows are clamped to row 0 of the chunk) and kept as
// raw bits, so nothing waits on them until the chunk is consumed.
template <int DK, bool F32IN>
struct ScanRegs {
    static constexpr int P = F32IN ? 2 : 1;
    using VT = typename std::conditional<F32IN, float, uint16_t>::type;
    int Lc;
    Raw8<F32IN> ksr[DK / 32], qsr[DK / 32];   // rows 16w.. of K, Q (raw inputs)
    Frag<P> ksh[DK / 32], qsh[DK / 32];       // the same from the workspace (gated forms)
    Frag<P> th[2], pm[2];                     // rows 16w.. of T^ and P
    VT vr[4];                                 // V tile (raw input), accumulator layout
    half_t vh[4][P];                          // V tile from the workspace (channel beta)
    float gam[4], gamq[4], lam[4];            // scalar-gate row factors (key rows, query rows, U)
    float g63[DK / 64 * 4];                   // state decay of this lane's S rows
    Raw8<F32IN> ktr[DK / 32];                 // Kl slice: token tid & 63, DK/4 channels (raw)
    half8 kth[DK / 32][P];                    // the same from the workspace
};

template <int DK, bool F32IN, bool CGATE, bool CBETA>
__device__ __forceinline__ void scan_fetch(const ChunkArgs& a, ScanRegs<DK, F32IN>& g, int seq,
                                           int c, int n0, int w, int l, int tid) {
    constexpr int P = F32IN ? 2 : 1;
    const int t0 = c * CH;
    const int Lc = min(CH, a.L - t0);
    g.Lc = Lc;
    const size_t tok0 = (size_t)seq * a.L + t0;
    const size_t cs = (size_t)seq * a.NC + c;
    const int ra = 16 * w + (l & 15);
    const int rac = ra < Lc ? ra : 0;                // clamped row for raw loads
    const size_t opl = (size_t)CH * DK;              // plane stride of [64][DK] operands
    const size_t obase = cs * (size_t)(P * CH * DK);
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
        const int k0 = 32 * s + 8 * (l >> 4);
        if constexpr (CGATE || CBETA) g.ksh[s] = load_frag_h<P>(a.wsKs, obase + ra * DK + k0, opl);
        else g.ksr[s] = ld_raw8<F32IN>(a.k, (tok0 + rac) * DK + k0);
        if constexpr (CGATE) g.qsh[s] = load_frag_h<P>(a.wsQ, obase + ra * DK + k0, opl);
        else g.qsr[s] = ld_raw8<F32IN>(a.q, (tok0 + rac) * DK + k0);
    }
    const size_t tbase = cs * (size_t)(P * CH * CH);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int k0 = 32 * s + 8 * (l >> 4);
        g.th[s] = load_frag_h<P>(a.wsT, tbase + ra * CH + k0, (size_t)CH * CH);
        g.pm[s] = load_frag_h<P>(a.wsP, tbase + ra * CH + k0, (size_t)CH * CH);
    }
    const int col = n0 + (l & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 16 * w + 4 * (l >> 4) + j;
        if constexpr (CBETA) {
#pragma unroll
            for (int p = 0; p < P; ++p) g.vh[j][p] = a.wsV[obase + p * opl + r * DK + col];
        } else {
            const int rc = r < Lc ? r : 0;
            g.vr[j] = static_cast<const typename ScanRegs<DK, F32IN>::VT*>(a.v)[(tok0 + rc) * a.Dv + col];
        }
        if constexpr (!CGATE) {
            // with normalised q and k: gamma/|k| for the key rows (gamma
            // itself when the workspace keys are already normalised), gamma/|q|
            // for the raw query rows
            g.gam[j] = a.wsG[cs * kGW + (a.qk_norm ? 128 : 0) + r];
            g.gamq[j] = a.wsG[cs * kGW + (a.qk_norm ? 192 : 0) + r];
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
    {
        const int r = tid & 63, c0 = (tid >> 6) * (DK / 4);
        const int rc = r < Lc ? r : 0;
#pragma unroll
        for (int i = 0; i < DK / 32; ++i) {
            if constexpr (CGATE || CBETA) {
                const half_t* src = (CGATE ? a.wsKl : a.wsKs) + obase + r * DK + c0 + 8 * i;
#pragma unroll
                for (int p = 0; p < P; ++p) g.kth[i][p] = *reinterpret_cast<const half8*>(src + p * opl);
            } else {
                g.ktr[i] = ld_raw8<F32IN>(a.k, (tok0 + rc) * DK + c0 + 8 * i);
            }
        }
    }
}

// One chunk of the scan for one workgroup: consumes the prefetched operands
// in `cur`, updates the fp32 state tile S (registers) and its fp16 copy in LDS.
template <int DK, bool F32IN, bool CGATE, bool CBETA>
__device__ __forceinline__ void scan_chunk(const ChunkArgs& a, const ScanRegs<DK, F32IN>& cur,
                                           f32x4 (&S)[DK / 64], half_t* smem, int seq, int c,
                                           int col, int w, int l, int tid) {
    constexpr int P = F32IN ? 2 : 1;
    constexpr int NTS = DK / 64;
    using SM = ScanSmem<DK, P>;
    half_t* sS = smem + SM::kS;
    half_t* sR = smem + SM::kR;
    half_t* sV = smem + SM::kV;
    half_t* sVl = smem + SM::kVl;
    half_t* sKT = smem + SM::kKT;
    constexpr int SPL = 16 * SM::SP;
    constexpr int RPL = 16 * SM::RP;
    constexpr int KPL = DK * SM::RP;
    const int t0 = c * CH;
    const int Lc = cur.Lc;
    const int ra = 16 * w + (l & 15);

    // Kl^T into LDS (read by the state update after the next barriers)
    {
        const int r = tid & 63, c0 = (tid >> 6) * (DK / 4);
#pragma unroll
        for (int i = 0; i < DK / 32; ++i) {
            if constexpr (CGATE || CBETA) {
                // already fp16 terms: copy each plane
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int p = 0; p < P; ++p) sKT[p * KPL + (c0 + 8 * i + j) * SM::RP + r] = cur.kth[i][p][j];
            } else {
                float x[8];
                cvt_raw8<F32IN>(cur.ktr[i], r < Lc, x);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if constexpr (P == 2) {
                        half_t hi, lo;
                        split2(x[j], hi, lo);
                        sKT[(c0 + 8 * i + j) * SM::RP + r] = hi;
                        sKT[KPL + (c0 + 8 * i + j) * SM::RP + r] = lo;
                    } else {
                        sKT[(c0 + 8 * i + j) * SM::RP + r] = (half_t)x[j];
                    }
                }
            }
        }
    }

    // step 1: X = Ks S, Y = Qs S for rows 16w..16w+15
    f32x4 X = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
        const int k0 = 32 * s + 8 * (l >> 4);
        Frag<P> sf = load_frag_h<P>(sS, (l & 15) * SM::SP + k0, SPL);
        Frag<P> kf, qf;
        if constexpr (CGATE || CBETA) kf = cur.ksh[s];
        else kf = raw_to_frag<F32IN, P>(cur.ksr[s], ra < Lc);
        if constexpr (CGATE) qf = cur.qsh[s];
        else qf = raw_to_frag<F32IN, P>(cur.qsr[s], ra < Lc);
        X = mma<P, P>(kf, sf, X);
        Y = mma<P, P>(qf, sf, Y);
    }
    // step 2: R = V - gamma X
    f32x4 Rv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 16 * w + 4 * (l >> 4) + j;
        float vv;
        if constexpr (CBETA) {
            vv = (float)cur.vh[j][0];
            if constexpr (P == 2) vv += (float)cur.vh[j][P - 1];
        } else if constexpr (F32IN) {
            vv = r < Lc ? cur.vr[j] : 0.f;
        } else {
            vv = r < Lc ? bf16_to_f32(cur.vr[j]) : 0.f;
        }
        Rv[j] = vv - (CGATE ? 1.f : cur.gam[j]) * X[j];
    }
    st4_lds<P>(sR + (l & 15) * SM::RP + 16 * w + 4 * (l >> 4), RPL, Rv);
    __syncthreads();

    // step 3: U = T^ R
    f32x4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int k0 = 32 * s + 8 * (l >> 4);
        U = mma<P, P>(cur.th[s], load_frag_h<P>(sR, (l & 15) * SM::RP + k0, RPL), U);
    }
    st4_lds<P>(sV + (l & 15) * SM::RP + 16 * w + 4 * (l >> 4), RPL, U);
    if constexpr (!CGATE) {
        f32x4 Ul;
#pragma unroll
        for (int j = 0; j < 4; ++j) Ul[j] = cur.lam[j] * U[j];
        st4_lds<P>(sVl + (l & 15) * SM::RP + 16 * w + 4 * (l >> 4), RPL, Ul);
    }
    __syncthreads();

    // step 4: O = gamma Y + P U
    f32x4 O;
#pragma unroll
    for (int j = 0; j < 4; ++j) O[j] = (CGATE ? 1.f : cur.gamq[j]) * Y[j];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int k0 = 32 * s + 8 * (l >> 4);
        O = mma<P, P>(cur.pm[s], load_frag_h<P>(sV, (l & 15) * SM::RP + k0, RPL), O);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 16 * w + 4 * (l >> 4) + j;
        if (r < Lc) {
            const size_t oi = ((size_t)seq * a.L + t0 + r) * a.Dv + col;
            if (a.out_bf16) static_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(O[j]);
            else static_cast<float*>(a.o)[oi] = O[j];
        }
    }

    // step 5: S = g63 S + Kl^T (lambda U)
    const half_t* sU = CGATE ? sV : sVl;
#pragma unroll
    for (int t = 0; t < NTS; ++t) {
        const int rt = 16 * (w * NTS + t);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int k0 = 32 * s + 8 * (l >> 4);
            Frag<P> ka = load_frag_h<P>(sKT, (rt + (l & 15)) * SM::RP + k0, KPL);
            acc = mma<P, P>(ka, load_frag_h<P>(sU, (l & 15) * SM::RP + k0, RPL), acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) S[t][j] = cur.g63[t * 4 + j] * S[t][j] + acc[j];
        st4_lds<P>(sS + (l & 15) * SM::SP + rt + 4 * (l >> 4), SPL, S[t]);
    }
    __syncthreads();
}

template <int DK, bool F32IN, bool CGATE, bool CBETA>
__global__ __launch_bounds__(256) void scan_kernel(ChunkArgs a) {
    constexpr int P = F32IN ? 2 : 1;
    constexpr int NTS = DK / 64;    // S row tiles (16 rows) per wave
    using SM = ScanSmem<DK, P>;
    __shared__ half_t smem[SM::HALFS];
    half_t* sS = smem + SM::kS;
    half_t* sR = smem + SM::kR;
    half_t* sV = smem + SM::kV;
    half_t* sVl = smem + SM::kVl;
    half_t* sKT = smem + SM::kKT;
    constexpr int SPL = 16 * SM::SP;   // plane strides
    constexpr int RPL = 16 * SM::RP;
    constexpr int KPL = DK * SM::RP;

    // XCD-aware mapping: consecutive workgroup ids go round-robin over the 8
    // XCDs, so put all column tiles of one sequence on the same XCD (they read
    // the same chunk operands) by striding sequences with the XCD index.
    const int NT = a.Dv / 16;
    const int bid = blockIdx.x;
    const int grp = bid / (8 * NT);
    const int seq = grp * 8 + (bid & 7);
    const int tile = (bid >> 3) % NT;
    if (seq >= a.nseq) return;
    const int n0 = tile * 16;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int col = n0 + (l & 15);

    // fp32 state tile in registers: rows 16*(w*NTS + t) + 4*(l>>4) + j, column col
    f32x4 S[NTS];
#pragma unroll
    for (int t = 0; t < NTS; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * (w * NTS + t) + 4 * (l >> 4) + j;
            S[t][j] = a.S0 ? a.S0[((size_t)seq * DK + row) * a.Dv + col] : 0.f;
        }
        st4_lds<P>(sS + (l & 15) * SM::SP + 16 * (w * NTS + t) + 4 * (l >> 4), SPL, S[t]);
    }

    // Two register sets, alternating: while one chunk is consumed the next
    // one's loads are in flight, with no loop-carried copies.
    ScanRegs<DK, F32IN> ra_, rb_;
    if (a.NC > 0) scan_fetch<DK, F32IN, CGATE, CBETA>(a, ra_, seq, 0, n0, w, l, tid);
    __syncthreads();
    // The fetches are unconditional (past the end they re-read the last chunk)
    // so that no control-flow join makes the compiler wait on the newer set.
    const int last = a.NC - 1;
    for (int c = 0; c < a.NC; c += 2) {
        scan_fetch<DK, F32IN, CGATE, CBETA>(a, rb_, seq, min(c + 1, last), n0, w, l, tid);
        __builtin_amdgcn_sched_barrier(0);   // keep every prefetch load at the top
        scan_chunk<DK, F32IN, CGATE, CBETA>(a, ra_, S, smem, seq, c, col, w, l, tid);
        if (c + 1 > last) break;
        scan_fetch<DK, F32IN, CGATE, CBETA>(a, ra_, seq, min(c + 2, last), n0, w, l, tid);
        __builtin_amdgcn_sched_barrier(0);
        scan_chunk<DK, F32IN, CGATE, CBETA>(a, rb_, S, smem, seq, c + 1, col, w, l, tid);
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

// ===========================================================================
// launchers
// ===========================================================================

// Workgroups of `kern` (with `threads` threads, static LDS only) resident on
// the current device at once: compute units times workgroups per unit.
// Cached per device and kernel (a device attribute and an occupancy query).
static long resident_groups(const void* kern, int threads) {
    struct Entry { const void* k; int dev; long n; };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& e : cache)
        if (e.k == kern && e.dev == dev) return e.n;
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, threads, 0) != hipSuccess || per <= 0) per = 1;
    const long n = (long)cus * per;
    cache.push_back({kern, dev, n});
    return n;
}

template <int DK, bool F32IN, bool CGATE, bool CBETA, bool SEPV = false, bool QKN = false, bool KS = false>
static hipError_t launch_chunk_t(const ChunkArgs& a, hipStream_t st) {
    const int nseq = a.nseq;
    if (a.NC > 0 && nseq > 0) {
        hipError_t e;
        if constexpr (!F32IN && !CGATE && !CBETA) {
            e = launch_prep16(a, DK, st);
        } else if constexpr (CGATE && !F32IN) {
            e = launch_prepcg16(a, DK, CBETA, SEPV, st);
        } else if constexpr (CGATE) {
            auto kern = prep_kernel<DK, F32IN, CGATE, CBETA, SEPV, QKN, KS>;
            const long njobs = (long)nseq * a.NC;
            constexpr int NTH = prep_threads<DK, CGATE>();
            const long slots = resident_groups((const void*)kern, NTH);
            const int grid = (int)(njobs < slots ? njobs : slots);
            e = launch_k(kProfPrep, kern, dim3(grid), dim3(NTH), 0, st, a);
        } else {
            dim3 g1(a.NC, a.H, a.B);
            e = launch_k(kProfPrep, prep_kernel<DK, F32IN, CGATE, CBETA>, g1, dim3(256), 0, st, a);
        }
        if (e != hipSuccess) return e;
    }
    if (nseq > 0) {
        if constexpr (!F32IN) {
            return launch_scan16(a, DK, CGATE, CBETA, st);
        } else {
            const int NT = a.Dv / 16;
            const int groups = (nseq + 7) / 8;
            return launch_k(kProfScan, scan_kernel<DK, F32IN, CGATE, CBETA>, dim3(groups * 8 * NT), dim3(256), 0,
                            st, a);
        }
    }
    return hipSuccess;
}

// A separate write strength changes only what the preparation writes for vt:
// the scalar-gate preparation reads a.beta_v as it is; the channel-gate one
// holds the next chunk's inputs in registers, so only the variant that needs
// beta_v carries room for it.
template <int DK, bool F32IN, bool QKN>
static hipError_t launch_chunk_cg(const ChunkArgs& a, bool cbeta, bool sepv, hipStream_t st) {
    if (a.key_scale) {   // write-side key scales: any gate mode, on this path
        return cbeta ? launch_chunk_t<DK, F32IN, true, true, false, QKN, true>(a, st)
                     : launch_chunk_t<DK, F32IN, true, false, false, QKN, true>(a, st);
    }
    if (!cbeta) return launch_chunk_t<DK, F32IN, true, false, false, QKN>(a, st);
    return sepv ? launch_chunk_t<DK, F32IN, true, true, true, QKN>(a, st)
                : launch_chunk_t<DK, F32IN, true, true, false, QKN>(a, st);
}

template <int DK, bool F32IN>
static hipError_t launch_chunk_d(const ChunkArgs& a, bool cgate, bool cbeta, bool sepv, hipStream_t st) {
    cgate = cgate || a.key_scale != nullptr;
    if (cgate) return a.qk_norm ? launch_chunk_cg<DK, F32IN, true>(a, cbeta, sepv, st)
                                : launch_chunk_cg<DK, F32IN, false>(a, cbeta, sepv, st);
    return cbeta ? launch_chunk_t<DK, F32IN, false, true>(a, st)
                 : launch_chunk_t<DK, F32IN, false, false>(a, st);
}

hipError_t launch_chunk(const ChunkArgs& a, int Dk, bool f32in, bool cgate, bool cbeta, bool sepv,
                        hipStream_t st) {
    if (Dk == 64) return f32in ? launch_chunk_d<64, true>(a, cgate, cbeta, sepv, st)
                               : launch_chunk_d<64, false>(a, cgate, cbeta, sepv, st);
    return f32in ? launch_chunk_d<128, true>(a, cgate, cbeta, sepv, st)
                 : launch_chunk_d<128, false>(a, cgate, cbeta, sepv, st);
}

}  // namespace dr
