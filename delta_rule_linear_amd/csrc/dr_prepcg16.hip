// dr_prepcg16.hip -- per-chunk preparation for bf16 inputs with a channel-wise
// gate (KDA, FG2-GDN, FG2-GDN+), and for write-side key scales with any gate,
// on gfx950.
//
// For one 64-token chunk of one (batch, head), with G_rc = sum_{j<=r} log
// alpha_jc the cumulative gate of key channel c inside the chunk (FG2-GDN
// page, section 2, channel-wise decay; the chunk algebra is written out at the
// top of dr_chunk.hip), it writes what the state scan reads:
//   Q e^G, Kt e^G, W e^{G_63 - G}  (and vt with channel strengths), fp16
//                                                   -> workspace Q, Ks, Kl (V)
//   e^{G_63}, the state decay over the chunk          -> workspace G
//   A_ri = b_r sum_c kt_rc w_ic e^{G_rc - G_ic}  (i < r),  T = (I + A)^-1,
//   T^ = T Diag(b)                                    -> workspace T (packed)
//   P_ri = sum_c q_rc w_ic e^{G_rc - G_ic}       (i <= r) -> workspace P (packed)
// kt = sqrt(beta) (.) k with channel-wise strengths (b = 1), kt = k with a
// scalar one (b = beta, the beta form); w = s (.) kt with write-side key
// scales s (OSDN page, method: the preconditioner on the write side), else
// w = kt.  Rows past the sequence's end are zero in every plane and in A and P.
//
// Layout.  Wave w owns chunk rows 16 w .. 16 w + 15; lane (i16, g), l = 16 g
// + i16, holds row 16 w + i16 at channels 32 s + 8 g .. + 7 for s < d_k / 32,
// which is the operand layout of the 16x16x32 matrix-core ops, so a row's
// inputs never leave their lane:
//  * the gate's prefix over the 16 rows of a block runs across the 16 lanes of
//    a DPP row; one thread per channel then combines the four blocks (LDS);
//  * the decay of a pair of blocks (R, I) splits as e^{G_r - G_i} = e^{G_r - M}
//    e^{M - G_i} with a reference M between them, each factor in fp16 range:
//    for R > I, M = G at the end of block I and both factors are at most 1;
//    for R = I, M = G at row 16 R + 8 and both lie within e^{+-9}, unless the
//    decay inside the block is stronger: then that block's products are summed
//    directly, with the exponent formed per element;
//  * every factor is a product of one of two per-element exponentials, y_r =
//    e^{G_r - G_start} and z_r = e^{G_end - G_r} inside the row's own block
//    (both at most 1), and a per-block, per-channel constant; the constants
//    come from LDS, so an element costs two exponentials;
//  * wave R forms the pairs (R, I), I <= R, from its own rows; for R > I the
//    row side is kt y (one fp16 fragment per channel slice, the same for
//    every I) and the column side w z times the pair's constant, which wave
//    I writes to LDS for each R > I (fp16 rows, XOR-swizzled 16-byte pieces).
// The triangular inverse follows (dr_tri16.h).  Three or four workgroups
// share a CU and hide each other's dependent chains and barriers.

#include <hip/hip_runtime.h>

#include "dr_device.h"
#include "dr_internal.h"
#include "dr_tri16.h"

namespace dr {

namespace {

// A diagonal block's factors e^{G_r - M} must lie in [e^-9, e^9] (fp16's
// normal range with room for the operands); past that the block is summed
// directly.
constexpr float kDiagLo16 = 1.2340980408667956e-4f, kDiagHi16 = 8103.083927575384f;

// LDS plan (bytes).  The column-side tiles of the six off-diagonal pairs
// [6][16][RB], over the in-block gate sums [4][DK] and the sums up to each
// block's row 8 [4][DK] (read before the tiles are written), then the
// per-block, per-channel constants (log2 units, blocks b, M_b = G at row
// 16 b + 8, E_b = G at the end of block b, E_{-1} = 0):
//   CT_T  + b   E_b - E_{b-1}                the block's own decay
//   CT_C1 + b   2^{E_{b-1}}                  e^{G_r} = CT_C1 y_r
//   CT_C2 + b   2^{E_3 - E_b}                e^{G_63 - G_r} = CT_C2 z_r
//   CT_C3 + b   2^{M_b - E_b}                e^{M_b - G_r} = CT_C3 z_r
//   CT_C4 + b   2^{E_{b-1} - M_b}            e^{G_r - M_b} = CT_C4 y_r
//   CT_C5 + p   2^{E_{R-1} - E_I}, pair p = (R, I), R > I:
//               e^{G_r - G_i} = y_r CT_C5 z_i  (r in block R, i in block I)
// Tiles and constants are dead once the products are formed: A (fp32, its
// ten lower 16 x 16 blocks packed with a row pitch of 17), T (fp32) and the
// solve's scratch then take their place.  After all of them: the row
// strengths [64], 1/|q_r| and 1/|k_r| [64] each.  38.7 KB at d_k = 128.
enum { CT_T = 0, CT_C1 = 4, CT_C2 = 8, CT_C3 = 12, CT_C4 = 16, CT_C5 = 20, CT_ROWS = 26 };

template <int DK>
struct PC16 {
    static constexpr int RB = DK * 2;
    static constexpr int KI = 0;
    static constexpr int GS = 0;                  // in-block sums [4][DK]
    static constexpr int GH = GS + 4 * DK * 4;    // in-block sums to row 8 [4][DK]
    static constexpr int CT = 96 * RB;
    static constexpr int CTE = CT + CT_ROWS * DK * 4;
    static constexpr int AB = 16 * 17;
    static constexpr int SA = 0;
    static constexpr int ST = SA + 10 * AB * 4;
    static constexpr int SX = ST + 64 * 65 * 4;
    static constexpr int SXE = SX + 4 * 16 * 17 * 4;
    static constexpr int SB = SXE > CTE ? SXE : CTE;
    static constexpr int SN = SB + 64 * 4;
    static constexpr int TOTAL = SN + 128 * 4;
    static_assert(GH + 4 * DK * 4 <= 96 * RB, "the gate sums fit under the tiles");
};

// Waves per SIMD the register allocation aims at: four for the plain
// channel gate at d_k = 128 (four workgroups per CU, which LDS allows), three
// for the variants with more inputs per element.
template <int DK, bool CBETA, bool SEPV, bool QN, bool KS>
constexpr int pc16_waves() { return !CBETA && !SEPV && !QN && !KS ? 4 : 3; }

// Lane i of each 16-lane row receives lane i - N of that row, 0 for i < N.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, false));
}

// Piece p of row r of a [rows][RB]-byte tile is stored at piece p ^ swz(r):
// the 16 rows a fragment read touches fall on distinct banks.
template <int RB>
__device__ __forceinline__ char* tile_piece(char* tile, int r, int p) {
    const int sw = RB == 256 ? (r & 15) : ((r >> 1) & 7);
    return tile + r * RB + 16 * (p ^ sw);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void ld8_f32(const float* p, float* x) {
    const float4 u = reinterpret_cast<const float4*>(p)[0];
    const float4 v = reinterpret_cast<const float4*>(p)[1];
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
}

__device__ __forceinline__ void st8_f32(float* p, const float* x) {
    reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

}  // namespace

template <int DK, bool CBETA, bool SEPV, bool QN, bool KS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(pc16_waves<DK, CBETA, SEPV, QN, KS>(), 8)))
void prepcg16_kernel(ChunkArgs a) {
    using L = PC16<DK>;
    constexpr int NS = DK / 32;
    constexpr float kL2E = 1.4426950408889634f;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float* sAp = reinterpret_cast<float*>(smem + L::SA);
    auto A_at = [&](int r, int c) -> float& {
        return sAp[tri_block(r >> 4, c >> 4) * L::AB + (r & 15) * 17 + (c & 15)];
    };
    float(*sT)[65] = reinterpret_cast<float(*)[65]>(smem + L::ST);
    float(*sX)[16][17] = reinterpret_cast<float(*)[16][17]>(smem + L::SX);
    char* sKi = smem + L::KI;
    float* sGS = reinterpret_cast<float*>(smem + L::GS);
    float* sGH = reinterpret_cast<float*>(smem + L::GH);
    float* sCT = reinterpret_cast<float*>(smem + L::CT);
    float* sb = reinterpret_cast<float*>(smem + L::SB);
    float* snq = reinterpret_cast<float*>(smem + L::SN);
    float* snk = snq + 64;

    const int c = blockIdx.x, h = blockIdx.y, bz = blockIdx.z;
    const int seq = bz * a.H + h;
    const size_t cs = (size_t)seq * a.NC + c;
    const int t0 = c * CH;
    const int Lc = min(CH, a.L - t0);
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: its branches are scalar
    const int i16 = l & 15, g = l >> 4;
    const int r = 16 * w + i16;
    const bool live = r < Lc;
    const size_t tok0 = (size_t)seq * a.L + t0;
    const size_t row = tok0 + (live ? r : 0);   // rows past the end load row 0 and are masked
    const int blg = a.beta_logit;
    const size_t pbase = cs * (size_t)(CH * DK) + (size_t)r * DK;   // this row of a workspace plane

    // log alpha of one element (the direct sums of a strongly decaying block)
    auto la_at = [&](size_t tr, int col) -> float {
        if constexpr (KS) {
            return a.gate_mode == 2 ? a.log_alpha[tr * DK + col] : a.gate_mode == 1 ? a.log_alpha[tr] : 0.f;
        } else {
            return a.log_alpha[tr * DK + col];
        }
    };

    // ------------------------------------------------------------ loads
    uint4 kr[NS], qr[NS];
    float G[NS][8];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int c0 = 32 * s + 8 * g;
        kr[s] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + row * DK + c0);
        qr[s] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + row * DK + c0);
        if constexpr (KS) {
            if (a.gate_mode == 2) {
                load_f32_n<8>(a.log_alpha + row * DK + c0, G[s]);
            } else {
                const float x = a.gate_mode == 1 ? a.log_alpha[row] : 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) G[s][j] = x;
            }
        } else {
            load_f32_n<8>(a.log_alpha + row * DK + c0, G[s]);
        }
    }

    if (!live) {
#pragma unroll
        for (int s = 0; s < NS; ++s) kr[s] = qr[s] = uint4{0u, 0u, 0u, 0u};
    }

    // input preparation: unit q and k rows (the row's squares summed over the
    // four lanes that hold it)
    float nk = 1.f, nq = 1.f;
    if constexpr (QN) {
        float ssk = 0.f, ssq = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            float kx[8], qx[8];
            unpack_bf16x8(kr[s], kx);
            unpack_bf16x8(qr[s], qx);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                ssk += kx[j] * kx[j];
                ssq += qx[j] * qx[j];
            }
        }
        ssk += __shfl_xor(ssk, 16);
        ssq += __shfl_xor(ssq, 16);
        ssk += __shfl_xor(ssk, 32);
        ssq += __shfl_xor(ssq, 32);
        nk = inv_norm(ssk);
        nq = inv_norm(ssq);
        if (g == 0) {
            snk[r] = nk;
            snq[r] = nq;
        }
    }
    if constexpr (!CBETA) {
        if (g == 0) sb[r] = live ? strength(a.beta[row], blg) : 0.f;
    }

    // ------------------------------------------ the gate's prefix over rows
    // (log2 units); inside the block: Gl_r = sum over rows 16 w .. r
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float x = live ? G[s][j] * kL2E : 0.f;
            x += row_shr<1>(x);
            x += row_shr<2>(x);
            x += row_shr<4>(x);
            x += row_shr<8>(x);
            G[s][j] = x;
        }
    if (i16 == 15) {
#pragma unroll
        for (int s = 0; s < NS; ++s) st8_f32(sGS + w * DK + 32 * s + 8 * g, G[s]);
    }
    if (i16 == 8) {
#pragma unroll
        for (int s = 0; s < NS; ++s) st8_f32(sGH + w * DK + 32 * s + 8 * g, G[s]);
    }
    __syncthreads();
    // one thread per channel: the block constants
    if (tid < DK) {
        float tot[4], E[4], M[4], run = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            tot[b] = sGS[b * DK + tid];
            M[b] = run + sGH[b * DK + tid];
            run += tot[b];
            E[b] = run;
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float ep = b > 0 ? E[b - 1] : 0.f;
            sCT[(CT_T + b) * DK + tid] = tot[b];
            sCT[(CT_C1 + b) * DK + tid] = ex2(ep);
            sCT[(CT_C2 + b) * DK + tid] = ex2(E[3] - E[b]);
            sCT[(CT_C3 + b) * DK + tid] = ex2(M[b] - E[b]);
            sCT[(CT_C4 + b) * DK + tid] = ex2(ep - M[b]);
        }
#pragma unroll
        for (int R = 1; R < 4; ++R)
#pragma unroll
            for (int I = 0; I < R; ++I) sCT[(CT_C5 + R * (R - 1) / 2 + I) * DK + tid] = ex2(E[R - 1] - E[I]);
        a.wsG[cs * kGW + tid] = ex2(E[3]);   // e^{G_63}: the state decay over the chunk
    }
    __syncthreads();

    // ----- planes, the column-side tiles and the diagonal pair (own rows);
    // the row side of the off-diagonal pairs (kt y, q y) stays as fp16 fragments
    uint4 fro[NS], fqo[NS];
    f32x4 dA = {0.f, 0.f, 0.f, 0.f}, dP = dA;
    bool bad = false;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int c0 = 32 * s + 8 * g;
        // (a) the two exponentials and the row / column bases
        float kay[8], qay[8], wz[8], y[8];
        {
            float tw[8], kx[8], qx[8], ks[8], sbk[8];
            ld8_f32(sCT + (CT_T + w) * DK + c0, tw);
            unpack_bf16x8(kr[s], kx);
            unpack_bf16x8(qr[s], qx);
            if constexpr (CBETA) {
                float bk[8];
                load_strength_n<8>(a.beta, a.beta_tok, row, DK, c0, bk);
#pragma unroll
                for (int j = 0; j < 8; ++j) sbk[j] = sqrtf(strength(bk[j], blg));
            }
            if constexpr (KS) load_f32_n<8>(a.key_scale + row * DK + c0, ks);
            half8 ao, qo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float gl = G[s][j];
                y[j] = ex2(gl);
                const float z = ex2(tw[j] - gl);
                const float kt = (CBETA ? sbk[j] : 1.f) * kx[j] * nk;
                const float qv = qx[j] * nq;
                const float wk = KS ? kt * ks[j] : kt;
                kay[j] = kt * y[j];
                qay[j] = qv * y[j];
                wz[j] = wk * z;
                ao[j] = (half_t)kay[j];
                qo[j] = (half_t)qay[j];
            }
            fro[s] = __builtin_bit_cast(uint4, ao);
            fqo[s] = __builtin_bit_cast(uint4, qo);
            if constexpr (CBETA) {
                // the value plane: sqrt(beta_v) v (beta_v = beta unless separate)
                float vx[8], sv[8];
                unpack_bf16x8(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) + row * a.Dv + c0),
                              vx);
                if constexpr (SEPV) {
                    float bv[8];
                    load_strength_n<8>(a.beta_v, a.beta_tok, row, DK, c0, bv);
#pragma unroll
                    for (int j = 0; j < 8; ++j) sv[j] = sqrtf(strength(bv[j], blg));
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) sv[j] = sbk[j];
                }
                half8 pv;
#pragma unroll
                for (int j = 0; j < 8; ++j) pv[j] = (half_t)(live ? sv[j] * vx[j] : 0.f);
                *reinterpret_cast<half8*>(a.wsV + pbase + c0) = pv;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // (b) the planes: Q e^G, Kt e^G, W e^{G_63 - G}
        {
            float c1[8], c2[8];
            ld8_f32(sCT + (CT_C1 + w) * DK + c0, c1);
            ld8_f32(sCT + (CT_C2 + w) * DK + c0, c2);
            half8 pq, pk, pl;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                pq[j] = (half_t)(qay[j] * c1[j]);
                pk[j] = (half_t)(kay[j] * c1[j]);
                pl[j] = (half_t)(wz[j] * c2[j]);
            }
            *reinterpret_cast<half8*>(a.wsQ + pbase + c0) = pq;
            *reinterpret_cast<half8*>(a.wsKs + pbase + c0) = pk;
            *reinterpret_cast<half8*>(a.wsKl + pbase + c0) = pl;
        }
        __builtin_amdgcn_sched_barrier(0);
        // (c) the diagonal pair, reference M = G at row 16 w + 8
        {
            float c3[8], c4[8];
            ld8_f32(sCT + (CT_C3 + w) * DK + c0, c3);
            ld8_f32(sCT + (CT_C4 + w) * DK + c0, c4);
            half8 fa, fq, fb;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float fr = y[j] * c4[j];   // e^{G_r - M}
                bad = bad || !(fr >= kDiagLo16 && fr <= kDiagHi16);
                fa[j] = (half_t)(kay[j] * c4[j]);
                fq[j] = (half_t)(qay[j] * c4[j]);
                fb[j] = (half_t)(wz[j] * c3[j]);
            }
            dA = mfma16(fa, fb, dA);
            dP = mfma16(fq, fb, dP);
        }
        __builtin_amdgcn_sched_barrier(0);
        // (d) column sides of the pairs (R, w), R > w
#pragma unroll
        for (int R = 1; R < 4; ++R) {
            if (R > w) {   // wave-uniform
                const int p = R * (R - 1) / 2 + w;
                float c5[8];
                ld8_f32(sCT + (CT_C5 + p) * DK + c0, c5);
                half8 kc;
#pragma unroll
                for (int j = 0; j < 8; ++j) kc[j] = (half_t)(wz[j] * c5[j]);
                *reinterpret_cast<half8*>(tile_piece<L::RB>(sKi, 16 * p + i16, 4 * s + g)) = kc;
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // one slice of channels at a time: fewer live registers
    }
    // a block whose in-block decay leaves the factor range takes the direct sums
    const bool badw = __builtin_amdgcn_ballot_w64(bad) != 0;
    __syncthreads();   // the column-side tiles are complete

    // -------------------------- off-diagonal pairs (w, I), I < w, on matrix cores
    f32x4 oA[3], oP[3];
#pragma unroll
    for (int I = 0; I < 3; ++I) oA[I] = oP[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int I = 0; I < 3; ++I) {
            if (I < w) {   // wave-uniform
                const int p = w * (w - 1) / 2 + I;
                const uint4 fb = *reinterpret_cast<const uint4*>(tile_piece<L::RB>(sKi, 16 * p + i16, 4 * s + g));
                oA[I] = mfma16(__builtin_bit_cast(half8, fro[s]), __builtin_bit_cast(half8, fb), oA[I]);
                oP[I] = mfma16(__builtin_bit_cast(half8, fqo[s]), __builtin_bit_cast(half8, fb), oP[I]);
            }
        }
    }

    // direct sums for a strongly decaying diagonal block: element (16 w + 4 g
    // + j, 16 w + i16), the exponent summed over the tokens between
    if (badw) {
#pragma unroll 1
        for (int j = 0; j < 4; ++j) {
            const int rr = 16 * w + 4 * g + j, ii = 16 * w + i16;
            float sa = 0.f, sp = 0.f;
            if (ii <= rr && rr < Lc) {
                const size_t tr = tok0 + rr, ti = tok0 + ii;
                const float nkr = QN ? snk[rr] : 1.f, nki = QN ? snk[ii] : 1.f, nqr = QN ? snq[rr] : 1.f;
#pragma unroll 1
                for (int col = 0; col < DK; ++col) {
                    float e = 0.f;
                    for (int t = ii + 1; t <= rr; ++t) e += la_at(tok0 + t, col);
                    const float dec = expf(e);
                    float kvr = bf16_to_f32(static_cast<const uint16_t*>(a.k)[tr * DK + col]) * nkr;
                    float kvi = bf16_to_f32(static_cast<const uint16_t*>(a.k)[ti * DK + col]) * nki;
                    const float qvr = bf16_to_f32(static_cast<const uint16_t*>(a.q)[tr * DK + col]) * nqr;
                    if constexpr (CBETA) {
                        kvr *= sqrtf(strength(strength_at(a.beta, a.beta_tok, tr, DK, col), blg));
                        kvi *= sqrtf(strength(strength_at(a.beta, a.beta_tok, ti, DK, col), blg));
                    }
                    if constexpr (KS) kvi *= a.key_scale[ti * DK + col];   // write side
                    sa += kvr * kvi * dec;
                    sp += qvr * kvi * dec;
                }
            }
            dA[j] = sa;
            dP[j] = sp;
        }
    }

    // ------------------------------------ masks, row strengths; P out, A kept
    float av[4][4];   // A values of the pairs (w, 0..w), rows 16 w + 4 g + j
    auto emit = [&](const int I, const f32x4& cA, const f32x4& cP, float (&out)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = 16 * w + 4 * g + j, ii = 16 * I + i16;
            const bool lv = rr < Lc;
            float va = cA[j];
            if constexpr (!CBETA) va *= sb[rr];
            out[j] = (lv && ii < rr) ? va : 0.f;
            // P to the workspace, packed: 16 lanes write one 32-byte block row
            a.wsP[cs * (size_t)(CH * CH) + tri_off(rr, ii)] = (half_t)((lv && ii <= rr) ? cP[j] : 0.f);
        }
    };
#pragma unroll
    for (int I = 0; I < 3; ++I)
        if (I < w) emit(I, oA[I], oP[I], av[I]);
    emit(w, dA, dP, av[3]);
    __syncthreads();   // every product is formed: A, T and the scratch take the tile's place
#pragma unroll
    for (int I = 0; I < 3; ++I)
        if (I < w)
#pragma unroll
            for (int j = 0; j < 4; ++j) A_at(16 * w + 4 * g + j, 16 * I + i16) = av[I][j];
#pragma unroll
    for (int j = 0; j < 4; ++j) A_at(16 * w + 4 * g + j, 16 * w + i16) = av[3][j];
    __syncthreads();

    tri_inverse_out<!CBETA>(A_at, sT, sX, sb, a.wsT, cs, tid, w, l, i16, g);
}

template <int DK, bool CBETA, bool SEPV, bool QN, bool KS>
static hipError_t launch_pc16(const ChunkArgs& a, hipStream_t st) {
    constexpr int lds = PC16<DK>::TOTAL;
    static_assert(lds <= 64 * 1024, "LDS plan of the channel-gate preparation");
    return launch_k(kProfPrep, prepcg16_kernel<DK, CBETA, SEPV, QN, KS>, dim3(a.NC, a.H, a.B), dim3(256), lds, st,
                    a);
}

template <int DK, bool QN>
static hipError_t launch_pc16_q(const ChunkArgs& a, bool cbeta, bool sepv, hipStream_t st) {
    if (a.key_scale) return cbeta ? launch_pc16<DK, true, false, QN, true>(a, st)
                                  : launch_pc16<DK, false, false, QN, true>(a, st);
    if (!cbeta) return launch_pc16<DK, false, false, QN, false>(a, st);
    return sepv ? launch_pc16<DK, true, true, QN, false>(a, st) : launch_pc16<DK, true, false, QN, false>(a, st);
}

hipError_t launch_prepcg16(const ChunkArgs& a, int Dk, bool cbeta, bool sepv, hipStream_t st) {
    if (Dk == 64) return a.qk_norm ? launch_pc16_q<64, true>(a, cbeta, sepv, st)
                                   : launch_pc16_q<64, false>(a, cbeta, sepv, st);
    return a.qk_norm ? launch_pc16_q<128, true>(a, cbeta, sepv, st) : launch_pc16_q<128, false>(a, cbeta, sepv, st);
}

}  // namespace dr
