// dr_bwd16.hip -- the backward's two state scans on the matrix cores, for bf16
// inputs with a scalar gate (or none) and a scalar beta, on gfx950.
//
// Same algebra as bwd_fscan_kernel and bwd_rscan_kernel in dr_bwd.hip (the
// reverse-mode derivative of the forward's chunk algebra; DeltaNet page,
// chunkwise form; FG2-GDN page, section 2 for the gated recurrence).  Per
// chunk of 64 tokens, with T^ = T Diag(beta), gamma_r = e^{g_r} and
// lambda_r = e^{g_63 - g_r}:
//   forward   R = V - Gamma K S,  U = T^ R,  S <- gamma_63 S + K^T Lambda U
//             (the start state S of every chunk is stored; the per-chunk
//             kernel forms R and U again from it);
//   reverse   dU = P^T dO + Lambda K H,  dR = T^T dU  (= dV),
//             H <- gamma_63 H + Q^T Gamma dO - K^T Gamma dR
//             (H at every chunk's end state and dU are stored, dR is dv,
//             and H after the first chunk is dS0).
// Each launch walks chunks [c0, c0 + cN) of its sequences: all of them, or
// one segment of a bounded-workspace backward, started from a checkpoint of
// S (forward) or from the gradient carried from the next segment (reverse).
// Built like the forward's scan16_kernel (dr_scan16.hip):
//  * one workgroup per (sequence, 16-column tile of the state), the tiles of
//    one sequence on one XCD; four compute waves and four copy waves.  The
//    copy waves bring each chunk's operand tiles straight into LDS with
//    16-byte global->LDS loads ahead of use (three buffers in the forward
//    scan, two in the reverse one, whose tiles are larger), touch the lines
//    of a chunk four ahead to start their HBM reads, and store the fp32
//    results that the compute waves stage in LDS (S; H, dU and dV), with
//    16-byte stores;
//  * fp32 values enter the bf16 matrix-core ops as hi + lo pairs (16
//    significant bits, the fp32 range): the states S and H and the per-chunk
//    R, U, dO, dU, Gamma dO, Gamma dR on the chunk's side, and T^, T^T, P^T
//    from the prep kernel, in the packed triangular block form.  A product
//    of two split values takes hi hi + hi lo + lo hi.  q and k are exact
//    bf16 operands; K^T and Q^T fragments come from the row-major tiles
//    through the transposing LDS read;
//  * three barriers per chunk, raw s_barrier with an LDS-only wait.
// Tokens past the end of a sequence: their R and dU rows are set to zero, and
// T^ and P^T (zero strength, zero rows of q and k in the prep kernel) make U
// and dR zero there, so the clamped rows that the copies bring in for them
// contribute nothing.
//
// Compute wave w owns chunk rows 16 w .. 16 w + 15 and state rows
// [DK/4 w, DK/4 (w + 1)).

#include <hip/hip_runtime.h>

#include "dr_device.h"
#include "dr_internal.h"
#include "dr_lds.h"

namespace dr {
namespace {

constexpr int FP = 16 * 4 + 16;      // bytes per staged fp32 row of 16 values
constexpr int RP = (CH + 8) * 2;     // bytes per token-major row of a split plane
#ifndef DR_BWD_PFD
#define DR_BWD_PFD 4                 // chunks ahead whose lines are touched
#endif

// A fragment (A operand) of a packed 64 x 64 block-triangular matrix: row
// 16 w + i16, columns 32 s + 8 g .. +7, i.e. block (w, 2 s + g / 2), half
// g & 1.  Lower: blocks I <= w at tri_block(w, I); upper: blocks I >= w at
// tri_block(3 - w, 3 - I).  Blocks outside the triangle read a valid block;
// tri_mask zeroes them once the read has landed.
template <bool UPPER>
__device__ __forceinline__ uint4 tri_frag(const lchar* tri, int w, int s, int i16, int g) {
    const int I = 2 * s + (g >> 1);
    const int Ic = UPPER ? (I >= w ? I : w) : (I <= w ? I : w);
    const int b = UPPER ? tri_block(3 - w, 3 - Ic) : tri_block(w, Ic);
    return lds16(tri + b * 512 + i16 * 32 + 16 * ((g & 1) ^ ((i16 >> 3) & 1)));
}
// The same fragment of T^T from the packed lower T^: T^ at rows 32 s + 8 g ..
// +7 of column 16 w + i16, through the transposing LDS read (lane q of a
// 16-lane group addresses row 8 (g & 1) + q / 4 (+ 4) of the block and its
// columns 4 (q & 3) .. +3).  Blocks above T^'s diagonal (2 s + g / 2 < w) read
// a valid block; tri_mask<true> zeroes them.
__device__ __forceinline__ uint4 tri_frag_t(const lchar* tri, int w, int s, int i16, int g) {
    const int mb = 2 * s + (g >> 1);
    const int b = tri_block(mb >= w ? mb : w, w);
    const int rho = 8 * (g & 1) + (i16 >> 2);
    const int cq = 4 * (i16 & 3);
    auto at = [&](int r) { return tri + b * 512 + r * 32 + 16 * (((cq >> 3) & 1) ^ ((r >> 3) & 1)) + 2 * (cq & 7); };
    const uint2 lo4 = lds_tr4(at(rho));
    const uint2 hi4 = lds_tr4(at(rho + 4));
    return {lo4.x, lo4.y, hi4.x, hi4.y};
}

template <bool UPPER>
__device__ __forceinline__ void tri_mask(uint4& f, int w, int s, int g) {
    const int I = 2 * s + (g >> 1);
    const uint32_t m = (UPPER ? I >= w : I <= w) ? ~0u : 0u;
    f.x &= m;
    f.y &= m;
    f.z &= m;
    f.w &= m;
}

// c += a b for split a and b (hi, lo): hi hi + hi lo + lo hi
__device__ __forceinline__ f32x4 mfma3(const uint4& ah, const uint4& al, const uint4& bh, const uint4& bl, f32x4 c) {
    c = mfma_raw<true>(ah, bh, c);
    c = mfma_raw<true>(ah, bl, c);
    return mfma_raw<true>(al, bh, c);
}

// 16-byte pieces of a token-major split plane (row i16, tokens 32 s + 8 g ..)
__device__ __forceinline__ uint4 plane16(const lchar* pl, int i16, int s, int g) {
    return lds16(pl + i16 * RP + 2 * (32 * s + 8 * g));
}

// Copy wave cw's share of a staged [ROWS][16] fp32 tile to dst (row r at
// dst + r * pitch floats): 16 rows per store, four lanes per row.  Rows at or
// past `valid` are not stored.
template <int ROWS>
__device__ __forceinline__ void store_staged(const lchar* st, float* dst, size_t pitch, int valid, int l, int cw) {
#pragma unroll
    for (int ii = 0; ii < ROWS / 64; ++ii) {
        const int row = 16 * (cw + 4 * ii) + (l >> 2);
        const float4 v = lds_ld<float4>(st + row * FP + 16 * (l & 3));
        if (row < valid) *reinterpret_cast<float4*>(dst + (size_t)row * pitch + 4 * (l & 3)) = v;
    }
}

// One line-touch plan: lane x of the workgroup's copy waves touches one
// dword of a 1/NT share of each chunk's operand lines (regions in order).
struct Warm {
    const char* base;
    unsigned stride;
    int x;
    const char* lastb;
    unsigned lastst;
    __device__ __forceinline__ void region(const void* b0, unsigned st, int n) {
        const char* bb = static_cast<const char*>(b0);
        if (!base && x >= 0 && x < n) {
            base = bb + 128 * x;
            stride = st;
        }
        lastb = bb + 128 * (n - 1);
        lastst = st;
        x -= n;
    }
    __device__ __forceinline__ void done() {
        if (!base) {
            base = lastb;
            stride = lastst;
        }
    }
};

// Copy wave cw's quarter of a chunk's [64][RB]-byte tile of raw bf16 rows
// (row r at src + r * RB bytes; rows >= valid read row 0) into swizzled LDS.
template <int RB>
__device__ __forceinline__ void copy_rows(const char* src, int valid, lchar* tile, int l, int cw) {
    constexpr int PPR = RB / 16, RPI = 64 / PPR, NI = 64 / RPI;
#pragma unroll
    for (int jj = 0; jj < NI / 4; ++jj) {
        const int j = cw + 4 * jj;
        const int r = j * RPI + l / PPR;
        const int rc = r < valid ? r : 0;
        const int lp = (l % PPR) ^ swz<RB>(r);
        dma16s(src, (unsigned)(rc * RB + 16 * lp), tile + j * 1024);
    }
}

// ------------------------------------------------------------ forward scan
// LDS: three operand buffers [K 64 x RB][T^ hi][T^ lo][V 64 x 32][gate 1024]
// and the working area [S^T hi/lo][R^T hi/lo][(lambda U)^T hi/lo][S fp32].
template <int DK>
struct FL {
    static constexpr int RB = DK * 2;
    static constexpr int KT = 0;
    static constexpr int TT = KT + 64 * RB;
    static constexpr int VT = TT + 2 * kTriBytes;
    static constexpr int GT = VT + 64 * 32;
    static constexpr int BUF = GT + 1024;
    static constexpr int SP = (DK + 8) * 2;
    static constexpr int WS = 0;
    static constexpr int WR = WS + 2 * 16 * SP;
    static constexpr int WUL = WR + 2 * 16 * RP;
    static constexpr int WSF = WUL + 2 * 16 * RP;
    static constexpr int WORK = WSF + DK * FP;
    static constexpr int TOTAL = 3 * BUF + WORK + 1024;
    static constexpr int NTI = RB / 16 / 4;   // K-tile copies per copy wave
    // a copy wave's vector-memory operations per chunk: the K tile, 4 part-2
    // slots, the stores of S (DK / 64), the line touch
    static constexpr int NOPS = NTI + 4 + DK / 64 + 1;
};

template <int DK>
__global__ __launch_bounds__(512) void bwd_fscan16_kernel(BwdArgs a) {
    using L = FL<DK>;
    constexpr int NTS = DK / 64;   // 16-row state tiles per compute wave
    __shared__ __attribute__((aligned(16))) char lds_b0[L::BUF];
    __shared__ __attribute__((aligned(16))) char lds_b1[L::BUF];
    __shared__ __attribute__((aligned(16))) char lds_b2[L::BUF];
    __shared__ __attribute__((aligned(16))) char lds_work[L::WORK];
    __shared__ __attribute__((aligned(16))) char lds_sink[1024];

    const int NT = a.Dv / 16;
    const int bid = blockIdx.x;
    const int seq = (bid / (8 * NT)) * 8 + (bid & 7);
    const int tile = (bid >> 3) % NT;
    if (seq >= a.nseq) return;
    const int n0 = tile * 16, Dv = a.Dv;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const bool copier = w >= 4;
    const int cw = __builtin_amdgcn_readfirstlane(w - 4);
    const int i16 = l & 15, g = l >> 4;
    const int ra = 16 * w + i16;
    lchar* b0 = (lchar*)lds_b0;
    lchar* b1 = (lchar*)lds_b1;
    lchar* b2 = (lchar*)lds_b2;
    lchar* work = (lchar*)lds_work;
    lchar* sink = (lchar*)lds_sink;
    lchar* sS = work + L::WS;
    lchar* sR = work + L::WR;
    lchar* sUl = work + L::WUL;
    lchar* sSf = work + L::WSF;
    auto sync = [&]() { lds_barrier(); };

    const char* kbase = static_cast<const char*>(a.k) + (size_t)seq * a.L * DK * 2;
    const char* vbase = static_cast<const char*>(a.v) + (size_t)seq * a.L * Dv * 2 + n0 * 2;
    const char* fbase = a.wF + (size_t)seq * a.NC * kBF;
    auto valid_of = [&](int c) { return min(CH, a.L - c * CH); };

    // part 0: the K tile; part 2: T^ hi/lo (slots 0-9), V (10-11), gate (12, repeated in 13-15)
    auto copy0 = [&](lchar* buf, int c) {
        copy_rows<L::RB>(uniform_ptr(kbase + (size_t)c * CH * L::RB), valid_of(c), buf + L::KT, l, cw);
    };
    auto copy2 = [&](lchar* buf, int c) {
        const char* fb = uniform_ptr(fbase + (size_t)c * kBF);
        const char* vb = uniform_ptr(vbase + (size_t)c * CH * Dv * 2);
        const int Lc = valid_of(c);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int k = cw + 4 * jj;   // wave-uniform
            if (k < 10) {
                dma16s(fb, 1024u * k + 16u * l, buf + L::TT + 1024 * k);
            } else if (k < 12) {
                const int r = 32 * (k - 10) + (l >> 1), rc = r < Lc ? r : 0;
                dma16s(vb, (unsigned)(rc * Dv * 2 + 16 * (l & 1)), buf + L::VT + 1024 * (k - 10));
            } else {
                dma16s(fb, kBfGate + 16u * (l & 31), buf + L::GT);
            }
        }
    };
    Warm wm{nullptr, 0, tile + NT * (64 * cw + l), nullptr, 0};
    if (copier) {
        wm.region(kbase, CH * L::RB, L::RB / 2);
        wm.region(fbase, kBF, 2 * kTriBytes / 128);
        wm.region(vbase - n0 * 2, CH * Dv * 2, Dv);
        wm.region(fbase + kBfGate, kBF, 4);
        wm.done();
    }
    const int NCF = a.L / CH;   // whole chunks (only those are touched ahead)
    const int cE = a.c0 + a.cN;  // chunks [c0, cE), from the state S0 points to

    f32x4 S[NTS];
    if (!copier) {
#pragma unroll
        for (int t = 0; t < NTS; ++t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * (w * NTS + t) + 4 * g + j;
                S[t][j] = a.S0 ? a.S0[((size_t)seq * DK + row) * Dv + n0 + i16] : 0.f;
            }
            st4_terms<true, 2>(sS + i16 * L::SP + 2 * (16 * (w * NTS + t) + 4 * g), 16 * L::SP, S[t]);
        }
    } else {
        copy0(b0, a.c0);
        copy2(b0, a.c0);
        const int c1 = min(a.c0 + 1, cE - 1);
        copy0(b1, c1);
        copy2(b1, c1);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(L::NTI + 4));   // chunk 0 has landed
    }
    sync();

    auto chunk = [&](const int c, const lchar* buf, lchar* cbuf) {
        const int cn = min(c + 2, cE - 1);
        const int Lc = valid_of(c);
        auto gt = [&](int i) { return lds_ld<float>(buf + L::GT + 4 * i); };
        uint4 tfr[2][2], kfr[NTS][2];
        float lam[4];

        // ---------------- phase 1: X = K S, R = V - Gamma X; stage S
        if (copier) {
            copy0(cbuf, cn);
        } else {
            uint4 kf[DK / 32], sfr[DK / 32][2];
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                kf[s] = lds16(tile_at<L::RB>(buf + L::KT, ra, 4 * s + g));
#pragma unroll
                for (int p = 0; p < 2; ++p) sfr[s][p] = lds16(sS + p * 16 * L::SP + i16 * L::SP + 2 * (32 * s + 8 * g));
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int p = 0; p < 2; ++p) tfr[s][p] = tri_frag<false>(buf + L::TT + p * kTriBytes, w, s, i16, g);
            uint16_t vb[4];
            float gam[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * w + 4 * g + j;
                vb[j] = lds_ld<uint16_t>(buf + L::VT + r * 32 + 2 * i16);
                gam[j] = gt(r);
                lam[j] = gt(64 + r);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int p = 0; p < 2; ++p) tri_mask<false>(tfr[s][p], w, s, g);
            f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < DK / 32; ++s)
#pragma unroll
                for (int p = 0; p < 2; ++p) X = mfma_raw<true>(kf[s], sfr[s][p], X);
            f32x4 Rv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * w + 4 * g + j;
                Rv[j] = r < Lc ? bf16_to_f32(vb[j]) - gam[j] * X[j] : 0.f;
            }
            st4_terms<true, 2>(sR + i16 * RP + 2 * (16 * w + 4 * g), 16 * RP, Rv);
#pragma unroll
            for (int t = 0; t < NTS; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    lds_st(sSf + (16 * (w * NTS + t) + 4 * g + j) * FP + 4 * i16, S[t][j]);
        }
        sync();

        // ---------------- phase 2: U = T^ R, lambda U
        if (copier) {
            // one store of S_c per chunk: its slot, or a checkpoint
            const bool ck = a.wCk && c > 0 && c < a.ckEnd && c % a.sC == 0;
            float* dst = ck ? a.wCk + ((size_t)(c / a.sC - 1) * a.nseq + seq) * DK * Dv
                            : a.wS + ((size_t)seq * a.sC + c % a.sC) * DK * Dv;
            store_staged<DK>(sSf, dst + n0, Dv, DK, l, cw);
        } else {
            uint4 rf[2][2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int p = 0; p < 2; ++p) rf[s][p] = plane16(sR + p * 16 * RP, i16, s, g);
            // K^T fragments for phase 3 (state row rt + i16, tokens 32 s + 8 g + 0..7)
#pragma unroll
            for (int t = 0; t < NTS; ++t) {
                const int rt = 16 * (w * NTS + t);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int tok = 32 * s + 8 * g + (i16 >> 2);
                    const int d = rt + 4 * (i16 & 3);
                    const uint2 lo4 = lds_tr4(tile_at<L::RB>(buf + L::KT, tok, d >> 3) + 2 * (d & 7));
                    const uint2 hi4 = lds_tr4(tile_at<L::RB>(buf + L::KT, tok + 4, d >> 3) + 2 * (d & 7));
                    kfr[t][s] = {lo4.x, lo4.y, hi4.x, hi4.y};
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) U = mfma3(tfr[s][0], tfr[s][1], rf[s][0], rf[s][1], U);
            f32x4 Ul;
#pragma unroll
            for (int j = 0; j < 4; ++j) Ul[j] = lam[j] * U[j];
            st4_terms<true, 2>(sUl + i16 * RP + 2 * (16 * w + 4 * g), 16 * RP, Ul);
        }
        sync();

        // ---------------- phase 3: S = gamma_63 S + K^T (lambda U)
        if (copier) {
            copy2(cbuf, cn);
            if (NCF > 0) dma4(wm.base + (size_t)min(c + DR_BWD_PFD, NCF - 1) * wm.stride, sink + 256 * cw);
            else dma4(fbase, sink + 256 * cw);
            // every operation of the previous chunks has completed, so the
            // copies of chunk c + 1 have landed
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(L::NOPS));
        } else {
            uint4 ulf[2][2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int p = 0; p < 2; ++p) ulf[s][p] = plane16(sUl + p * 16 * RP, i16, s, g);
            const float d63 = gt(63);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < NTS; ++t) {
                const int rt = 16 * (w * NTS + t);
                f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int p = 0; p < 2; ++p) acc[s] = mfma_raw<true>(kfr[t][s], ulf[s][p], acc[s]);
#pragma unroll
                for (int j = 0; j < 4; ++j) S[t][j] = d63 * S[t][j] + (acc[0][j] + acc[1][j]);
                st4_terms<true, 2>(sS + i16 * L::SP + 2 * (rt + 4 * g), 16 * L::SP, S[t]);
            }
        }
        sync();
    };

    for (int c = a.c0; c < cE; c += 3) {
        chunk(c, b0, b2);
        if (c + 1 < cE) chunk(c + 1, b1, b0);
        if (c + 2 < cE) chunk(c + 2, b2, b1);
    }
    if (copier) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no copy may land after the workgroup ends
}

// ------------------------------------------------------------ reverse scan
// LDS: two operand buffers [K 64 x RB][Q 64 x RB][T^ hi][T^ lo][P^T hi]
// [P^T lo][gate 1024] (the last five are the chunk's kBF slot, one contiguous
// run) and the working area [H^T hi/lo][dO^T hi/lo][(Gamma dO)^T hi/lo]
// [dU^T hi/lo][(Gamma dR)^T hi/lo][H fp32][dU fp32][dR fp32].  The compute
// waves load their own dO values one chunk ahead into registers.
template <int DK>
struct RL {
    static constexpr int RB = DK * 2;
    static constexpr int KT = 0;
    static constexpr int QT = KT + 64 * RB;
    static constexpr int MT = QT + 64 * RB;           // T^ hi, lo, P^T hi, lo, gate
    static constexpr int GT = MT + 4 * kTriBytes;
    static constexpr int BUF = GT + 1024;
    static constexpr int SP = (DK + 8) * 2;
    static constexpr int WH = 0;
    static constexpr int WO = WH + 2 * 16 * SP;
    static constexpr int WGO = WO + 2 * 16 * RP;
    static constexpr int WDU = WGO + 2 * 16 * RP;
    static constexpr int WGR = WDU + 2 * 16 * RP;
    static constexpr int WHF = WGR + 2 * 16 * RP;
    static constexpr int WDUF = WHF + DK * FP;
    static constexpr int WDRF = WDUF + 64 * FP;
    static constexpr int WORK = WDRF + 64 * FP;
    static constexpr int TOTAL = 2 * BUF + WORK + 1024;
    static constexpr int NTI = RB / 16 / 4;            // K- (and Q-) tile copies per copy wave
    static constexpr int NSLOT = (4 * kTriBytes + 1024) / 1024;   // 21 one-KiB slots
    static constexpr int NS2 = (NSLOT + 3) / 4;        // part-2 copies per copy wave
    // operations after a chunk's last copy: the stores of H (DK / 64) and dU, the line touch
    static constexpr int NAFTER = DK / 64 + 2;
};

template <int DK>
__global__ __launch_bounds__(512) void bwd_rscan16_kernel(BwdArgs a) {
    using L = RL<DK>;
    constexpr int NTS = DK / 64;
    __shared__ __attribute__((aligned(16))) char lds_b0[L::BUF];
    __shared__ __attribute__((aligned(16))) char lds_b1[L::BUF];
    __shared__ __attribute__((aligned(16))) char lds_work[L::WORK];
    __shared__ __attribute__((aligned(16))) char lds_sink[1024];

    const int NT = a.Dv / 16;
    const int bid = blockIdx.x;
    const int seq = (bid / (8 * NT)) * 8 + (bid & 7);
    const int tile = (bid >> 3) % NT;
    if (seq >= a.nseq) return;
    const int n0 = tile * 16, Dv = a.Dv;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const bool copier = w >= 4;
    const int cw = __builtin_amdgcn_readfirstlane(w - 4);
    const int i16 = l & 15, g = l >> 4;
    const int ra = 16 * w + i16;
    lchar* b0 = (lchar*)lds_b0;
    lchar* b1 = (lchar*)lds_b1;
    lchar* work = (lchar*)lds_work;
    lchar* sink = (lchar*)lds_sink;
    lchar* sH = work + L::WH;
    lchar* sO = work + L::WO;
    lchar* sGO = work + L::WGO;
    lchar* sDU = work + L::WDU;
    lchar* sGR = work + L::WGR;
    lchar* sHf = work + L::WHF;
    lchar* sDUf = work + L::WDUF;
    lchar* sDRf = work + L::WDRF;
    auto sync = [&]() { lds_barrier(); };

    const char* kbase = static_cast<const char*>(a.k) + (size_t)seq * a.L * DK * 2;
    const char* qbase = static_cast<const char*>(a.q) + (size_t)seq * a.L * DK * 2;
    const char* fbase = a.wF + (size_t)seq * a.NC * kBF;
    const float* obase = a.dO + (size_t)seq * a.L * Dv + n0;
    auto valid_of = [&](int c) { return min(CH, a.L - c * CH); };

    auto copy0 = [&](lchar* buf, int c) {
        const int Lc = valid_of(c);
        copy_rows<L::RB>(uniform_ptr(kbase + (size_t)c * CH * L::RB), Lc, buf + L::KT, l, cw);
        copy_rows<L::RB>(uniform_ptr(qbase + (size_t)c * CH * L::RB), Lc, buf + L::QT, l, cw);
    };
    auto copy2 = [&](lchar* buf, int c) {
        const char* fb = uniform_ptr(fbase + (size_t)c * kBF);
#pragma unroll
        for (int jj = 0; jj < L::NS2; ++jj) {
            const int k = min(cw + 4 * jj, L::NSLOT - 1);   // wave-uniform; the last slot (gate) repeated
            dma16s(fb, 1024u * k + (k == L::NSLOT - 1 ? 16u * (l & 31) : 16u * l), buf + L::MT + 1024 * k);
        }
    };
    Warm wm{nullptr, 0, tile + NT * (64 * cw + l), nullptr, 0};
    if (copier) {
        wm.region(kbase, CH * L::RB, L::RB / 2);
        wm.region(qbase, CH * L::RB, L::RB / 2);
        wm.region(fbase, kBF, (4 * kTriBytes + 512) / 128);
        wm.region(obase - n0, CH * Dv * 4, 2 * Dv);
        wm.done();
    }
    const int NCF = a.L / CH;
    const int cE = a.c0 + a.cN;   // chunks [c0, cE) in reverse, from the gradient dS_final points to

    // dO of chunk c, rows 16 w + 4 g + j, column n0 + i16 (zero past the end)
    auto load_do = [&](int c, float* od) {
        const int Lc = valid_of(c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * w + 4 * g + j;
            od[j] = obase[((size_t)c * CH + (r < Lc ? r : 0)) * Dv + i16];
        }
    };
    auto mask_do = [&](int c, float* od) {
        const int Lc = valid_of(c);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (16 * w + 4 * g + j >= Lc) od[j] = 0.f;
    };

    f32x4 H[NTS];
    float oc[4], on[4] = {0.f, 0.f, 0.f, 0.f};   // dO of the chunk being computed and of the next one
    if (!copier) {
#pragma unroll
        for (int t = 0; t < NTS; ++t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * (w * NTS + t) + 4 * g + j;
                H[t][j] = a.dS_final ? a.dS_final[((size_t)seq * DK + row) * Dv + n0 + i16] : 0.f;
            }
            st4_terms<true, 2>(sH + i16 * L::SP + 2 * (16 * (w * NTS + t) + 4 * g), 16 * L::SP, H[t]);
        }
        load_do(cE - 1, oc);
        mask_do(cE - 1, oc);
        st4_terms<true, 2>(sO + i16 * RP + 2 * (16 * w + 4 * g), 16 * RP, f32x4{oc[0], oc[1], oc[2], oc[3]});
        if (cE - 1 > a.c0) load_do(cE - 2, on);
    } else {
        copy0(b0, cE - 1);
        copy2(b0, cE - 1);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    sync();

    // chunk c (operands in buf); the copy waves fill cbuf with chunk c - 1
    auto chunk = [&](const int c, const lchar* buf, lchar* cbuf) {
        const int cn = max(c - 1, a.c0);
        const int Lc = valid_of(c);
        const size_t cs = (size_t)seq * a.sC + c % a.sC;   // slot of H_c and dU
        auto gt = [&](int i) { return lds_ld<float>(buf + L::GT + 4 * i); };
        uint4 tfr[2][2], kfr[NTS][2], qfr[NTS][2];
        float gam[4];

        // ---------------- phase A: dU = P^T dO + Lambda K H; stage H and dU
        if (copier) {
            if (c + 1 < cE)   // dV of chunk c + 1
                store_staged<64>(sDRf, a.dv + ((size_t)seq * a.L + (size_t)(c + 1) * CH) * Dv + n0, Dv,
                                 valid_of(c + 1), l, cw);
            copy0(cbuf, cn);
        } else {
            uint4 kf[DK / 32], hfr[DK / 32][2], pfr[2][2], ofr[2][2];
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                kf[s] = lds16(tile_at<L::RB>(buf + L::KT, ra, 4 * s + g));
#pragma unroll
                for (int p = 0; p < 2; ++p) hfr[s][p] = lds16(sH + p * 16 * L::SP + i16 * L::SP + 2 * (32 * s + 8 * g));
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    pfr[s][p] = tri_frag<true>(buf + L::MT + kBfPt + p * kTriBytes, w, s, i16, g);
                    tfr[s][p] = tri_frag_t(buf + L::MT + p * kTriBytes, w, s, i16, g);
                    ofr[s][p] = plane16(sO + p * 16 * RP, i16, s, g);
                }
            float lam[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * w + 4 * g + j;
                gam[j] = gt(r);
                lam[j] = gt(64 + r);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    tri_mask<true>(pfr[s][p], w, s, g);
                    tri_mask<true>(tfr[s][p], w, s, g);
                }
            f32x4 Z = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < DK / 32; ++s)
#pragma unroll
                for (int p = 0; p < 2; ++p) Z = mfma_raw<true>(kf[s], hfr[s][p], Z);
#pragma unroll
            for (int s = 0; s < 2; ++s) Y = mfma3(pfr[s][0], pfr[s][1], ofr[s][0], ofr[s][1], Y);
            f32x4 du;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * w + 4 * g + j;
                du[j] = r < Lc ? lam[j] * Z[j] + Y[j] : 0.f;
                lds_st(sDUf + r * FP + 4 * i16, du[j]);
            }
            st4_terms<true, 2>(sDU + i16 * RP + 2 * (16 * w + 4 * g), 16 * RP, du);
#pragma unroll
            for (int t = 0; t < NTS; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    lds_st(sHf + (16 * (w * NTS + t) + 4 * g + j) * FP + 4 * i16, H[t][j]);
        }
        sync();

        // ---------------- phase B: dR = T^T dU; Gamma dR, Gamma dO
        if (copier) {
            copy2(cbuf, cn);
            store_staged<DK>(sHf, a.wH + cs * DK * Dv + n0, Dv, DK, l, cw);
            store_staged<64>(sDUf, a.wdU + cs * CH * Dv + n0, Dv, CH, l, cw);
        } else {
            uint4 duf[2][2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int p = 0; p < 2; ++p) duf[s][p] = plane16(sDU + p * 16 * RP, i16, s, g);
            // K^T and Q^T fragments for phase C
#pragma unroll
            for (int t = 0; t < NTS; ++t) {
                const int rt = 16 * (w * NTS + t);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int tok = 32 * s + 8 * g + (i16 >> 2);
                    const int d = rt + 4 * (i16 & 3);
                    uint2 lo4 = lds_tr4(tile_at<L::RB>(buf + L::KT, tok, d >> 3) + 2 * (d & 7));
                    uint2 hi4 = lds_tr4(tile_at<L::RB>(buf + L::KT, tok + 4, d >> 3) + 2 * (d & 7));
                    kfr[t][s] = {lo4.x, lo4.y, hi4.x, hi4.y};
                    lo4 = lds_tr4(tile_at<L::RB>(buf + L::QT, tok, d >> 3) + 2 * (d & 7));
                    hi4 = lds_tr4(tile_at<L::RB>(buf + L::QT, tok + 4, d >> 3) + 2 * (d & 7));
                    qfr[t][s] = {lo4.x, lo4.y, hi4.x, hi4.y};
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x4 dr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) dr = mfma3(tfr[s][0], tfr[s][1], duf[s][0], duf[s][1], dr);
            f32x4 gr, go;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lds_st(sDRf + (16 * w + 4 * g + j) * FP + 4 * i16, dr[j]);
                gr[j] = gam[j] * dr[j];
                go[j] = gam[j] * oc[j];
            }
            st4_terms<true, 2>(sGR + i16 * RP + 2 * (16 * w + 4 * g), 16 * RP, gr);
            st4_terms<true, 2>(sGO + i16 * RP + 2 * (16 * w + 4 * g), 16 * RP, go);
        }
        sync();

        // ---------------- phase C: H = gamma_63 H + Q^T (Gamma dO) - K^T (Gamma dR);
        // the next chunk's dO into sO
        if (copier) {
            if (NCF > 0) dma4(wm.base + (size_t)min(max(c - DR_BWD_PFD, 0), NCF - 1) * wm.stride, sink + 256 * cw);
            else dma4(fbase, sink + 256 * cw);
            // the copies of chunk c - 1 (issued in phases A and B) have landed
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(L::NAFTER));
        } else {
            uint4 gof[2][2], grf[2][2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    gof[s][p] = plane16(sGO + p * 16 * RP, i16, s, g);
                    grf[s][p] = plane16(sGR + p * 16 * RP, i16, s, g);
                }
            const float d63 = gt(63);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < NTS; ++t) {
                const int rt = 16 * (w * NTS + t);
                f32x4 hq = {0.f, 0.f, 0.f, 0.f}, hk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        hq = mfma_raw<true>(qfr[t][s], gof[s][p], hq);
                        hk = mfma_raw<true>(kfr[t][s], grf[s][p], hk);
                    }
#pragma unroll
                for (int j = 0; j < 4; ++j) H[t][j] = d63 * H[t][j] + (hq[j] - hk[j]);
                st4_terms<true, 2>(sH + i16 * L::SP + 2 * (rt + 4 * g), 16 * L::SP, H[t]);
            }
            if (c > a.c0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) oc[j] = on[j];
                mask_do(c - 1, oc);
                st4_terms<true, 2>(sO + i16 * RP + 2 * (16 * w + 4 * g), 16 * RP, f32x4{oc[0], oc[1], oc[2], oc[3]});
                if (c > a.c0 + 1) load_do(c - 2, on);
            }
        }
        sync();
    };

    for (int i = 0; i < a.cN; i += 2) {
        const int c = cE - 1 - i;
        chunk(c, b0, b1);
        if (c - 1 >= a.c0) chunk(c - 1, b1, b0);
    }
    if (copier) {
        // dV of chunk c0
        store_staged<64>(sDRf, a.dv + ((size_t)seq * a.L + (size_t)a.c0 * CH) * Dv + n0, Dv, valid_of(a.c0), l, cw);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else if (a.dS0) {
#pragma unroll
        for (int t = 0; t < NTS; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * (w * NTS + t) + 4 * g + j;
                a.dS0[((size_t)seq * DK + row) * Dv + n0 + i16] = H[t][j];
            }
    }
}

template <int DK>
hipError_t launch_f(const BwdArgs& a, hipStream_t st) {
    static_assert(FL<DK>::TOTAL <= 160 * 1024, "LDS plan exceeds 160 KiB");
    static_assert(FL<DK>::NOPS <= 63, "operations per chunk exceed the vector-memory counter");
    const unsigned n = (unsigned)((a.nseq + 7) / 8) * 8u * (unsigned)(a.Dv / 16);
    return launch_k(kProfBwdFscan, bwd_fscan16_kernel<DK>, dim3(n), dim3(512), 0, st, a);
}

template <int DK>
hipError_t launch_r(const BwdArgs& a, hipStream_t st) {
    static_assert(RL<DK>::TOTAL <= 160 * 1024, "LDS plan exceeds 160 KiB");
    static_assert(RL<DK>::NS2 * 4 >= RL<DK>::NSLOT, "part-2 slots cover the run");
    const unsigned n = (unsigned)((a.nseq + 7) / 8) * 8u * (unsigned)(a.Dv / 16);
    return launch_k(kProfBwdRscan, bwd_rscan16_kernel<DK>, dim3(n), dim3(512), 0, st, a);
}

}  // namespace

hipError_t launch_bwd_fscan16(const BwdArgs& a, int Dk, hipStream_t st) {
    return Dk == 128 ? launch_f<128>(a, st) : launch_f<64>(a, st);
}

hipError_t launch_bwd_rscan16(const BwdArgs& a, int Dk, hipStream_t st) {
    return Dk == 128 ? launch_r<128>(a, st) : launch_r<64>(a, st);
}

}  // namespace dr
