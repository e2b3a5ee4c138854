// dr_prep16.hip -- per-chunk preparation for bf16 inputs with a scalar (or no)
// gate and a scalar beta, on gfx950.
//
// For one 64-token chunk of one (batch, head) it produces what the state scan
// needs (the chunk algebra is written out at the top of dr_chunk.hip):
//   G_r     cumulative log gate inside the chunk; gamma_r = e^{G_r},
//           lambda_r = e^{G_63 - G_r}                         -> workspace G
//   A_ri  = beta_r (k_r . k_i) e^{G_r - G_i}   (i < r),   T = (I + A)^-1
//   T^    = T Diag(beta)                                    -> workspace T (fp16)
//   P_ri  = (q_r . k_i) e^{G_r - G_i}          (i <= r)    -> workspace P (fp16)
// Rows past the sequence end are masked out of A and P, so their T^ rows are
// zero and the scan's U vanishes there.
//
// With the input preparation (q and k made unit vectors, DeltaNet page, step
// list, step 2), the raw bf16 tiles stay the matrix-core operands and the
// normalisation becomes row and column factors: A_ri gains 1/(|k_r| |k_i|),
// P_ri gains 1/(|q_r| |k_i|), and the workspace G record adds gamma_r/|k_r|
// and gamma_r/|q_r| and stores lambda_r/|k_r|, which the scan applies to the
// rows of K S, Q S and U.  beta given as logits is passed through a sigmoid
// where it is loaded.
//
// Data path: the chunk's k and q tiles are copied once into LDS (coalesced
// 16-byte global->LDS loads, XOR-swizzled rows).  k.k and q.k products are
// exact on bf16 matrix cores (bf16 x bf16 products are exact in fp32).  The
// triangular inverse is blocked in 16 x 16 tiles: diagonal tiles by a
// 16-step column sweep in fp32, off-diagonal tiles on fp32 matrix cores,
//   T_RI = -T_RR sum_{J=I}^{R-1} A_RJ T_JI,
// one block row R at a time.

#include <hip/hip_runtime.h>

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x4 mfma_bf16(const uint4& a, const uint4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ void dma16(const void* g, char* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 16, 0, 0);
#endif
}

template <int RB>
__device__ __forceinline__ int swz(int r) {
    return RB == 256 ? (r & 15) : ((r >> 1) & 7);
}

template <int RB>
__device__ __forceinline__ const char* tile_at(const char* tile, int r, int piece) {
    return tile + r * RB + 16 * (piece ^ swz<RB>(r));
}

// [64][RB]-byte tile of 16-bit values into swizzled LDS (rows >= valid read
// row 0; those rows are masked out of every product that uses them).
template <int RB>
__device__ __forceinline__ void dma_tile(const uint16_t* src, size_t pitch, int valid, char* tile, int w, int l) {
    constexpr int PPR = RB / 16;
    constexpr int RPI = 64 / PPR;
    constexpr int NI = 64 / RPI / 4;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int blk = w * NI + j;
        const int r = blk * RPI + l / PPR;
        const int rc = r < valid ? r : 0;
        const int lp = (l % PPR) ^ swz<RB>(r);
        dma16(src + (size_t)rc * pitch + 8 * lp, tile + blk * 1024);
    }
}

}  // namespace

// LDS plan (bytes): k tile, q tile.  A (fp32, its ten lower 16 x 16 blocks
// packed with a row pitch of 17), T (fp32), the per-wave 16 x 16 scratch of
// the triangular solve and the chunk's strengths reuse the k / q tiles, which
// are dead once A and P are formed (the waves hold their A blocks in
// registers until then); at d = 64 the tiles are too small and A, T and the
// scratch follow them.  P goes straight to the workspace.  The gates live in
// registers (every wave forms the chunk's prefix sums itself); only with the
// input preparation are 1/|q_r| and 1/|k_r| exchanged through LDS, after the
// tiles.  32 KB at d = 128 (five workgroups per CU), 32.5 KB with the input
// preparation (four).
template <int DK>
struct P16 {
    static constexpr int RB = DK * 2;
    static constexpr int KT = 0;
    static constexpr int QT = KT + 64 * RB;
    static constexpr int AP = 65;                 // fp32 pitch of T
    static constexpr int AB = 16 * 17;            // floats per packed A block
    static constexpr int ABYTES = 10 * AB * 4;
    static constexpr int TXA = ABYTES + 64 * AP * 4 + 4 * 16 * 17 * 4;   // A, T and the scratch
    static constexpr bool ALIAS = TXA <= 2 * 64 * RB;                    // they fit in the tiles
    static constexpr int SA = ALIAS ? KT : QT + 64 * RB;
    static constexpr int ST = SA + ABYTES;
    static constexpr int SX = ST + 64 * AP * 4;   // [4][16][17] fp32
    static constexpr int SB = ALIAS ? TXA : SX + 4 * 16 * 17 * 4;       // beta [64], once the tiles are dead
    static constexpr int SN = ALIAS ? QT + 64 * RB : SB + 64 * 4;         // 1/|q|, 1/|k| [64] each
    static constexpr int TOTAL = ALIAS ? 2 * 64 * RB : SN;
    static constexpr int TOTAL_QN = SN + 128 * 4;
    static_assert(!ALIAS || TXA + 64 * 4 <= 2 * 64 * RB, "beta fits beside A, T and the scratch");
};

template <int DK, bool QN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void prep16_kernel(ChunkArgs a) {
    using L = P16<DK>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float* sAp = reinterpret_cast<float*>(smem + L::SA);
    // element (r, c), c <= r rounded to blocks, of the packed A
    auto A_at = [&](int r, int c) -> float& {
        return sAp[tri_block(r >> 4, c >> 4) * L::AB + (r & 15) * 17 + (c & 15)];
    };
    float(*sT)[L::AP] = reinterpret_cast<float(*)[L::AP]>(smem + L::ST);
    float* sb = reinterpret_cast<float*>(smem + L::SB);    // beta, written once the tiles are dead
    float* snq = reinterpret_cast<float*>(smem + L::SN);   // 1 / |q_r| (input preparation)
    float* snk = snq + 64;                                 // 1 / |k_r|
    float(*sX)[16][17] = reinterpret_cast<float(*)[16][17]>(smem + L::SX);

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int seq = b * a.H + h;
    const size_t cs = (size_t)seq * a.NC + c;
    const int t0 = c * CH;
    const int Lc = min(CH, a.L - t0);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int i16 = l & 15, g = l >> 4;
    const size_t tok0 = (size_t)seq * a.L + t0;

    dma_tile<L::RB>(static_cast<const uint16_t*>(a.k) + tok0 * DK, DK, Lc, smem + L::KT, w, l);
    dma_tile<L::RB>(static_cast<const uint16_t*>(a.q) + tok0 * DK, DK, Lc, smem + L::QT, w, l);
    // every wave: lane l holds row l's cumulative log gate gl and strength bl
    // (zero past the end)
    float gl, bl;
    {
        const int lc = l < Lc ? l : 0;
        gl = a.has_gate ? a.log_alpha[tok0 + lc] : 0.f;
        gl = l < Lc ? gl : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(gl, off);
            if (l >= off) gl += y;
        }
        bl = l < Lc ? strength(a.beta[tok0 + lc], a.beta_logit) : 0.f;
    }
    const float g63 = __shfl(gl, 63);
    if (w == 0) {
        a.wsG[cs * kGW + l] = expf(gl);                         // gamma_r
        if (!QN) a.wsG[cs * kGW + 64 + l] = expf(g63 - gl);    // lambda_r
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's tile copies landed
    __syncthreads();

    // input preparation: 1/|q_r| and 1/|k_r| from the tiles (four lanes per
    // row, each summing a quarter of the row), and the scaled gate factors
    if constexpr (QN) {
        const int r = tid >> 2, qd = tid & 3;
        float ssq = 0.f, ssk = 0.f;
#pragma unroll
        for (int pc = qd; pc < L::RB / 16; pc += 4) {
            const uint4 kv = *reinterpret_cast<const uint4*>(tile_at<L::RB>(smem + L::KT, r, pc));
            const uint4 qv = *reinterpret_cast<const uint4*>(tile_at<L::RB>(smem + L::QT, r, pc));
            const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w}, qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float k0 = bf16_to_f32((uint16_t)kw[e]), k1 = bf16_to_f32((uint16_t)(kw[e] >> 16));
                const float q0 = bf16_to_f32((uint16_t)qw[e]), q1 = bf16_to_f32((uint16_t)(qw[e] >> 16));
                ssk += k0 * k0 + k1 * k1;
                ssq += q0 * q0 + q1 * q1;
            }
        }
        ssk = group_sum<4>(ssk);
        ssq = group_sum<4>(ssq);
        if (qd == 0) {
            snk[r] = inv_norm(ssk);
            snq[r] = inv_norm(ssq);
        }
        __syncthreads();
        if (w == 0) {
            const float gam = expf(gl), nk = snk[l];
            a.wsG[cs * kGW + 64 + l] = expf(g63 - gl) * nk;   // lambda_r / |k_r|
            a.wsG[cs * kGW + 128 + l] = gam * nk;             // gamma_r / |k_r|
            a.wsG[cs * kGW + 192 + l] = gam * snq[l];         // gamma_r / |q_r|
        }
    }

    // gate values this lane needs, in registers (log2 units): rows
    // 16 R + 4 g + j of every block row R, column 16 I + i16 of every block
    // column I; beta of the rows (times 1/|k_r| with the input preparation),
    // 1/|q_r| of the rows and 1/|k_i| of the column (1 without it)
    constexpr float kLog2e = 1.4426950408889634f;
    float grow[4][4], brow[4][4], gcol[4], qrow[4][4], kcol[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * R + 4 * g + j;
            grow[R][j] = __shfl(gl, r) * kLog2e;
            const float br = __shfl(bl, r);
            brow[R][j] = QN ? br * snk[r] : br;
            qrow[R][j] = QN ? snq[r] : 1.f;
        }
        gcol[R] = __shfl(gl, 16 * R + i16) * kLog2e;
        kcol[R] = QN ? snk[16 * R + i16] : 1.f;
    }

    // A and P, 16 x 16 block pairs (R, I), R >= I, on the bf16 matrix cores.
    // A and P of a pair share the k_I fragments and the decay factors
    // e^{G_r - G_i}; the pairs of a wave share the block row R, so its k_R and
    // q_R fragments are read once: wave 0 takes (3, 0..2), wave 1 (2, 0..2),
    // wave 2 (1, 0..1), wave 3 (0, 0) and (3, 3).
    float areg[3][4];   // this wave's A values (pair slot, row j) until the tiles are dead
    auto pair_group = [&](const int R, const int I0, const int NI, const int slot0) {
        f32x4 accA[3], accP[3];
#pragma unroll
        for (int t = 0; t < 3; ++t) accA[t] = accP[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            const uint4 ka = *reinterpret_cast<const uint4*>(tile_at<L::RB>(smem + L::KT, 16 * R + i16, 4 * s + g));
            const uint4 qa = *reinterpret_cast<const uint4*>(tile_at<L::RB>(smem + L::QT, 16 * R + i16, 4 * s + g));
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                if (t < NI) {   // wave-uniform
                    const int I = I0 + t;
                    const uint4 kb = I == R ? ka
                                            : *reinterpret_cast<const uint4*>(
                                                  tile_at<L::RB>(smem + L::KT, 16 * I + i16, 4 * s + g));
                    accA[t] = mfma_bf16(ka, kb, accA[t]);
                    accP[t] = mfma_bf16(qa, kb, accP[t]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            if (t < NI) {
                const int I = I0 + t;
                const float gi = I == 0 ? gcol[0] : I == 1 ? gcol[1] : I == 2 ? gcol[2] : gcol[3];
                const float ki = I == 0 ? kcol[0] : I == 1 ? kcol[1] : I == 2 ? kcol[2] : kcol[3];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * R + 4 * g + j, i = 16 * I + i16;
                    const float gr = R == 0 ? grow[0][j] : R == 1 ? grow[1][j] : R == 2 ? grow[2][j] : grow[3][j];
                    const float br = R == 0 ? brow[0][j] : R == 1 ? brow[1][j] : R == 2 ? brow[2][j] : brow[3][j];
                    const float qr = R == 0 ? qrow[0][j] : R == 1 ? qrow[1][j] : R == 2 ? qrow[2][j] : qrow[3][j];
                    const float f = __builtin_amdgcn_exp2f(gr - gi);   // e^{G_r - G_i} <= 1
                    const bool live = r < Lc;
                    areg[slot0 + t][j] = (live && i < r) ? accA[t][j] * f * br * ki : 0.f;
                    // P to the workspace, packed: 16 lanes write one 32-byte block row
                    a.wsP[cs * (size_t)(CH * CH) + tri_off(r, i)] =
                        (half_t)((live && i <= r) ? accP[t][j] * f * qr * ki : 0.f);
                }
            }
        }
    };
    auto write_a = [&](const int R, const int I0, const int NI, const int slot0) {
#pragma unroll
        for (int t = 0; t < 3; ++t)
            if (t < NI)
#pragma unroll
                for (int j = 0; j < 4; ++j) A_at(16 * R + 4 * g + j, 16 * (I0 + t) + i16) = areg[slot0 + t][j];
    };
    if (w == 0) pair_group(3, 0, 3, 0);
    else if (w == 1) pair_group(2, 0, 3, 0);
    else if (w == 2) pair_group(1, 0, 2, 0);
    else {
        pair_group(0, 0, 1, 0);
        pair_group(3, 3, 1, 1);
    }
    if constexpr (L::ALIAS) __syncthreads();   // the tiles are dead: A may take their place
    if (w == 0) sb[l] = bl;                     // the strengths, for T^ = T Diag(beta)
    if (w == 0) write_a(3, 0, 3, 0);
    else if (w == 1) write_a(2, 0, 3, 0);
    else if (w == 2) write_a(1, 0, 2, 0);
    else {
        write_a(0, 0, 1, 0);
        write_a(3, 3, 1, 1);
    }
    __syncthreads();

    // diagonal 16 x 16 blocks of T: wave w inverts block w by a column sweep,
    // lane j < 16 owns column j (16 dependent steps, the updates within a
    // step are independent)
    if (l < 16) {
        const int base = 16 * w, j = l;
        float acc[16], t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            t[i] = (i == j ? 1.f : 0.f) - acc[i];
            if (i < j) t[i] = 0.f;
#pragma unroll
            for (int r = i + 1; r < 16; ++r) acc[r] += A_at(base + r, base + i) * t[i];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[base + r][base + j] = t[r];
    }
    __syncthreads();

    // T^ = T Diag(beta) in the packed lower-block form, fp16, from the fp32
    // blocks of block row R, one 8-column piece (of 32 R + 32) per thread
    // index e = 0, nthr, 2 nthr, ... starting at e0
    auto out_row = [&](const int R, int e0, const int nthr) {
        for (int e = e0; e < 32 * (R + 1); e += nthr) {
            const int I = e >> 5, r = (e >> 1) & 15, h = e & 1;
            const int row = 16 * R + r, c0 = 16 * I + 8 * h;
            half8 hv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = c0 + j;
                hv[j] = (half_t)(col <= row ? sT[row][col] * sb[col] : 0.f);
            }
            *reinterpret_cast<half8*>(a.wsT + cs * (size_t)(CH * CH) + tri_off(row, c0)) = hv;
        }
    };

    // off-diagonal blocks, block row R = 1..3; wave I < R computes T_RI:
    //   X = sum_{m in [16 I, 16 R)} A[16 R + .][m] T[m][16 I + .],  T_RI = -T_RR X
    // while the idle waves (w >= R) write block row R - 1 of T^, final by now
    for (int R = 1; R < 4; ++R) {
        if (w < R) {
            const int I = w;
            // two accumulators (even / odd k-steps) halve the dependent chain
            f32x4 X0 = {0.f, 0.f, 0.f, 0.f}, X1 = X0;
            for (int s = 0; s < 4 * (R - I); s += 2) {
                const int m = 16 * I + 4 * s + g;
                X0 = mfma_f32x4(A_at(16 * R + i16, m), sT[m][16 * I + i16], X0);
                X1 = mfma_f32x4(A_at(16 * R + i16, m + 4), sT[m + 4][16 * I + i16], X1);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) sX[w][4 * g + j][i16] = X0[j] + X1[j];
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's scratch is written
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");
            f32x4 Tn0 = {0.f, 0.f, 0.f, 0.f}, Tn1 = Tn0;
#pragma unroll
            for (int s = 0; s < 4; s += 2) {
                Tn0 = mfma_f32x4(sT[16 * R + i16][16 * R + 4 * s + g], sX[w][4 * s + g][i16], Tn0);
                Tn1 = mfma_f32x4(sT[16 * R + i16][16 * R + 4 * s + 4 + g], sX[w][4 * s + 4 + g][i16], Tn1);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) sT[16 * R + 4 * g + j][16 * I + i16] = -(Tn0[j] + Tn1[j]);
        } else {
            out_row(R - 1, tid - 64 * R, 64 * (4 - R));
        }
        __syncthreads();
    }
    out_row(3, tid, 256);
}

template <int DK, bool QN>
static hipError_t launch_p16(const ChunkArgs& a, hipStream_t st) {
    using L = P16<DK>;
    constexpr int lds = QN ? L::TOTAL_QN : L::TOTAL;
    auto kern = prep16_kernel<DK, QN>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    return launch_k(kProfPrep, kern, dim3(a.NC, a.H, a.B), dim3(256), lds, st, a);
}

hipError_t launch_prep16(const ChunkArgs& a, int Dk, hipStream_t st) {
    if (a.qk_norm) return Dk == 64 ? launch_p16<64, true>(a, st) : launch_p16<128, true>(a, st);
    return Dk == 64 ? launch_p16<64, false>(a, st) : launch_p16<128, false>(a, st);
}

}  // namespace dr
