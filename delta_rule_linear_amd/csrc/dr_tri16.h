// dr_tri16.h -- the blocked triangular inverse of the channel-gate
// preparation kernel for bf16 inputs (dr_prepcg16.hip).  The scalar-gate
// kernel (dr_prep16.hip) keeps its own inline copy of the same steps: with
// this function inlined there instead, the compiler allocates it 112 VGPRs
// rather than 88, one workgroup per CU fewer.
//
// T = (I + A)^-1 for the 64 x 64 unit lower-triangular I + A of one chunk (the
// chunkwise form's triangular factor, DeltaNet page, chunkwise training step;
// FG2-GDN page, section 2), in 16 x 16 blocks: diagonal blocks by a 16-step
// column sweep in fp32, off-diagonal blocks on fp32 matrix cores,
//   T_RI = -T_RR sum_{J=I}^{R-1} A_RJ T_JI,
// one block row R at a time.  The result leaves as T^ = T Diag(b) (or T
// itself) in the packed lower-block fp16 form (tri_off).
#pragma once

#include <hip/hip_runtime.h>

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {

// Called by all 256 threads (four waves) of a workgroup, after a barrier that
// makes A visible; tid = 64 w + l, l = 16 g + i16.
//   A_at(r, c)  fp32 element (r, c) of A for c < r (any element of the lower
//               16 x 16 blocks may be asked for; only the strict lower part
//               is used)
//   sT          [64][65] fp32 LDS scratch that receives T
//   sX          [4][16][17] fp32 LDS scratch
//   sb          column factors b [64] (BETA), else unused
//   wsT, cs     the packed T^ (fp16, tri_off) of chunk slot cs
template <bool BETA, class AAt>
__device__ __forceinline__ void tri_inverse_out(AAt A_at, float (*sT)[65], float (*sX)[16][17], const float* sb,
                                                half_t* wsT, size_t cs, int tid, int w, int l, int i16, int g) {

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

    // T^ in the packed lower-block form, fp16, from the fp32 blocks of block
    // row R, one 8-column piece (of 32 R + 32) per thread index e = e0,
    // e0 + nthr, ...
    auto out_row = [&](const int R, int e0, const int nthr) {
        for (int e = e0; e < 32 * (R + 1); e += nthr) {
            const int I = e >> 5, r = (e >> 1) & 15, h = e & 1;
            const int row = 16 * R + r, c0 = 16 * I + 8 * h;
            half8 hv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = c0 + j;
                if constexpr (BETA) hv[j] = (half_t)(col <= row ? sT[row][col] * sb[col] : 0.f);
                else hv[j] = (half_t)(col <= row ? sT[row][col] : 0.f);
            }
            *reinterpret_cast<half8*>(wsT + cs * (size_t)(CH * CH) + tri_off(row, c0)) = hv;
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

}  // namespace dr
