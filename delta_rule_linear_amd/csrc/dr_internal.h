// dr_internal.h -- argument blocks and launchers shared by the host ABI and
// the kernel translation units (not part of the public interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "dr_device.h"

namespace dr {

// floats of per-chunk gate data in the workspace.  Channel gate: the chunk's
// state decay e^{G_63}[Dk].  Scalar gate: gamma_r = e^{G_r} at [0, 64) and
// lambda_r = e^{G_63 - G_r} at [64, 128); when q and k are normalised inside
// the kernels and the raw inputs are the scan's operands (scalar gate and
// beta), lambda_r is stored times 1/|k_r|, and [128, 192) holds gamma_r/|k_r|
// (the key reads) and [192, 256) gamma_r/|q_r| (the query reads).
constexpr int kGW = 256;

// Packed lower-triangular form of the 64 x 64 per-chunk matrices T^ and P for
// bf16 inputs: the ten 16 x 16 blocks (R, I), R >= I, in the order
// (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ..., 512 bytes each; row r of a
// block is 32 bytes whose two 8-column halves are swapped when (r & 8), so
// that 16 lanes reading one half of 16 consecutive rows hit distinct banks.
// 5120 bytes per matrix, at the start of its 64 x 64 workspace slot.
constexpr int kTriBytes = 10 * 512;
__host__ __device__ constexpr int tri_block(int R, int I) { return R * (R + 1) / 2 + I; }
// offset (in 16-bit elements) of element (r, c), c <= r rounded to blocks
__host__ __device__ constexpr int tri_off(int r, int c) {
    return tri_block(r >> 4, c >> 4) * 256 + (r & 15) * 16 + 8 * (((c >> 3) & 1) ^ ((r >> 3) & 1)) + (c & 7);
}

// Everything the chunked-forward kernels read.  Workspace planes, per chunk
// slot cs = (b * H + h) * NC + c, with P = 1 (bf16 inputs) or 2 (fp32 inputs)
// fp16 terms per value:
//   wsT, wsP  [NCH][P][64][64]   T^ = (I + A)^-1 (beta-scaled columns) and P
//                                (bf16 inputs: packed lower blocks, see tri_off)
//   wsG       [NCH][kGW]         gate factors
//   wsQ/Ks/Kl [NCH][P][64][Dk]   gated operands (channel gate; with a channel
//                                beta and scalar gate Ks holds sqrt(beta) k and
//                                Q a copy of q)
//   wsV       [NCH][P][64][Dk]   sqrt(beta_v) v (channel beta)
// beta_v is the write strength that scales v; it is beta itself unless the
// caller gives a separate one (channel beta only).
// Input preparation: qk_norm makes every q_t and k_t a unit vector (the zero
// vector stays zero), beta_logit reads beta (and beta_v) as logits,
// beta = 1 / (1 + e^{-x}).  key_scale (write-side key scales s_t) makes the
// write key w = s (.) kt: S_t = (I - w kt^T) Diag(alpha) S + w vt^T; such calls
// run on the channel-gate path whatever the gate (scalar and absent gates are
// broadcast to every channel).
struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const float* beta_v;
    const float* S0;
    void* o;
    float* S_final;
    int B, H, L, Dv, NC, nseq;
    int has_gate;
    int out_bf16;
    int qk_norm;
    int beta_logit;
    int gate_mode;              // 0 none, 1 scalar, 2 channel
    const float* key_scale;     // write-side key scales [B][H][L][Dk], or null
    half_t* wsT;
    half_t* wsP;
    float* wsG;
    half_t* wsQ;
    half_t* wsKs;
    half_t* wsKl;
    half_t* wsV;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const float* beta_v;   // write strength on v (== beta unless separate)
    float* S;
    void* o;
    int N, H, Dv;
    int has_gate;
    int out_bf16;
    int qk_norm;      // input preparation, as in ChunkArgs
    int beta_logit;
    const float* key_scale;   // write-side key scales [N][H][Dk], or null
};

// Everything the backward kernels read and write (scalar gate or none, scalar
// beta; fp32 gradients).  Workspace planes, fp32, per chunk slot
// cs = (b * H + h) * NC + c:
//   wT, wP, wA  [NCH][64][64]   T = (I + A)^-1, P, and K K^T o E (strict lower)
//   wG          [NCH][64]       cumulative log-decay g_r within the chunk
//                               ([NCH][64][Dk] per channel with a channel gate)
// With a channel gate (cgate) also the gated operands, [NCH][64][Dk] each:
//   wQh = q o e^G, wKh = k o e^G, wKc = k o e^-G, wKt = k o e^(G_63 - G)
//   wS, wH      [NCH][Dk][Dv]   chunk start state, gradient at its end state
//   wU, wR, wdU [NCH][64][Dv]   U, R = V - Gamma K S, and dU
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const float* S0;
    const float* dO;
    const float* dS_final;
    float* dq;
    float* dk;
    float* dv;
    float* dlog_alpha;
    float* dbeta;
    float* dS0;
    int B, H, L, Dv, NC, nseq;
    int has_gate;
    float* wT;
    float* wP;
    float* wA;
    float* wG;
    float* wS;
    float* wH;
    float* wU;
    float* wR;
    float* wdU;
    int cgate;
    float* wQh;
    float* wKh;
    float* wKc;
    float* wKt;
};

// Optional per-kernel timing: launchers mark the start of each kernel and the
// end of their last one (dr_profile_begin / dr_profile_end).
enum ProfSlot {
    kProfPrep = 0, kProfScan = 1, kProfDecode = 2,
    kProfBwdPrep = 3, kProfBwdFscan = 4, kProfBwdRscan = 5, kProfBwdPost = 6,
    kProfSlots = 7, kProfEnd = 7
};
void prof_mark(hipStream_t st, int slot);

// sepv: a.beta_v differs from a.beta (channel beta only)
hipError_t launch_chunk(const ChunkArgs& a, int Dk, bool f32in, bool cgate, bool cbeta, bool sepv,
                        hipStream_t st);
// chunk preparation for bf16 inputs, scalar gate and scalar beta (dr_prep16.hip)
hipError_t launch_prep16(const ChunkArgs& a, int Dk, hipStream_t st);
// the state scan for bf16 inputs (dr_scan16.hip)
hipError_t launch_scan16(const ChunkArgs& a, int Dk, bool cgate, bool cbeta, hipStream_t st);
// the backward (dr_bwd.hip)
hipError_t launch_bwd(const BwdArgs& a, int Dk, bool f32in, hipStream_t st);
// channel-wise beta: q, sqrt(beta_k) k, sqrt(beta_v) v as fp32 and unit
// strengths before the backward (n = tokens x Dk, ntok = tokens); the
// gradients of k, v and the strengths from those of the scaled key and value
// after it (dbeta_v NULL: one strength, beta_v == beta_k)
hipError_t launch_bwd_cbeta_in(const void* q, const void* k, const void* v, const float* beta_k,
                               const float* beta_v, bool f32in, size_t n, size_t ntok, float* q32, float* k32,
                               float* v32, float* ones, hipStream_t st);
hipError_t launch_bwd_cbeta_out(const void* k, const void* v, const float* beta_k, const float* beta_v, bool f32in,
                                size_t n, float* dk, float* dv, float* dbeta_k, float* dbeta_v, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int Dk, bool f32in, bool cgate, bool cbeta,
                         hipStream_t st);

}  // namespace dr
