// dr_internal.h -- argument blocks and launchers shared by the host ABI and
// the kernel translation units (not part of the public interface).
#pragma once

#include <hip/hip_ext.h>
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
    // beta and beta_v hold one value per token ([B][H][L]) that every channel
    // shares, on the channel-beta kernels (separate scalar strengths)
    int beta_tok;
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
// For bf16 inputs without a channel gate (wF not NULL) the prep kernel writes,
// per chunk, the operands of the matrix-core scans and of the per-chunk
// kernel (kBF bytes) in place of wP and wA (wU and wR are not used either):
//   [T^ hi][T^ lo]      T^ = T Diag(beta), packed lower blocks (tri_off)
//   [P^T hi][P^T lo]    P transposed, packed upper blocks (kBfPt)
//   [gamma 64][lambda 64] fp32 at kBfGate
// as bf16 hi + lo pairs (x = hi + lo to 16 significant bits).  A packed upper
// block (R, I), I >= R, of a 64 x 64 matrix sits where tri_block(3 - R, 3 - I)
// puts a lower one, with the same layout inside the block.  T^T is read from
// T^ through the transposing LDS read.
constexpr int kBfPt = 2 * kTriBytes;
constexpr int kBfGate = 4 * kTriBytes;
constexpr int kBF = kBfGate + 1024;
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
    // channel-gate kernels only: gmode 2 reads log alpha per channel, 1 one
    // value per token (broadcast to every channel), 0 none; the per-channel
    // d log alpha goes to dla_cg (NULL: not written)
    int gmode;
    float* dla_cg;
    // write-side key scales (NULL: none): the write key is ks (.) k, on the
    // column side of A and P and in the state update; dks its gradient
    const float* ks;
    float* dks;
    // the matrix-core scans' operands (bf16 inputs, no channel gate), or NULL
    char* wF;
    // Chunk range and state slots.  A launch of the scans or of the per-chunk
    // kernel covers chunks [c0, c0 + cN) of every sequence.  The per-chunk
    // S_c, H_c and dU sit in slot seq * sC + c % sC of wS, wH and wdU (sC ==
    // NC: one slot per chunk).  With sC < NC (bounded workspace, matrix-core
    // path only) the host walks segments of sC chunks, last to first; the
    // forward scan's first pass over all chunks then stores S_c of every
    // chunk c = j sC with 0 < c < ckEnd into the checkpoint slot
    // wCk[(j - 1) nseq + seq] in place of its slot in wS.
    // wHc carries the reverse scan's gradient from one segment to the next.
    int c0, cN, sC;
    float* wCk;
    int ckEnd;
    float* wHc;
};

// Optional per-kernel timing (dr_profile_begin / dr_profile_end).  While it is
// on, launch_k gives each kernel launch a start and a stop event of its own,
// set from the dispatch's own timestamps, so that no marker packets sit
// between the kernels being timed; the pair is kept under the kernel's slot.
enum ProfSlot {
    kProfPrep = 0, kProfScan = 1, kProfDecode = 2,
    kProfBwdPrep = 3, kProfBwdFscan = 4, kProfBwdRscan = 5, kProfBwdPost = 6,
    kProfSlots = 7, kProfNone = -1
};
// two new timing events while timing is on (false otherwise)
bool prof_events(hipEvent_t* start, hipEvent_t* stop);
void prof_record(hipEvent_t start, hipEvent_t stop, int slot);

template <typename F, typename... Args>
hipError_t launch_k(int slot, F kernel, dim3 grid, dim3 block, unsigned shmem, hipStream_t st, Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const bool timed = slot != kProfNone && prof_events(&e0, &e1);
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, e0, e1, 0u, args...);
    const hipError_t e = hipGetLastError();
    if (timed) prof_record(e0, e1, slot);
    return e;
}

// sepv: a.beta_v differs from a.beta (channel beta only)
hipError_t launch_chunk(const ChunkArgs& a, int Dk, bool f32in, bool cgate, bool cbeta, bool sepv,
                        hipStream_t st);
// chunk preparation for bf16 inputs, scalar gate and scalar beta (dr_prep16.hip)
hipError_t launch_prep16(const ChunkArgs& a, int Dk, hipStream_t st);
// the same with a channel-wise gate, or with write-side key scales and any
// gate (dr_prepcg16.hip)
hipError_t launch_prepcg16(const ChunkArgs& a, int Dk, bool cbeta, bool sepv, hipStream_t st);
// the state scan for bf16 inputs (dr_scan16.hip)
hipError_t launch_scan16(const ChunkArgs& a, int Dk, bool cgate, bool cbeta, hipStream_t st);
// the backward (dr_bwd.hip)
hipError_t launch_bwd(const BwdArgs& a, int Dk, bool f32in, hipStream_t st);
// the backward's two state scans on the matrix cores for bf16 inputs with a
// scalar gate (or none) and a scalar beta, from the operands in a.wF
// (dr_bwd16.hip)
hipError_t launch_bwd_fscan16(const BwdArgs& a, int Dk, hipStream_t st);
hipError_t launch_bwd_rscan16(const BwdArgs& a, int Dk, hipStream_t st);
// The backward kernels differentiate the recurrence with respect to q, k, v
// and a scalar beta as they receive them.  When a call's inputs are not those
// (a channel-wise or separate beta, or the input preparation), a per-token
// pass writes fp32 copies of what the recurrence sees, the kernels run on the
// copies, and a second per-token pass maps the gradients back:
//   qh = q / |q|, kh = k / |k| with the normalisation (1/|x| kept per token),
//   beta = sigmoid(x) for logits,
//   on the channel-beta route (channel-wise or separate strengths) the copies
//   are kt = sqrt(beta^k) (.) kh and vt = sqrt(beta^v) (.) v with unit
//   strength; otherwise kh, v and the scalar beta itself (with logits alone
//   only the strengths are written: q, k and v are used as they are);
// back: dk = sqrt(beta^k) (.) dkt, dv = sqrt(beta^v) (.) dvt,
//   dbeta^k = dkt (.) kh / (2 sqrt(beta^k)) (summed over the token's channels
//   for per-token strengths; one strength adds dbeta^v to it), times
//   beta (1 - beta) for logits; dq = (dqh - qh (qh . dqh)) / |q|, likewise dk.
struct BwdMap {
    const void* q;
    const void* k;
    const void* v;
    const float* beta;
    const float* beta_v;   // == beta with one strength
    int f32in, cbeta, per_token, sepv, l2, logit, Dk, Dv;
    int copy;              // q, k, v copied (channel-beta route or normalisation); else only b32
    size_t ntok;
    float* q32;
    float* k32;
    float* v32;
    float* b32;            // unit strengths (channel-beta route) or the scalar beta's values
    float* rq;             // 1/|q_t|, 1/|k_t| (normalisation only)
    float* rk;
};
hipError_t launch_bwd_map_in(const BwdMap& m, hipStream_t st);
// dla[t] = sum over the DK channels of dla_ch[t][.] (a scalar gate through the
// channel-gate kernels)
hipError_t launch_bwd_gate_sum(const float* dla_ch, float* dla, size_t ntok, int dk, hipStream_t st);
// dq, dk, dv (and dbeta for a scalar beta) hold the copies' gradients on entry
hipError_t launch_bwd_map_out(const BwdMap& m, float* dq, float* dk, float* dv, float* dbeta, float* dbeta_v,
                              hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int Dk, bool f32in, bool cgate, bool cbeta,
                         hipStream_t st);

}  // namespace dr
