/*
 * deltarule.h -- C ABI of the MI355X (gfx950) delta-rule linear-attention forward.
 *
 * The operation (FG2-GDN page, section 2 "Kerninnovation", the scaled
 * key/value equation and the state-update equation; DeltaNet page, the
 * seven-step list, steps 3-6):
 *
 *     kt_t = sqrt(beta_t) (.) k_t,      vt_t = sqrt(beta_t) (.) v_t
 *     S_t  = (I - kt_t kt_t^T) Diag(alpha_t) S_{t-1} + kt_t vt_t^T
 *     o_t  = S_t^T q_t                   (the output reads the updated state)
 *
 * per (batch b, head h), S a d_k x d_v matrix.  Variants, chosen by mode enums:
 *   plain DeltaNet  alpha == 1, scalar beta          (DeltaNet page, step list)
 *   Gated DeltaNet  scalar alpha_t                   (FG2-GDN page, section 1)
 *   KDA             alpha_t a d_k-vector             (FG2-GDN page, section 1)
 *   FG2-GDN         beta_t a d_k-vector, as sqrt on both k and v (section 2)
 *   FG2-GDN+        separate strengths: the erase strength beta^k on k and
 *                   the write strength beta^v on v (section "Erweiterung:
 *                   FG2-GDN+"; d_k-vectors, or one scalar each per token,
 *                   which the page's ablation also decouples), through the
 *                   *_kv entry points:
 *                     kt_t = sqrt(beta^k_t) (.) k_t,  vt_t = sqrt(beta^v_t) (.) v_t
 *                   and the same S_t and o_t.  The page gives no formula; this
 *                   is the reading that reduces to FG2-GDN at beta^v == beta^k.
 *   preconditioned  a diagonal preconditioner s_t on the delta rule's gradient
 *                   step (OSDN page, section "Method"; the preconditioned
 *                   delta rule page, abstract), which amounts to scaling the
 *                   write-side key per feature; through the *_precond entry
 *                   points, with s_t an input (its online update is not
 *                   printed) and w_t = s_t (.) kt_t:
 *                     S_t = (I - w_t kt_t^T) Diag(alpha_t) S_{t-1} + w_t vt_t^T
 * No query scaling is applied; callers pre-scale q if they want one.
 *
 * Input preparation (optional, descriptor field input_flags), the steps in
 * front of the recurrence, done inside the kernels so that the prepared
 * tensors never pass through memory:
 *   DR_IN_QK_L2NORM   q_t and k_t are replaced by q_t / |q_t|_2 and
 *                     k_t / |k_t|_2 (per token and head, computed in fp32 from
 *                     the input values; a zero vector stays zero) -- the
 *                     L2 normalisation after the key/query feature map of the
 *                     DeltaNet page, step list, step 2.  The learned parts of
 *                     that map (a projection, SiLU, a short convolution) are
 *                     the caller's.
 *   DR_IN_BETA_LOGIT  the beta arrays (beta_k and beta_v too) hold logits x,
 *                     and beta = 1 / (1 + e^{-x}) -- beta from a sigmoid
 *                     projection (DeltaNet page, list of design choices).
 * log_alpha is always taken as given: the pages fix no parametrisation of the
 * gate.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every tensor pointer is a DEVICE pointer owned by the caller; the
 *   library never allocates, frees or retains memory, and keeps no state
 *   between calls apart from the per-thread error text.  Every tensor pointer
 *   must be 16-byte aligned.  Tensors are dense, row-major (C order).
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Work is enqueued asynchronously; inputs, outputs and workspace
 *   must stay untouched until the stream reaches the enqueued work's end.
 * Errors.  Arguments are validated on the host before any device work, so on
 *   any error status nothing has been enqueued and nothing written.  A HIP
 *   launch failure returns DR_ERR_HIP; faults inside kernels surface at the
 *   caller's next synchronisation.  dr_last_error() returns the detail text of
 *   the calling thread's most recent failure.
 * Numerics.  The state and every accumulation are fp32.  Matrix-core
 *   operands: with bf16 inputs, a scalar gate and a scalar beta, the raw bf16
 *   q and k feed bf16 ops as they are, and the fp32 quantities they meet (the
 *   state, lambda U) are carried as bf16 hi + lo pairs (16 significant bits);
 *   with a channel-wise gate or beta, the gated operands and the state are
 *   single fp16 terms; fp32 inputs use a two-term fp16 split (about 22
 *   significant bits).  The chunk matrices T^ and P are stored in fp16 (two
 *   terms for fp32 inputs).  NaN/Inf inputs propagate and are not checked.
 *   For a channel-wise gate, each chunk's cumulative log-gate must stay above
 *   -80 per channel (i.e. alpha products over 64 tokens above e^-80);
 *   stronger decay underflows fp32 in the chunk algebra.
 * Magnitudes.  The operands derived from v and the state (R = V - gamma K S
 *   and U with every mode; with a channel-wise gate or beta also the state and
 *   the gated operands) are fp16 terms, finite up to 65504 and normal down to
 *   2^-14.  With unit-norm keys the parity bounds (relative to each output's
 *   largest entry: 3e-3 for bf16 inputs, 1e-4 for fp32) hold for v and S0
 *   whose entries are N(0, 1)-like scaled by 2^e, e in [-12, 13] for bf16
 *   inputs and [-8, 13] for fp32 inputs (largest |v| entries about 3.5e4).
 *   Larger values overflow, and the outputs then hold Inf or NaN; smaller ones
 *   lose precision to fp16 subnormals.  Neither is checked: callers scale v
 *   and S0 by a power of two (the outputs scale with them exactly).
 * Overlaps.  Outputs (o, S_final, the states of a decode step, gradients)
 *   must not overlap any input, the workspace or each other; S_final may be
 *   S0 itself.  Any other overlap is DR_ERR_UNSUPPORTED.
 * Empty work.  B, H, N or L equal to 0 is valid: nothing is computed, and
 *   with L == 0 S_final receives S0 (zeros if S0 is NULL).
 */
#ifndef DELTARULE_H
#define DELTARULE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DR_ABI_VERSION 10

typedef enum {
    DR_OK = 0,
    DR_ERR_NULL = 1,        /* a required pointer is NULL (or a forbidden one is not) */
    DR_ERR_SHAPE = 2,       /* a dimension is negative (0 is valid: no work) */
    DR_ERR_UNSUPPORTED = 3, /* d_k / d_v / mode / dtype combination not provided */
    DR_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
    DR_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
    DR_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed */
} dr_status;

typedef enum { DR_F32 = 0, DR_BF16 = 1 } dr_dtype;

/* alpha_t: none (alpha == 1), one scalar per token, or one per key channel. */
typedef enum { DR_GATE_NONE = 0, DR_GATE_SCALAR = 1, DR_GATE_CHANNEL = 2 } dr_gate_mode;

/* beta_t: one scalar per token, or one per key channel (needs d_v == d_k). */
typedef enum { DR_BETA_SCALAR = 0, DR_BETA_CHANNEL = 1 } dr_beta_mode;

/* Input preparation flags (bitwise or; 0 = inputs used as given). */
typedef enum { DR_IN_QK_L2NORM = 1, DR_IN_BETA_LOGIT = 2 } dr_input_flags;

/* Shapes and modes of a chunked forward.
 *   B, H >= 0 sequences x heads; L >= 0 tokens; Dk in {64, 128};
 *   Dv a multiple of 16 in [16, 256] (Dv == Dk when beta == DR_BETA_CHANNEL).
 *   in_dtype types q, k, v; out_dtype types o.
 *   input_flags: dr_input_flags bits (other bits: DR_ERR_UNSUPPORTED). */
typedef struct {
    int B, H, L, Dk, Dv;
    dr_dtype in_dtype;
    dr_dtype out_dtype;
    dr_gate_mode gate;
    dr_beta_mode beta;
    unsigned input_flags;
} dr_chunk_desc;

/* Shapes and modes of one recurrent decode step on N x H independent states
 * (same limits as dr_chunk_desc for Dk, Dv, the modes and input_flags). */
typedef struct {
    int N, H, Dk, Dv;
    dr_dtype in_dtype;
    dr_dtype out_dtype;
    dr_gate_mode gate;
    dr_beta_mode beta;
    unsigned input_flags;
} dr_decode_desc;

/* Bytes of device workspace dr_chunk_fwd needs for `d` (0 if d is invalid or
 * there is no work).  Depends only on the shape and the modes. */
size_t dr_chunk_fwd_workspace_bytes(const dr_chunk_desc* d);

/*
 * dr_chunk_fwd -- chunked prefill over whole sequences.
 *
 * Computes, for every (b, h), o_t for t = 0..L-1 and the final state S_L of
 * the recurrence above, started from S0.  The method (DeltaNet page, step 7,
 * and the FG2-GDN page, section 2, on the WY form) is chunkwise: 64-token
 * chunks, a per-chunk triangular solve, and a sequential pass that carries
 * the fp32 state between chunks.  Any L >= 0 is accepted; a partial last chunk
 * is masked.
 *
 *   q          [B][H][L][Dk]  in_dtype
 *   k          [B][H][L][Dk]  in_dtype
 *   v          [B][H][L][Dv]  in_dtype
 *   log_alpha  [B][H][L] (GATE_SCALAR) or [B][H][L][Dk] (GATE_CHANNEL) fp32,
 *              natural log of alpha_t; must be NULL iff gate == DR_GATE_NONE
 *   beta       [B][H][L] (BETA_SCALAR) or [B][H][L][Dk] (BETA_CHANNEL) fp32,
 *              expected in [0, 1] (not checked), or logits (DR_IN_BETA_LOGIT)
 *   S0         [B][H][Dk][Dv] fp32 initial states, or NULL for zeros
 *   o          [B][H][L][Dv]  out_dtype, written
 *   S_final    [B][H][Dk][Dv] fp32, written, or NULL to skip; may alias S0
 *              exactly (in-place state carry) but no other argument
 *   workspace  device scratch of at least dr_chunk_fwd_workspace_bytes(d)
 *              bytes (may be NULL when that is 0); its contents on entry are
 *              ignored and on exit are unspecified
 * o must not overlap any input (DR_ERR_UNSUPPORTED).  Returns DR_OK or an error
 * status (see above).
 */
dr_status dr_chunk_fwd(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* beta, const float* S0, void* o,
                       float* S_final, void* workspace, size_t workspace_bytes, void* stream);

/* Size of the per-GPU device scratch array that dr_chunk_fwd_noalloc uses in
 * place of a workspace (256 MiB: the workspace of B * H * L up to about
 * 16 * 2^14 tokens with bf16 inputs, a scalar gate and a scalar beta). */
#define DR_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/*
 * dr_chunk_fwd_noalloc -- dr_chunk_fwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same computation, arguments and error behaviour as
 * dr_chunk_fwd, without the workspace arguments: the library's own device
 * scratch array of DR_NOALLOC_SCRATCH_BYTES serves as the workspace.  Each GPU
 * the library runs on holds one such array from the library's first use on it
 * until the process ends; the call allocates and frees nothing.
 *   Limit: a call whose dr_chunk_fwd_workspace_bytes(d) exceeds
 *   DR_NOALLOC_SCRATCH_BYTES returns DR_ERR_WORKSPACE (nothing launched).
 *   Sharing: every call on one GPU uses that GPU's array, whose contents a
 *   call neither needs on entry nor leaves defined; two calls on one GPU that
 *   overlap in time (different streams or host threads without ordering
 *   between them) race and give undefined results.  Calls ordered on one
 *   stream are safe.
 */
dr_status dr_chunk_fwd_noalloc(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const float* S0, void* o,
                               float* S_final, void* stream);

/* Bytes of device workspace dr_chunk_fwd_kv needs for `d` (0 if d is invalid
 * for it or there is no work): dr_chunk_fwd_workspace_bytes(d) with a channel
 * beta; with scalar strengths also the channel-beta operand planes. */
size_t dr_chunk_fwd_kv_workspace_bytes(const dr_chunk_desc* d);

/*
 * dr_chunk_fwd_kv -- dr_chunk_fwd with separate erase and write strengths
 * (FG2-GDN page, section "Erweiterung: FG2-GDN+"; its ablation study decouples
 * them as vectors and as scalars): beta_k takes the place of beta on kt in both
 * the erase and the write term, beta_v scales v.
 *
 *   d->beta    DR_BETA_CHANNEL: d_k-vectors; DR_BETA_SCALAR: one value per
 *              token each.  Either way Dv == Dk (else DR_ERR_UNSUPPORTED):
 *              scalar strengths run on the channel-beta kernels, every
 *              channel taking its token's value.
 *   beta_k     [B][H][L][Dk] or [B][H][L] fp32, expected in [0, 1] (not checked)
 *   beta_v     beta_k's shape, fp32, expected in [0, 1] (not checked)
 *   workspace  at least dr_chunk_fwd_kv_workspace_bytes(d) bytes
 * Every other argument and the error behaviour are those of dr_chunk_fwd;
 * beta_v == beta_k gives dr_chunk_fwd's result up to rounding.
 */
dr_status dr_chunk_fwd_kv(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                          const float* log_alpha, const float* beta_k, const float* beta_v,
                          const float* S0, void* o, float* S_final, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Bytes of device workspace dr_chunk_fwd_precond needs for `d` (the channel-gate
 * operand planes are always used; 0 if d is invalid or there is no work). */
size_t dr_chunk_fwd_precond_workspace_bytes(const dr_chunk_desc* d);

/*
 * dr_chunk_fwd_precond -- dr_chunk_fwd with a diagonal preconditioner on the
 * delta rule's gradient step, i.e. write-side key scales (OSDN page, section
 * "Method"; the preconditioned delta rule page, abstract): with w = s (.) kt,
 *   S_t = (I - w_t kt_t^T) Diag(alpha_t) S_{t-1} + w_t vt_t^T,  o_t = S_t^T q_t.
 * s == 1 gives dr_chunk_fwd's recurrence.
 *
 *   key_scale  [B][H][L][Dk] fp32, the preconditioner's diagonal per token
 *   workspace  at least dr_chunk_fwd_precond_workspace_bytes(d) bytes
 * Every other argument, every mode (gate, beta, dtypes, input_flags) and the
 * error behaviour are those of dr_chunk_fwd.  Whatever the gate, the call runs
 * the channel-gate kernels (a scalar or absent gate broadcast per channel).
 */
dr_status dr_chunk_fwd_precond(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const float* key_scale,
                               const float* S0, void* o, float* S_final, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * dr_decode_step -- one recurrent step (DeltaNet page, property list: inference
 * uses the recurrent form with a constant-size state) for N x H independent
 * states, one new token each, updating the states in place:
 *
 *   S[n][h] <- (I - kt kt^T) Diag(alpha) S[n][h] + kt vt^T,  o[n][h] = S[n][h]^T q
 *
 *   q, k       [N][H][Dk] in_dtype;  v [N][H][Dv] in_dtype
 *   log_alpha  [N][H] or [N][H][Dk] fp32, NULL iff gate == DR_GATE_NONE
 *   beta       [N][H] or [N][H][Dk] fp32
 *   S          [N][H][Dk][Dv] fp32, read and overwritten
 *   o          [N][H][Dv] out_dtype, written; must not overlap S or the inputs
 * Equivalent to dr_chunk_fwd with L == 1, S0 == S_final == S.
 */
dr_status dr_decode_step(const dr_decode_desc* d, const void* q, const void* k, const void* v,
                         const float* log_alpha, const float* beta, float* S, void* o,
                         void* stream);

/*
 * dr_decode_step_kv -- dr_decode_step with separate erase and write strengths
 * (FG2-GDN page, section "Erweiterung: FG2-GDN+"):
 *
 *   S[n][h] <- (I - kt kt^T) Diag(alpha) S[n][h] + kt vt^T,
 *   kt = sqrt(beta_k) (.) k,  vt = sqrt(beta_v) (.) v
 *
 *   beta_k, beta_v  [N][H][Dk] (DR_BETA_CHANNEL, needs Dv == Dk) or [N][H]
 *                   (DR_BETA_SCALAR) fp32
 * Every other argument as for dr_decode_step.  Equivalent to dr_chunk_fwd_kv
 * with L == 1, S0 == S_final == S.
 */
dr_status dr_decode_step_kv(const dr_decode_desc* d, const void* q, const void* k, const void* v,
                            const float* log_alpha, const float* beta_k, const float* beta_v,
                            float* S, void* o, void* stream);

/*
 * dr_decode_step_precond -- dr_decode_step with write-side key scales (the
 * preconditioner's diagonal, as in dr_chunk_fwd_precond):
 *   S[n][h] <- (I - w kt^T) Diag(alpha) S[n][h] + w vt^T,  w = s (.) kt
 *   key_scale  [N][H][Dk] fp32
 * Every other argument as for dr_decode_step.
 */
dr_status dr_decode_step_precond(const dr_decode_desc* d, const void* q, const void* k, const void* v,
                                 const float* log_alpha, const float* beta, const float* key_scale,
                                 float* S, void* o, void* stream);

/* Bytes of device workspace dr_chunk_bwd needs for `d` (0 if d is invalid for
 * the backward or there is no work): per 64-token chunk of every sequence,
 * three 64 x 64 matrices, 64 gate values, two Dk x Dv states and three
 * 64 x Dv blocks, all fp32 (for bf16 inputs without a channel gate, channel
 * beta or DR_IN_QK_L2NORM: one 64 x Dv block and 31744 bytes of packed
 * operands in place of the other two); with a channel gate 64 x Dk gate
 * values and four more 64 x Dk blocks (the gated keys and queries); with a channel beta or
 * DR_IN_QK_L2NORM fp32 copies of q, k and v and up to four floats per token;
 * with DR_IN_BETA_LOGIT alone one float per token. */
size_t dr_chunk_bwd_workspace_bytes(const dr_chunk_desc* d);

/* The least workspace dr_chunk_bwd accepts for `d` (0 if d is invalid or
 * there is no work).  For bf16 inputs with a scalar gate or none, a scalar
 * beta and no input preparation, a workspace below
 * dr_chunk_bwd_workspace_bytes(d) makes the call run in segments of at least
 * 32 chunks (2048 tokens), the longest that fit: it keeps S_c, H_c and dU of
 * one segment of every sequence instead of every chunk's, plus a checkpoint
 * of S at each later segment's start and the state gradient carried between
 * segments.  That costs one more forward state pass (every segment's start
 * states are recomputed from their checkpoints) and three launches per
 * segment; the gradients are bit-identical to those of a call with the full
 * workspace (the arithmetic per chunk is unchanged).  For every other mode
 * this equals dr_chunk_bwd_workspace_bytes(d). */
size_t dr_chunk_bwd_workspace_bytes_min(const dr_chunk_desc* d);

/*
 * dr_chunk_bwd -- gradients of dr_chunk_fwd's o and S_final with respect to
 * every input, for the loss whose gradients with respect to o and S_final
 * are dO and dS_final.  The pages print no backward; this is the exact
 * reverse-mode derivative of the chunkwise form that dr_chunk_fwd computes
 * (DeltaNet page, step 7 and the hardware notes; FG2-GDN page, section 2),
 * evaluated chunk by chunk: a sequential pass recomputes each chunk's start
 * state, a reverse pass carries the state gradient, and a per-chunk pass
 * forms the gradients of q, k, beta and log alpha.  Everything runs in fp32,
 * and every sum in a fixed order: repeated calls give the same bits.
 *
 * Covered modes: every gate and beta mode (plain DeltaNet, Gated DeltaNet,
 * KDA, FG2-GDN), every input_flags combination, d->out_dtype DR_F32 (the
 * dtype of dO); anything else is DR_ERR_UNSUPPORTED.  The gradients are with
 * respect to the arrays as passed: with DR_IN_QK_L2NORM those of the raw q
 * and k (through the normalisation; a zero row has a zero gradient), with
 * DR_IN_BETA_LOGIT those of the logits (through the sigmoid).  With
 * DR_BETA_CHANNEL or the input preparation a per-token pass first writes fp32
 * copies of what the recurrence sees (normalised q and k, the strengths'
 * values; with DR_BETA_CHANNEL sqrt(beta) (.) k and sqrt(beta) (.) v with
 * unit strength), the kernels run on those, and a second per-token pass maps
 * the gradients back (DR_BETA_CHANNEL: beta > 0 assumed, the square root has
 * no derivative at 0; logits always satisfy it).  in_dtype (fp32 or bf16) is the dtype
 * of q, k, v; Dk, Dv as for dr_chunk_fwd.  With DR_GATE_CHANNEL the kernels
 * work on keys and queries scaled by e^{+-G}, G a channel's cumulative log
 * decay within a 64-token chunk; a chunk in which some channel's decay falls
 * below -60 takes those products relative to the channel's mid-chunk decay,
 * so every channel's decay over a chunk must stay above about -170 (an
 * average log alpha of about -2.7 per token; not checked).
 *
 *   q, k, v, log_alpha, beta, S0   as for dr_chunk_fwd (S0 may be NULL: zeros)
 *   dO         [B][H][L][Dv] fp32, gradient with respect to o
 *   dS_final   [B][H][Dk][Dv] fp32, gradient with respect to S_final, or NULL
 *              (zero)
 *   dq, dk     [B][H][L][Dk] fp32, written
 *   dv         [B][H][L][Dv] fp32, written
 *   dlog_alpha log_alpha's shape ([B][H][L] or [B][H][L][Dk]) fp32, written;
 *              required with a gate, must be NULL without one
 *   dbeta      beta's shape ([B][H][L] or [B][H][L][Dk]) fp32, written
 *   dS0        [B][H][Dk][Dv] fp32, gradient with respect to S0, written, or
 *              NULL to skip
 *   workspace  device scratch of workspace_bytes bytes, at least
 *              dr_chunk_bwd_workspace_bytes_min(d); with less than
 *              dr_chunk_bwd_workspace_bytes(d) the call runs in segments
 *              (see dr_chunk_bwd_workspace_bytes_min); contents on entry
 *              ignored, on exit unspecified; fewer bytes: DR_ERR_WORKSPACE
 * Outputs must not overlap each other or any input.  Returns DR_OK or an
 * error status; nothing is launched on an error.
 */
dr_status dr_chunk_bwd(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* beta, const float* S0, const float* dO,
                       const float* dS_final, float* dq, float* dk, float* dv, float* dlog_alpha,
                       float* dbeta, float* dS0, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace dr_chunk_bwd_kv needs for `d` (0 if d is invalid
 * for it or there is no work). */
size_t dr_chunk_bwd_kv_workspace_bytes(const dr_chunk_desc* d);

/*
 * dr_chunk_bwd_kv -- dr_chunk_bwd for dr_chunk_fwd_kv: gradients with separate
 * erase and write strengths (FG2-GDN page, section "Erweiterung: FG2-GDN+";
 * the same reading as the forward, kt = sqrt(beta_k) (.) k,
 * vt = sqrt(beta_v) (.) v).
 *
 *   d->beta    DR_BETA_CHANNEL or DR_BETA_SCALAR as for dr_chunk_fwd_kv;
 *              Dv == Dk either way
 *   beta_k, beta_v    [B][H][L][Dk] or [B][H][L] fp32, > 0
 *   dbeta_k, dbeta_v  beta_k's shape, fp32, written (with scalar strengths the
 *                     sum over the token's channels)
 *   workspace  at least dr_chunk_bwd_kv_workspace_bytes(d) bytes
 * Every other argument and the error behaviour are those of dr_chunk_bwd;
 * beta_v == beta_k gives dr_chunk_bwd's gradients, with dbeta_k + dbeta_v its
 * dbeta.
 */
dr_status dr_chunk_bwd_kv(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                          const float* log_alpha, const float* beta_k, const float* beta_v, const float* S0,
                          const float* dO, const float* dS_final, float* dq, float* dk, float* dv,
                          float* dlog_alpha, float* dbeta_k, float* dbeta_v, float* dS0, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Bytes of device workspace dr_chunk_bwd_precond needs for `d` (0 if d is
 * invalid for it or there is no work): that of the channel-gate backward for
 * every gate mode, plus Dk floats per token with a scalar gate. */
size_t dr_chunk_bwd_precond_workspace_bytes(const dr_chunk_desc* d);

/*
 * dr_chunk_bwd_precond -- dr_chunk_bwd for dr_chunk_fwd_precond: gradients of
 * the preconditioned rule, write key w_t = s_t (.) kt (OSDN page, "Method";
 * the reading of dr_chunk_fwd_precond).  In the chunk algebra w takes kt's
 * place on the column side of A and P and in the state update, and the read
 * side keeps kt, so the gradient of kt gathers both roles:
 * dk = dk_read + s (.) dw and ds = kt (.) dw (through the input preparation
 * and sqrt(beta) as in dr_chunk_bwd).  Every gate mode runs the channel-gate
 * kernels, a scalar or absent gate broadcast to every channel (the same limit
 * on each channel's cumulative log decay within a chunk applies); with a
 * scalar gate, d log alpha is summed over the channels at the end.
 *
 *   key_scale   [B][H][L][Dk] fp32, the diagonal s_t
 *   dkey_scale  [B][H][L][Dk] fp32, written
 *   workspace   at least dr_chunk_bwd_precond_workspace_bytes(d) bytes
 * Every other argument, the modes (every gate and beta mode, input_flags) and
 * the error behaviour are those of dr_chunk_bwd; key_scale and dkey_scale are
 * required when there are tokens.
 */
dr_status dr_chunk_bwd_precond(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const float* key_scale, const float* S0,
                               const float* dO, const float* dS_final, float* dq, float* dk, float* dv,
                               float* dlog_alpha, float* dbeta, float* dkey_scale, float* dS0, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Per-kernel timing, for benchmarks and profiling (not part of the method).
 * Between dr_profile_begin and dr_profile_end every chunked-forward, backward
 * and decode call launches each of its kernels with a start and a stop event
 * of its own, set from the kernel dispatch's timestamps (no marker packets
 * between the kernels); dr_profile_end waits for those events and reports the
 * summed kernel durations.  Calls made while profiling must come from one
 * host thread.  dr_profile_begin discards any earlier unreported records.  The
 * events belong to the library: dr_profile_begin creates a pool of 1024 (more
 * only if a window needs them), and the library keeps them for reuse until
 * the process ends, so that no event is created while kernels are timed.
 * Returns DR_ERR_NULL for a NULL report, DR_ERR_HIP if an event fails.
 */
typedef struct dr_profile_report {
    int chunk_calls;    /* dr_chunk_fwd(_kv) calls that launched kernels */
    int decode_calls;   /* dr_decode_step(_kv) calls that launched kernels */
    double prep_ms;     /* chunk preparation kernel (gates, A, T, P) */
    double scan_ms;     /* inter-chunk state scan kernel (o and S_final) */
    double decode_ms;   /* recurrent decode kernel */
    int bwd_calls;      /* dr_chunk_bwd calls that launched kernels */
    double bwd_prep_ms;   /* backward: per-chunk T, P and K K^T */
    double bwd_fscan_ms;  /* backward: forward state scan (chunk start states) */
    double bwd_rscan_ms;  /* backward: reverse scan of the state gradient */
    double bwd_post_ms;   /* backward: per-chunk gradients of q, k, beta, log alpha */
} dr_profile_report;

dr_status dr_profile_begin(void);
dr_status dr_profile_end(dr_profile_report* report);

/* Static text for a status code. */
const char* dr_status_str(dr_status s);

/* Detail text of the calling thread's last failing call ("" if none). */
const char* dr_last_error(void);

/* DR_ABI_VERSION of the built library. */
int dr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DELTARULE_H */
