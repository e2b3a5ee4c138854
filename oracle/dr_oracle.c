/*
 * dr_oracle.c -- plain fp64 CPU oracle of the delta-rule forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path may include, link or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code with the HIP kernels.
 *
 * What it computes, token by token, for every (batch b, head h) independently:
 *
 *   FG2-GDN page, section 2 ("Kerninnovation"), the scaled key/value equation:
 *       kt = sqrt(beta_t) (.) k_t        vt = sqrt(beta_t) (.) v_t
 *     beta_t is a scalar (DeltaNet / GDN / KDA) or a d_k-vector (FG2-GDN);
 *     a scalar beta scales every channel alike.
 *   FG2-GDN page, section 2, the state-update equation:
 *       S_t = (I - kt kt^T) Diag(alpha_t) S_{t-1} + kt vt^T
 *     S is d_k x d_v.  alpha_t is 1 (plain DeltaNet), a scalar (Gated
 *     DeltaNet, section 1 of the same page) or a d_k-vector (KDA, idem);
 *     it is passed as log alpha.
 *   DeltaNet page, the seven-step list, step 6: the output reads the updated
 *   state, o_t = S_t^T q_t (the page writes S q with S stored d_v x d_k).
 *   FG2-GDN page, section "Erweiterung: FG2-GDN+": separate erase and write
 *   strengths beta^k_t and beta^v_t.  The page prints no equation; the reading
 *   taken here is kt = sqrt(beta^k_t) (.) k_t (in both the erase and the
 *   write term) and vt = sqrt(beta^v_t) (.) v_t (dro_forward_kv); with
 *   beta^v = beta^k it is the equation above.
 *
 * Write-side key scaling (dro_forward_ex, key_scale non-NULL): the OSDN page
 * (section "Method") and the preconditioned delta rule page (its abstract)
 * precondition the delta rule's gradient step with a diagonal matrix, which
 * the OSDN page states is the same as scaling the key on the write side per
 * feature.  The preconditioner's own online update is not printed; here it is
 * an input s_t (a d_k-vector per token), and with w_t = s_t (.) kt_t
 *       S_t = (I - w_t kt_t^T) Diag(alpha_t) S_{t-1} + w_t vt_t^T,
 * i.e. S' = Diag(alpha_t) S_{t-1}, S_t = S' - Diag(s_t) grad, grad = kt (S'^T kt
 * - vt)^T the gradient of 1/2 |S^T kt - vt|^2 at S'.  s = 1 is the update
 * above.
 *
 * Optional input preparation (dro_forward_ex, input_flags), the steps in
 * front of the recurrence:
 *   DRO_IN_QK_L2NORM  DeltaNet page, step list, step 2, and its note on the
 *     key/query map: keys pass through a feature map followed by L2
 *     normalisation, and queries get the same map.  Here q_t and k_t are
 *     replaced by q_t / |q_t|_2 and k_t / |k_t|_2 before anything else (a zero
 *     vector stays zero).  The learned parts of the map (a projection, SiLU, a
 *     short convolution) belong to the layer in front and are not modelled.
 *   DRO_IN_BETA_LOGIT  DeltaNet page, list of design choices: beta_t from a
 *     sigmoid projection.  The strength arrays (beta, and beta^v) hold the
 *     projection's output x, and beta = 1 / (1 + e^{-x}).
 *
 * The update is evaluated in the rank-one form that the DeltaNet page's steps
 * 3-5 describe (read the current map, form the error, add the outer product):
 *       S'  = Diag(alpha_t) S_{t-1}
 *       p   = S'^T kt                     (what the memory returns for kt)
 *       S_t = S' + kt (vt - p)^T
 * which is the printed product expanded: (I - kt kt^T) S' + kt vt^T.  A test
 * checks it against the literal dense product.
 *
 * No query scaling is applied.  All arithmetic is IEEE fp64.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { DRO_GATE_NONE = 0, DRO_GATE_SCALAR = 1, DRO_GATE_CHANNEL = 2 };
enum { DRO_BETA_SCALAR = 0, DRO_BETA_CHANNEL = 1 };
enum { DRO_IN_QK_L2NORM = 1, DRO_IN_BETA_LOGIT = 2 };

/* Return codes. */
enum { DRO_OK = 0, DRO_EINVAL = 1, DRO_ENOMEM = 2 };

/* 1 / |x|_2 over n entries, 0 for the zero vector. */
static double inv_l2(const double* x, int n)
{
    double s = 0.0;
    for (int c = 0; c < n; ++c) s += x[c] * x[c];
    return s > 0.0 ? 1.0 / sqrt(s) : 0.0;
}

/* A strength as given, or the sigmoid of the given logit. */
static double strength(double x, int logit)
{
    return logit ? 1.0 / (1.0 + exp(-x)) : x;
}

/* One (b, h) sequence.  Pointers are already offset to that sequence:
 *   q, k   [L][Dk]      v, o [L][Dv]
 *   la     [L] or [L][Dk] (NULL when gate == NONE)
 *   beta   [L] or [L][Dk]      scales kt
 *   betav  [L] or [L][Dk]      scales vt (the same array as beta unless the
 *                              write strength is separate)
 *   ks     [L][Dk] write-side key scales, or NULL (all ones)
 *   S      [Dk][Dv]  in: initial state, out: final state
 *   kt, vt scratch of Dk and Dv doubles, p scratch of Dv doubles. */
static void run_sequence(int L, int Dk, int Dv,
                         const double* q, const double* k, const double* v,
                         const double* la, int gate, const double* beta, const double* betav,
                         int beta_mode, const double* ks, int flags, double* S, double* o, double* kt,
                         double* vt, double* p)
{
    const int l2 = (flags & DRO_IN_QK_L2NORM) != 0;
    const int logit = (flags & DRO_IN_BETA_LOGIT) != 0;
    for (int t = 0; t < L; ++t) {
        const double* qt = q + (size_t)t * Dk;
        const double* k_t = k + (size_t)t * Dk;
        const double* v_t = v + (size_t)t * Dv;

        /* input preparation: the factors that make q_t and k_t unit vectors */
        const double qn = l2 ? inv_l2(qt, Dk) : 1.0;
        const double kn = l2 ? inv_l2(k_t, Dk) : 1.0;

        /* scaled key and value */
        for (int c = 0; c < Dk; ++c) {
            double b = beta_mode == DRO_BETA_SCALAR ? beta[t] : beta[(size_t)t * Dk + c];
            kt[c] = sqrt(strength(b, logit)) * (kn * k_t[c]);
        }
        for (int j = 0; j < Dv; ++j) {
            /* channel beta scales v's channel j by beta's channel j (d_v == d_k) */
            double b = beta_mode == DRO_BETA_SCALAR ? betav[t] : betav[(size_t)t * Dk + j];
            vt[j] = sqrt(strength(b, logit)) * v_t[j];
        }

        /* S' = Diag(alpha_t) S : row c of S is scaled by alpha_t[c] */
        if (gate != DRO_GATE_NONE) {
            for (int c = 0; c < Dk; ++c) {
                double a = gate == DRO_GATE_SCALAR ? exp(la[t]) : exp(la[(size_t)t * Dk + c]);
                double* row = S + (size_t)c * Dv;
                for (int j = 0; j < Dv; ++j) row[j] *= a;
            }
        }

        /* p = S'^T kt */
        for (int j = 0; j < Dv; ++j) p[j] = 0.0;
        for (int c = 0; c < Dk; ++c) {
            const double* row = S + (size_t)c * Dv;
            for (int j = 0; j < Dv; ++j) p[j] += row[j] * kt[c];
        }

        /* S_t = S' + w (vt - p)^T, the write-side key w = s (.) kt */
        for (int c = 0; c < Dk; ++c) {
            const double w = ks ? ks[(size_t)t * Dk + c] * kt[c] : kt[c];
            double* row = S + (size_t)c * Dv;
            for (int j = 0; j < Dv; ++j) row[j] += w * (vt[j] - p[j]);
        }

        /* o_t = S_t^T q_t */
        double* ot = o + (size_t)t * Dv;
        for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
        for (int c = 0; c < Dk; ++c) {
            const double* row = S + (size_t)c * Dv;
            for (int j = 0; j < Dv; ++j) ot[j] += row[j] * (qn * qt[c]);
        }
    }
}

/*
 * dro_forward_ex -- the whole batch, with separate key and value strengths and
 * the optional input preparation.
 *   q, k      [B][H][L][Dk] fp64
 *   v         [B][H][L][Dv] fp64
 *   log_alpha [B][H][L] (gate SCALAR) or [B][H][L][Dk] (gate CHANNEL); NULL for NONE
 *   beta      [B][H][L] (SCALAR) or [B][H][L][Dk] (CHANNEL; needs Dv == Dk): beta^k
 *   beta_v    beta^v, the same shape as beta
 *   key_scale [B][H][L][Dk] write-side key scales s_t, or NULL (no scaling)
 *   input_flags  DRO_IN_QK_L2NORM | DRO_IN_BETA_LOGIT, or 0
 *   S0        [B][H][Dk][Dv] or NULL (zeros)
 *   o         [B][H][L][Dv]     out
 *   S_final   [B][H][Dk][Dv]    out, may be NULL
 *   nthreads  worker threads over (b, h); <= 0 means the OpenMP default
 * Decode is the same call with L == 1 and S0 the current states.
 */
int dro_forward_ex(int B, int H, int L, int Dk, int Dv,
                   const double* q, const double* k, const double* v,
                   const double* log_alpha, int gate, const double* beta, const double* beta_v,
                   int beta_mode, const double* key_scale, int input_flags, const double* S0,
                   double* o, double* S_final, int nthreads)
{
    if (B <= 0 || H <= 0 || L < 0 || Dk <= 0 || Dv <= 0) return DRO_EINVAL;
    if (input_flags & ~(DRO_IN_QK_L2NORM | DRO_IN_BETA_LOGIT)) return DRO_EINVAL;
    if (!q || !k || !v || !beta || !beta_v || !o) return DRO_EINVAL;
    if (gate < DRO_GATE_NONE || gate > DRO_GATE_CHANNEL) return DRO_EINVAL;
    if (beta_mode != DRO_BETA_SCALAR && beta_mode != DRO_BETA_CHANNEL) return DRO_EINVAL;
    if ((gate == DRO_GATE_NONE) != (log_alpha == NULL)) return DRO_EINVAL;
    if (beta_mode == DRO_BETA_CHANNEL && Dv != Dk) return DRO_EINVAL;

    const long nseq = (long)B * H;
    const size_t sz = (size_t)Dk * Dv;
    int err = DRO_OK;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (long s = 0; s < nseq; ++s) {
        double* S = (double*)malloc(sizeof(double) * (sz + 2 * (size_t)Dk + 2 * (size_t)Dv));
        if (!S) {
            err = DRO_ENOMEM;
            continue;
        }
        double* kt = S + sz;
        double* vt = kt + Dk;
        double* p = vt + Dv;
        if (S0) memcpy(S, S0 + (size_t)s * sz, sizeof(double) * sz);
        else memset(S, 0, sizeof(double) * sz);
        const size_t lw = (gate == DRO_GATE_CHANNEL) ? (size_t)L * Dk : (size_t)L;
        const size_t bw = (beta_mode == DRO_BETA_CHANNEL) ? (size_t)L * Dk : (size_t)L;
        run_sequence(L, Dk, Dv,
                     q + (size_t)s * L * Dk, k + (size_t)s * L * Dk, v + (size_t)s * L * Dv,
                     log_alpha ? log_alpha + (size_t)s * lw : NULL, gate,
                     beta + (size_t)s * bw, beta_v + (size_t)s * bw, beta_mode,
                     key_scale ? key_scale + (size_t)s * L * Dk : NULL, input_flags,
                     S, o + (size_t)s * L * Dv, kt, vt, p);
        if (S_final) memcpy(S_final + (size_t)s * sz, S, sizeof(double) * sz);
        free(S);
    }
    (void)nthreads;
    return err;
}

/* Separate strengths, inputs as given. */
int dro_forward_kv(int B, int H, int L, int Dk, int Dv,
                   const double* q, const double* k, const double* v,
                   const double* log_alpha, int gate, const double* beta, const double* beta_v,
                   int beta_mode, const double* S0, double* o, double* S_final, int nthreads)
{
    return dro_forward_ex(B, H, L, Dk, Dv, q, k, v, log_alpha, gate, beta, beta_v, beta_mode, NULL, 0,
                          S0, o, S_final, nthreads);
}

/* The same with one strength for both the key and the value (beta^v = beta). */
int dro_forward(int B, int H, int L, int Dk, int Dv,
                const double* q, const double* k, const double* v,
                const double* log_alpha, int gate, const double* beta, int beta_mode,
                const double* S0, double* o, double* S_final, int nthreads)
{
    return dro_forward_kv(B, H, L, Dk, Dv, q, k, v, log_alpha, gate, beta, beta, beta_mode, S0, o,
                          S_final, nthreads);
}

/*
 * dro_backward -- gradients of the forward above by reverse-mode
 * differentiation of the token recurrence (dro_backward: one strength, inputs
 * as given; dro_backward_kv: separate strengths; dro_backward_ex: any of
 * these with write-side key scales and the input preparation).
 * The pages give no backward (the DeltaNet page, step 7, only says training
 * uses the chunkwise form); this is the chain rule applied to the update as
 * written, in the order of the forward's steps, with qh, kh the prepared query
 * and key (the inputs themselves, or their unit vectors) and w = s (.) kt the
 * write-side key (kt itself without key scales):
 *   S' = Diag(alpha) S_{t-1},  p = S'^T kt,  u = vt - p,
 *   S_t = S' + w u^T,  o_t = S_t^T qh_t.
 * With G the gradient of the loss with respect to S_t (dS_final for t = L,
 * plus qh_t do_t^T from the output):
 *   dqh_t = S_t do_t,   du = G^T w,   dw = G u,   dvt = du,
 *   dkt = s (.) dw - S' du,   ds = kt (.) dw,
 *   dS' = G - kt du^T,   dalpha_c = sum_j dS'_cj S_{t-1,cj},
 *   G <- Diag(alpha) dS'   (the gradient with respect to S_{t-1}),
 * then through kt = sqrt(beta) kh, vt = sqrt(beta) v, alpha = e^{log alpha},
 * beta = sigmoid(x) (logits: dx = dbeta beta (1 - beta)) and the
 * normalisation qh = q / |q| (dq = (dqh - qh (qh . dqh)) / |q|; the
 * normalisation is not differentiable at the zero vector, which it leaves
 * at zero: its gradient there is taken as zero), likewise for k.
 *   dO        [B][H][L][Dv]  gradient of the loss with respect to o
 *   dS_final  [B][H][Dk][Dv] with respect to S_final, or NULL (zero)
 *   dq, dk    [B][H][L][Dk]  out;  dv [B][H][L][Dv] out
 *   dlog_alpha  out, log_alpha's shape, or NULL (gate NONE)
 *   dbeta     out, beta's shape (the derivative of sqrt at 0 is infinite:
 *             beta > 0 is assumed; with logits it always is)
 *   dS0       [B][H][Dk][Dv] out, or NULL
 * dro_backward_kv takes a separate write strength beta_v (beta's shape; the
 * forward's FG2-GDN+ reading: vt = sqrt(beta_v) v, beta on kt only) and
 * returns its gradient in dbeta_v; dbeta then holds beta's (erase strength's)
 * part alone.  dro_backward_ex: beta_v and dbeta_v as for dro_backward_kv or
 * both NULL (one strength); key_scale [B][H][L][Dk] and its gradient
 * dkey_scale, both NULL without key scales; input_flags as for the forward.
 */
static int backward_impl(int B, int H, int L, int Dk, int Dv,
                         const double* q, const double* k, const double* v,
                         const double* log_alpha, int gate, const double* beta, const double* beta_v,
                         int beta_mode, const double* key_scale, int flags, const double* S0, const double* dO,
                         const double* dS_final, double* dq, double* dk, double* dv, double* dlog_alpha,
                         double* dbeta, double* dbeta_v, double* dkey_scale, double* dS0, int nthreads)
{
    if (B <= 0 || H <= 0 || L < 0 || Dk <= 0 || Dv <= 0) return DRO_EINVAL;
    if (!q || !k || !v || !beta || !dO || !dq || !dk || !dv || !dbeta) return DRO_EINVAL;
    if (gate < DRO_GATE_NONE || gate > DRO_GATE_CHANNEL) return DRO_EINVAL;
    if (beta_mode != DRO_BETA_SCALAR && beta_mode != DRO_BETA_CHANNEL) return DRO_EINVAL;
    if ((gate == DRO_GATE_NONE) != (log_alpha == NULL)) return DRO_EINVAL;
    if (gate != DRO_GATE_NONE && !dlog_alpha) return DRO_EINVAL;
    if (beta_mode == DRO_BETA_CHANNEL && Dv != Dk) return DRO_EINVAL;
    if ((key_scale == NULL) != (dkey_scale == NULL)) return DRO_EINVAL;
    if (flags & ~(DRO_IN_QK_L2NORM | DRO_IN_BETA_LOGIT)) return DRO_EINVAL;
    const int l2 = (flags & DRO_IN_QK_L2NORM) != 0;
    const int logit = (flags & DRO_IN_BETA_LOGIT) != 0;

    const long nseq = (long)B * H;
    const size_t sz = (size_t)Dk * Dv;
    int err = DRO_OK;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (long s = 0; s < nseq; ++s) {
        /* the states S_0 .. S_L, then the working arrays */
        double* St = (double*)malloc(sizeof(double) * ((size_t)(L + 1) * sz + 2 * sz + 11 * (size_t)Dk +
                                                       6 * (size_t)Dv));
        if (!St) {
            err = DRO_ENOMEM;
            continue;
        }
        double* G = St + (size_t)(L + 1) * sz;
        double* Sp = G + sz;
        double* kt = Sp + sz;       /* Dk each: */
        double* al = kt + Dk;
        double* sbk = al + Dk;
        double* dkt = sbk + Dk;
        double* qh = dkt + Dk;
        double* kh = qh + Dk;
        double* w = kh + Dk;
        double* dw = w + Dk;
        double* dqh = dw + Dk;
        double* dkh = dqh + Dk;
        double* bkv = dkh + Dk;
        double* vt = bkv + Dk;      /* Dv each: */
        double* u = vt + Dv;
        double* dvt = u + Dv;
        double* sbv = dvt + Dv;
        double* bvv = sbv + Dv;
        double* pp = bvv + Dv;
        (void)pp;
        const size_t lw = (gate == DRO_GATE_CHANNEL) ? (size_t)L * Dk : (size_t)L;
        const size_t bw = (beta_mode == DRO_BETA_CHANNEL) ? (size_t)L * Dk : (size_t)L;
        const double* qs = q + (size_t)s * L * Dk;
        const double* ks_ = k + (size_t)s * L * Dk;
        const double* vs = v + (size_t)s * L * Dv;
        const double* las = log_alpha ? log_alpha + (size_t)s * lw : NULL;
        const double* bs = beta + (size_t)s * bw;
        const double* bvs = beta_v ? beta_v + (size_t)s * bw : bs;   /* the write strength */
        const double* kss = key_scale ? key_scale + (size_t)s * L * Dk : NULL;
        /* outputs, then the forward step's scratch: kt (Dk), vt (Dv), p (Dv) */
        double* tmp_o = (double*)malloc(sizeof(double) * ((size_t)L * Dv + (size_t)Dk + 2 * (size_t)Dv));
        if (!tmp_o) {
            free(St);
            err = DRO_ENOMEM;
            continue;
        }
        /* forward, keeping every state */
        if (S0) memcpy(St, S0 + (size_t)s * sz, sizeof(double) * sz);
        else memset(St, 0, sizeof(double) * sz);
        {
            double* ktmp = tmp_o + (size_t)L * Dv;
            double* vtmp = ktmp + Dk;
            double* ptmp = vtmp + Dv;
            for (int t = 0; t < L; ++t) {
                memcpy(St + (size_t)(t + 1) * sz, St + (size_t)t * sz, sizeof(double) * sz);
                run_sequence(1, Dk, Dv, qs + (size_t)t * Dk, ks_ + (size_t)t * Dk, vs + (size_t)t * Dv,
                             las ? las + (gate == DRO_GATE_CHANNEL ? (size_t)t * Dk : (size_t)t) : NULL, gate,
                             bs + (beta_mode == DRO_BETA_CHANNEL ? (size_t)t * Dk : (size_t)t),
                             bvs + (beta_mode == DRO_BETA_CHANNEL ? (size_t)t * Dk : (size_t)t), beta_mode,
                             kss ? kss + (size_t)t * Dk : NULL, flags, St + (size_t)(t + 1) * sz,
                             tmp_o + (size_t)t * Dv, ktmp, vtmp, ptmp);
            }
        }
        /* reverse */
        if (dS_final) memcpy(G, dS_final + (size_t)s * sz, sizeof(double) * sz);
        else memset(G, 0, sizeof(double) * sz);
        for (int t = L - 1; t >= 0; --t) {
            const double* qt = qs + (size_t)t * Dk;
            const double* k_t = ks_ + (size_t)t * Dk;
            const double* v_t = vs + (size_t)t * Dv;
            const double* dot = dO + ((size_t)s * L + t) * Dv;
            const double* Sprev = St + (size_t)t * sz;
            const double* Snew = St + (size_t)(t + 1) * sz;
            const double* st_ = kss ? kss + (size_t)t * Dk : NULL;
            /* the prepared query and key, the strengths, kt, w and alpha */
            const double rq = l2 ? inv_l2(qt, Dk) : 1.0;   /* 1 / |q_t| */
            const double rk = l2 ? inv_l2(k_t, Dk) : 1.0;   /* 1 / |k_t| */
            for (int c = 0; c < Dk; ++c) {
                qh[c] = rq * qt[c];
                kh[c] = rk * k_t[c];
                bkv[c] = strength(beta_mode == DRO_BETA_SCALAR ? bs[t] : bs[(size_t)t * Dk + c], logit);
                sbk[c] = sqrt(bkv[c]);
                kt[c] = sbk[c] * kh[c];
                w[c] = st_ ? st_[c] * kt[c] : kt[c];
                al[c] = gate == DRO_GATE_NONE ? 1.0
                      : gate == DRO_GATE_SCALAR ? exp(las[t]) : exp(las[(size_t)t * Dk + c]);
            }
            for (int j = 0; j < Dv; ++j) {
                bvv[j] = strength(beta_mode == DRO_BETA_SCALAR ? bvs[t] : bvs[(size_t)t * Dk + j], logit);
                sbv[j] = sqrt(bvv[j]);
                vt[j] = sbv[j] * v_t[j];
            }
            /* S' and u = vt - S'^T kt */
            for (int c = 0; c < Dk; ++c)
                for (int j = 0; j < Dv; ++j) Sp[(size_t)c * Dv + j] = al[c] * Sprev[(size_t)c * Dv + j];
            for (int j = 0; j < Dv; ++j) {
                double pj = 0.0;
                for (int c = 0; c < Dk; ++c) pj += Sp[(size_t)c * Dv + j] * kt[c];
                u[j] = vt[j] - pj;
            }
            /* the output: G += qh do^T, dqh = S_t do */
            for (int c = 0; c < Dk; ++c) {
                double a = 0.0;
                for (int j = 0; j < Dv; ++j) {
                    G[(size_t)c * Dv + j] += qh[c] * dot[j];
                    a += Snew[(size_t)c * Dv + j] * dot[j];
                }
                dqh[c] = a;
            }
            /* du = G^T w (= dvt);  dw = G u;  dkt = s (.) dw - S' du;  ds = kt (.) dw */
            for (int j = 0; j < Dv; ++j) {
                double a = 0.0;
                for (int c = 0; c < Dk; ++c) a += G[(size_t)c * Dv + j] * w[c];
                dvt[j] = a;
            }
            for (int c = 0; c < Dk; ++c) {
                double a = 0.0, b = 0.0;
                for (int j = 0; j < Dv; ++j) {
                    a += G[(size_t)c * Dv + j] * u[j];
                    b += Sp[(size_t)c * Dv + j] * dvt[j];
                }
                dw[c] = a;
                dkt[c] = (st_ ? st_[c] : 1.0) * a - b;
                if (st_) dkey_scale[((size_t)s * L + t) * Dk + c] = kt[c] * a;
            }
            /* dS' = G - kt du^T;  dalpha;  G <- Diag(alpha) dS' */
            double dla_s = 0.0;
            for (int c = 0; c < Dk; ++c) {
                double da = 0.0;
                for (int j = 0; j < Dv; ++j) {
                    const double g = G[(size_t)c * Dv + j] - kt[c] * dvt[j];
                    da += g * Sprev[(size_t)c * Dv + j];
                    G[(size_t)c * Dv + j] = al[c] * g;
                }
                /* d/dlog alpha = alpha d/dalpha */
                if (gate == DRO_GATE_CHANNEL) dlog_alpha[((size_t)s * L + t) * Dk + c] = al[c] * da;
                dla_s += al[c] * da;
            }
            if (gate == DRO_GATE_SCALAR) dlog_alpha[(size_t)s * L + t] = dla_s;
            /* through kt = sqrt(beta) kh and vt = sqrt(beta) v; a logit adds
               beta (1 - beta) */
            double db_s = 0.0;
            for (int c = 0; c < Dk; ++c) {
                dkh[c] = sbk[c] * dkt[c];
                double g = dkt[c] * kh[c] / (2.0 * sbk[c]);
                if (logit) g *= bkv[c] * (1.0 - bkv[c]);
                if (beta_mode == DRO_BETA_CHANNEL) dbeta[((size_t)s * L + t) * Dk + c] = g;
                db_s += g;
            }
            /* the value's part goes to the write strength when it is separate */
            double* dbv = dbeta_v ? dbeta_v : dbeta;
            double dbv_s = 0.0;
            for (int j = 0; j < Dv; ++j) {
                dv[((size_t)s * L + t) * Dv + j] = sbv[j] * dvt[j];
                double g = dvt[j] * v_t[j] / (2.0 * sbv[j]);
                if (logit) g *= bvv[j] * (1.0 - bvv[j]);
                if (beta_mode == DRO_BETA_CHANNEL) {
                    if (dbeta_v) dbv[((size_t)s * L + t) * Dk + j] = g;
                    else dbv[((size_t)s * L + t) * Dk + j] += g;
                }
                dbv_s += g;
            }
            if (beta_mode == DRO_BETA_SCALAR) {
                if (dbeta_v) {
                    dbeta[(size_t)s * L + t] = db_s;
                    dbeta_v[(size_t)s * L + t] = dbv_s;
                } else {
                    dbeta[(size_t)s * L + t] = db_s + dbv_s;
                }
            }
            /* through the normalisation: dx = (dxh - xh (xh . dxh)) / |x| */
            double pq = 0.0, pk = 0.0;
            for (int c = 0; c < Dk; ++c) {
                pq += qh[c] * dqh[c];
                pk += kh[c] * dkh[c];
            }
            for (int c = 0; c < Dk; ++c) {
                dq[((size_t)s * L + t) * Dk + c] = l2 ? rq * (dqh[c] - qh[c] * pq) : dqh[c];
                dk[((size_t)s * L + t) * Dk + c] = l2 ? rk * (dkh[c] - kh[c] * pk) : dkh[c];
            }
        }
        if (dS0) memcpy(dS0 + (size_t)s * sz, G, sizeof(double) * sz);
        free(tmp_o);
        free(St);
    }
    (void)nthreads;
    return err;
}

int dro_backward(int B, int H, int L, int Dk, int Dv,
                 const double* q, const double* k, const double* v,
                 const double* log_alpha, int gate, const double* beta, int beta_mode,
                 const double* S0, const double* dO, const double* dS_final,
                 double* dq, double* dk, double* dv, double* dlog_alpha, double* dbeta, double* dS0,
                 int nthreads)
{
    return backward_impl(B, H, L, Dk, Dv, q, k, v, log_alpha, gate, beta, NULL, beta_mode, NULL, 0, S0, dO,
                         dS_final, dq, dk, dv, dlog_alpha, dbeta, NULL, NULL, dS0, nthreads);
}

int dro_backward_kv(int B, int H, int L, int Dk, int Dv,
                    const double* q, const double* k, const double* v,
                    const double* log_alpha, int gate, const double* beta, const double* beta_v, int beta_mode,
                    const double* S0, const double* dO, const double* dS_final,
                    double* dq, double* dk, double* dv, double* dlog_alpha, double* dbeta, double* dbeta_v,
                    double* dS0, int nthreads)
{
    if (!beta_v || !dbeta_v) return DRO_EINVAL;
    return backward_impl(B, H, L, Dk, Dv, q, k, v, log_alpha, gate, beta, beta_v, beta_mode, NULL, 0, S0, dO,
                         dS_final, dq, dk, dv, dlog_alpha, dbeta, dbeta_v, NULL, dS0, nthreads);
}

int dro_backward_ex(int B, int H, int L, int Dk, int Dv,
                    const double* q, const double* k, const double* v,
                    const double* log_alpha, int gate, const double* beta, const double* beta_v, int beta_mode,
                    const double* key_scale, int input_flags, const double* S0, const double* dO,
                    const double* dS_final, double* dq, double* dk, double* dv, double* dlog_alpha,
                    double* dbeta, double* dbeta_v, double* dkey_scale, double* dS0, int nthreads)
{
    if ((beta_v == NULL) != (dbeta_v == NULL)) return DRO_EINVAL;
    return backward_impl(B, H, L, Dk, Dv, q, k, v, log_alpha, gate, beta, beta_v, beta_mode, key_scale,
                         input_flags, S0, dO, dS_final, dq, dk, dv, dlog_alpha, dbeta, dbeta_v, dkey_scale, dS0,
                         nthreads);
}

/* Threads the OpenMP runtime would use by default (1 without OpenMP). */
int dro_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
