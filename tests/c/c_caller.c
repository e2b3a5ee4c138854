/*
 * c_caller.c -- the library used from plain C through include/deltarule.h.
 *
 * TEST PROGRAM.  "cpu" mode needs no GPU: it checks the version, the status
 * text and host-side validation.  "gpu" mode runs a small chunked forward
 * (fp32 inputs, scalar gate and beta, a ragged last chunk), its backward, the
 * backward of the preconditioned rule with the input preparation, and one
 * decode step through the C ABI with device buffers from the HIP runtime, and
 * compares them with the fp64 oracle (oracle/libdr_oracle.so, test
 * infrastructure).
 * Exit status 0 on success.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "deltarule.h"

/* the oracle's entry point (oracle/dr_oracle.c) */
int dro_forward(int B, int H, int L, int Dk, int Dv, const double* q, const double* k, const double* v,
                const double* log_alpha, int gate, const double* beta, int beta_mode, const double* S0,
                double* o, double* S_final, int nthreads);
int dro_backward(int B, int H, int L, int Dk, int Dv, const double* q, const double* k, const double* v,
                 const double* log_alpha, int gate, const double* beta, int beta_mode, const double* S0,
                 const double* dO, const double* dS_final, double* dq, double* dk, double* dv, double* dlog_alpha,
                 double* dbeta, double* dS0, int nthreads);

int dro_backward_ex(int B, int H, int L, int Dk, int Dv, const double* q, const double* k, const double* v,
                    const double* log_alpha, int gate, const double* beta, const double* beta_v, int beta_mode,
                    const double* key_scale, int input_flags, const double* S0, const double* dO,
                    const double* dS_final, double* dq, double* dk, double* dv, double* dlog_alpha,
                    double* dbeta, double* dbeta_v, double* dkey_scale, double* dS0, int nthreads);

static int fails = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                 \
            fprintf(stderr, "\n");                        \
            ++fails;                                      \
        }                                                 \
    } while (0)

static int cpu_checks(void) {
    CHECK(dr_abi_version() == DR_ABI_VERSION, "abi %d != %d", dr_abi_version(), DR_ABI_VERSION);
    CHECK(strncmp(dr_status_str(DR_ERR_SHAPE), "DR_ERR_SHAPE", 12) == 0, "status text");
    dr_chunk_desc d = {2, 3, 100, 96, 128, DR_BF16, DR_F32, DR_GATE_SCALAR, DR_BETA_SCALAR, 0};
    CHECK(dr_chunk_fwd_workspace_bytes(&d) == 0, "workspace for an invalid descriptor");
    dr_status s = dr_chunk_fwd(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
    CHECK(s == DR_ERR_UNSUPPORTED, "Dk = 96 gives %d", (int)s);
    CHECK(strlen(dr_last_error()) > 0, "detail text");
    d.Dk = 128;
    CHECK(dr_chunk_fwd_workspace_bytes(&d) > 0, "workspace size");
    d.B = 0;
    s = dr_chunk_fwd(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
    CHECK(s == DR_OK, "empty batch gives %d", (int)s);
    return fails;
}

/* a small counter-based generator: uniform in [-1, 1) */
static double urand(unsigned long long* st) {
    *st = *st * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(*st >> 11) / 4503599627370496.0 - 1.0;
}

static double max_rel(const float* x, const double* y, size_t n) {
    double e = 0.0, m = 0.0;
    for (size_t i = 0; i < n; ++i) {
        e = fmax(e, fabs((double)x[i] - y[i]));
        m = fmax(m, fabs(y[i]));
    }
    return m > 0.0 ? e / m : e;
}

#define HIPOK(x)                                                            \
    do {                                                                    \
        hipError_t e_ = (x);                                                \
        if (e_ != hipSuccess) {                                             \
            fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            exit(2);                                                        \
        }                                                                   \
    } while (0)

static int gpu_checks(void) {
    const int B = 1, H = 3, L = 150, D = 64;
    const size_t nq = (size_t)B * H * L * D, ng = (size_t)B * H * L, ns = (size_t)B * H * D * D;
    unsigned long long st = 12345;
    float *q = malloc(nq * 4), *k = malloc(nq * 4), *v = malloc(nq * 4), *la = malloc(ng * 4),
          *be = malloc(ng * 4), *S0 = malloc(ns * 4), *o = malloc(nq * 4), *Sf = malloc(ns * 4);
    double *qd = malloc(nq * 8), *kd = malloc(nq * 8), *vd = malloc(nq * 8), *lad = malloc(ng * 8),
           *bed = malloc(ng * 8), *S0d = malloc(ns * 8), *od = malloc(nq * 8), *Sfd = malloc(ns * 8);
    for (size_t t = 0; t < (size_t)B * H * L; ++t) {
        double nqv = 0.0, nkv = 0.0;
        for (int c = 0; c < D; ++c) {
            q[t * D + c] = (float)urand(&st);
            k[t * D + c] = (float)urand(&st);
            v[t * D + c] = (float)urand(&st);
            nqv += (double)q[t * D + c] * q[t * D + c];
            nkv += (double)k[t * D + c] * k[t * D + c];
        }
        for (int c = 0; c < D; ++c) {   /* unit keys and queries, as the layer in front would give */
            q[t * D + c] = (float)(q[t * D + c] / sqrt(nqv));
            k[t * D + c] = (float)(k[t * D + c] / sqrt(nkv));
        }
        la[t] = (float)(-0.05 + 0.049 * urand(&st));
        be[t] = (float)(0.5 + 0.45 * urand(&st));
    }
    for (size_t i = 0; i < ns; ++i) S0[i] = (float)(0.1 * urand(&st));
    for (size_t i = 0; i < nq; ++i) { qd[i] = q[i]; kd[i] = k[i]; vd[i] = v[i]; }
    for (size_t i = 0; i < ng; ++i) { lad[i] = la[i]; bed[i] = be[i]; }
    for (size_t i = 0; i < ns; ++i) S0d[i] = S0[i];

    dr_chunk_desc d = {B, H, L, D, D, DR_F32, DR_F32, DR_GATE_SCALAR, DR_BETA_SCALAR, 0};
    const size_t wsb = dr_chunk_fwd_workspace_bytes(&d);
    void *dq, *dk, *dv, *dla, *dbe, *dS, *dO, *dws;
    HIPOK(hipMalloc(&dq, nq * 4)); HIPOK(hipMalloc(&dk, nq * 4)); HIPOK(hipMalloc(&dv, nq * 4));
    HIPOK(hipMalloc(&dla, ng * 4)); HIPOK(hipMalloc(&dbe, ng * 4)); HIPOK(hipMalloc(&dS, ns * 4));
    HIPOK(hipMalloc(&dO, nq * 4)); HIPOK(hipMalloc(&dws, wsb));
    HIPOK(hipMemcpy(dq, q, nq * 4, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dk, k, nq * 4, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dv, v, nq * 4, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dla, la, ng * 4, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dbe, be, ng * 4, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dS, S0, ns * 4, hipMemcpyHostToDevice));
    /* in-place state carry: S_final aliases S0 */
    dr_status s = dr_chunk_fwd(&d, dq, dk, dv, dla, dbe, dS, dO, dS, dws, wsb, NULL);
    CHECK(s == DR_OK, "dr_chunk_fwd: %s (%s)", dr_status_str(s), dr_last_error());
    HIPOK(hipDeviceSynchronize());
    HIPOK(hipMemcpy(o, dO, nq * 4, hipMemcpyDeviceToHost));
    HIPOK(hipMemcpy(Sf, dS, ns * 4, hipMemcpyDeviceToHost));
    CHECK(dro_forward(B, H, L, D, D, qd, kd, vd, lad, 1, bed, 0, S0d, od, Sfd, 1) == 0, "oracle");
    const double eo = max_rel(o, od, nq), es = max_rel(Sf, Sfd, ns);
    printf("chunk forward: o %.2e  S %.2e\n", eo, es);
    CHECK(eo <= 1e-4 && es <= 1e-4, "forward parity o %.2e S %.2e", eo, es);

    /* the backward of the same forward, for seeded gradients of o and S_final */
    {
        float *gO = malloc(nq * 4), *gS = malloc(ns * 4);
        double *gOd = malloc(nq * 8), *gSd = malloc(ns * 8);
        for (size_t i = 0; i < nq; ++i) { gO[i] = (float)urand(&st); gOd[i] = gO[i]; }
        for (size_t i = 0; i < ns; ++i) { gS[i] = (float)urand(&st); gSd[i] = gS[i]; }
        const size_t wbb = dr_chunk_bwd_workspace_bytes(&d);
        CHECK(wbb > 0, "backward workspace size");
        void *dgO, *dgS, *dS0b, *gq, *gk, *gv, *gla, *gbe, *gS0, *dwb;
        HIPOK(hipMalloc(&dgO, nq * 4)); HIPOK(hipMalloc(&dgS, ns * 4)); HIPOK(hipMalloc(&dS0b, ns * 4));
        HIPOK(hipMalloc(&gq, nq * 4)); HIPOK(hipMalloc(&gk, nq * 4)); HIPOK(hipMalloc(&gv, nq * 4));
        HIPOK(hipMalloc(&gla, ng * 4)); HIPOK(hipMalloc(&gbe, ng * 4)); HIPOK(hipMalloc(&gS0, ns * 4));
        HIPOK(hipMalloc(&dwb, wbb));
        HIPOK(hipMemcpy(dgO, gO, nq * 4, hipMemcpyHostToDevice));
        HIPOK(hipMemcpy(dgS, gS, ns * 4, hipMemcpyHostToDevice));
        HIPOK(hipMemcpy(dS0b, S0, ns * 4, hipMemcpyHostToDevice));
        s = dr_chunk_bwd(&d, dq, dk, dv, dla, dbe, dS0b, dgO, dgS, gq, gk, gv, gla, gbe, gS0, dwb, wbb, NULL);
        CHECK(s == DR_OK, "dr_chunk_bwd: %s (%s)", dr_status_str(s), dr_last_error());
        HIPOK(hipDeviceSynchronize());
        float* hg[6];
        const size_t cnt[6] = {nq, nq, nq, ng, ng, ns};
        void* dev[6] = {gq, gk, gv, gla, gbe, gS0};
        double* ref[6];
        for (int i = 0; i < 6; ++i) {
            hg[i] = malloc(cnt[i] * 4);
            ref[i] = malloc(cnt[i] * 8);
            HIPOK(hipMemcpy(hg[i], dev[i], cnt[i] * 4, hipMemcpyDeviceToHost));
        }
        CHECK(dro_backward(B, H, L, D, D, qd, kd, vd, lad, 1, bed, 0, S0d, gOd, gSd, ref[0], ref[1], ref[2], ref[3],
                           ref[4], ref[5], 1) == 0, "oracle backward");
        double eb = 0.0;
        for (int i = 0; i < 6; ++i) {
            const double e = max_rel(hg[i], ref[i], cnt[i]);
            if (e > eb) eb = e;
        }
        printf("chunk backward: max over dq, dk, dv, dlog_alpha, dbeta, dS0 %.2e\n", eb);
        CHECK(eb <= 1e-4, "backward parity %.2e", eb);
        for (int i = 0; i < 6; ++i) { free(hg[i]); free(ref[i]); }

        /* the preconditioned rule with the input preparation: key scales in
           [0.5, 1.5), q and k normalised in the library, strengths as logits */
        {
            dr_chunk_desc dp = d;
            dp.input_flags = DR_IN_QK_L2NORM | DR_IN_BETA_LOGIT;
            float *ks = malloc(nq * 4), *lg = malloc(ng * 4);
            double *ksd = malloc(nq * 8), *lgd = malloc(ng * 8);
            for (size_t i = 0; i < nq; ++i) { ks[i] = (float)(1.0 + 0.5 * urand(&st)); ksd[i] = ks[i]; }
            for (size_t i = 0; i < ng; ++i) { lg[i] = (float)log(be[i] / (1.0 - be[i])); lgd[i] = lg[i]; }
            const size_t wpb = dr_chunk_bwd_precond_workspace_bytes(&dp);
            CHECK(wpb > 0, "precond backward workspace size");
            void *dks, *dlg, *gks, *dwp;
            HIPOK(hipMalloc(&dks, nq * 4)); HIPOK(hipMalloc(&dlg, ng * 4)); HIPOK(hipMalloc(&gks, nq * 4));
            HIPOK(hipMalloc(&dwp, wpb));
            HIPOK(hipMemcpy(dks, ks, nq * 4, hipMemcpyHostToDevice));
            HIPOK(hipMemcpy(dlg, lg, ng * 4, hipMemcpyHostToDevice));
            s = dr_chunk_bwd_precond(&dp, dq, dk, dv, dla, dlg, dks, dS0b, dgO, dgS, gq, gk, gv, gla, gbe, gks, gS0,
                                     dwp, wpb, NULL);
            CHECK(s == DR_OK, "dr_chunk_bwd_precond: %s (%s)", dr_status_str(s), dr_last_error());
            HIPOK(hipDeviceSynchronize());
            const size_t pc[7] = {nq, nq, nq, ng, ng, ns, nq};
            void* pdev[7] = {gq, gk, gv, gla, gbe, gS0, gks};
            float* ph[7];
            double* pref[7];
            for (int i = 0; i < 7; ++i) {
                ph[i] = malloc(pc[i] * 4);
                pref[i] = malloc(pc[i] * 8);
                HIPOK(hipMemcpy(ph[i], pdev[i], pc[i] * 4, hipMemcpyDeviceToHost));
            }
            CHECK(dro_backward_ex(B, H, L, D, D, qd, kd, vd, lad, 1, lgd, NULL, 0, ksd, 3, S0d, gOd, gSd, pref[0],
                                  pref[1], pref[2], pref[3], pref[4], NULL, pref[6], pref[5], 1) == 0,
                  "oracle backward_ex");
            double ep = 0.0;
            for (int i = 0; i < 7; ++i) {
                const double e = max_rel(ph[i], pref[i], pc[i]);
                if (e > ep) ep = e;
            }
            printf("preconditioned backward with input preparation: max over the gradients %.2e\n", ep);
            CHECK(ep <= 1e-4, "precond backward parity %.2e", ep);
            for (int i = 0; i < 7; ++i) { free(ph[i]); free(pref[i]); }
            HIPOK(hipFree(dks)); HIPOK(hipFree(dlg)); HIPOK(hipFree(gks)); HIPOK(hipFree(dwp));
            free(ks); free(lg); free(ksd); free(lgd);
        }
        HIPOK(hipFree(dgO)); HIPOK(hipFree(dgS)); HIPOK(hipFree(dS0b)); HIPOK(hipFree(gq)); HIPOK(hipFree(gk));
        HIPOK(hipFree(gv)); HIPOK(hipFree(gla)); HIPOK(hipFree(gbe)); HIPOK(hipFree(gS0)); HIPOK(hipFree(dwb));
        free(gO); free(gS); free(gOd); free(gSd);
    }

    /* one decode step on the final states with the first token's inputs */
    dr_decode_desc dd = {B, H, D, D, DR_F32, DR_F32, DR_GATE_SCALAR, DR_BETA_SCALAR, 0};
    float *q1 = malloc((size_t)H * D * 4), *k1 = malloc((size_t)H * D * 4), *v1 = malloc((size_t)H * D * 4);
    float la1[3], be1[3];
    double *q1d = malloc((size_t)H * D * 8), *k1d = malloc((size_t)H * D * 8), *v1d = malloc((size_t)H * D * 8);
    double la1d[3], be1d[3], *o1d = malloc((size_t)H * D * 8), *S1d = malloc(ns * 8);
    for (int h = 0; h < H; ++h) {
        for (int c = 0; c < D; ++c) {
            q1[h * D + c] = q[((size_t)h * L) * D + c];
            k1[h * D + c] = k[((size_t)h * L) * D + c];
            v1[h * D + c] = v[((size_t)h * L) * D + c];
            q1d[h * D + c] = q1[h * D + c]; k1d[h * D + c] = k1[h * D + c]; v1d[h * D + c] = v1[h * D + c];
        }
        la1[h] = la[(size_t)h * L]; be1[h] = be[(size_t)h * L]; la1d[h] = la1[h]; be1d[h] = be1[h];
    }
    void *dq1, *dk1, *dv1, *dla1, *dbe1, *dO1;
    HIPOK(hipMalloc(&dq1, (size_t)H * D * 4)); HIPOK(hipMalloc(&dk1, (size_t)H * D * 4));
    HIPOK(hipMalloc(&dv1, (size_t)H * D * 4)); HIPOK(hipMalloc(&dla1, 16)); HIPOK(hipMalloc(&dbe1, 16));
    HIPOK(hipMalloc(&dO1, (size_t)H * D * 4));
    HIPOK(hipMemcpy(dq1, q1, (size_t)H * D * 4, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dk1, k1, (size_t)H * D * 4, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dv1, v1, (size_t)H * D * 4, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dla1, la1, (size_t)H * 4, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dbe1, be1, (size_t)H * 4, hipMemcpyHostToDevice));
    s = dr_decode_step(&dd, dq1, dk1, dv1, dla1, dbe1, dS, dO1, NULL);
    CHECK(s == DR_OK, "dr_decode_step: %s (%s)", dr_status_str(s), dr_last_error());
    HIPOK(hipDeviceSynchronize());
    float* o1 = malloc((size_t)H * D * 4);
    HIPOK(hipMemcpy(o1, dO1, (size_t)H * D * 4, hipMemcpyDeviceToHost));
    HIPOK(hipMemcpy(Sf, dS, ns * 4, hipMemcpyDeviceToHost));
    CHECK(dro_forward(1, H, 1, D, D, q1d, k1d, v1d, la1d, 1, be1d, 0, Sfd, o1d, S1d, 1) == 0, "oracle decode");
    const double e1 = max_rel(o1, o1d, (size_t)H * D), eS = max_rel(Sf, S1d, ns);
    printf("decode step: o %.2e  S %.2e\n", e1, eS);
    CHECK(e1 <= 1e-4 && eS <= 1e-4, "decode parity o %.2e S %.2e", e1, eS);
    return fails;
}

int main(int argc, char** argv) {
    const int gpu = argc > 1 && strcmp(argv[1], "gpu") == 0;
    int f = gpu ? gpu_checks() : cpu_checks();
    printf("%s: %s\n", gpu ? "gpu" : "cpu", f ? "FAILED" : "ok");
    return f ? 1 : 0;
}
