// dr_abi.hip -- host side of the C ABI declared in include/deltarule.h:
// argument validation, workspace layout, dispatch to the kernel launchers and
// the per-thread error text.  Nothing here allocates device memory.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <limits>
#include <mutex>
#include <vector>

#include "deltarule.h"
#include "dr_internal.h"

namespace {

thread_local char g_err[512] = "";

dr_status fail(dr_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dr_status fail(dr_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_dtype(int x) { return x == DR_F32 || x == DR_BF16; }
bool valid_gate(int x) { return x == DR_GATE_NONE || x == DR_GATE_SCALAR || x == DR_GATE_CHANNEL; }
bool valid_beta(int x) { return x == DR_BETA_SCALAR || x == DR_BETA_CHANNEL; }

// Shared shape/mode checks.  `nseq` sequences (or states) of Dk x Dv.
dr_status check_modes(int Dk, int Dv, int in_dtype, int out_dtype, int gate, int beta, unsigned flags) {
    if (flags & ~(unsigned)(DR_IN_QK_L2NORM | DR_IN_BETA_LOGIT))
        return fail(DR_ERR_UNSUPPORTED, "unknown input_flags bits 0x%x", flags);
    if (Dk != 64 && Dk != 128) return fail(DR_ERR_UNSUPPORTED, "Dk=%d: supported Dk are 64 and 128", Dk);
    if (Dv < 16 || Dv > 256 || Dv % 16 != 0)
        return fail(DR_ERR_UNSUPPORTED, "Dv=%d: Dv must be a multiple of 16 in [16, 256]", Dv);
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
        return fail(DR_ERR_UNSUPPORTED, "unknown dtype (in %d, out %d)", in_dtype, out_dtype);
    if (!valid_gate(gate)) return fail(DR_ERR_UNSUPPORTED, "unknown gate mode %d", gate);
    if (!valid_beta(beta)) return fail(DR_ERR_UNSUPPORTED, "unknown beta mode %d", beta);
    if (beta == DR_BETA_CHANNEL && Dv != Dk)
        return fail(DR_ERR_UNSUPPORTED, "channel-wise beta scales v by beta's channels: needs Dv == Dk (%d != %d)", Dv, Dk);
    return DR_OK;
}

// Workspace regions, each 256-byte aligned, for a validated descriptor.
struct WsLayout {
    size_t T, Pm, G, Q, Ks, Kl, V, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// precond: write-side key scales, which run on the channel-gate path
WsLayout ws_layout(const dr_chunk_desc& d, bool precond = false) {
    WsLayout w{};
    const size_t P = d.in_dtype == DR_F32 ? 2 : 1;
    const size_t NC = ((size_t)d.L + dr::CH - 1) / dr::CH;
    const size_t NCH = (size_t)d.B * d.H * NC;
    const bool cg = d.gate == DR_GATE_CHANNEL || precond, cb = d.beta == DR_BETA_CHANNEL;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    const size_t opnd = NCH * P * dr::CH * d.Dk * sizeof(dr::half_t);
    w.T = take(NCH * P * dr::CH * dr::CH * sizeof(dr::half_t));
    w.Pm = take(NCH * P * dr::CH * dr::CH * sizeof(dr::half_t));
    w.G = take(NCH * dr::kGW * sizeof(float));
    w.Q = (cg || cb) ? take(opnd) : 0;
    w.Ks = (cg || cb) ? take(opnd) : 0;
    w.Kl = cg ? take(opnd) : 0;
    w.V = cb ? take(opnd) : 0;
    w.total = NCH ? off : 0;
    return w;
}

dr_status check_chunk_desc(const dr_chunk_desc* d) {
    if (!d) return fail(DR_ERR_NULL, "descriptor is NULL");
    if (d->B < 0 || d->H < 0 || d->L < 0)
        return fail(DR_ERR_SHAPE, "negative dimension (B=%d H=%d L=%d)", d->B, d->H, d->L);
    dr_status s = check_modes(d->Dk, d->Dv, d->in_dtype, d->out_dtype, d->gate, d->beta, d->input_flags);
    if (s != DR_OK) return s;
    if (d->B > 65535 || d->H > 65535)
        return fail(DR_ERR_UNSUPPORTED, "B and H are limited to 65535 (grid dimensions)");
    const size_t nseq = (size_t)d->B * d->H;
    if (nseq > (size_t)std::numeric_limits<int>::max() / 256)
        return fail(DR_ERR_UNSUPPORTED, "B*H=%zu too large", nseq);
    return DR_OK;
}

__global__ void copy_state_kernel(float* dst, const float* src, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}


// ---------------------------------------------------------------- profiling
struct ProfRec {
    hipEvent_t ev;
    int slot;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRec> g_prof;
hipError_t g_prof_err = hipSuccess;

void prof_clear() {
    for (auto& r : g_prof) hipEventDestroy(r.ev);
    g_prof.clear();
}

}  // namespace

namespace dr {
void prof_mark(hipStream_t st, int slot) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipEvent_t ev;
    hipError_t e = hipEventCreate(&ev);
    if (e == hipSuccess) e = hipEventRecord(ev, st);
    if (e != hipSuccess) {
        if (g_prof_err == hipSuccess) g_prof_err = e;
        return;
    }
    g_prof.push_back({ev, slot});
}
}  // namespace dr

extern "C" {

dr_status dr_profile_begin(void) {
    g_err[0] = '\0';
    std::lock_guard<std::mutex> lk(g_prof_mu);
    prof_clear();
    g_prof_err = hipSuccess;
    g_prof_on.store(true);
    return DR_OK;
}

dr_status dr_profile_end(dr_profile_report* report) {
    g_err[0] = '\0';
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on.store(false);
    if (!report) {
        prof_clear();
        return fail(DR_ERR_NULL, "report is NULL");
    }
    *report = dr_profile_report{};
    hipError_t e = g_prof_err;
    double ms[dr::kProfSlots] = {};
    for (size_t i = 0; e == hipSuccess && i < g_prof.size(); ++i) {
        const int slot = g_prof[i].slot;
        if (slot == dr::kProfPrep) ++report->chunk_calls;
        if (slot == dr::kProfDecode) ++report->decode_calls;
        if (slot == dr::kProfBwdPrep) ++report->bwd_calls;
        if (slot == dr::kProfEnd || i + 1 == g_prof.size()) continue;
        e = hipEventSynchronize(g_prof[i + 1].ev);
        float t = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, g_prof[i].ev, g_prof[i + 1].ev);
        if (e == hipSuccess) ms[slot] += t;
    }
    prof_clear();
    if (e != hipSuccess) return fail(DR_ERR_HIP, "profiling events: %s", hipGetErrorString(e));
    report->prep_ms = ms[dr::kProfPrep];
    report->scan_ms = ms[dr::kProfScan];
    report->decode_ms = ms[dr::kProfDecode];
    report->bwd_prep_ms = ms[dr::kProfBwdPrep];
    report->bwd_fscan_ms = ms[dr::kProfBwdFscan];
    report->bwd_rscan_ms = ms[dr::kProfBwdRscan];
    report->bwd_post_ms = ms[dr::kProfBwdPost];
    return DR_OK;
}

int dr_abi_version(void) { return DR_ABI_VERSION; }

const char* dr_last_error(void) { return g_err; }

const char* dr_status_str(dr_status s) {
    switch (s) {
        case DR_OK: return "DR_OK";
        case DR_ERR_NULL: return "DR_ERR_NULL: required pointer missing";
        case DR_ERR_SHAPE: return "DR_ERR_SHAPE: invalid dimension";
        case DR_ERR_UNSUPPORTED: return "DR_ERR_UNSUPPORTED: unsupported size, mode or dtype";
        case DR_ERR_ALIGN: return "DR_ERR_ALIGN: pointer not 16-byte aligned";
        case DR_ERR_WORKSPACE: return "DR_ERR_WORKSPACE: workspace missing or too small";
        case DR_ERR_HIP: return "DR_ERR_HIP: HIP runtime or launch failure";
    }
    return "unknown dr_status";
}

size_t dr_chunk_fwd_workspace_bytes(const dr_chunk_desc* d) {
    if (check_chunk_desc(d) != DR_OK) return 0;
    return ws_layout(*d).total;
}

}  // extern "C"

namespace {

// The chunked forward; beta_v is the write strength on v (beta itself for
// dr_chunk_fwd, a separate channel-wise array for dr_chunk_fwd_kv).
dr_status chunk_fwd(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                    const float* log_alpha, const float* beta, const float* beta_v, const float* key_scale,
                    bool precond, const float* S0, void* o, float* S_final, void* workspace,
                    size_t workspace_bytes, void* stream) {
    dr_status s = check_chunk_desc(d);
    if (s != DR_OK) return s;
    const size_t nseq = (size_t)d->B * d->H;
    const bool tokens = nseq > 0 && d->L > 0;
    if (tokens) {
        if (!q || !k || !v || !beta || !beta_v || !o)
            return fail(DR_ERR_NULL, "q, k, v, beta (beta_k and beta_v) and o are required");
        if (precond && !key_scale) return fail(DR_ERR_NULL, "key_scale is required");
        if ((d->gate == DR_GATE_NONE) != (log_alpha == nullptr))
            return fail(DR_ERR_NULL, "log_alpha must be NULL exactly when gate is DR_GATE_NONE");
    }
    const void* ptrs[] = {q, k, v, log_alpha, beta, beta_v, key_scale, S0, o, S_final, workspace};
    const char* names[] = {"q", "k", "v", "log_alpha", "beta", "beta_v", "key_scale", "S0", "o", "S_final",
                           "workspace"};
    for (int i = 0; i < 11; ++i)
        if (ptrs[i] && !aligned16(ptrs[i])) return fail(DR_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    if (S_final && S0 && S_final != S0) {
        const size_t bytes = nseq * d->Dk * d->Dv * sizeof(float);
        const char* a0 = (const char*)S0;
        const char* a1 = (const char*)S_final;
        if (a0 < a1 + bytes && a1 < a0 + bytes)
            return fail(DR_ERR_UNSUPPORTED, "S_final overlaps S0 without being the same array");
    }
    const WsLayout w = ws_layout(*d, precond);
    if (w.total) {
        if (!workspace) return fail(DR_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", w.total);
        if (workspace_bytes < w.total)
            return fail(DR_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, w.total);
    }
    hipStream_t st = (hipStream_t)stream;
    if (nseq == 0) return DR_OK;
    if (d->L == 0) {
        // no tokens: the final state is the initial state
        if (S_final && S_final != S0) {
            const size_t n = nseq * d->Dk * d->Dv;
            hipLaunchKernelGGL(copy_state_kernel, dim3(256), dim3(256), 0, st, S_final, S0, n);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return fail(DR_ERR_HIP, "state copy launch: %s", hipGetErrorString(e));
        }
        return DR_OK;
    }
    dr::ChunkArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.log_alpha = log_alpha; a.beta = beta; a.beta_v = beta_v; a.S0 = S0;
    a.o = o; a.S_final = S_final;
    a.B = d->B; a.H = d->H; a.L = d->L; a.Dv = d->Dv;
    a.NC = (d->L + dr::CH - 1) / dr::CH;
    a.nseq = (int)nseq;
    a.has_gate = d->gate != DR_GATE_NONE;
    a.out_bf16 = d->out_dtype == DR_BF16;
    a.qk_norm = (d->input_flags & DR_IN_QK_L2NORM) != 0;
    a.beta_logit = (d->input_flags & DR_IN_BETA_LOGIT) != 0;
    a.gate_mode = d->gate;
    a.key_scale = precond ? key_scale : nullptr;
    char* ws = (char*)workspace;
    a.wsT = (dr::half_t*)(ws + w.T);
    a.wsP = (dr::half_t*)(ws + w.Pm);
    a.wsG = (float*)(ws + w.G);
    a.wsQ = w.Q ? (dr::half_t*)(ws + w.Q) : nullptr;
    a.wsKs = w.Ks ? (dr::half_t*)(ws + w.Ks) : nullptr;
    a.wsKl = w.Kl ? (dr::half_t*)(ws + w.Kl) : nullptr;
    a.wsV = w.V ? (dr::half_t*)(ws + w.V) : nullptr;
    hipError_t e = dr::launch_chunk(a, d->Dk, d->in_dtype == DR_F32, d->gate == DR_GATE_CHANNEL || precond,
                                    d->beta == DR_BETA_CHANNEL, beta_v != beta, st);
    if (e != hipSuccess) return fail(DR_ERR_HIP, "chunk kernels launch: %s", hipGetErrorString(e));
    return DR_OK;
}

dr_status decode_step(const dr_decode_desc* d, const void* q, const void* k, const void* v,
                      const float* log_alpha, const float* beta, const float* beta_v,
                      const float* key_scale, bool precond, float* S, void* o, void* stream) {
    if (!d) return fail(DR_ERR_NULL, "descriptor is NULL");
    if (d->N < 0 || d->H < 0) return fail(DR_ERR_SHAPE, "negative dimension (N=%d H=%d)", d->N, d->H);
    dr_status s = check_modes(d->Dk, d->Dv, d->in_dtype, d->out_dtype, d->gate, d->beta, d->input_flags);
    if (s != DR_OK) return s;
    const size_t nst = (size_t)d->N * d->H;
    const size_t blocks = nst * ((d->Dv + 63) / 64);
    if (blocks > (size_t)std::numeric_limits<int>::max())
        return fail(DR_ERR_UNSUPPORTED, "N*H=%zu too large", nst);
    if (nst == 0) return DR_OK;
    if (!q || !k || !v || !beta || !beta_v || !S || !o)
        return fail(DR_ERR_NULL, "q, k, v, beta (beta_k and beta_v), S and o are required");
    if (precond && !key_scale) return fail(DR_ERR_NULL, "key_scale is required");
    if ((d->gate == DR_GATE_NONE) != (log_alpha == nullptr))
        return fail(DR_ERR_NULL, "log_alpha must be NULL exactly when gate is DR_GATE_NONE");
    const void* ptrs[] = {q, k, v, log_alpha, beta, beta_v, key_scale, S, o};
    const char* names[] = {"q", "k", "v", "log_alpha", "beta", "beta_v", "key_scale", "S", "o"};
    for (int i = 0; i < 9; ++i)
        if (ptrs[i] && !aligned16(ptrs[i])) return fail(DR_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    dr::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.log_alpha = log_alpha; a.beta = beta; a.beta_v = beta_v;
    a.S = S; a.o = o;
    a.N = d->N; a.H = d->H; a.Dv = d->Dv;
    a.has_gate = d->gate != DR_GATE_NONE;
    a.out_bf16 = d->out_dtype == DR_BF16;
    a.qk_norm = (d->input_flags & DR_IN_QK_L2NORM) != 0;
    a.beta_logit = (d->input_flags & DR_IN_BETA_LOGIT) != 0;
    a.key_scale = precond ? key_scale : nullptr;
    hipError_t e = dr::launch_decode(a, d->Dk, d->in_dtype == DR_F32, d->gate == DR_GATE_CHANNEL,
                                     d->beta == DR_BETA_CHANNEL, (hipStream_t)stream);
    if (e != hipSuccess) return fail(DR_ERR_HIP, "decode kernel launch: %s", hipGetErrorString(e));
    return DR_OK;
}

// ----------------------------------------------------------------- backward
struct BwdLayout {
    size_t T, Pm, A, G, S, H, U, R, dU, Qh, Kh, Kc, Kt, q32, k32, v32, ones, db1, total;
};

BwdLayout bwd_layout(const dr_chunk_desc& d) {
    BwdLayout w{};
    const size_t NC = ((size_t)d.L + dr::CH - 1) / dr::CH;
    const size_t NCH = (size_t)d.B * d.H * NC;
    const size_t f = sizeof(float);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    w.T = take(NCH * dr::CH * dr::CH * f);
    w.Pm = take(NCH * dr::CH * dr::CH * f);
    w.A = take(NCH * dr::CH * dr::CH * f);
    const bool cg = d.gate == DR_GATE_CHANNEL;
    w.G = take(NCH * dr::CH * (cg ? d.Dk : 1) * f);
    w.S = take(NCH * d.Dk * d.Dv * f);
    w.H = take(NCH * d.Dk * d.Dv * f);
    w.U = take(NCH * dr::CH * d.Dv * f);
    w.R = take(NCH * dr::CH * d.Dv * f);
    w.dU = take(NCH * dr::CH * d.Dv * f);
    if (cg) {
        w.Qh = take(NCH * dr::CH * d.Dk * f);
        w.Kh = take(NCH * dr::CH * d.Dk * f);
        w.Kc = take(NCH * dr::CH * d.Dk * f);
        w.Kt = take(NCH * dr::CH * d.Dk * f);
    }
    if (d.beta == DR_BETA_CHANNEL) {
        // q, sqrt(beta) k, sqrt(beta) v in fp32, unit strengths and their (unused) gradient
        const size_t ntok = (size_t)d.B * d.H * d.L;
        w.q32 = take(ntok * d.Dk * f);
        w.k32 = take(ntok * d.Dk * f);
        w.v32 = take(ntok * d.Dv * f);
        w.ones = take(ntok * f);
        w.db1 = take(ntok * f);
    }
    w.total = NCH ? off : 0;
    return w;
}

dr_status check_bwd_desc(const dr_chunk_desc* d) {
    dr_status s = check_chunk_desc(d);
    if (s != DR_OK) return s;
    if (d->input_flags) return fail(DR_ERR_UNSUPPORTED, "the backward takes no input_flags");
    if (d->out_dtype != DR_F32) return fail(DR_ERR_UNSUPPORTED, "dO and the gradients are fp32: out_dtype must be DR_F32");
    const size_t NCH = (size_t)d->B * d->H * (((size_t)d->L + dr::CH - 1) / dr::CH);
    if (NCH > (size_t)std::numeric_limits<int>::max())
        return fail(DR_ERR_UNSUPPORTED, "B*H*ceil(L/64)=%zu chunks: too many", NCH);
    return DR_OK;
}

// beta_v and dbeta_v: the separate write strength and its gradient (channel
// beta only), or NULL for one strength
dr_status chunk_bwd(const dr_chunk_desc* d, const void* q, const void* k, const void* v, const float* log_alpha,
                    const float* beta, const float* beta_v, const float* S0, const float* dO,
                    const float* dS_final, float* dq, float* dk, float* dv, float* dlog_alpha, float* dbeta,
                    float* dbeta_v, float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
    dr_status s = check_bwd_desc(d);
    if (s != DR_OK) return s;
    const size_t nseq = (size_t)d->B * d->H;
    const bool tokens = nseq > 0 && d->L > 0;
    if (tokens) {
        if (!q || !k || !v || !beta || !dO || !dq || !dk || !dv || !dbeta)
            return fail(DR_ERR_NULL, "q, k, v, beta, dO, dq, dk, dv and dbeta are required");
        if ((beta_v == nullptr) != (dbeta_v == nullptr))
            return fail(DR_ERR_NULL, "beta_v and dbeta_v are required together");
        if ((d->gate == DR_GATE_NONE) != (log_alpha == nullptr))
            return fail(DR_ERR_NULL, "log_alpha must be NULL exactly when gate is DR_GATE_NONE");
        if ((d->gate == DR_GATE_NONE) != (dlog_alpha == nullptr))
            return fail(DR_ERR_NULL, "dlog_alpha must be NULL exactly when gate is DR_GATE_NONE");
    }
    const void* ptrs[] = {q, k, v, log_alpha, beta, beta_v, S0, dO, dS_final, dq, dk, dv, dlog_alpha, dbeta,
                          dbeta_v, dS0, workspace};
    const char* names[] = {"q", "k", "v", "log_alpha", "beta", "beta_v", "S0", "dO", "dS_final", "dq", "dk", "dv",
                           "dlog_alpha", "dbeta", "dbeta_v", "dS0", "workspace"};
    for (int i = 0; i < 17; ++i)
        if (ptrs[i] && !aligned16(ptrs[i])) return fail(DR_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    const BwdLayout w = bwd_layout(*d);
    if (w.total) {
        if (!workspace) return fail(DR_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", w.total);
        if (workspace_bytes < w.total)
            return fail(DR_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, w.total);
    }
    hipStream_t st = (hipStream_t)stream;
    if (nseq == 0) return DR_OK;
    if (d->L == 0) {
        // no tokens: S_final is S0, so dS0 is dS_final
        if (dS0) {
            const size_t n = nseq * d->Dk * d->Dv;
            hipLaunchKernelGGL(copy_state_kernel, dim3(256), dim3(256), 0, st, dS0, dS_final, n);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return fail(DR_ERR_HIP, "state copy launch: %s", hipGetErrorString(e));
        }
        return DR_OK;
    }
    dr::BwdArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.log_alpha = log_alpha; a.beta = beta; a.S0 = S0;
    a.dO = dO; a.dS_final = dS_final;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dlog_alpha = dlog_alpha; a.dbeta = dbeta; a.dS0 = dS0;
    a.B = d->B; a.H = d->H; a.L = d->L; a.Dv = d->Dv;
    a.NC = (d->L + dr::CH - 1) / dr::CH;
    a.nseq = (int)nseq;
    a.has_gate = d->gate != DR_GATE_NONE;
    char* ws = (char*)workspace;
    a.wT = (float*)(ws + w.T);
    a.wP = (float*)(ws + w.Pm);
    a.wA = (float*)(ws + w.A);
    a.wG = (float*)(ws + w.G);
    a.wS = (float*)(ws + w.S);
    a.wH = (float*)(ws + w.H);
    a.wU = (float*)(ws + w.U);
    a.wR = (float*)(ws + w.R);
    a.wdU = (float*)(ws + w.dU);
    a.cgate = d->gate == DR_GATE_CHANNEL;
    if (a.cgate) {
        a.wQh = (float*)(ws + w.Qh);
        a.wKh = (float*)(ws + w.Kh);
        a.wKc = (float*)(ws + w.Kc);
        a.wKt = (float*)(ws + w.Kt);
    }
    bool f32in = d->in_dtype == DR_F32;
    const bool cbeta = d->beta == DR_BETA_CHANNEL;
    const size_t ntok = nseq * d->L, nel = ntok * d->Dk;   // Dv == Dk with a channel beta
    hipError_t e = hipSuccess;
    if (cbeta) {
        // the scaled inputs with unit strengths; the beta gradient of that run is discarded
        float* q32 = (float*)(ws + w.q32);
        float* k32 = (float*)(ws + w.k32);
        float* v32 = (float*)(ws + w.v32);
        float* ones = (float*)(ws + w.ones);
        e = dr::launch_bwd_cbeta_in(q, k, v, beta, beta_v ? beta_v : beta, f32in, nel, ntok, q32, k32, v32, ones,
                                    st);
        if (e != hipSuccess) return fail(DR_ERR_HIP, "backward input scaling launch: %s", hipGetErrorString(e));
        a.q = q32; a.k = k32; a.v = v32;
        a.beta = ones;
        a.dbeta = (float*)(ws + w.db1);
        f32in = true;
    }
    e = dr::launch_bwd(a, d->Dk, f32in, st);
    if (e != hipSuccess) return fail(DR_ERR_HIP, "backward kernels launch: %s", hipGetErrorString(e));
    if (cbeta) {
        e = dr::launch_bwd_cbeta_out(k, v, beta, beta_v ? beta_v : beta, d->in_dtype == DR_F32, nel, dk, dv, dbeta,
                                     dbeta_v, st);
        if (e != hipSuccess) return fail(DR_ERR_HIP, "backward gradient mapping launch: %s", hipGetErrorString(e));
    }
    return DR_OK;
}

// The separate-strength entry points take channel-wise strengths only.
dr_status check_kv_mode(int beta_mode) {
    if (beta_mode != DR_BETA_CHANNEL)
        return fail(DR_ERR_UNSUPPORTED, "separate erase and write strengths are channel-wise: "
                                        "beta mode must be DR_BETA_CHANNEL");
    return DR_OK;
}

}  // namespace

extern "C" {

dr_status dr_chunk_fwd(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* beta, const float* S0, void* o,
                       float* S_final, void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    return chunk_fwd(d, q, k, v, log_alpha, beta, beta, nullptr, false, S0, o, S_final, workspace,
                     workspace_bytes, stream);
}

dr_status dr_chunk_fwd_kv(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                          const float* log_alpha, const float* beta_k, const float* beta_v,
                          const float* S0, void* o, float* S_final, void* workspace,
                          size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    if (d && check_kv_mode(d->beta) != DR_OK) return DR_ERR_UNSUPPORTED;
    return chunk_fwd(d, q, k, v, log_alpha, beta_k, beta_v, nullptr, false, S0, o, S_final, workspace,
                     workspace_bytes, stream);
}

size_t dr_chunk_fwd_precond_workspace_bytes(const dr_chunk_desc* d) {
    if (check_chunk_desc(d) != DR_OK) return 0;
    return ws_layout(*d, true).total;
}

dr_status dr_chunk_fwd_precond(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const float* key_scale,
                               const float* S0, void* o, float* S_final, void* workspace,
                               size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    return chunk_fwd(d, q, k, v, log_alpha, beta, beta, key_scale, true, S0, o, S_final, workspace,
                     workspace_bytes, stream);
}

dr_status dr_decode_step(const dr_decode_desc* d, const void* q, const void* k, const void* v,
                         const float* log_alpha, const float* beta, float* S, void* o,
                         void* stream) {
    g_err[0] = '\0';
    return decode_step(d, q, k, v, log_alpha, beta, beta, nullptr, false, S, o, stream);
}

dr_status dr_decode_step_precond(const dr_decode_desc* d, const void* q, const void* k, const void* v,
                                 const float* log_alpha, const float* beta, const float* key_scale,
                                 float* S, void* o, void* stream) {
    g_err[0] = '\0';
    return decode_step(d, q, k, v, log_alpha, beta, beta, key_scale, true, S, o, stream);
}

dr_status dr_decode_step_kv(const dr_decode_desc* d, const void* q, const void* k, const void* v,
                            const float* log_alpha, const float* beta_k, const float* beta_v,
                            float* S, void* o, void* stream) {
    g_err[0] = '\0';
    if (d && check_kv_mode(d->beta) != DR_OK) return DR_ERR_UNSUPPORTED;
    return decode_step(d, q, k, v, log_alpha, beta_k, beta_v, nullptr, false, S, o, stream);
}

size_t dr_chunk_bwd_workspace_bytes(const dr_chunk_desc* d) {
    if (check_bwd_desc(d) != DR_OK) return 0;
    return bwd_layout(*d).total;
}

dr_status dr_chunk_bwd(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* beta, const float* S0, const float* dO,
                       const float* dS_final, float* dq, float* dk, float* dv, float* dlog_alpha,
                       float* dbeta, float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    return chunk_bwd(d, q, k, v, log_alpha, beta, nullptr, S0, dO, dS_final, dq, dk, dv, dlog_alpha, dbeta, nullptr,
                     dS0, workspace, workspace_bytes, stream);
}

dr_status dr_chunk_bwd_kv(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                          const float* log_alpha, const float* beta_k, const float* beta_v, const float* S0,
                          const float* dO, const float* dS_final, float* dq, float* dk, float* dv,
                          float* dlog_alpha, float* dbeta_k, float* dbeta_v, float* dS0, void* workspace,
                          size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    if (d && check_kv_mode(d->beta) != DR_OK) return DR_ERR_UNSUPPORTED;
    const size_t ntok = d ? (size_t)(d->B > 0 ? d->B : 0) * (d->H > 0 ? d->H : 0) * (d->L > 0 ? d->L : 0) : 0;
    if (ntok && (!beta_v || !dbeta_v)) return fail(DR_ERR_NULL, "beta_v and dbeta_v are required");
    return chunk_bwd(d, q, k, v, log_alpha, beta_k, beta_v, S0, dO, dS_final, dq, dk, dv, dlog_alpha, dbeta_k,
                     dbeta_v, dS0, workspace, workspace_bytes, stream);
}

}  // extern "C"
