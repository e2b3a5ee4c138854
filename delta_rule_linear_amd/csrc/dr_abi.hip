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

// The allocation-free forward's workspace: one array per GPU, from the
// library's first use on that GPU until the process ends.  In host code the
// name stands for a host-side shadow, not the device address: the device
// address comes from hipGetSymbolAddress, once per device (scratch_for_device).
static __device__ __align__(256) unsigned char scratch[DR_NOALLOC_SCRATCH_BYTES];

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

// A tensor argument as a byte range (p may be NULL: an absent tensor).
struct Span {
    const void* p;
    size_t bytes;
    const char* name;
};

bool overlap(const Span& a, const Span& b) {
    if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
    const char* x = (const char*)a.p;
    const char* y = (const char*)b.p;
    return x < y + b.bytes && y < x + a.bytes;
}

// Every output in `outs` must be disjoint from every input in `ins` and from
// the other outputs, except that output alias_out may be input alias_in
// exactly (the same address and size: the in-place state carry); any other
// overlap is an error.
dr_status check_disjoint(const Span* outs, int nout, const Span* ins, int nin, const void* alias_out = nullptr,
                         const void* alias_in = nullptr) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j) {
            if (!overlap(outs[i], ins[j])) continue;
            if (alias_out && outs[i].p == alias_out && ins[j].p == alias_in && outs[i].p == ins[j].p &&
                outs[i].bytes == ins[j].bytes)
                continue;
            return fail(DR_ERR_UNSUPPORTED, "%s overlaps %s", outs[i].name, ins[j].name);
        }
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j]))
                return fail(DR_ERR_UNSUPPORTED, "%s overlaps %s", outs[i].name, outs[j].name);
    }
    return DR_OK;
}

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

// precond: write-side key scales, which run on the channel-gate path;
// kvtok: separate scalar strengths, which run on the channel-beta path
WsLayout ws_layout(const dr_chunk_desc& d, bool precond = false, bool kvtok = false) {
    WsLayout w{};
    const size_t P = d.in_dtype == DR_F32 ? 2 : 1;
    const size_t NC = ((size_t)d.L + dr::CH - 1) / dr::CH;
    const size_t NCH = (size_t)d.B * d.H * NC;
    const bool cg = d.gate == DR_GATE_CHANNEL || precond, cb = d.beta == DR_BETA_CHANNEL || kvtok;
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

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call per device, with that device current).
dr_status scratch_for_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(DR_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(DR_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DR_OK;
}

__global__ void copy_state_kernel(float* dst, const float* src, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}


// ---------------------------------------------------------------- profiling
struct ProfRec {
    hipEvent_t start, stop;
    int slot;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRec> g_prof;
hipError_t g_prof_err = hipSuccess;
// Events are kept for reuse: none is created or destroyed while a profiling
// window is open once the pool holds enough (creating events allocates in
// the runtime, which would run beside the kernels being timed).
std::vector<hipEvent_t> g_pool;
constexpr size_t kPoolFill = 1024;

void prof_clear() {
    for (auto& r : g_prof) {
        g_pool.push_back(r.start);
        g_pool.push_back(r.stop);
    }
    g_prof.clear();
}

// tops the pool up to kPoolFill events (called with g_prof_mu held)
hipError_t pool_fill() {
    while (g_pool.size() < kPoolFill) {
        hipEvent_t e;
        const hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) return r;
        g_pool.push_back(e);
    }
    return hipSuccess;
}

}  // namespace

namespace dr {
bool prof_events(hipEvent_t* start, hipEvent_t* stop) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return false;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipError_t e = hipSuccess;
    if (g_pool.size() < 2) e = pool_fill();
    if (e != hipSuccess) {
        if (g_prof_err == hipSuccess) g_prof_err = e;
        *start = *stop = nullptr;
        return false;
    }
    *stop = g_pool.back();
    g_pool.pop_back();
    *start = g_pool.back();
    g_pool.pop_back();
    return true;
}

void prof_record(hipEvent_t start, hipEvent_t stop, int slot) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back({start, stop, slot});
}
}  // namespace dr

extern "C" {

dr_status dr_profile_begin(void) {
    g_err[0] = '\0';
    std::lock_guard<std::mutex> lk(g_prof_mu);
    prof_clear();
    g_prof_err = pool_fill();
    if (g_prof_err != hipSuccess) return fail(DR_ERR_HIP, "profiling events: %s", hipGetErrorString(g_prof_err));
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
        e = hipEventSynchronize(g_prof[i].stop);
        float t = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, g_prof[i].start, g_prof[i].stop);
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
// kvtok: separate strengths of one value per token (beta and beta_v [B][H][L]),
// run on the channel-beta kernels with every channel sharing its token's value
dr_status chunk_fwd(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                    const float* log_alpha, const float* beta, const float* beta_v, const float* key_scale,
                    bool precond, const float* S0, void* o, float* S_final, void* workspace,
                    size_t workspace_bytes, void* stream, bool kvtok = false) {
    dr_status s = check_chunk_desc(d);
    if (s != DR_OK) return s;
    if (kvtok && d->Dv != d->Dk)
        return fail(DR_ERR_UNSUPPORTED, "separate scalar strengths run on the channel-beta kernels: needs Dv == Dk "
                                        "(%d != %d)", d->Dv, d->Dk);
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
    const WsLayout w = ws_layout(*d, precond, kvtok);
    {
        // o and S_final are disjoint from every input, the workspace and each
        // other; S_final may be S0 itself (in-place state carry)
        const size_t ntok = nseq * (size_t)d->L;
        const size_t inb = d->in_dtype == DR_F32 ? 4 : 2, outb = d->out_dtype == DR_F32 ? 4 : 2;
        const size_t gw = d->gate == DR_GATE_CHANNEL ? d->Dk : 1, bw = d->beta == DR_BETA_CHANNEL ? d->Dk : 1;
        const size_t sb = nseq * d->Dk * d->Dv * sizeof(float);
        const Span ins[] = {{q, ntok * d->Dk * inb, "q"},
                            {k, ntok * d->Dk * inb, "k"},
                            {v, ntok * d->Dv * inb, "v"},
                            {log_alpha, ntok * gw * 4, "log_alpha"},
                            {beta, ntok * bw * 4, "beta"},
                            {beta_v, ntok * bw * 4, "beta_v"},
                            {key_scale, ntok * d->Dk * 4, "key_scale"},
                            {S0, sb, "S0"},
                            {workspace, w.total, "workspace"}};
        const Span outs[] = {{o, ntok * d->Dv * outb, "o"}, {S_final, sb, "S_final"}};
        s = check_disjoint(outs, 2, ins, 9, S_final, S0);
        if (s != DR_OK) return s;
    }
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
    a.beta_tok = kvtok;
    char* ws = (char*)workspace;
    a.wsT = (dr::half_t*)(ws + w.T);
    a.wsP = (dr::half_t*)(ws + w.Pm);
    a.wsG = (float*)(ws + w.G);
    a.wsQ = w.Q ? (dr::half_t*)(ws + w.Q) : nullptr;
    a.wsKs = w.Ks ? (dr::half_t*)(ws + w.Ks) : nullptr;
    a.wsKl = w.Kl ? (dr::half_t*)(ws + w.Kl) : nullptr;
    a.wsV = w.V ? (dr::half_t*)(ws + w.V) : nullptr;
    hipError_t e = dr::launch_chunk(a, d->Dk, d->in_dtype == DR_F32, d->gate == DR_GATE_CHANNEL || precond,
                                    d->beta == DR_BETA_CHANNEL || kvtok, beta_v != beta, st);
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
    {
        // o is disjoint from the states and the inputs; the states from the inputs
        const size_t inb = d->in_dtype == DR_F32 ? 4 : 2, outb = d->out_dtype == DR_F32 ? 4 : 2;
        const size_t gw = d->gate == DR_GATE_CHANNEL ? d->Dk : 1, bw = d->beta == DR_BETA_CHANNEL ? d->Dk : 1;
        const Span ins[] = {{q, nst * d->Dk * inb, "q"},           {k, nst * d->Dk * inb, "k"},
                            {v, nst * d->Dv * inb, "v"},           {log_alpha, nst * gw * 4, "log_alpha"},
                            {beta, nst * bw * 4, "beta"},          {beta_v, nst * bw * 4, "beta_v"},
                            {key_scale, nst * d->Dk * 4, "key_scale"}};
        const Span outs[] = {{o, nst * d->Dv * outb, "o"}, {S, nst * d->Dk * d->Dv * sizeof(float), "S"}};
        s = check_disjoint(outs, 2, ins, 7);
        if (s != DR_OK) return s;
    }
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
    size_t T, Pm, A, G, S, H, U, R, dU, Qh, Kh, Kc, Kt, q32, k32, v32, b32, db1, rq, rk, dla, F, Ck, Hc, total;
    size_t sC;   // chunks per segment (the chunk count of a sequence: no segments)
};

// The shortest segment a bounded-workspace backward takes, in 64-token chunks
// (each segment costs three launches).
constexpr size_t kMinSegChunks = 32;

// Whether a backward call runs on prepared fp32 copies of its inputs: a
// channel-wise strength, separate strengths (kvtok: of one value per token),
// or the input preparation.
bool bwd_mapped(const dr_chunk_desc& d, bool kvtok) {
    return d.beta == DR_BETA_CHANNEL || kvtok || d.input_flags != 0;
}

bool bwd_copies(const dr_chunk_desc& d, bool kvtok) {
    return d.beta == DR_BETA_CHANNEL || kvtok || (d.input_flags & DR_IN_QK_L2NORM);
}

// Whether the backward's state scans run on the matrix cores: bf16 inputs
// seen by the kernels as they are, no channel gate.
bool bwd_mc(const dr_chunk_desc& d, bool kvtok, bool precond) {
    return d.in_dtype == DR_BF16 && d.gate != DR_GATE_CHANNEL && !precond && !bwd_copies(d, kvtok);
}

// precond: write-side key scales, which take the channel-gate kernels for
// every gate mode.  seg: chunks per segment of a bounded-workspace backward
// (matrix-core path only; 0 or >= the chunk count: none), which keeps S_c,
// H_c and dU for one segment of every sequence, plus a checkpoint of S per
// later segment and the carried state gradient.
BwdLayout bwd_layout(const dr_chunk_desc& d, bool kvtok = false, bool precond = false, size_t seg = 0) {
    BwdLayout w{};
    const size_t NC = ((size_t)d.L + dr::CH - 1) / dr::CH;
    const size_t NCH = (size_t)d.B * d.H * NC;
    const size_t nseq = (size_t)d.B * d.H;
    w.sC = seg == 0 || seg >= NC ? NC : seg;
    const size_t NSL = nseq * w.sC;   // state slots
    const size_t f = sizeof(float);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    // the matrix-core path keeps P, U and R in other forms (packed operands,
    // formed again) and K K^T o E not at all
    const bool mc = bwd_mc(d, kvtok, precond);
    w.T = take(NCH * dr::CH * dr::CH * f);
    if (!mc) {
        w.Pm = take(NCH * dr::CH * dr::CH * f);
        w.A = take(NCH * dr::CH * dr::CH * f);
    }
    const bool cg = d.gate == DR_GATE_CHANNEL || precond;
    w.G = take(NCH * dr::CH * (cg ? d.Dk : 1) * f);
    w.S = take(NSL * d.Dk * d.Dv * f);
    w.H = take(NSL * d.Dk * d.Dv * f);
    if (!mc) {
        w.U = take(NCH * dr::CH * d.Dv * f);
        w.R = take(NCH * dr::CH * d.Dv * f);
    }
    w.dU = take(NSL * dr::CH * d.Dv * f);
    if (w.sC < NC) {
        w.Ck = take(((NC + w.sC - 1) / w.sC - 1) * nseq * d.Dk * d.Dv * f);
        w.Hc = take(nseq * d.Dk * d.Dv * f);
    }
    if (cg) {
        w.Qh = take(NCH * dr::CH * d.Dk * f);
        w.Kh = take(NCH * dr::CH * d.Dk * f);
        w.Kc = take(NCH * dr::CH * d.Dk * f);
        w.Kt = take(NCH * dr::CH * d.Dk * f);
    }
    if (bwd_mapped(d, kvtok)) {
        // the fp32 copies (not with logits alone) and their strengths (with
        // the unused gradient of the unit strengths on the channel-beta
        // route), 1/|q|, 1/|k|
        const size_t ntok = (size_t)d.B * d.H * d.L;
        if (bwd_copies(d, kvtok)) {
            w.q32 = take(ntok * d.Dk * f);
            w.k32 = take(ntok * d.Dk * f);
            w.v32 = take(ntok * d.Dv * f);
        }
        w.b32 = take(ntok * f);
        if (d.beta == DR_BETA_CHANNEL || kvtok) w.db1 = take(ntok * f);
        if (d.input_flags & DR_IN_QK_L2NORM) {
            w.rq = take(ntok * f);
            w.rk = take(ntok * f);
        }
    }
    if (precond && d.gate == DR_GATE_SCALAR)   // d log alpha per channel, summed per token at the end
        w.dla = take((size_t)d.B * d.H * d.L * d.Dk * f);
    if (mc) w.F = take(NCH * dr::kBF);
    w.total = NCH ? off : 0;
    return w;
}

// The workspace layout for `bytes` of workspace: every chunk's states when
// they fit (or segments are not available), else the longest segments that
// fit (total > bytes: none does).
BwdLayout bwd_layout_for(const dr_chunk_desc& d, bool kvtok, bool precond, size_t bytes) {
    const BwdLayout full = bwd_layout(d, kvtok, precond);
    const size_t NC = ((size_t)d.L + dr::CH - 1) / dr::CH;
    if (full.total <= bytes || !bwd_mc(d, kvtok, precond)) return full;
    for (size_t seg = NC - 1; seg >= kMinSegChunks; --seg) {
        const BwdLayout w = bwd_layout(d, kvtok, precond, seg);
        if (w.total <= bytes) return w;
    }
    return full;
}

// The least workspace over the segment lengths (the full layout when
// segments are not available)
size_t bwd_min_bytes(const dr_chunk_desc& d) {
    size_t best = bwd_layout(d).total;
    if (!bwd_mc(d, false, false)) return best;
    const size_t NC = ((size_t)d.L + dr::CH - 1) / dr::CH;
    for (size_t seg = kMinSegChunks; seg < NC; ++seg) best = std::min(best, bwd_layout(d, false, false, seg).total);
    return best;
}

dr_status check_bwd_desc(const dr_chunk_desc* d) {
    dr_status s = check_chunk_desc(d);
    if (s != DR_OK) return s;
    if (d->out_dtype != DR_F32) return fail(DR_ERR_UNSUPPORTED, "dO and the gradients are fp32: out_dtype must be DR_F32");
    const size_t NCH = (size_t)d->B * d->H * (((size_t)d->L + dr::CH - 1) / dr::CH);
    if (NCH > (size_t)std::numeric_limits<int>::max())
        return fail(DR_ERR_UNSUPPORTED, "B*H*ceil(L/64)=%zu chunks: too many", NCH);
    return DR_OK;
}

// beta_v and dbeta_v: the separate write strength and its gradient, or NULL
// for one strength; kvtok: the two strengths hold one value per token
// key_scale and dkey_scale (precond): the write-side key scales and their gradient
dr_status chunk_bwd(const dr_chunk_desc* d, const void* q, const void* k, const void* v, const float* log_alpha,
                    const float* beta, const float* beta_v, const float* S0, const float* dO,
                    const float* dS_final, float* dq, float* dk, float* dv, float* dlog_alpha, float* dbeta,
                    float* dbeta_v, float* dS0, void* workspace, size_t workspace_bytes, void* stream,
                    bool kvtok = false, const float* key_scale = nullptr, float* dkey_scale = nullptr,
                    bool precond = false) {
    dr_status s = check_bwd_desc(d);
    if (s != DR_OK) return s;
    if (kvtok && d->Dv != d->Dk)
        return fail(DR_ERR_UNSUPPORTED, "separate scalar strengths take the channel-beta route: needs Dv == Dk "
                                        "(%d != %d)", d->Dv, d->Dk);
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
        if (precond && (!key_scale || !dkey_scale))
            return fail(DR_ERR_NULL, "key_scale and dkey_scale are required");
    }
    const void* ptrs[] = {q, k, v, log_alpha, beta, beta_v, S0, dO, dS_final, dq, dk, dv, dlog_alpha, dbeta,
                          dbeta_v, dS0, workspace, key_scale, dkey_scale};
    const char* names[] = {"q", "k", "v", "log_alpha", "beta", "beta_v", "S0", "dO", "dS_final", "dq", "dk", "dv",
                           "dlog_alpha", "dbeta", "dbeta_v", "dS0", "workspace", "key_scale", "dkey_scale"};
    for (int i = 0; i < 19; ++i)
        if (ptrs[i] && !aligned16(ptrs[i])) return fail(DR_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    const BwdLayout w = bwd_layout_for(*d, kvtok, precond, workspace ? workspace_bytes : 0);
    {
        // the gradients are disjoint from every input, the workspace and each other
        const size_t ntok = nseq * (size_t)d->L;
        const size_t inb = d->in_dtype == DR_F32 ? 4 : 2;
        const size_t gw = d->gate == DR_GATE_CHANNEL ? d->Dk : 1, bw = d->beta == DR_BETA_CHANNEL ? d->Dk : 1;
        const size_t sb = nseq * d->Dk * d->Dv * sizeof(float);
        const Span ins[] = {{q, ntok * d->Dk * inb, "q"},        {k, ntok * d->Dk * inb, "k"},
                            {v, ntok * d->Dv * inb, "v"},        {log_alpha, ntok * gw * 4, "log_alpha"},
                            {beta, ntok * bw * 4, "beta"},       {beta_v, ntok * bw * 4, "beta_v"},
                            {S0, sb, "S0"},                      {dO, ntok * d->Dv * 4, "dO"},
                            {dS_final, sb, "dS_final"},          {workspace, w.total, "workspace"},
                            {key_scale, ntok * d->Dk * 4, "key_scale"}};
        const Span outs[] = {{dq, ntok * d->Dk * 4, "dq"},
                             {dk, ntok * d->Dk * 4, "dk"},
                             {dv, ntok * d->Dv * 4, "dv"},
                             {dlog_alpha, ntok * gw * 4, "dlog_alpha"},
                             {dbeta, ntok * bw * 4, "dbeta"},
                             {dbeta_v, ntok * bw * 4, "dbeta_v"},
                             {dS0, sb, "dS0"},
                             {dkey_scale, ntok * d->Dk * 4, "dkey_scale"}};
        s = check_disjoint(outs, 8, ins, 11);
        if (s != DR_OK) return s;
    }
    if (w.total) {
        if (!workspace) return fail(DR_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", w.total);
        if (workspace_bytes < w.total)
            return fail(DR_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed (%zu at least, in segments)",
                        workspace_bytes, w.total, kvtok || precond ? w.total : bwd_min_bytes(*d));
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
    a.c0 = 0;
    a.cN = a.NC;
    a.sC = (int)w.sC;
    a.has_gate = d->gate != DR_GATE_NONE;
    char* ws = (char*)workspace;
    const bool mc = bwd_mc(*d, kvtok, precond);
    a.wT = (float*)(ws + w.T);
    a.wP = mc ? nullptr : (float*)(ws + w.Pm);
    a.wA = mc ? nullptr : (float*)(ws + w.A);
    a.wG = (float*)(ws + w.G);
    a.wS = (float*)(ws + w.S);
    a.wH = (float*)(ws + w.H);
    a.wU = mc ? nullptr : (float*)(ws + w.U);
    a.wR = mc ? nullptr : (float*)(ws + w.R);
    a.wdU = (float*)(ws + w.dU);
    if (w.sC < (size_t)a.NC) {
        a.wCk = (float*)(ws + w.Ck);
        a.wHc = (float*)(ws + w.Hc);
    }
    a.cgate = d->gate == DR_GATE_CHANNEL || precond;
    if (a.cgate) {
        a.wQh = (float*)(ws + w.Qh);
        a.wKh = (float*)(ws + w.Kh);
        a.wKc = (float*)(ws + w.Kc);
        a.wKt = (float*)(ws + w.Kt);
        a.gmode = d->gate == DR_GATE_CHANNEL ? 2 : d->gate == DR_GATE_SCALAR ? 1 : 0;
        a.dla_cg = d->gate == DR_GATE_CHANNEL ? dlog_alpha : d->gate == DR_GATE_SCALAR ? (float*)(ws + w.dla) : nullptr;
    }
    if (precond) {
        a.ks = key_scale;
        a.dks = dkey_scale;
    }
    if (mc) a.wF = ws + w.F;
    const bool cbeta = d->beta == DR_BETA_CHANNEL || kvtok;
    const bool mapped = bwd_mapped(*d, kvtok);
    hipError_t e = hipSuccess;
    dr::BwdMap m{};
    if (mapped) {
        // the recurrence's inputs as fp32 copies; on the channel-beta route
        // the unit strengths' gradient goes to db1 and is discarded
        m.q = q; m.k = k; m.v = v;
        m.beta = beta; m.beta_v = beta_v ? beta_v : beta;
        m.f32in = d->in_dtype == DR_F32;
        m.cbeta = cbeta;
        m.per_token = kvtok;
        m.sepv = beta_v != nullptr;
        m.l2 = (d->input_flags & DR_IN_QK_L2NORM) != 0;
        m.logit = (d->input_flags & DR_IN_BETA_LOGIT) != 0;
        m.Dk = d->Dk; m.Dv = d->Dv;
        m.ntok = nseq * d->L;
        m.copy = bwd_copies(*d, kvtok);
        if (m.copy) {
            m.q32 = (float*)(ws + w.q32);
            m.k32 = (float*)(ws + w.k32);
            m.v32 = (float*)(ws + w.v32);
        }
        m.b32 = (float*)(ws + w.b32);
        if (m.l2) {
            m.rq = (float*)(ws + w.rq);
            m.rk = (float*)(ws + w.rk);
        }
        e = dr::launch_bwd_map_in(m, st);
        if (e != hipSuccess) return fail(DR_ERR_HIP, "backward input mapping launch: %s", hipGetErrorString(e));
        if (m.copy) {
            a.q = m.q32; a.k = m.k32; a.v = m.v32;
        }
        a.beta = m.b32;
        if (cbeta) a.dbeta = (float*)(ws + w.db1);
    }
    e = dr::launch_bwd(a, d->Dk, m.copy || d->in_dtype == DR_F32, st);
    if (e != hipSuccess) return fail(DR_ERR_HIP, "backward kernels launch: %s", hipGetErrorString(e));
    if (precond && d->gate == DR_GATE_SCALAR) {
        e = dr::launch_bwd_gate_sum(a.dla_cg, dlog_alpha, nseq * d->L, d->Dk, st);
        if (e != hipSuccess) return fail(DR_ERR_HIP, "backward gate sum launch: %s", hipGetErrorString(e));
    }
    if (mapped) {
        e = dr::launch_bwd_map_out(m, dq, dk, dv, dbeta, dbeta_v, st);
        if (e != hipSuccess) return fail(DR_ERR_HIP, "backward gradient mapping launch: %s", hipGetErrorString(e));
    }
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

dr_status dr_chunk_fwd_noalloc(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const float* S0, void* o,
                               float* S_final, void* stream) {
    g_err[0] = '\0';
    dr_status s = check_chunk_desc(d);
    if (s != DR_OK) return s;
    const size_t need = ws_layout(*d).total;
    if (need > DR_NOALLOC_SCRATCH_BYTES)
        return fail(DR_ERR_WORKSPACE, "the call needs %zu bytes of workspace, the scratch array holds %zu", need,
                    (size_t)DR_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need) {
        s = scratch_for_device(&ws);
        if (s != DR_OK) return s;
    }
    return chunk_fwd(d, q, k, v, log_alpha, beta, beta, nullptr, false, S0, o, S_final, ws,
                     need ? (size_t)DR_NOALLOC_SCRATCH_BYTES : 0, stream);
}

dr_status dr_chunk_fwd_kv(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                          const float* log_alpha, const float* beta_k, const float* beta_v,
                          const float* S0, void* o, float* S_final, void* workspace,
                          size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    // scalar strengths: one value per token each, on the channel-beta kernels
    const bool kvtok = d && d->beta == DR_BETA_SCALAR;
    return chunk_fwd(d, q, k, v, log_alpha, beta_k, beta_v, nullptr, false, S0, o, S_final, workspace,
                     workspace_bytes, stream, kvtok);
}

size_t dr_chunk_fwd_kv_workspace_bytes(const dr_chunk_desc* d) {
    if (check_chunk_desc(d) != DR_OK) return 0;
    const bool kvtok = d->beta == DR_BETA_SCALAR;
    if (kvtok && d->Dv != d->Dk) return 0;
    return ws_layout(*d, false, kvtok).total;
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
    return decode_step(d, q, k, v, log_alpha, beta_k, beta_v, nullptr, false, S, o, stream);
}

size_t dr_chunk_bwd_workspace_bytes(const dr_chunk_desc* d) {
    if (check_bwd_desc(d) != DR_OK) return 0;
    return bwd_layout(*d).total;
}

size_t dr_chunk_bwd_workspace_bytes_min(const dr_chunk_desc* d) {
    if (check_bwd_desc(d) != DR_OK) return 0;
    return bwd_min_bytes(*d);
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
    const size_t ntok = d ? (size_t)(d->B > 0 ? d->B : 0) * (d->H > 0 ? d->H : 0) * (d->L > 0 ? d->L : 0) : 0;
    if (ntok && (!beta_v || !dbeta_v)) return fail(DR_ERR_NULL, "beta_v and dbeta_v are required");
    return chunk_bwd(d, q, k, v, log_alpha, beta_k, beta_v, S0, dO, dS_final, dq, dk, dv, dlog_alpha, dbeta_k,
                     dbeta_v, dS0, workspace, workspace_bytes, stream, d && d->beta == DR_BETA_SCALAR);
}

size_t dr_chunk_bwd_precond_workspace_bytes(const dr_chunk_desc* d) {
    if (check_bwd_desc(d) != DR_OK) return 0;
    return bwd_layout(*d, false, true).total;
}

dr_status dr_chunk_bwd_precond(const dr_chunk_desc* d, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const float* key_scale, const float* S0,
                               const float* dO, const float* dS_final, float* dq, float* dk, float* dv,
                               float* dlog_alpha, float* dbeta, float* dkey_scale, float* dS0, void* workspace,
                               size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    return chunk_bwd(d, q, k, v, log_alpha, beta, nullptr, S0, dO, dS_final, dq, dk, dv, dlog_alpha, dbeta, nullptr,
                     dS0, workspace, workspace_bytes, stream, false, key_scale, dkey_scale, true);
}

size_t dr_chunk_bwd_kv_workspace_bytes(const dr_chunk_desc* d) {
    if (check_bwd_desc(d) != DR_OK) return 0;
    const bool kvtok = d->beta == DR_BETA_SCALAR;
    if (kvtok && d->Dv != d->Dk) return 0;
    return bwd_layout(*d, kvtok).total;
}

}  // extern "C"
