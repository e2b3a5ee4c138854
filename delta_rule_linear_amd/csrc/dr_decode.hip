// dr_decode.hip -- one recurrent decode step for a batch of independent states.
//
// Optional input preparation (DeltaNet page, step list, step 2 and its notes on
// the key/query map and on choosing beta): q and k made unit vectors, beta
// (and beta_v) given as logits.  Optional write-side key scales s (OSDN page,
// "Method"): the write key is w = s (.) kt, S = S' + w u^T, o = S'^T q + (q . w) u.
//
// Per state S (d_k x d_v, fp32) and one new token (FG2-GDN page, section 2,
// the state-update equation; DeltaNet page, step list, steps 3-6; with a
// separate write strength, vt = sqrt(beta_v) v, section "Erweiterung:
// FG2-GDN+"):
//   S' = Diag(alpha) S;  p = S'^T kt;  r = S'^T q;  u = vt - p;
//   S  = S' + kt u^T;    o = S^T q = r + (q . kt) u.
// Each state is read once and written once, so the step is bound by HBM
// bandwidth; the kernel streams the state in 16-byte non-temporal accesses,
// keeps its slice in registers between the read and the write, and reduces
// the two column dot products through LDS.
//
// Geometry: one workgroup of 256 threads per (state, 64-column slab).  Thread
// (rg = tid >> 4, cg = tid & 15) holds rows rg + 16 i (i < Dk / 16) of columns
// slab*64 + 4 cg .. +3, so each wave reads four full 256-byte row segments per
// load instruction.

#include <hip/hip_runtime.h>

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {

// The state is streamed once in and once out per step; between two steps on
// the same state a layer's other states (or other layers) pass through the
// caches, so the state traffic carries the non-temporal hint: it does not
// displace what the caches hold for other work.  Measured on a batch twice the
// size of the last-level cache, this is the faster form.
__device__ __forceinline__ float4 ld_state(const float* p) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void st_state(float* p, const float4& v) {
    const f32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(p));
}

template <int DK, bool F32IN, bool CGATE, bool CBETA>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    constexpr int RPT = DK / 16;   // rows per thread
    __shared__ float sk[DK];       // kt (the read side)
    __shared__ float sw[DK];       // the write-side key: kt, or s (.) kt with key scales
    __shared__ float sq[DK];       // q
    __shared__ float sa[DK];       // alpha per row
    __shared__ float red[2][16][64];
    __shared__ float su[64];
    __shared__ float sdot[3][4];

    const int nslab = (a.Dv + 63) / 64;
    const int sidx = blockIdx.x / nslab;       // state index n * H + h
    const int slab = blockIdx.x % nslab;
    const int tid = threadIdx.x;
    const int rg = tid >> 4, cg = tid & 15;
    const int col0 = slab * 64 + 4 * cg;
    const bool colok = col0 < a.Dv;            // Dv is a multiple of 16, so 4 columns at once

    float4 s[RPT];
    float* S = a.S + (size_t)sidx * DK * a.Dv;
    if (colok) {
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            s[i] = ld_state(S + (size_t)(rg + 16 * i) * a.Dv + col0);
    }

    // token vectors: kt = sqrt(beta) k, alpha, q;  q . kt.  With the input
    // preparation, q and k are first made unit vectors: the three sums q . kt,
    // |q|^2 and |k|^2 are reduced together, then the vectors are rescaled.
    float dotp = 0.f, ssq = 0.f, ssk = 0.f, kt = 0.f, qv = 0.f, ksc = 1.f;
    if (tid < DK) {
        const int c = tid;
        const size_t ti = (size_t)sidx * DK + c;
        const float kv = load1<F32IN>(a.k, ti);
        qv = load1<F32IN>(a.q, ti);
        const float bv = strength(CBETA ? a.beta[ti] : a.beta[sidx], a.beta_logit);
        kt = sqrtf(bv) * kv;
        if (a.key_scale) ksc = a.key_scale[ti];
        float al = 1.f;
        if (a.has_gate) al = expf(CGATE ? a.log_alpha[ti] : a.log_alpha[sidx]);
        sa[c] = al;
        dotp = qv * (kt * ksc);   // q . w
        ssq = qv * qv;
        ssk = kv * kv;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        dotp += __shfl_xor(dotp, off);
        ssq += __shfl_xor(ssq, off);
        ssk += __shfl_xor(ssk, off);
    }
    if ((tid & 63) == 0) {
        sdot[0][tid >> 6] = dotp;
        sdot[1][tid >> 6] = ssq;
        sdot[2][tid >> 6] = ssk;
    }
    __syncthreads();
    float rq = 1.f, rk = 1.f;
    if (a.qk_norm) {
        rq = inv_norm(sdot[1][0] + sdot[1][1] + sdot[1][2] + sdot[1][3]);
        rk = inv_norm(sdot[2][0] + sdot[2][1] + sdot[2][2] + sdot[2][3]);
    }
    const float qk = (sdot[0][0] + sdot[0][1] + sdot[0][2] + sdot[0][3]) * (rq * rk);
    if (tid < DK) {
        sk[tid] = kt * rk;
        sw[tid] = (kt * rk) * ksc;
        sq[tid] = qv * rq;
    }
    __syncthreads();

    // this thread's slice of S, read once (issued above, before the token
    // vectors' barriers)
    float pp[4] = {0.f, 0.f, 0.f, 0.f}, pr[4] = {0.f, 0.f, 0.f, 0.f};
    if (colok) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int c = rg + 16 * i;
            const float ka = sa[c] * sk[c], qa = sa[c] * sq[c];
            pp[0] += ka * s[i].x; pp[1] += ka * s[i].y; pp[2] += ka * s[i].z; pp[3] += ka * s[i].w;
            pr[0] += qa * s[i].x; pr[1] += qa * s[i].y; pr[2] += qa * s[i].z; pr[3] += qa * s[i].w;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        red[0][rg][4 * cg + j] = pp[j];
        red[1][rg][4 * cg + j] = pr[j];
    }
    __syncthreads();

    // column totals, new value u = vt - p, output o = r + (q . w) u
    if (tid < 64) {
        const int col = slab * 64 + tid;
        float p = 0.f, r = 0.f;
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            p += red[0][g][tid];
            r += red[1][g][tid];
        }
        float u = 0.f;
        if (col < a.Dv) {
            const size_t vi = (size_t)sidx * a.Dv + col;
            const float bv = strength(CBETA ? a.beta_v[(size_t)sidx * DK + col] : a.beta_v[sidx],
                                      a.beta_logit);
            const float vt = sqrtf(bv) * load1<F32IN>(a.v, vi);
            u = vt - p;
            const float o = r + qk * u;
            if (a.out_bf16) static_cast<uint16_t*>(a.o)[vi] = f32_to_bf16(o);
            else static_cast<float*>(a.o)[vi] = o;
        }
        su[tid] = u;
    }
    __syncthreads();

    // S = Diag(alpha) S + w u^T, written once
    if (colok) {
        const float u0 = su[4 * cg], u1 = su[4 * cg + 1], u2 = su[4 * cg + 2], u3 = su[4 * cg + 3];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int c = rg + 16 * i;
            const float al = sa[c], w = sw[c];
            float4 n;
            n.x = al * s[i].x + w * u0;
            n.y = al * s[i].y + w * u1;
            n.z = al * s[i].z + w * u2;
            n.w = al * s[i].w + w * u3;
            st_state(S + (size_t)c * a.Dv + col0, n);
        }
    }
}

template <int DK, bool F32IN>
static hipError_t launch_decode_d(const DecodeArgs& a, bool cgate, bool cbeta, hipStream_t st) {
    const int nslab = (a.Dv + 63) / 64;
    dim3 grid((unsigned)((size_t)a.N * a.H * nslab));
    if (cgate) {
        if (cbeta) return launch_k(kProfDecode, decode_kernel<DK, F32IN, true, true>, grid, dim3(256), 0, st, a);
        return launch_k(kProfDecode, decode_kernel<DK, F32IN, true, false>, grid, dim3(256), 0, st, a);
    }
    if (cbeta) return launch_k(kProfDecode, decode_kernel<DK, F32IN, false, true>, grid, dim3(256), 0, st, a);
    return launch_k(kProfDecode, decode_kernel<DK, F32IN, false, false>, grid, dim3(256), 0, st, a);
}

hipError_t launch_decode(const DecodeArgs& a, int Dk, bool f32in, bool cgate, bool cbeta,
                         hipStream_t st) {
    if ((size_t)a.N * a.H == 0) return hipSuccess;
    hipError_t e;
    if (Dk == 64) e = f32in ? launch_decode_d<64, true>(a, cgate, cbeta, st)
                            : launch_decode_d<64, false>(a, cgate, cbeta, st);
    else e = f32in ? launch_decode_d<128, true>(a, cgate, cbeta, st)
                   : launch_decode_d<128, false>(a, cgate, cbeta, st);
    return e;
}

}  // namespace dr
