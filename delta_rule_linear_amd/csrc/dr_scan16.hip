// dr_scan16.hip -- the inter-chunk state scan for bf16 inputs on gfx950.
//
// Same algebra as the scan in dr_chunk.hip (per chunk, with T^ and P from the
// prep kernel):  X = Ks S,  R = V - g X,  U = T^ R,  O = g Q S + P U,
// S <- g63 S + Kl^T (l U).  Built around the data movement:
//
//  * One workgroup per (sequence, 16-column tile of S): four compute waves
//    and four copy waves.  The copy waves issue the chunk loop's global
//    memory operations: the chunk operand tiles (Kl, Ks and Q with a channel
//    gate, T^, P, the V tile, gate factors) straight into LDS with 16-byte
//    global->LDS loads, two chunks ahead into a triple buffer (double with a
//    channel gate, whose tiles are larger), a one-dword touch of the chunk
//    four ahead to start its HBM reads early, and the coalesced store of the
//    previous chunk's output from LDS.  Vector-memory issue stalls thus fall
//    on the copy waves.  Without a channel gate the compute waves load their
//    own Q rows into registers one chunk ahead (four 16-byte loads per lane
//    and chunk), which leaves the copy waves less to issue.
//  * On gfx950 a wave's LDS counter also covers its global->LDS copies in
//    flight: each barrier's LDS wait makes the copy waves' copies of that
//    phase complete, and so does the LDS read of the output tile.
//  * Rows of a K / Q tile are stored with their 16-byte pieces XOR-swizzled
//    by row, so fragment reads are free of bank conflicts; T^ and P arrive in
//    the packed lower-block form written by the prep kernels.
//  * Operand types.  With a scalar beta and no channel gate, Ks = Kl = k and
//    Q = q are the raw bf16 inputs: they feed bf16 matrix-core ops directly,
//    with the fp32 state S and l U carried as bf16 hi + lo pairs (16
//    significant bits).  With a channel-wise gate or beta the gated operands
//    come from the workspace in fp16 and S, U are single fp16 terms.  T^ R and
//    P U are fp16 ops in both cases.
//  * Kl^T fragments come from the row-major Kl tile through the transposing
//    LDS read (ds_read_b64_tr_b16): no transposition in registers.
//  * No masking: rows past a sequence's end load a valid clamped row; their
//    U is exactly zero (beta or the prep kernel's zero rows make it so), so
//    they contribute nothing to S, and their O is never stored.
//  * Three barriers per chunk, all raw s_barrier with an LDS-only wait.  The
//    copy waves also wait for the copies of the next chunk before the last
//    one, by count.
//  * The copies are inline assembly, invisible to the compiler, which would
//    otherwise wait for every copy in flight before each LDS read; the
//    operand buffers and the working area are separate LDS objects as well.
//
// Compute wave w owns chunk rows 16w..16w+15 for X, Y, R, U, O and state rows
// [DK/4 w, DK/4 (w+1)) for the state update.

#include <hip/hip_runtime.h>

#include "dr_device.h"
#include "dr_internal.h"
#include "dr_lds.h"

namespace dr {

// LDS plan (bytes).  NB operand buffers, each
//   [Kl 64 x RB][Ks 64 x RB, channel gate only][Q 64 x RB, channel gate only]
//   [T^ packed][P packed][V 64 x 32][gate factors 1024]
// Without a channel gate (QREG) Q is not staged: the compute waves load their
// Q fragments into registers one chunk ahead, which leaves the copy waves
// less to issue.  With a channel gate the copy waves carry Q as well (the
// compute waves' own loads would queue behind the larger copies).
// and the working area [S^T NPL x 16 x SP][R^T 16 x RP][U^T 16 x RP]
// [(lU)^T NPL x 16 x RP][O 64 x OP].
template <int DK, bool RAW, bool CGATE>
struct SD {
    static constexpr int NPL = RAW ? 2 : 1;
    static constexpr bool QREG = !CGATE;
    static constexpr int NB = QREG ? 3 : 2;
    static constexpr int RB = DK * 2;               // bytes per K / Q row
    static constexpr int KL = 0;
    static constexpr int KS = CGATE ? KL + 64 * RB : KL;   // Ks == Kl unless the gate is per channel
    static constexpr int QT = KS + 64 * RB;
    static constexpr int TT = QT + (QREG ? 0 : 64 * RB);
    static constexpr int PT = TT + kTriBytes;
    static constexpr int VT = PT + kTriBytes;
    static constexpr int GT = VT + 64 * 32;
    static constexpr int BUF = GT + 1024;
    static constexpr int SP = (DK + 8) * 2;          // bytes per S^T row
    static constexpr int RP = (CH + 8) * 2;          // bytes per token-major row
    static constexpr int WS = 0;
    static constexpr int WR = WS + NPL * 16 * SP;
    static constexpr int WU = WR + 16 * RP;
    static constexpr int WUL = WU + 16 * RP;
    static constexpr int OP = 16 * 4 + 16;           // bytes per O row (fp32)
    static constexpr int WO = WUL + NPL * 16 * RP;
    static constexpr int WORK = WO + 64 * OP;
    static constexpr int TOTAL = NB * BUF + WORK + 1024;
    // copy waves, and the copy instructions each issues per chunk: a quarter
    // of every K (and Q) tile (RB / 16 instructions each) and four of the 16
    // slots holding T^ (5), P (5), the V tile (2), the gate factors (1) and
    // three repeats of the gate copy, so that every copy wave issues the same
    // count
    static constexpr int NCW = 4;
    static constexpr int NCOPY = ((CGATE ? 2 : 1) + (QREG ? 0 : 1)) * (RB / 16) / NCW + 4;
};

// Lanes (16 bytes each) that copy a chunk's gate record into the 1 KiB gate
// area; the other lanes repeat them.  Channel gate: the state decay [DK].
// Scalar gate: gamma and lambda, and with normalised q and k on raw operands
// (QN) also gamma/|k| and gamma/|q|.
template <int DK, bool CGATE, bool QN>
__host__ __device__ constexpr int gate_lanes() {
    return CGATE ? DK / 4 : QN ? 64 : 32;
}

// Copy wave cw's quarter of a [64][RB]-byte tile of 16-bit values (row r at
// src + r * pitch elements; rows >= valid read row 0) into swizzled LDS.
template <int RB>
__device__ __forceinline__ void copy_tile(const uint16_t* src, size_t pitch, int valid, lchar* tile, int l, int cw) {
    constexpr int PPR = RB / 16;      // pieces per row
    constexpr int RPI = 64 / PPR;     // rows per 1 KiB instruction
    constexpr int NI = 64 / RPI;      // instructions per tile
#pragma unroll
    for (int jj = 0; jj < NI / 4; ++jj) {
        const int j = cw + 4 * jj;
        const int r = j * RPI + l / PPR;
        const int rc = r < valid ? r : 0;
        const int lp = (l % PPR) ^ swz<RB>(r);
        dma16(src + (size_t)rc * pitch + 8 * lp, tile + j * 1024);
    }
}

// Part `PART` of the copies of chunk c into buffer `buf`, copy wave cw's share:
//   0: Kl;  1: Q (channel gate);  2: Ks (channel gate), T^, P, the V tile, the gate factors.
template <int DK, bool RAW, bool CGATE, bool CBETA, bool QN, int PART>
__device__ __forceinline__ void s16_copy(const ChunkArgs& a, lchar* buf, int seq, int c, int n0, int l, int cw) {
    using L = SD<DK, RAW, CGATE>;
    const int t0 = c * CH;
    const int Lc = min(CH, a.L - t0);
    const size_t tok0 = (size_t)seq * a.L + t0;
    const size_t cs = (size_t)seq * a.NC + c;
    const size_t obase = cs * (size_t)(CH * DK);
    if constexpr (PART == 0) {
        if constexpr (RAW)
            copy_tile<L::RB>(static_cast<const uint16_t*>(a.k) + tok0 * DK, DK, Lc, buf + L::KL, l, cw);
        else
            copy_tile<L::RB>(reinterpret_cast<const uint16_t*>(CGATE ? a.wsKl : a.wsKs) + obase, DK, CH,
                             buf + L::KL, l, cw);
    } else if constexpr (PART == 2) {
        if constexpr (CGATE)
            copy_tile<L::RB>(reinterpret_cast<const uint16_t*>(a.wsKs) + obase, DK, CH, buf + L::KS, l, cw);
        // slots k = cw, cw + 4, cw + 8, cw + 12 of: T^ (0-4), P (5-9), the V
        // tile (10-11: 64 rows x 16 columns, two 16-byte pieces per row), the
        // gate factors (12-15; lanes past the data repeat it into the unused
        // upper part of the 1 KiB area)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int k = cw + 4 * jj;
            if (k < 5) {
                dma16(a.wsT + cs * (size_t)(CH * CH) + 512 * k + 8 * l, buf + L::TT + 1024 * k);
            } else if (k < 10) {
                dma16(a.wsP + cs * (size_t)(CH * CH) + 512 * (k - 5) + 8 * l, buf + L::PT + 1024 * (k - 5));
            } else if (k < 12) {
                const int hh = k - 10;
                const int r = 32 * hh + (l >> 1), piece = l & 1;
                if constexpr (CBETA) {
                    dma16(reinterpret_cast<const uint16_t*>(a.wsV) + obase + r * DK + n0 + 8 * piece,
                          buf + L::VT + hh * 1024);
                } else {
                    const int rc = r < Lc ? r : 0;
                    dma16(static_cast<const uint16_t*>(a.v) + (tok0 + rc) * a.Dv + n0 + 8 * piece,
                          buf + L::VT + hh * 1024);
                }
            } else {
                constexpr int NG = gate_lanes<DK, CGATE, QN>();
                dma16(a.wsG + cs * kGW + 4 * (l % NG), buf + L::GT);
            }
        }
    } else {
        copy_tile<L::RB>(reinterpret_cast<const uint16_t*>(a.wsQ) + obase, DK, CH, buf + L::QT, l, cw);
    }
}

// How many chunks ahead of the one being computed the copy waves touch the
// operands to start their HBM reads early: each workgroup of a sequence
// touches one dword in each of a 1/NT share of the chunk's 128-byte operand
// lines, as one global->LDS load per copy wave into a scratch row that is
// never read (Copier::warm).
#ifndef DR_SCAN_PFD
#define DR_SCAN_PFD 4
#endif

// A copy wave's per-lane address plan: byte offsets inside each operand tile
// it copies, computed once, so that every copy in the chunk loop is a scalar
// base (per chunk) plus a fixed lane offset.  A partial last chunk, whose raw
// rows must be clamped, goes through s16_copy instead.
template <int DK, bool RAW, bool CGATE, bool CBETA, bool QN>
struct Copier {
    using L = SD<DK, RAW, CGATE>;
    static constexpr int PPR = L::RB / 16;   // 16-byte pieces per tile row
    static constexpr int RPI = 64 / PPR;     // tile rows per 1 KiB instruction
    static constexpr int NTI = PPR / 4;      // tile instructions per copy wave
    unsigned toff[NTI];   // lane offsets in a K / Q tile (row pitch DK)
    unsigned soff[4];     // lane offsets of the part-1 slots
    unsigned ooff;        // output lane offset (elements)
    const char* wbase;    // this lane's warm-up line in chunk 0
    unsigned wstride;     // and its per-chunk stride
    int cw;

    __device__ __forceinline__ void init(const ChunkArgs& a, int seq, int n0, int l, int cw_, int tile, int NT) {
        cw = cw_;
#pragma unroll
        for (int jj = 0; jj < NTI; ++jj) {
            const int j = cw + 4 * jj;
            const int r = j * RPI + l / PPR;
            const int lp = (l % PPR) ^ swz<L::RB>(r);
            toff[jj] = (unsigned)(r * DK + 8 * lp) * 2u;
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int k = cw + 4 * jj;
            unsigned o;
            if (k < 5) o = 1024u * k + 16u * l;
            else if (k < 10) o = 1024u * (k - 5) + 16u * l;
            else if (k < 12) {
                const int r = 32 * (k - 10) + (l >> 1), piece = l & 1;
                o = (unsigned)(r * (CBETA ? DK : a.Dv) + n0 + 8 * piece) * 2u;
            } else {
                constexpr int NG = gate_lanes<DK, CGATE, QN>();
                o = 16u * (l % NG);
            }
            soff[jj] = o;
        }
        ooff = (unsigned)((16 * cw + (l >> 2)) * a.Dv + n0 + 4 * (l & 3));
        // warm-up line: regions of one full chunk, in order
        const size_t seq0 = (size_t)seq * a.L;           // first token of the sequence
        const size_t cs0 = (size_t)seq * a.NC;           // its first chunk slot
        int x = tile + NT * (64 * cw + l);
        const char* b = nullptr;
        unsigned st = 0;
        const char* lastb = nullptr;
        unsigned lastst = 0;
        auto region = [&](const void* base0, unsigned stride, int n) {
            const char* bb = static_cast<const char*>(base0);
            if (!b && x >= 0 && x < n) { b = bb + 128 * x; st = stride; }
            lastb = bb + 128 * (n - 1);
            lastst = stride;
            x -= n;
        };
        if constexpr (RAW) {
            region(static_cast<const char*>(a.k) + seq0 * DK * 2, CH * DK * 2, DK);
            region(static_cast<const char*>(a.q) + seq0 * DK * 2, CH * DK * 2, DK);
        } else {
            region(reinterpret_cast<const char*>(CGATE ? a.wsKl : a.wsKs) + cs0 * CH * DK * 2, CH * DK * 2, DK);
            if constexpr (CGATE) region(reinterpret_cast<const char*>(a.wsKs) + cs0 * CH * DK * 2, CH * DK * 2, DK);
            region(reinterpret_cast<const char*>(a.wsQ) + cs0 * CH * DK * 2, CH * DK * 2, DK);
        }
        region(a.wsT + cs0 * CH * CH, CH * CH * 2, kTriBytes / 128);
        region(a.wsP + cs0 * CH * CH, CH * CH * 2, kTriBytes / 128);
        if constexpr (CBETA) region(reinterpret_cast<const char*>(a.wsV) + cs0 * CH * DK * 2, CH * DK * 2, DK);
        else region(static_cast<const char*>(a.v) + seq0 * a.Dv * 2, CH * a.Dv * 2, a.Dv);
        region(a.wsG + cs0 * kGW, kGW * 4, gate_lanes<DK, CGATE, QN>() * 16 / 128);
        wbase = b ? b : lastb;
        wstride = b ? st : lastst;
    }

    // chunk cn's raw rows need clamping (partial last chunk)?
    __device__ __forceinline__ static bool tail(const ChunkArgs& a, int cn) { return (cn + 1) * CH > a.L; }

    // part PART of chunk cn's copies (numbered as in s16_copy)
    template <int PART>
    __device__ __forceinline__ void copy(const ChunkArgs& a, lchar* buf, int seq, int cn, int n0, int l) const {
        constexpr bool RAWROWS = PART == 2 ? !CBETA : RAW;
        if (RAWROWS && tail(a, cn)) {
            s16_copy<DK, RAW, CGATE, CBETA, QN, PART>(a, buf, seq, cn, n0, l, cw);
            return;
        }
        const size_t tok0 = (size_t)seq * a.L + (size_t)cn * CH;
        const size_t cs = (size_t)seq * a.NC + cn;
        const size_t obase = cs * (size_t)(CH * DK) * 2;   // bytes
        if constexpr (PART == 0) {
            const char* src = uniform_ptr(RAW ? static_cast<const char*>(a.k) + tok0 * DK * 2
                                              : reinterpret_cast<const char*>(CGATE ? a.wsKl : a.wsKs) + obase);
#pragma unroll
            for (int jj = 0; jj < NTI; ++jj) dma16s(src, toff[jj], buf + L::KL + (cw + 4 * jj) * 1024);
        } else if constexpr (PART == 1) {
            const char* src = uniform_ptr(reinterpret_cast<const char*>(a.wsQ) + obase);
#pragma unroll
            for (int jj = 0; jj < NTI; ++jj) dma16s(src, toff[jj], buf + L::QT + (cw + 4 * jj) * 1024);
        } else {
            if constexpr (CGATE) {
                const char* src = uniform_ptr(reinterpret_cast<const char*>(a.wsKs) + obase);
#pragma unroll
                for (int jj = 0; jj < NTI; ++jj) dma16s(src, toff[jj], buf + L::KS + (cw + 4 * jj) * 1024);
            }
            const char* tb = uniform_ptr(a.wsT + cs * (size_t)(CH * CH));
            const char* pb = uniform_ptr(a.wsP + cs * (size_t)(CH * CH));
            const char* vb = uniform_ptr(CBETA ? reinterpret_cast<const char*>(a.wsV) + obase
                                               : static_cast<const char*>(a.v) + tok0 * a.Dv * 2);
            const char* gb = uniform_ptr(a.wsG + cs * kGW);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int k = cw + 4 * jj;   // wave-uniform: selects, no branches
                const char* src = k < 5 ? tb : k < 10 ? pb : k < 12 ? vb : gb;
                const int dst = k < 5 ? L::TT + 1024 * k
                              : k < 10 ? L::PT + 1024 * (k - 5)
                              : k < 12 ? L::VT + 1024 * (k - 10) : L::GT;
                dma16s(src, soff[jj], buf + dst);
            }
        }
    }

    // one dword of chunk cc's lines (cc < 0: the first workspace line)
    __device__ __forceinline__ void warm(const ChunkArgs& a, int seq, int cc, lchar* sink) const {
        const char* p = cc >= 0 ? wbase + (size_t)cc * wstride
                                : reinterpret_cast<const char*>(a.wsT + (size_t)seq * a.NC * (CH * CH));
        dma4(p, sink);
    }

    // chunk cc's output rows 16 cw .. 16 cw + 15 from sO.  The LDS read waits
    // (lgkmcnt) for this wave's global->LDS copies issued before it as well,
    // so it is placed where those have long landed.
    __device__ __forceinline__ void store_o(const ChunkArgs& a, const lchar* sO, int seq, int cc, int l) const {
        const int t0 = cc * CH;
        const int Lc = min(CH, a.L - t0);
        const int row = 16 * cw + (l >> 2);
        const float4 v = lds_ld<float4>(sO + row * L::OP + 16 * (l & 3));
        const size_t e0 = ((size_t)seq * a.L + t0) * a.Dv;   // first element of the chunk's rows
        const bf16x4 h = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
        const bool bf = a.out_bf16;
        if (row < Lc && bf) *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(a.o) + e0 + ooff) = h;
        if (row < Lc && !bf) *reinterpret_cast<float4*>(static_cast<float*>(a.o) + e0 + ooff) = v;
    }
};

// QN: q and k are made unit vectors in the kernels while the raw inputs are
// the operands (scalar gate and beta); the rows of K S take gamma/|k|, those
// of Q S gamma/|q| (lambda/|k| is stored in lambda's place).
template <int DK, bool RAW, bool CGATE, bool CBETA, bool QN = false>
__global__ __launch_bounds__(512) void scan16_kernel(ChunkArgs a) {
    using L = SD<DK, RAW, CGATE>;
    constexpr int NB = L::NB;
    constexpr int NPL = L::NPL;
    constexpr int NTS = DK / 64;   // 16-row state tiles per compute wave
    constexpr bool BF = RAW;       // raw bf16 operands use bf16 ops, workspace ones fp16
    // Separate LDS objects for the operand buffers and the working area: the
    // compiler then sees that copies into one buffer cannot alias the reads
    // of another, and does not wait for copies before every LDS access.
    __shared__ __attribute__((aligned(16))) char lds_b0[L::BUF];
    __shared__ __attribute__((aligned(16))) char lds_b1[L::BUF];
    __shared__ __attribute__((aligned(16))) char lds_b2[NB == 3 ? L::BUF : 16];
    __shared__ __attribute__((aligned(16))) char lds_work[L::WORK];
    __shared__ __attribute__((aligned(16))) char lds_sink[1024];

    // all column tiles of one sequence on one XCD (workgroups are dealt
    // round-robin to the 8 XCDs), so they share the chunk operands in L2
    const int NT = a.Dv / 16;
    const int bid = blockIdx.x;
    const int seq = (bid / (8 * NT)) * 8 + (bid & 7);
    const int tile = (bid >> 3) % NT;
    if (seq >= a.nseq) return;
    const int n0 = tile * 16;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const bool copier = w >= 4;   // waves 4-7 copy, 0-3 compute (wave-uniform)
    const int cw = __builtin_amdgcn_readfirstlane(w - 4);
    const int i16 = l & 15, g = l >> 4;
    const int col = n0 + i16;
    const int ra = 16 * w + i16;
    lchar* b0 = (lchar*)lds_b0;
    lchar* b1 = (lchar*)lds_b1;
    lchar* b2 = (lchar*)lds_b2;
    lchar* work = (lchar*)lds_work;
    lchar* sink = (lchar*)lds_sink;
    lchar* sS = work + L::WS;
    lchar* sR = work + L::WR;
    lchar* sU = work + L::WU;
    lchar* sUl = work + L::WUL;
    lchar* sO = work + L::WO;

    // Barrier.  On gfx950 a wave's LDS counter also covers its global->LDS
    // copies in flight, so at each barrier the copy waves wait for the copies
    // they issued in that phase.  Measured, that is faster than letting the
    // copies run on: unthrottled copies fill the memory pipeline, and the
    // compute waves' own loads and stores then wait at issue.
    auto sync = [&]() { lds_barrier(); };

    Copier<DK, RAW, CGATE, CBETA, QN> cp;
    if (copier) cp.init(a, seq, n0, l, cw, tile, NT);
    // chunks that are whole (only those are touched ahead)
    const int NCF = a.L / CH;

    f32x4 S[NTS];
    if (!copier) {
#pragma unroll
        for (int t = 0; t < NTS; ++t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * (w * NTS + t) + 4 * g + j;
                S[t][j] = a.S0 ? a.S0[((size_t)seq * DK + row) * a.Dv + col] : 0.f;
            }
            st4_terms<BF, NPL>(sS + i16 * L::SP + 2 * (16 * (w * NTS + t) + 4 * g), 16 * L::SP, S[t]);
        }
    } else {
        cp.template copy<0>(a, b0, seq, 0, n0, l);
        if constexpr (!L::QREG) cp.template copy<1>(a, b0, seq, 0, n0, l);
        cp.template copy<2>(a, b0, seq, 0, n0, l);
        if constexpr (NB == 3) {
            const int c1 = min(1, a.NC - 1);
            cp.template copy<0>(a, b1, seq, c1, n0, l);
            cp.template copy<2>(a, b1, seq, c1, n0, l);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(L::NCOPY));   // this wave's copies of chunk 0 have landed
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
    }
    // Q fragments of row 16 w + i16 (columns 32 s + 8 g .. +7), loaded into
    // registers by the compute waves one chunk ahead; rows past a sequence's
    // end load row 0 of the chunk (their output is never stored)
    uint4 qn[DK / 32];
    auto fetch_q = [&](int cq) {
        const int t0 = cq * CH;
        const int Lc = min(CH, a.L - t0);
        const int r = ra < Lc ? ra : 0;
        const uint16_t* src = RAW ? static_cast<const uint16_t*>(a.q) + ((size_t)seq * a.L + t0 + r) * DK
                                  : reinterpret_cast<const uint16_t*>(a.wsQ) +
                                        ((size_t)seq * a.NC + cq) * (size_t)(CH * DK) + (size_t)ra * DK;
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) qn[s] = *reinterpret_cast<const uint4*>(src + 32 * s + 8 * g);
    };
    if constexpr (L::QREG) {
        if (!copier) fetch_q(0);
    }
    sync();

    // one chunk: operands in `buf`; the copy wave fills `cbuf` with chunk
    // c + NB - 1 (clamped to the last chunk: a buffer nobody reads again)
    auto chunk = [&](const int c, const lchar* buf, lchar* cbuf) {
        const int cn = min(c + NB - 1, a.NC - 1);
        auto gt = [&](int i) { return lds_ld<float>(buf + L::GT + 4 * i); };
        f32x4 Y, gam, lam, gamq;
        // A fragment of a packed triangle: row 16 w + i16, columns 32 s + 8 g
        // .. +7, i.e. block (w, 2 s + g / 2), half g & 1; zero above the
        // diagonal blocks.
        // (read with tri_frag, zeroed above the diagonal blocks with
        // tri_mask once the read has landed)
        auto tri_frag = [&](const lchar* tri, int s) {
            const int I = 2 * s + (g >> 1);
            const int Ic = I <= w ? I : w;
            return lds16(tri + tri_block(w, Ic) * 512 + i16 * 32 + 16 * ((g & 1) ^ ((i16 >> 3) & 1)));
        };
        auto tri_mask = [&](uint4& f, int s) {
            const uint32_t m = 2 * s + (g >> 1) <= w ? ~0u : 0u;
            f.x &= m;
            f.y &= m;
            f.z &= m;
            f.w &= m;
        };
        // operands of phases 2 and 3 that depend only on the chunk's tiles,
        // read during phase 1 so that their LDS latency is off the chain
        uint4 tfr[2], pfr[2], kfr[NTS][2], sfr[DK / 32][NPL];

        // ---------------- phase 1: X = Ks S, R = V - g X
        if (copier) {
            if constexpr (!L::QREG) {
                if (c > 0) cp.store_o(a, sO, seq, c - 1, l);
            }
            cp.template copy<0>(a, cbuf, seq, cn, n0, l);
        } else {
            // X only: the state fragments are kept for Y = Q S, which is off
            // the chain and done in phase 2.  Every LDS read of the phase is
            // issued first, so that one read latency is exposed, not one per
            // k-step.
            uint4 kf[DK / 32];
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                kf[s] = lds16(tile_at<L::RB>(buf + L::KS, ra, 4 * s + g));
#pragma unroll
                for (int p = 0; p < NPL; ++p)
                    sfr[s][p] = lds16(sS + p * 16 * L::SP + i16 * L::SP + 2 * (32 * s + 8 * g));
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) tfr[s] = tri_frag(buf + L::TT, s);
            uint16_t vb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * w + 4 * g + j;
                vb[j] = lds_ld<uint16_t>(buf + L::VT + r * 32 + 2 * i16);
                gam[j] = CGATE ? 1.f : gt(QN ? 128 + r : r);
                lam[j] = CGATE ? 1.f : gt(64 + r);
                if constexpr (QN) gamq[j] = gt(192 + r);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 2; ++s) tri_mask(tfr[s], s);
            f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < DK / 32; ++s)
#pragma unroll
                for (int p = 0; p < NPL; ++p) X = mfma_raw<BF>(kf[s], sfr[s][p], X);
            f32x4 Rv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float vv = CBETA ? (float)__builtin_bit_cast(half_t, vb[j]) : bf16_to_f32(vb[j]);
                Rv[j] = vv - gam[j] * X[j];
            }
            st4_terms<false, 1>(sR + i16 * L::RP + 2 * (16 * w + 4 * g), 0, Rv);
        }
        sync();

        // ---------------- phase 2: U = T^ R (and l U for the state update), Y = Q S
        f32x4 U;
        if (copier) {
            if constexpr (!L::QREG) {
                cp.template copy<1>(a, cbuf, seq, cn, n0, l);
            } else {
                // the previous chunk's output (sO is rewritten in phase 3)
                if (c > 0) cp.store_o(a, sO, seq, c - 1, l);
            }
        } else {
            // all LDS reads first: R, then Q and the phase-3 operands that
            // depend only on the chunk's tiles
            uint4 rf[2], qf[DK / 32];
#pragma unroll
            for (int s = 0; s < 2; ++s) rf[s] = lds16(sR + i16 * L::RP + 2 * (32 * s + 8 * g));
#pragma unroll
            for (int s = 0; s < DK / 32; ++s)
                qf[s] = L::QREG ? qn[s] : lds16(tile_at<L::RB>(buf + L::QT, ra, 4 * s + g));
#pragma unroll
            for (int s = 0; s < 2; ++s) pfr[s] = tri_frag(buf + L::PT, s);
            // Kl^T fragments (state row rt + i16, tokens 32 s + 8 g + 0..7) from
            // two transposed reads: lane q of each 16-lane group points at
            // token 32 s + 8 g + (q >> 2) (+4) and key column rt + 4 (q & 3);
            // lane i then holds column rt + i.
#pragma unroll
            for (int t = 0; t < NTS; ++t) {
                const int rt = 16 * (w * NTS + t);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int tok = 32 * s + 8 * g + (i16 >> 2);
                    const int d = rt + 4 * (i16 & 3);
                    const uint2 lo4 = lds_tr4(tile_at<L::RB>(buf + L::KL, tok, d >> 3) + 2 * (d & 7));
                    const uint2 hi4 = lds_tr4(tile_at<L::RB>(buf + L::KL, tok + 4, d >> 3) + 2 * (d & 7));
                    kfr[t][s] = {lo4.x, lo4.y, hi4.x, hi4.y};
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 2; ++s) tri_mask(pfr[s], s);
            U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s) U = mfma_raw<false>(tfr[s], rf[s], U);
            st4_terms<false, 1>(sU + i16 * L::RP + 2 * (16 * w + 4 * g), 0, U);
            f32x4 Ul;
#pragma unroll
            for (int j = 0; j < 4; ++j) Ul[j] = lam[j] * U[j];
            st4_terms<BF, NPL>(sUl + i16 * L::RP + 2 * (16 * w + 4 * g), 16 * L::RP, Ul);
            // off the chain: Y = Q S
            Y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < DK / 32; ++s)
#pragma unroll
                for (int p = 0; p < NPL; ++p) Y = mfma_raw<BF>(qf[s], sfr[s][p], Y);
            if constexpr (L::QREG) fetch_q(min(c + 1, a.NC - 1));
        }
        sync();

        // ---------------- phase 3: O = g Y + P U; S = g63 S + Kl^T (l U)
        if (copier) {
            cp.template copy<2>(a, cbuf, seq, cn, n0, l);
            cp.warm(a, seq, NCF > 0 ? min(c + DR_SCAN_PFD, NCF - 1) : -1, sink + 256 * cw);
            // the copies of chunk c + 1 have landed: with three buffers every
            // operation but the NCOPY + 1 just issued for later chunks is
            // complete; with two, every one but the touch
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(NB == 3 ? L::NCOPY + 1 : 1));
        } else {
            // all LDS reads first: U, l U and the state decay
            uint4 uf[2], ulf[2][NPL];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                uf[s] = lds16(sU + i16 * L::RP + 2 * (32 * s + 8 * g));
#pragma unroll
                for (int p = 0; p < NPL; ++p)
                    ulf[s][p] = lds16(sUl + p * 16 * L::RP + i16 * L::RP + 2 * (32 * s + 8 * g));
            }
            float d63[NTS][4];
#pragma unroll
            for (int t = 0; t < NTS; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) d63[t][j] = CGATE ? gt(16 * (w * NTS + t) + 4 * g + j) : gt(63);
            __builtin_amdgcn_sched_barrier(0);
            f32x4 O;
#pragma unroll
            for (int j = 0; j < 4; ++j) O[j] = (QN ? gamq[j] : gam[j]) * Y[j];
#pragma unroll
            for (int s = 0; s < 2; ++s) O = mfma_raw<false>(pfr[s], uf[s], O);
            // to LDS; the copy waves store it to global memory during the
            // next chunk (global stores would block these waves at issue
            // behind the copies)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                lds_st(sO + (16 * w + 4 * g + j) * L::OP + 4 * i16, O[j]);

#pragma unroll
            for (int t = 0; t < NTS; ++t) {
                const int rt = 16 * (w * NTS + t);
                f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int p = 0; p < NPL; ++p) acc[s] = mfma_raw<BF>(kfr[t][s], ulf[s][p], acc[s]);
#pragma unroll
                for (int j = 0; j < 4; ++j) S[t][j] = d63[t][j] * S[t][j] + (acc[0][j] + acc[1][j]);
                st4_terms<BF, NPL>(sS + i16 * L::SP + 2 * (rt + 4 * g), 16 * L::SP, S[t]);
            }
        }
        sync();
    };

    for (int c = 0; c < a.NC; c += NB) {
        if constexpr (NB == 3) {
            chunk(c, b0, b2);
            if (c + 1 < a.NC) chunk(c + 1, b1, b0);
            if (c + 2 < a.NC) chunk(c + 2, b2, b1);
        } else {
            chunk(c, b0, b1);
            if (c + 1 < a.NC) chunk(c + 1, b1, b0);
        }
    }

    if (copier) {
        cp.store_o(a, sO, seq, a.NC - 1, l);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no copy may land after the workgroup ends
    } else if (a.S_final) {
#pragma unroll
        for (int t = 0; t < NTS; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * (w * NTS + t) + 4 * g + j;
                a.S_final[((size_t)seq * DK + row) * a.Dv + col] = S[t][j];
            }
    }
}

template <int DK, bool CGATE, bool CBETA>
static hipError_t launch_s16(const ChunkArgs& a, hipStream_t st) {
    constexpr bool RAW = !CGATE && !CBETA;
    using L = SD<DK, RAW, CGATE>;
    static_assert(L::TOTAL <= 160 * 1024, "LDS plan exceeds 160 KiB");
    static_assert(L::NCOPY + 1 <= 63, "copies per chunk exceed the vector-memory counter");
    static_assert(gate_lanes<DK, CGATE, RAW>() * 16 <= 1024, "gate record exceeds its LDS area");
    auto kern = RAW && a.qk_norm ? scan16_kernel<DK, RAW, CGATE, CBETA, RAW>
                                 : scan16_kernel<DK, RAW, CGATE, CBETA>;
    const int NT = a.Dv / 16;
    const int groups = (a.nseq + 7) / 8;
    return launch_k(kProfScan, kern, dim3(groups * 8 * NT), dim3(512), 0, st, a);
}

hipError_t launch_scan16(const ChunkArgs& a, int Dk, bool cgate, bool cbeta, hipStream_t st) {
    if (Dk == 64) {
        if (cgate) return cbeta ? launch_s16<64, true, true>(a, st) : launch_s16<64, true, false>(a, st);
        return cbeta ? launch_s16<64, false, true>(a, st) : launch_s16<64, false, false>(a, st);
    }
    if (cgate) return cbeta ? launch_s16<128, true, true>(a, st) : launch_s16<128, true, false>(a, st);
    return cbeta ? launch_s16<128, false, true>(a, st) : launch_s16<128, false, false>(a, st);
}

}  // namespace dr
