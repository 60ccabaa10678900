// Fused chunked Titans memory scan with each memory split over a PAIR (or a QUAD) of
// workgroups, for the 64 -> 256 -> 64 SiLU memory with chunks of 64 tokens and bf16
// q/k/v/y (fp32 gates and state).
//
// Why split: one (b, h) memory per workgroup leaves most of the GPU's compute units idle
// when there are fewer memories than compute units, and its 256 KB of fp32 state fills the
// register file of one CU.  Here side s of kS = 2 (pairs) or 4 (quads) owns hidden units
// kHidSide s .. kHidSide (s + 1) - 1 (kHidSide = 256 / kS); wave w of a side owns 32 (pairs)
// or 16 (quads) of them (rows of W1 / S1, columns of W2 / S2), held in registers as MFMA
// accumulators for the whole sequence.  Quads serve small B*H (four workgroups per memory
// fit the compute units); pairs the rest.
//
// Per chunk the algebra is that of the single-workgroup kernel (the unrolled momentum /
// forget-gated write rule of the Titans pages with gradients frozen at the chunk start,
// each gradient an outer product delta h^T).  What depends on the gates only (the
// coefficient vectors and Cm) comes from a pass over all chunks before the scan
// (pair_coef_kernel); the rest that does not depend on the hidden units (scaled Q / K
// copies, Cm o Q K^T, E2 layouts) is formed by every side; every sum over hidden units
// is computed per side:
//   O = Hk W2^T      every side needs the full O for E2 = 2 (O - V): each side posts its
//                    partial (64 x 64 fp32) and adds the other sides';
//   Y                each side writes y for its 64 / kS rows of the chunk's tokens and
//                    posts its partials of the other rows to their owners, which add them
//                    one chunk later (off the critical path).
// The sides' partials are added in side order ((O_0 + O_1) for pairs, (O_0 + O_1) +
// (O_2 + O_3) for quads; each side forms it as (own + side^1) + (side^2 + side^3), equal
// bit for bit since fp32 addition is commutative), so every side holds bitwise the same
// E2 and the result is reproducible.
//
// Exchange protocol.  The workgroups of a memory are blockIdx x + 8 s, s < kS (the
// dispatcher places them on one XCD).  Every word of the exchange area is written and
// read only with agent-scope relaxed atomics: per-instruction coherent loads and stores
// that meet beyond the per-XCD L2s, so no L2 writeback or invalidate is ever issued.
// Thread t of wave w writes its own words, the wave waits for its stores to complete
// (s_waitcnt vmcnt(0)), then lane 0 stores the wave's flag = exchange number e.  The
// other sides' waves w poll those flags (all in one bounded loop), then thread t reads
// exactly the words the other sides' threads t wrote.  Exchange e (one per chunk, plus
// one after the last) carries chunk e's O partial and chunk e-1's y partials.  O and Y
// areas are double-buffered by the parity of the chunk; a wave posts e + 1 only after its
// reads of exchange e have returned, which is what lets the writer reuse a buffer two
// exchanges later.  The launch is cooperative, so all workgroups of a memory are resident
// together.  A wait that exceeds its bound (never expected) stops all further waits of that
// wave, and from then on the wave sends NaN in place of its O and y partials and writes NaN
// y rows: the other sides' E2 turns NaN at the next exchange, so every side of the memory
// ends with NaN y rows and a NaN theta_T / s_T, never with finite values built from a
// missing partial.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "mfma_util.h"
#include "titans_internal.h"

namespace titans {
namespace {

using namespace fused;

constexpr int kD = 64;                   // key / value / query width
constexpr int kHid = 256;                // hidden width of the memory MLP
constexpr int kC = 64;                   // chunk length
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMat = kC * kLd;           // elements of one padded 64 x 64 matrix
constexpr int kMaxSpin = 1 << 21;        // flag polls before a wait gives up (about 2 s)

// A memory split over kS workgroups ("sides": 2 for pairs, 4 for quads).  Side s owns hidden
// units kHidSide s .. kHidSide (s + 1) - 1, a wave kHidW of them, and y rows kYRows s ..
// kYRows (s + 1) - 1 of every chunk.
//
// Exchange area of one memory (byte offsets): flags [side][wave] 128 bytes apart, then
// O words [slot 2][side][i 8][thread], then Y words [slot 2][source side][destination
// d][i][thread], destination side (source + 1 + d) mod kS; a word is two fp32 values.
template <int kS>
struct Split {
    static_assert(kS == 2 || kS == 4, "pairs or quads");
    static constexpr int kHidSide = kHid / kS;        // hidden units per workgroup
    static constexpr int kHidW = kHidSide / kWaves;   // hidden units per wave (32, 16)
    static constexpr int kHt = kHidW / 16;            // 16-wide hidden tiles per wave (2, 1)
    static constexpr int kLd2 = kHidSide + 8;         // padded row of the frozen W2 slice
    static constexpr int kYRows = kC / kS;            // y rows a side owns per chunk
    static constexpr int kYE = kYRows * kD / kThreads;  // y elements per thread and side
    static constexpr int kYW = kYE / 2;               // ... in exchange words
    static constexpr int64_t kFlagBytes = kS * kWaves * 128;
    static constexpr int64_t kOWords = 2 * kS * 8 * kThreads;
    static constexpr int64_t kYWords = 2 * kS * (kS - 1) * kYW * kThreads;
    static constexpr int64_t kBytes = kFlagBytes + 8 * (kOWords + kYWords);
    static_assert(kBytes % 256 == 0, "exchange areas stay 256-byte aligned");
};

// Sum of one value per side, own = this side's, p[d] = side (this side ^ (d + 1))'s:
// (own + p0) for pairs, (own + p0) + (p1 + p2) for quads.  fp32 addition is commutative, so
// every side gets bitwise (v0 + v1) resp. (v0 + v1) + (v2 + v3), side order.
template <int kS>
__device__ __forceinline__ float sum_sides(float own, const float (&p)[kS - 1]) {
    if constexpr (kS == 2)
        return own + p[0];
    else
        return (own + p[0]) + (p[1] + p[2]);
}

__device__ __forceinline__ uint64_t pack2(float a, float b) {
    return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
}
__device__ __forceinline__ float lo32(uint64_t u) { return __uint_as_float((uint32_t)u); }
__device__ __forceinline__ float hi32(uint64_t u) { return __uint_as_float((uint32_t)(u >> 32)); }
__device__ __forceinline__ void xstore(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t xload(uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// This wave's exchange stores are complete, then lane 0 publishes exchange number e.
__device__ __forceinline__ void post_flag(int* flag, int e, int lane) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if (lane == 0) __hip_atomic_store(flag, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wave-uniform bounded wait for the partner waves' flags (one per other side) to reach e:
// every poll loads all of them at once, so partners that post at different times cost one
// round trip per poll, not one per partner.  `bad` latches a timeout; a wave that has timed
// out does not wait again.
template <int N>
__device__ __forceinline__ void wait_flags(int* const (&flag)[N], int e, bool& bad, int max_spin) {
    if (bad) return;
    for (int s = 0; s < max_spin; ++s) {
        int v[N];
#pragma unroll
        for (int d = 0; d < N; ++d)
            v[d] = __hip_atomic_load(flag[d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int m = __builtin_amdgcn_readfirstlane(v[0]);
#pragma unroll
        for (int d = 1; d < N; ++d) m = min(m, __builtin_amdgcn_readfirstlane(v[d]));
        if (m >= e) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");  // no load moves above
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    bad = true;
}

struct __attribute__((aligned(16))) Smem {
    // Regions are reused within a chunk; the comment gives each region's lives in order.
    float r[2][kMat];          // O partials (pairwise reduction) -> Y partial slots 0, 1
                               //   ([c][dd] fp32)
    __bf16 qa[kMat];           // diag(a) Q [c][d]              } Y partial slot 2
    __bf16 qb[kMat];           // -diag(b) Q [c][d]             }
    __bf16 mq[kMat];           // -(Cm o Q K^T) [c][c']         } Y partial slot 3
    __bf16 e2l[kMat];          // E2 [c][dd]                    }
    __bf16 kk[kMat];           // K [c][d]
    __bf16 qq[kMat];           // Q [c][d]
    __bf16 e2t[kMat];          // E2^T [dd][c]
    __bf16 e2c[kMat];          // -(diag(c_C) E2)^T [dd][c]
    __bf16 e2w[kMat];          // (diag(w) E2)^T [dd][c]
    __bf16 cm[kMat];           // c_{t,j}, t, j < 64 (rows t)
    float a[kC], b[kC], cc[kC], w[kC];  // one chunk's coefficient vectors
    float tail[4];                       // a_C, b_C, p (right after w: one copy fills all)
    int fail;
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");

// Gradient chunks longer than the 64-token sub-chunk (C = 128, 192, 256): the gradients of
// every sub-chunk are taken at the weights of the chunk start, kept here in bf16 (the
// precision every product reads them in) and refreshed at each chunk start; the reads and
// the carry use the running weights in registers as for C = 64.
template <int kS>
struct __attribute__((aligned(16))) SmemFrozen : Smem {
    __bf16 w1c[Split<kS>::kHidSide * kLd];  // W1 at the chunk start [h][d], this side's rows
    __bf16 w2c[kD * Split<kS>::kLd2];       // W2 at the chunk start [dd][h], this side's columns
};
static_assert(sizeof(SmemFrozen<2>) <= 160 * 1024, "LDS budget");

// C = 64: the LDS the frozen copy would take holds two more O partial slots instead, so all
// four waves store their partials at once and the sum needs no second stage or barrier.
struct __attribute__((aligned(16))) SmemFour : Smem {
    float o2[2][kMat];  // O partials of waves 2, 3
};
static_assert(sizeof(SmemFour) <= 160 * 1024, "LDS budget");

// k operand over a wave's hidden units: its two 16-wide tiles, or its one tile and zeros.
template <int kHt>
__device__ __forceinline__ bf16x8 hcat(const bf16x4 (&x)[kHt][4], int i) {
    if constexpr (kHt == 2)
        return cat(x[0][i], x[1][i]);
    else
        return cat(x[0][i], bf16x4{});
}

// bf16 operand fragment from a k-contiguous fp32 LDS row (as frag(), rounding each element).
__device__ __forceinline__ bf16x8 frag32(const float* p, int off) {
    return cat(bf4(*reinterpret_cast<const f32x4*>(p + off)),
               bf4(*reinterpret_cast<const f32x4*>(p + off + 16)));
}

__device__ __forceinline__ float* yslot(Smem& sm, int w) {
    switch (w) {
        case 0: return sm.r[0];
        case 1: return sm.r[1];
        case 2: return reinterpret_cast<float*>(sm.qa);
        default: return reinterpret_cast<float*>(sm.mq);
    }
}

// ---------------------------------------------------------------- chunk coefficients
//
// Everything the scan needs from the gates alone, per (memory, chunk), computed for all
// chunks at once before the scan (they do not depend on the memory's state):
//   a_t = prod_{m<t} (1 - alpha_m), t = 0..C          (a_C: the chunk-end decay)
//   b_t: b_0 = 0, b_{t+1} = (1 - alpha_t) b_t + eta_t prod_{m<=t} beta_m
//   p = prod_m beta_m,  w_j = (1 - beta_j) prod_{j<m<C} beta_m
//   c_{t,j} = sum_{j<=i<t} L1[t][i] L2[i][j]          (strictly lower, t = 0..C)
//     L1[t][i] = prod_{i<m<t} (1 - alpha_m),  L2[i][j] = eta_i (1 - beta_j) prod_{j<m<=i} beta_m
// The carry's coefficients (the chunk-end row c_C and w) are scans of plain fp32 products
// (suffix scans: the lane order reversed by a lane permutation): S_j = sum_{i>=j} L1[C][i]
// eta_i prod_{j<m<=i} beta_m satisfies S_j = eta_j L1[C][j] + beta_{j+1} S_{j+1}, and
// c_C[j] = (1 - beta_j) S_j.  The in-chunk matrix Cm (the reads only) is one bf16 MFMA
// product of L1 and L2 entries, each exp2 of a difference of log2 prefix sums (positive
// factors only; a zero factor enters as log2 = -1024 and comes out as exactly zero).
// Tokens past the sequence end are padding: no decay, no write, momentum kept (alpha = eta
// = 0, beta = 1).
//
// Record of one chunk (bytes): Cm [t][j] bf16 64 x 64 | a[0..63] | b[0..63] | c_C[0..63] |
// w[0..63] (fp32) | a_C, b_C, p, 0.
constexpr int64_t kCoefCm = kC * kC * 2;
constexpr int64_t kCoefBytes = kCoefCm + 5 * kC * 4;
static_assert(kCoefBytes % 256 == 0, "records stay 256-byte aligned");

struct __attribute__((aligned(16))) CoefSmem {  // one wave's per-token vectors
    float la2i[kC];  // sum_{m<=t} log2(1 - alpha_m)
    float la2x[kC];  // sum_{m<t} log2(1 - alpha_m)
    float lb2[kC];   // sum_{m<=t} log2(beta_m)
    float et[kC];    // eta_t
    float omb[kC];   // 1 - beta_t
};

// L1 / L2 entries are formed directly in the MFMA operand layout: lane (g, j) holds, for
// reduction block kb, the eight entries with i = 32 kb + {4g .. 4g+3, 16+4g .. 16+4g+3}.
__device__ __forceinline__ bf16x8 l1_frag(const CoefSmem& cs, float la2t, int t, int kb, int g) {
    bf16x8 f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int i0 = 32 * kb + 16 * h + 4 * g;
        const f32x4 li = *reinterpret_cast<const f32x4*>(cs.la2i + i0);
#pragma unroll
        for (int v = 0; v < 4; ++v)  // out-of-triangle exponents may be +inf: discarded
            f[4 * h + v] = (__bf16)(i0 + v < t ? __builtin_amdgcn_exp2f(la2t - li[v]) : 0.f);
    }
    return f;
}
__device__ __forceinline__ bf16x8 l2_frag(const CoefSmem& cs, float lbj, float ombj, int jr, int kb,
                                          int g) {
    bf16x8 f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int i0 = 32 * kb + 16 * h + 4 * g;
        const f32x4 lb = *reinterpret_cast<const f32x4*>(cs.lb2 + i0);
        const f32x4 et = *reinterpret_cast<const f32x4*>(cs.et + i0);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            f[4 * h + v] =
                (__bf16)(i0 + v >= jr ? et[v] * __builtin_amdgcn_exp2f(lb[v] - lbj) * ombj : 0.f);
    }
    return f;
}

// Value of lane 63 - l (the wave's lane order reversed).
__device__ __forceinline__ float lane_rev(float x, int l) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((63 - l) << 2, __float_as_int(x)));
}

__global__ void __launch_bounds__(kThreads) pair_coef_kernel(ScanArgs A, char* coef, int64_t nchunks) {
    __shared__ CoefSmem csm[kWaves];
    const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    const int64_t task = (int64_t)blockIdx.x * kWaves + wv;  // one chunk per wave
    if (task >= A.B * A.H * nchunks) return;
    const int64_t seq = task / nchunks, n = task % nchunks;
    const int64_t bi = seq / A.H, hi = seq % A.H;
    CoefSmem& cs = csm[wv];
    char* rec = coef + task * kCoefBytes;
    float* rv = reinterpret_cast<float*>(rec + kCoefCm);

    const int64_t t = n * kC + l;
    float al = 0.f, et_l = 0.f, be_l = 1.f;
    if (t < A.T) {
        const int64_t go = bi * A.gs[0] + t * A.gs[1] + hi * A.gs[2];
        al = A.alpha[go];
        et_l = A.eta[go];
        be_l = A.beta[go];
    }
    const float keep = 1.f - al;
    const float pa = wave_scan_mul(keep);    // prod_{m<=l} (1 - alpha_m)
    const float pbl = wave_scan_mul(be_l);   // prod_{m<=l} beta_m
    const float lk = wave_scan_add(keep > 0.f ? __log2f(keep) : -1024.f);
    const float lb = wave_scan_add(be_l > 0.f ? __log2f(be_l) : -1024.f);
    float mk = keep, mc = et_l * pbl;        // affine maps x -> keep_t x + eta_t p_t, composed
    wave_scan_affine(mk, mc);
    // suffix products and the suffix affine scan, on the reversed lane order (lane
    // r = 63 - j holds token j): L1[C][j] = prod_{j<m<C} (1 - alpha_m), prod_{j<m<C} beta_m,
    // S_j = eta_j L1[C][j] + beta_{j+1} S_{j+1}
    const float keep_r = lane_rev(keep, l), be_r = lane_rev(be_l, l), et_r = lane_rev(et_l, l);
    const float l1c_r = lane_prev(wave_scan_mul(keep_r), 1.f);
    const float pw_r = lane_prev(wave_scan_mul(be_r), 1.f);
    float sk = lane_prev(be_r, 1.f), sc = et_r * l1c_r;
    wave_scan_affine(sk, sc);
    cs.la2i[l] = lk;
    cs.la2x[l] = lane_prev(lk, 0.f);
    cs.lb2[l] = lb;
    cs.et[l] = et_l;
    cs.omb[l] = 1.f - be_l;
    rv[l] = lane_prev(pa, 1.f);                       // a_l
    rv[kC + l] = lane_prev(mc, 0.f);                  // b_l
    rv[2 * kC + l] = (1.f - be_l) * lane_rev(sc, l);  // c_C[l]
    rv[3 * kC + l] = (1.f - be_l) * lane_rev(pw_r, l);  // w_l
    if (l == 63) {
        rv[4 * kC + 0] = pa;
        rv[4 * kC + 1] = mc;
        rv[4 * kC + 2] = pbl;
        rv[4 * kC + 3] = 0.f;
    }
    wave_lds_sync();
    // Cm^T[j][t] = sum_i L2^T[j][i] L1^T[i][t], tiles (j-block jt, t-block tb), jt <= tb
    bf16x8 l2f[4][2];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const int jr = 16 * jt + j;
        const float lbj = cs.lb2[jr], ombj = cs.omb[jr];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) l2f[jt][kb] = l2_frag(cs, lbj, ombj, jr, kb, g);
    }
    __bf16* cmg = reinterpret_cast<__bf16*>(rec);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int tr = 16 * tb + j;
        const float la2t = cs.la2x[tr];
        const bf16x8 b0 = l1_frag(cs, la2t, tr, 0, g), b1 = l1_frag(cs, la2t, tr, 1, g);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            f32x4 x = zero4();
            if (jt <= tb) {
                x = mfma(l2f[jt][0], b0, x);
                x = mfma(l2f[jt][1], b1, x);
            }
            *reinterpret_cast<bf16x4*>(cmg + tr * kC + 16 * jt + 4 * g) = bf4(x);
        }
    }
}

// Per-token surprise (kSurp): the norm of the gradient token t writes with, at the chunk-start
// weights.  For the 64 -> 256 -> 64 memory g_t = {E2_t Hk_t^T, D1_t k_t^T}, so
// ||g_t||^2 = ||E2_t||^2 ||Hk_t||^2 + ||D1_t||^2 ||k_t||^2.  Each lane's 16 per-token sums
// of squares (its hidden units) are first added over its quad of lanes by two DPP steps
// (register moves, no LDS round trip), then stored: 32 shares per token and quantity
// (2 sides x 4 waves x 4 quads); side 0 stores ||E2_t||^2; pair_surprise_kernel adds the
// shares with ||k_t||^2 after the scan.  Partials per (memory, token): Hk shares [32], D1
// shares [32], then ||E2||^2 apart.
constexpr int kSurpShares = 32;

template <int kCtrl>
__device__ __forceinline__ float dpp_quad(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xf, 0xf, true));
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]

// v[ct][r]: this lane's sums for tokens 16 ct + 4 g + r.  Returns in c[r] the sums over the
// lane's quad (j = 4 q .. 4 q + 3) for tokens 16 p + 4 g + r, p = j & 3: each step keeps the
// half of the entries whose ct bit matches the lane's and adds the partner's copy of it.
__device__ __forceinline__ void quad_reduce_scatter(const float (&v)[4][4], int j, float (&c)[4]) {
    const bool b0 = j & 1, b1 = j & 2;
    float h[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float send = b0 ? v[2 * k][r] : v[2 * k + 1][r];
            const float keep = b0 ? v[2 * k + 1][r] : v[2 * k][r];
            h[k][r] = keep + dpp_quad<kQuadXor1>(send);
        }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float send = b1 ? h[0][r] : h[1][r];
        const float keep = b1 ? h[1][r] : h[0][r];
        c[r] = keep + dpp_quad<kQuadXor2>(send);
    }
}

template <int kS, bool kFrozen, bool kSurp>
__global__ void __launch_bounds__(kThreads, 1) scan_pair_kernel(ScanArgs A) {
    static_assert(!kSurp || kS == 2, "the surprise shares are laid out for pairs");
    using SX = Split<kS>;
    constexpr int kHidSide = SX::kHidSide, kHidW = SX::kHidW, kHt = SX::kHt;
    constexpr int kYRows = SX::kYRows, kYE = SX::kYE, kYW = SX::kYW;
    __shared__ std::conditional_t<kFrozen, SmemFrozen<kS>, SmemFour> sm;
    const int kSub = A.C / kC;  // sub-chunks per gradient chunk
    const int tid = threadIdx.x;
    const int wv = tid >> 6, l = tid & 63, g = l >> 4, j = l & 15;
    // workgroups i + 8 s, s < kS (i % 8 = x, one XCD), serve memory 8 (i / (8 kS)) + x
    const int bid = blockIdx.x;
    const int side = (bid >> 3) % kS;
    const int64_t seq = 8 * (int64_t)(bid / (8 * kS)) + (bid & 7);
    if (seq >= A.B * A.H) return;  // all workgroups of a padding memory leave together
    const int64_t bi = seq / A.H, hi = seq % A.H;

    char* pbase = static_cast<char*>(A.ws) + seq * SX::kBytes;
    int* myflag = reinterpret_cast<int*>(pbase) + (side * kWaves + wv) * 32;
    // the other sides: other(d) = side ^ (d + 1), d < kS - 1
    auto other = [&](int d) { return side ^ (d + 1); };
    auto flag_of = [&](int s) { return reinterpret_cast<int*>(pbase) + (s * kWaves + wv) * 32; };
    int* pflag[kS - 1];  // the same wave's flag on every other side
#pragma unroll
    for (int d = 0; d < kS - 1; ++d) pflag[d] = flag_of(other(d));
    uint64_t* xo = reinterpret_cast<uint64_t*>(pbase + SX::kFlagBytes);
    uint64_t* xy = xo + SX::kOWords;
    auto oslot = [&](int e, int s) { return xo + ((e & 1) * kS + s) * 8 * kThreads + tid; };
    const int64_t nchunks = (A.T + kC - 1) / kC;
    const char* coef = static_cast<const char*>(A.ws) + ((A.B * A.H + 7) / 8 * 8) * SX::kBytes +
                       seq * nchunks * kCoefBytes;
    // the y words side `src` posts for side `dst` (dst != src)
    auto yxslot = [&](int e, int src, int dst) {
        const int d = (src ^ dst) - 1;
        return xy + (((e & 1) * kS + src) * (kS - 1) + d) * kYW * kThreads + tid;
    };
    float* const spart = kSurp ? reinterpret_cast<float*>(static_cast<char*>(A.ws) +
                                                         ((A.B * A.H + 7) / 8 * 8) * SX::kBytes +
                                                         A.B * A.H * nchunks * kCoefBytes)
                               : nullptr;
    float* const shk = kSurp ? spart + seq * A.T * 2 * kSurpShares : nullptr;   // [t][2][128]
    float* const se2 = kSurp ? spart + A.B * A.H * A.T * 2 * kSurpShares + seq * A.T : nullptr;
    const int share = side * 16 + wv * 4 + (j >> 2);  // this quad's share index
    bool bad = false;
    // test hook (debug bit 0): side 1 never posts, every wait gives up after 1024 polls
    const bool mute = (A.debug & 1) && side == 1;
    const int max_spin = (A.debug & 1) ? 1024 : kMaxSpin;

    const float* th0 = A.theta0 + bi * A.s0s[0] + hi * A.s0s[1];
    const float* mo0 = A.s0 + bi * A.s0s[0] + hi * A.s0s[1];
    float* thT = A.thetaT + bi * A.ss[0] + hi * A.ss[1];
    float* moT = A.sT + bi * A.ss[0] + hi * A.ss[1];
    constexpr int kOff2 = kHid * kD;  // W2 follows W1 (256 x 64) in a memory
    const int hb = kHidSide * side + kHidW * wv;  // this wave's first hidden unit

    // ---- state: W1T[dt][ht] = W1[h][d] (rows d = 16dt+4g+r, cols h = hb+16ht+j),
    //             W2T[ht][dt] = W2[dd][h] (rows h = hb+16ht+4g+r, cols dd = 16dt+j)
    f32x4 W1T[4][kHt], S1T[4][kHt], W2T[kHt][4], S2T[kHt][4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ht = 0; ht < kHt; ++ht) {
            const int h = hb + 16 * ht + j;
            const int d = 16 * dt + 4 * g;
            W1T[dt][ht] = *reinterpret_cast<const f32x4*>(th0 + h * kD + d);
            S1T[dt][ht] = *reinterpret_cast<const f32x4*>(mo0 + h * kD + d);
            const int h2 = hb + 16 * ht + 4 * g;
            const int dd = 16 * dt + j;
            W2T[ht][dt] = *reinterpret_cast<const f32x4*>(th0 + kOff2 + dd * kHid + h2);
            S2T[ht][dt] = *reinterpret_cast<const f32x4*>(mo0 + kOff2 + dd * kHid + h2);
        }
    if (tid == 0) sm.fail = 0;

    const __bf16* qg = static_cast<const __bf16*>(A.q);
    const __bf16* kg = static_cast<const __bf16*>(A.k);
    const __bf16* vg = static_cast<const __bf16*>(A.v);
    __bf16* yg = static_cast<__bf16*>(A.y);
    const int64_t qbase = bi * A.qs[0] + hi * A.qs[2];
    const int64_t ybase = bi * A.ys[0] + hi * A.ys[2];
    // this thread's slice of a chunk's 64 x 64 token tiles: row rc, columns cl0 .. cl0+15
    const int rc = tid >> 2, cl0 = 16 * (tid & 3);
    // this thread's y elements: row yr of each side's kYRows rows, columns yd0 .. yd0 + kYE - 1
    const int yr = tid / (kD / kYE), yd0 = kYE * (tid % (kD / kYE));
    const int yrow_own = kYRows * side + yr;
    float yown[kYE];

    // B = [I16; 0] and [0; I16] in the MFMA k order (lane (g, j) slot v < 4 is row 4g + v of
    // the block's first 16 rows, slot v >= 4 row 4g + v - 4 of its second 16)
    bf16x8 eye, eye1;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        eye[v] = (__bf16)((v < 4 && 4 * g + v == j) ? 1.f : 0.f);
        eye1[v] = (__bf16)((v >= 4 && 4 * g + v - 4 == j) ? 1.f : 0.f);
    }

    bf16x8 kpre[2], qpre[2], cpre[2];
    f32x4 vpre = zero4();
    auto prefetch = [&](int64_t t0) {
        // the chunk's coefficient record: Cm row rc, columns cl0 .. cl0+15; threads 0..64
        // also one 16-byte piece of a | b | c_C | w | (a_C, b_C, p)
        const char* rec = coef + (t0 / kC) * kCoefBytes;
        cpre[0] = *reinterpret_cast<const bf16x8*>(rec + 32 * tid);
        cpre[1] = *reinterpret_cast<const bf16x8*>(rec + 32 * tid + 16);
        if (tid <= kC) vpre = *reinterpret_cast<const f32x4*>(rec + kCoefCm + 16 * tid);
        const int64_t t = t0 + rc;
        if (t < A.T) {
            const int64_t o = qbase + t * A.qs[1] + cl0;
            kpre[0] = *reinterpret_cast<const bf16x8*>(kg + o);
            kpre[1] = *reinterpret_cast<const bf16x8*>(kg + o + 8);
            qpre[0] = *reinterpret_cast<const bf16x8*>(qg + o);
            qpre[1] = *reinterpret_cast<const bf16x8*>(qg + o + 8);
        } else {
            kpre[0] = kpre[1] = qpre[0] = qpre[1] = bf16x8{};
        }
    };
    // y for this side's rows of the chunk starting at token t0: the sum of every side's
    // partial in side order (px[d]: the words of side other(d))
    auto write_y = [&](int64_t t0, const uint64_t (&px)[kS - 1][kYW]) {
        const int64_t t = t0 + yrow_own;
        __bf16 out[kYE];
#pragma unroll
        for (int i = 0; i < kYW; ++i)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                float pv[kS - 1];
#pragma unroll
                for (int d = 0; d < kS - 1; ++d) pv[d] = h2 ? hi32(px[d][i]) : lo32(px[d][i]);
                out[2 * i + h2] = (__bf16)(bad ? __builtin_nanf("") : sum_sides<kS>(yown[2 * i + h2], pv));
            }
        if (t < A.T) {
            __bf16* dst = yg + ybase + t * A.ys[1] + yd0;
            if constexpr (kYE == 8)
                *reinterpret_cast<bf16x8*>(dst) = bf16x8{out[0], out[1], out[2], out[3], out[4], out[5], out[6], out[7]};
            else
                *reinterpret_cast<bf16x4*>(dst) = bf16x4{out[0], out[1], out[2], out[3]};
        }
    };
    // the prefetched chunk's Q and Cm into LDS (both dead once the Y partials are stored)
    auto commit_qc = [&]() {
        const int xb = opq(rc * kLd + cl0);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            *reinterpret_cast<bf16x4*>(sm.qq + xb + 4 * q4) = half4(qpre[q4 >> 1], q4 & 1);
            *reinterpret_cast<bf16x4*>(sm.cm + xb + 4 * q4) = half4(cpre[q4 >> 1], q4 & 1);
        }
    };
    // ... and its K and coefficient vectors (read by the carry: after the last barrier)
    auto commit_kv = [&]() {
        const int xb = opq(rc * kLd + cl0);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<bf16x4*>(sm.kk + xb + 4 * q4) = half4(kpre[q4 >> 1], q4 & 1);
        if (tid <= kC) *reinterpret_cast<f32x4*>(sm.a + 4 * tid) = vpre;  // a|b|cc|w|tail
    };
    // Chunk n+1's loads are issued early in chunk n (after B4) and land in LDS once chunk n
    // has stopped reading each region: Q and Cm after the Y partials are stored, K and the
    // coefficient vectors after the last barrier.
    prefetch(0);
    commit_qc();
    commit_kv();

    int e = 0;  // exchange number of the current sub-chunk (1, 2, ...)
    for (int64_t c0 = 0; c0 < A.T; c0 += kC) {
        ++e;
        if constexpr (kFrozen) {
            if ((e - 1) % kSub == 0) {
                // a gradient chunk starts: freeze this wave's W1 rows and W2 columns (each
                // wave reads back only its own slice; B1 orders the writes before the reads)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int ht = 0; ht < kHt; ++ht) {
                        *reinterpret_cast<bf16x4*>(sm.w1c + (kHidW * wv + 16 * ht + j) * kLd +
                                                   16 * dt + 4 * g) = bf4(W1T[dt][ht]);
                        *reinterpret_cast<bf16x4*>(sm.w2c + (16 * dt + j) * SX::kLd2 + kHidW * wv +
                                                   16 * ht + 4 * g) = bf4(W2T[ht][dt]);
                    }
            }
        }
        // ================= P0: load V
        bf16x8 vr[2];
        {
            const int64_t t = c0 + rc;
            if (t < A.T) {
                const int64_t o = qbase + t * A.qs[1] + cl0;
                vr[0] = *reinterpret_cast<const bf16x8*>(vg + o);
                vr[1] = *reinterpret_cast<const bf16x8*>(vg + o + 8);
            } else {
                vr[0] = vr[1] = bf16x8{};
            }
        }
        __syncthreads();  // B1

        // ================= P1: key forward and O partials
        // Z = K W1^T (rows c, cols h) for this wave's hidden units; Hk^T (rows h, cols c)
        // by an exact MFMA against the identity (D = A [I; 0] is the transpose of A's first
        // 16 x 16 tile when A is an accumulator tile in registers)
        bf16x4 Hk[4][kHt], Sp[4][kHt], HkT[kHt][4];
        float hsq[4][4] = {};  // kSurp: this wave's share of ||Hk_t||^2, t = 16 ct + 4 g + r
        {
            const int rb = opq(j * kLd + 4 * g);
            const __bf16* ks = sm.kk + rb;
#pragma unroll
            for (int ht = 0; ht < kHt; ++ht) {
                bf16x8 bw0, bw1;
                if constexpr (kFrozen) {
                    const __bf16* wr = sm.w1c + (kHidW * wv + 16 * ht + j) * kLd + 4 * g;
                    bw0 = frag(wr, 0);
                    bw1 = frag(wr, 32);
                } else {
                    bw0 = state_frag(W1T[0][ht], W1T[1][ht]);
                    bw1 = state_frag(W1T[2][ht], W1T[3][ht]);
                }
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    f32x4 z = mfma(frag(ks, fo(ct, 0)), bw0, zero4());
                    z = mfma(frag(ks, fo(ct, 1)), bw1, z);
                    f32x4 hk, sp;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float sg = sigmoid(z[r]);
                        const float hh = z[r] * sg;
                        hk[r] = hh;
                        sp[r] = sg + hh * (1.f - sg);  // SiLU'(z) = s (1 + z (1 - s))
                        if constexpr (kSurp) hsq[ct][r] += hh * hh;
                    }
                    Hk[ct][ht] = bf4(hk);
                    Sp[ct][ht] = bf4(sp);
                    HkT[ht][ct] = bf4(mfma(cat(Hk[ct][ht], bf16x4{}), eye, zero4()));
                }
            }
        }
        if constexpr (kSurp) {
            float cs[4];
            quad_reduce_scatter(hsq, j, cs);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = c0 + 16 * (j & 3) + 4 * g + r;
                if (t < A.T) shk[t * 2 * kSurpShares + share] = cs[r];
            }
        }
        // O^T partial over this wave's hidden units: O^T[dd][c] = sum_h W2[dd][h] Hk[c][h]
        f32x4 Ot[4][4];
        {
            const int rb = opq(j * kLd + 4 * g);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                // k = this wave's hidden units (16 of them: the upper k half is zero)
                bf16x8 a0;
                const __bf16* w2r = nullptr;
                if constexpr (kFrozen) w2r = sm.w2c + (16 * dt + j) * SX::kLd2 + kHidW * wv + 4 * g;
                if constexpr (kFrozen && kHt == 2)
                    a0 = frag(w2r, 0);
                else if constexpr (kFrozen)
                    a0 = cat(*reinterpret_cast<const bf16x4*>(w2r), bf16x4{});
                else if constexpr (kHt == 2)
                    a0 = state_frag(W2T[0][dt], W2T[1][dt]);
                else
                    a0 = state_frag(W2T[0][dt], zero4());
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) Ot[dt][ct] = mfma(a0, hcat(HkT, ct), zero4());
            }
            // deterministic reduction, fixed order (w0 + w2) + (w1 + w3):
            //   C = 64: every wave stores its partial in its own slot;
            //   longer chunks (less LDS): waves 2, 3 store, waves 0, 1 add theirs in P2
            if constexpr (!kFrozen) {
                float* slot = (wv < 2 ? sm.r[wv] : sm.o2[wv - 2]) + rb;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        *reinterpret_cast<f32x4*>(slot + 16 * ct * kLd + 16 * dt) = Ot[dt][ct];
            } else if (wv >= 2) {
                float* slot = sm.r[wv - 2] + rb;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        *reinterpret_cast<f32x4*>(slot + 16 * ct * kLd + 16 * dt) = Ot[dt][ct];
            }
        }
        if constexpr (!kFrozen) {
            // diag(a) Q and -diag(b) Q
            const float ar = sm.a[rc], br = -sm.b[rc];
            const int xb = opq(rc * kLd + cl0);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 qv = f4(*reinterpret_cast<const bf16x4*>(sm.qq + xb + 4 * q4));
                *reinterpret_cast<bf16x4*>(sm.qa + xb + 4 * q4) = bf4(qv * ar);
                *reinterpret_cast<bf16x4*>(sm.qb + xb + 4 * q4) = bf4(qv * br);
            }
        }
        __syncthreads();  // B2: O partials (C = 64: and the scaled Q copies)

        if constexpr (kFrozen) {
            // ================= P2: stage 2 of O; scaled Q copies
            if (wv < 2) {
                // all reads first, then all writes (the slot never aliases within itself; a
                // read-add-write per tile would wait out one LDS round trip per tile)
                float* slot = sm.r[wv] + opq(j * kLd + 4 * g);
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    f32x4 prev[2][4];
#pragma unroll
                    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
                        for (int ct = 0; ct < 4; ++ct)
                            prev[d2][ct] = *reinterpret_cast<const f32x4*>(
                                slot + 16 * ct * kLd + 16 * (2 * half + d2));
                    reload();
#pragma unroll
                    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
                        for (int ct = 0; ct < 4; ++ct)
                            *reinterpret_cast<f32x4*>(slot + 16 * ct * kLd + 16 * (2 * half + d2)) =
                                Ot[2 * half + d2][ct] + prev[d2][ct];
                }
            }
            // waves 2, 3 meanwhile: diag(a) Q and -diag(b) Q (thread u: row u / 2, 32 columns)
            if (wv >= 2) {
                const int u = tid & 127, row = u >> 1, c32 = 32 * (u & 1);
                const float ar = sm.a[row], br = -sm.b[row];
                const int xb = opq(row * kLd + c32);
#pragma unroll
                for (int q4 = 0; q4 < 8; ++q4) {
                    const f32x4 qv = f4(*reinterpret_cast<const bf16x4*>(sm.qq + xb + 4 * q4));
                    *reinterpret_cast<bf16x4*>(sm.qa + xb + 4 * q4) = bf4(qv * ar);
                    *reinterpret_cast<bf16x4*>(sm.qb + xb + 4 * q4) = bf4(qv * br);
                }
            }
            __syncthreads();  // B3: this side's O partial, diag(a) Q, -diag(b) Q
        }

        // ================= P2x: exchange O; Mq and the state terms of Zq meanwhile
        float oo[16];
        {
            const int xb = opq(rc * kLd + cl0);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 o;
                if constexpr (!kFrozen)
                    o = (*reinterpret_cast<const f32x4*>(sm.r[0] + xb + 4 * q4) +
                         *reinterpret_cast<const f32x4*>(sm.o2[0] + xb + 4 * q4)) +
                        (*reinterpret_cast<const f32x4*>(sm.r[1] + xb + 4 * q4) +
                         *reinterpret_cast<const f32x4*>(sm.o2[1] + xb + 4 * q4));
                else
                    o = *reinterpret_cast<const f32x4*>(sm.r[0] + xb + 4 * q4) +
                        *reinterpret_cast<const f32x4*>(sm.r[1] + xb + 4 * q4);
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) oo[4 * q4 + e4] = bad ? __builtin_nanf("") : o[e4];
            }
            // the O words go out now; the flag follows once they have landed (below)
            uint64_t* dst = oslot(e, side);
#pragma unroll
            for (int i = 0; i < 8; ++i) xstore(dst + i * kThreads, pack2(oo[2 * i], oo[2 * i + 1]));
        }
        {
            // Mq[c][c'] = -c_{c,c'} (Q K^T)[c][c'] for column tile c = 16 wv + j
            const int rb = opq(j * kLd + 4 * g);
            const __bf16* ks = sm.kk + rb;
            const __bf16* qr = sm.qq + rb + 16 * wv * kLd;
            const __bf16* cmr = sm.cm + rb + 16 * wv * kLd;
            __bf16* mqw = sm.mq + rb + 16 * wv * kLd;
#pragma unroll
            for (int ctp = 0; ctp < 4; ++ctp) {
                f32x4 x = zero4();
                if (ctp <= wv) {
                    x = mfma(frag(ks, fo(ctp, 0)), frag(qr, 0), x);
                    x = mfma(frag(ks, fo(ctp, 1)), frag(qr, 32), x);
                    const f32x4 cmv = f4(*reinterpret_cast<const bf16x4*>(cmr + 16 * ctp));
                    x = -(x * cmv);
                }
                *reinterpret_cast<bf16x4*>(mqw + 16 * ctp) = bf4(x);
            }
        }
        const float aC = sm.tail[0], bC = sm.tail[1], pC = sm.tail[2];  // chunk-end factors
        // Zq^T state terms (rows h, cols c): W1 (diag(a) Q)^T + S1 (-diag(b) Q)^T
        f32x4 zqp[kHt][4];
        {
            const int rb = opq(j * kLd + 4 * g);
            const __bf16* qar = sm.qa + rb;
            const __bf16* qbr = sm.qb + rb;
#pragma unroll
            for (int ht = 0; ht < kHt; ++ht) {
                const bf16x8 aw0 = state_frag(W1T[0][ht], W1T[1][ht]);
                const bf16x8 aw1 = state_frag(W1T[2][ht], W1T[3][ht]);
                const bf16x8 as0 = state_frag(S1T[0][ht], S1T[1][ht]);
                const bf16x8 as1 = state_frag(S1T[2][ht], S1T[3][ht]);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    f32x4 zq = mfma(aw0, frag(qar, fo(ct, 0)), zero4());
                    zq = mfma(aw1, frag(qar, fo(ct, 1)), zq);
                    zq = mfma(as0, frag(qbr, fo(ct, 0)), zq);
                    zqp[ht][ct] = mfma(as1, frag(qbr, fo(ct, 1)), zq);
                }
                // the O words went out before Mq: they have landed by now; the partner's
                // flag then travels while this wave finishes its state terms
                if (ht == 0 && !mute) post_flag(myflag, e, l);
            }
        }
        {
            // W1 and S1 are not read again before the carry: apply its rescale now
            // (a_C W1 - b_C S1, p S1; the carry's products add onto these)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int ht = 0; ht < kHt; ++ht) {
                    W1T[dt][ht] = aC * W1T[dt][ht] - bC * S1T[dt][ht];
                    S1T[dt][ht] = pC * S1T[dt][ht];
                }
        }
        wait_flags(pflag, e, bad, max_spin);
        {
            // the other sides' O partials of this chunk and their partials of this side's y
            // rows of the previous chunk, all loads issued together (one round trip)
            uint64_t po[kS - 1][8], px[kS - 1][kYW];
#pragma unroll
            for (int d = 0; d < kS - 1; ++d) {
                const uint64_t* src = oslot(e, other(d));
#pragma unroll
                for (int i = 0; i < 8; ++i) po[d][i] = xload(const_cast<uint64_t*>(src + i * kThreads));
            }
            if (e > 1) {
#pragma unroll
                for (int d = 0; d < kS - 1; ++d) {
                    const uint64_t* srcy = yxslot(e - 1, other(d), side);
#pragma unroll
                    for (int i = 0; i < kYW; ++i)
                        px[d][i] = xload(const_cast<uint64_t*>(srcy + i * kThreads));
                }
            }
            // E2 = loss'(O - V) (2 (O - V) for the squared error), O = the sides' partials
            // summed in side order (bitwise the same O on every side), in its four layouts
            const int xb = opq(rc * kLd + cl0), xt = opq(cl0 * kLd + rc);
            // gradient chunks longer than 64 tokens: E2's low part E2 - bf16(E2) (exact in
            // fp32) for the product G below, fp32 [c][dd] in O partial slot 0, which is dead
            // from the O sum to the Y partials; each thread writes exactly the elements it
            // read in the O sum, so the write needs no barrier before it
            float* const elw = sm.r[0] + xb;
            const float ccr = -sm.cc[rc], wr = sm.w[rc];
            float esq = 0.f;  // kSurp: this thread's 16 columns of ||E2_rc||^2
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 o;
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int k = 4 * q4 + e4;
                    float op[kS - 1];
#pragma unroll
                    for (int d = 0; d < kS - 1; ++d)
                        op[d] = (k & 1) ? hi32(po[d][k >> 1]) : lo32(po[d][k >> 1]);
                    o[e4] = sum_sides<kS>(oo[k], op);
                }
                const f32x4 v4 = f4(half4(vr[q4 >> 1], q4 & 1));
                const f32x4 e2 = bias_grad4(o - v4, A.bias, A.bias_param);
                if constexpr (kSurp) esq += (e2[0] * e2[0] + e2[1] * e2[1]) + (e2[2] * e2[2] + e2[3] * e2[3]);
                const bf16x4 el = bf4(e2), ec = bf4(e2 * ccr), ew = bf4(e2 * wr);
                *reinterpret_cast<bf16x4*>(sm.e2l + xb + 4 * q4) = el;
                if constexpr (kFrozen) *reinterpret_cast<f32x4*>(elw + 4 * q4) = e2 - f4(el);
#pragma unroll
                for (int ee = 0; ee < 4; ++ee) {
                    const int o2 = xt + (4 * q4 + ee) * kLd;
                    sm.e2t[o2] = el[ee];
                    sm.e2c[o2] = ec[ee];
                    sm.e2w[o2] = ew[ee];
                }
            }
            if constexpr (kSurp) {
                esq += __shfl_xor(esq, 1);
                esq += __shfl_xor(esq, 2);
                if (side == 0 && (tid & 3) == 0 && c0 + rc < A.T) se2[c0 + rc] = esq;
            }
            if (e > 1) write_y(c0 - kC, px);
        }
        __syncthreads();  // B4

        // ================= P4: backward, reads at the in-chunk weights
        // The next chunk's K, Q and coefficients load from here to the end of the chunk
        // (registers stay free through the phases above; about 4 us of cover).
        if (c0 + kC < A.T) prefetch(c0 + kC);
        // G = E2 W2 (rows c, cols h); D1 = G o SiLU'(Z).  The B operand W2 [dd][h] is the
        // transpose of the state tiles W2T [h][dd]: one exact identity MFMA per tile.
        bf16x4 D1[4][kHt];
        float dsq[4][4] = {};  // kSurp: this wave's share of ||D1_t||^2
        {
            bf16x4 W2n[4][kHt];  // rows dd = 16 dt + 4g + r, cols h = 16 ht + j
#pragma unroll
            for (int ht = 0; ht < kHt; ++ht)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    // lane (g, j): W2[16 dt + j][16 ht + 4g + v], v < 4, of the weights the
                    // gradient is taken at (operand A of the identity product)
                    bf16x4 tile;
                    if constexpr (kFrozen)
                        tile = *reinterpret_cast<const bf16x4*>(sm.w2c + (16 * dt + j) * SX::kLd2 +
                                                                 kHidW * wv + 16 * ht + 4 * g);
                    else
                        tile = bf4(W2T[ht][dt]);
                    W2n[dt][ht] = bf4(mfma(cat(tile, bf16x4{}), eye, zero4()));
                }
            // With gradient chunks longer than 64 tokens (the long-context configurations)
            // E2 enters as bf16 high + low parts, two products each: of the kernel's bf16
            // rounding points this is the one that moves long runs furthest from the exact
            // recurrence (emulated point by point over 256K tokens of a slowly forgetting
            // memory, C = 256: alone it moves single reads by up to 20 %, all the others
            // together by 3 %; at 2M tokens it takes y from 4.9e-3 to 3.1e-2 of the exact
            // result).  With C = 64 one product is kept (it costs 5 % there, and on the
            // 16K-token workload the split changes the error by nothing measurable).
            const int rb = opq(j * kLd + 4 * g);
            const __bf16* er = sm.e2l + rb;
            const float* erl = sm.r[0] + rb;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const bf16x8 a0 = frag(er, fo(ct, 0)), a1 = frag(er, fo(ct, 1));
                bf16x8 l0{}, l1{};
                if constexpr (kFrozen) {
                    l0 = frag32(erl, fo(ct, 0));
                    l1 = frag32(erl, fo(ct, 1));
                }
#pragma unroll
                for (int ht = 0; ht < kHt; ++ht) {
                    const bf16x8 b0 = cat(W2n[0][ht], W2n[1][ht]);
                    const bf16x8 b1 = cat(W2n[2][ht], W2n[3][ht]);
                    f32x4 gg = mfma(a0, b0, zero4());
                    if constexpr (kFrozen) {
                        f32x4 gl = mfma(l0, b0, zero4());
                        gg = mfma(a1, b1, gg);
                        gl = mfma(l1, b1, gl);
                        gg += gl;
                    } else {
                        gg = mfma(a1, b1, gg);
                    }
                    const f32x4 d1 = gg * f4(Sp[ct][ht]);
                    D1[ct][ht] = bf4(d1);
                    if constexpr (kSurp)
#pragma unroll
                        for (int r = 0; r < 4; ++r) dsq[ct][r] += d1[r] * d1[r];
                }
            }
        }
        if constexpr (kSurp) {
            float cs[4];
            quad_reduce_scatter(dsq, j, cs);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = c0 + 16 * (j & 3) + 4 * g + r;
                if (t < A.T) shk[t * 2 * kSurpShares + kSurpShares + share] = cs[r];
            }
        }
        // Zq^T += D1^T Mq^T; Hq = SiLU(Zq), also scaled by a_c and -b_c (its column c is
        // token c) for the W2 / S2 terms of Y
        bf16x4 Hq[kHt][4], Hqa[kHt][4], Hqb[kHt][4];
        {
            const int rb = opq(j * kLd + 4 * g);
            const __bf16* mqr = sm.mq + rb;
            float ac[4], nbc[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                ac[ct] = sm.a[16 * ct + j];
                nbc[ct] = -sm.b[16 * ct + j];
            }
#pragma unroll
            for (int ht = 0; ht < kHt; ++ht) {
                const bf16x8 ad0 = cat(D1[0][ht], D1[1][ht]);
                const bf16x8 ad1 = cat(D1[2][ht], D1[3][ht]);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    f32x4 zq = mfma(ad0, frag(mqr, fo(ct, 0)), zqp[ht][ct]);
                    if (ct >= 2) zq = mfma(ad1, frag(mqr, fo(ct, 1)), zq);
                    f32x4 hq;
#pragma unroll
                    for (int r = 0; r < 4; ++r) hq[r] = zq[r] * sigmoid(zq[r]);
                    Hq[ht][ct] = bf4(hq);
                    Hqa[ht][ct] = bf4(hq * ac[ct]);
                    Hqb[ht][ct] = bf4(hq * nbc[ct]);
                }
            }
        }
        __syncthreads();  // B5: Q, Mq and E2 [c][dd] are dead -> Y slots
        // Y^T (rows dd, cols c) = W2 (a_c Hq)^T + S2 (-b_c Hq)^T + E2^T Pm^T over this wave's
        // hidden units, Pm^T[c'][c] = -c_{c,c'} (Hk Hq^T)[c'][c]; each wave stores its
        // partial in its slot
        {
            const int rb = opq(j * kLd + 4 * g);
            bf16x4 pm[4][4];  // [ct][ctp]
            {
                const __bf16* cmr = sm.cm + rb;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const bf16x8 bq = hcat(Hq, ct);
#pragma unroll
                    for (int ctp = 0; ctp < 4; ++ctp) {
                        f32x4 pt = zero4();
                        if (ctp <= ct) {
                            pt = mfma(hcat(HkT, ctp), bq, pt);
                            const f32x4 cmv =
                                f4(*reinterpret_cast<const bf16x4*>(cmr + 16 * ct * kLd + 16 * ctp));
                            pt = -(pt * cmv);
                        }
                        pm[ct][ctp] = bf4(pt);
                    }
                }
            }
            float* slot = yslot(sm, wv) + rb;
            const __bf16* etr = sm.e2t + rb;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                bf16x8 aw, as;
                if constexpr (kHt == 2) {
                    aw = state_frag(W2T[0][dt], W2T[1][dt]);
                    as = state_frag(S2T[0][dt], S2T[1][dt]);
                } else {
                    aw = state_frag(W2T[0][dt], zero4());
                    as = state_frag(S2T[0][dt], zero4());
                }
                const bf16x8 e0 = frag(etr, fo(dt, 0));
                const bf16x8 e1 = frag(etr, fo(dt, 1));
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    f32x4 yt = mfma(aw, hcat(Hqa, ct), zero4());
                    yt = mfma(as, hcat(Hqb, ct), yt);
                    yt = mfma(e0, cat(pm[ct][0], pm[ct][1]), yt);
                    if (ct >= 2) yt = mfma(e1, cat(pm[ct][2], pm[ct][3]), yt);
                    *reinterpret_cast<f32x4*>(slot + 16 * ct * kLd + 16 * dt) = yt;
                }
            }
        }
        __syncthreads();  // B6: all Y partials stored

        // ================= P5: this side's Y; post the other sides' rows; carry
        {
            // hlf 0: this side's rows; hlf d + 1: side other(d)'s rows
            float ys[kS][kYE];
#pragma unroll
            for (int hlf = 0; hlf < kS; ++hlf) {
                const int e0 = (kYRows * (hlf == 0 ? side : other(hlf - 1)) + yr) * kLd + yd0;
#pragma unroll
                for (int q = 0; q < kYE / 4; ++q) {
                    const int e4 = e0 + 4 * q;
                    const f32x4 yv = (*reinterpret_cast<const f32x4*>(yslot(sm, 0) + e4) +
                                      *reinterpret_cast<const f32x4*>(yslot(sm, 1) + e4)) +
                                     (*reinterpret_cast<const f32x4*>(yslot(sm, 2) + e4) +
                                      *reinterpret_cast<const f32x4*>(yslot(sm, 3) + e4));
#pragma unroll
                    for (int k = 0; k < 4; ++k) ys[hlf][4 * q + k] = yv[k];
                }
            }
#pragma unroll
            for (int k = 0; k < kYE; ++k) yown[k] = ys[0][k];
#pragma unroll
            for (int d = 0; d < kS - 1; ++d) {
                uint64_t* dst = yxslot(e, side, other(d));
#pragma unroll
                for (int i = 0; i < kYW; ++i)
                    xstore(dst + i * kThreads, pack2(bad ? __builtin_nanf("") : ys[d + 1][2 * i],
                                                     bad ? __builtin_nanf("") : ys[d + 1][2 * i + 1]));
            }
        }
        if (c0 + kC < A.T) commit_qc();  // every wave is past B6: Q and Cm are no longer read
        {
            // The carry's K operands: A = (-c_C o K)^T and (w o K)^T, rows d, k = tokens c.
            // An identity MFMA on K's LDS rows gives K tiles in accumulator layout (lane
            // (g, j): K[16 ct + 4g + r][16 dt + j], exact); as operand A that is K^T, scaled
            // by c_C / w of its token per element.
            const int rb = opq(j * kLd + 4 * g);
            f32x4 ncc[4], wv4[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                ncc[ct] = -*reinterpret_cast<const f32x4*>(sm.cc + 16 * ct + 4 * g);
                wv4[ct] = *reinterpret_cast<const f32x4*>(sm.w + 16 * ct + 4 * g);
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                bf16x4 kc[4], kw[4];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const f32x4 kd = mfma(frag(sm.kk + rb, fo(ct, dt >> 1)), (dt & 1) ? eye1 : eye,
                                          zero4());
                    kc[ct] = bf4(kd * ncc[ct]);
                    kw[ct] = bf4(kd * wv4[ct]);
                }
                const bf16x8 kc0 = cat(kc[0], kc[1]), kc1 = cat(kc[2], kc[3]);
                const bf16x8 kw0 = cat(kw[0], kw[1]), kw1 = cat(kw[2], kw[3]);
                const bf16x8 ec0 = frag(sm.e2c + rb, fo(dt, 0));
                const bf16x8 ec1 = frag(sm.e2c + rb, fo(dt, 1));
                const bf16x8 ew0 = frag(sm.e2w + rb, fo(dt, 0));
                const bf16x8 ew1 = frag(sm.e2w + rb, fo(dt, 1));
#pragma unroll
                for (int ht = 0; ht < kHt; ++ht) {
                    const bf16x8 bd0 = cat(D1[0][ht], D1[1][ht]);  // B: D1 [c][h]
                    const bf16x8 bd1 = cat(D1[2][ht], D1[3][ht]);
                    const bf16x8 ah0 = cat(Hk[0][ht], Hk[1][ht]);  // A: Hk^T [h][c]
                    const bf16x8 ah1 = cat(Hk[2][ht], Hk[3][ht]);
                    // W1 and S1 were rescaled before the exchange wait; W2, S2 here
                    // (a_C W - b_C S, p S fused into the accumulator input)
                    W1T[dt][ht] = mfma(kc1, bd1, mfma(kc0, bd0, W1T[dt][ht]));
                    S1T[dt][ht] = mfma(kw1, bd1, mfma(kw0, bd0, S1T[dt][ht]));
                    const f32x4 tw2 = aC * W2T[ht][dt] - bC * S2T[ht][dt];
                    const f32x4 ts2 = pC * S2T[ht][dt];
                    W2T[ht][dt] = mfma(ah1, ec1, mfma(ah0, ec0, tw2));
                    S2T[ht][dt] = mfma(ah1, ew1, mfma(ah0, ew0, ts2));
                }
            }
        }
        __syncthreads();  // B7: the Y slots, K, Q, Cm and the vectors are no longer read
        if (c0 + kC < A.T) commit_kv();
    }

    // ---- y of the last chunk: one more exchange (no O words)
    {
        const int ef = e + 1;
        if (!mute) post_flag(myflag, ef, l);
        wait_flags(pflag, ef, bad, max_spin);
        uint64_t px[kS - 1][kYW];
#pragma unroll
        for (int d = 0; d < kS - 1; ++d) {
            const uint64_t* src = yxslot(e, other(d), side);
#pragma unroll
            for (int i = 0; i < kYW; ++i) px[d][i] = xload(const_cast<uint64_t*>(src + i * kThreads));
        }
        write_y((int64_t)(e - 1) * kC, px);
    }
    if (bad) sm.fail = 1;
    __syncthreads();
    const float nan = __builtin_nanf("");
    const bool failed = sm.fail != 0;

    // ---- final memory and momentum of this side's hidden units
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ht = 0; ht < kHt; ++ht) {
            const int h = hb + 16 * ht + j;
            const int d = 16 * dt + 4 * g;
            const f32x4 nn = {nan, nan, nan, nan};
            *reinterpret_cast<f32x4*>(thT + h * kD + d) = failed ? nn : W1T[dt][ht];
            *reinterpret_cast<f32x4*>(moT + h * kD + d) = failed ? nn : S1T[dt][ht];
            const int h2 = hb + 16 * ht + 4 * g;
            const int dd = 16 * dt + j;
            *reinterpret_cast<f32x4*>(thT + kOff2 + dd * kHid + h2) = failed ? nn : W2T[ht][dt];
            *reinterpret_cast<f32x4*>(moT + kOff2 + dd * kHid + h2) = failed ? nn : S2T[ht][dt];
        }
}

// Clears the flags of every memory's exchange area before a launch (exchange numbers
// restart at 1).
__global__ void clear_pair_flags(char* ws, int64_t nmem, int64_t area_bytes, int flag_bytes) {
    const int64_t m = blockIdx.x;
    if (m >= nmem) return;
    int* f = reinterpret_cast<int*>(ws + m * area_bytes);
    for (int i = threadIdx.x; i < flag_bytes / 4; i += blockDim.x) f[i] = 0;
}

// Workgroups per memory of a call (ScanArgs::sides, 2 unless the dispatcher chose 4).
int sides_of(const ScanArgs& a) { return a.sides == 4 ? 4 : 2; }
int64_t area_bytes(const ScanArgs& a) {
    return sides_of(a) == 4 ? Split<4>::kBytes : Split<2>::kBytes;
}
int64_t padded_pairs(const ScanArgs& a) { return (a.B * a.H + 7) / 8 * 8; }
int64_t num_chunks(const ScanArgs& a) { return (a.T + kC - 1) / kC; }

// ||g_t|| from the 32 shares of ||Hk_t||^2 and of ||D1_t||^2, ||E2_t||^2 and ||k_t||^2 read
// from k; 16 lanes per (memory, token): lane l adds four shares (l < 8: Hk, else D1) and
// four components of k, then the group sums by xor shuffles inside its 16 lanes.
__global__ void __launch_bounds__(256) pair_surprise_kernel(ScanArgs A, const float* part) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    if (i >= A.B * A.H * A.T) return;  // whole 16-lane groups leave together
    const int64_t seq = i / A.T, t = i % A.T, b = seq / A.H, h = seq % A.H;
    const f32x4 s4 = *reinterpret_cast<const f32x4*>(part + i * 2 * kSurpShares + 4 * l);
    float sh = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    const __bf16* kp = static_cast<const __bf16*>(A.k) + b * A.qs[0] + t * A.qs[1] + h * A.qs[2];
    const f32x4 k4 = f4(*reinterpret_cast<const bf16x4*>(kp + 4 * l));
    float ks = (k4[0] * k4[0] + k4[1] * k4[1]) + (k4[2] * k4[2] + k4[3] * k4[3]);
#pragma unroll
    for (int m = 4; m >= 1; m >>= 1) sh += __shfl_xor(sh, m);  // within each 8-lane half
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) ks += __shfl_xor(ks, m);
    const float d1 = __shfl_xor(sh, 8);  // lane 0: the D1 half's sum
    if (l == 0) {
        const float e2 = part[A.B * A.H * A.T * 2 * kSurpShares + i];
        A.surprise[b * A.gs[0] + t * A.gs[1] + h * A.gs[2]] = sqrtf(e2 * sh + d1 * ks);
    }
}

// Scratch of the allocation-free entry point (titans_mem_scan_noalloc): the pair path's
// exchange areas and chunk coefficient records in one static device array, which every
// GPU the library runs on holds from the library's first use on it until the process
// ends.  Host code reaches it only through the address hipGetSymbolAddress returns for the
// current device (the array's name is a host-side stand-in, not a device address).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

size_t scan_pair_scratch_capacity() { return kScratchBytes; }

hipError_t scan_pair_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        // once per device, with that device current: this GPU's copy of the array
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

size_t scan_pair_scratch_exchange_bytes(const ScanArgs& a) {
    return (size_t)padded_pairs(a) * (size_t)area_bytes(a);
}

size_t scan_pair_scratch_chunk_bytes(const ScanArgs& a) {
    return (size_t)(a.B * a.H) * (size_t)(a.C / kC) * (size_t)kCoefBytes;
}

size_t scan_pair_surprise_bytes(const ScanArgs& a) {
    return (size_t)(a.B * a.H) * (size_t)a.T * (2 * kSurpShares + 1) * sizeof(float);
}

bool scan_pair_supported(const ScanArgs& a) {
    return a.L == 2 && a.n[0] == kD && a.n[1] == kHid && a.n[2] == kD && a.C >= kC &&
           a.C % kC == 0 && a.io == TITANS_BF16;
}

size_t scan_pair_workspace_bytes(const ScanArgs& a) {
    return (size_t)padded_pairs(a) * (size_t)area_bytes(a) +
           (size_t)(a.B * a.H) * (size_t)num_chunks(a) * (size_t)kCoefBytes;
}

int64_t scan_pair_workgroups(const ScanArgs& a) { return sides_of(a) * padded_pairs(a); }

hipError_t launch_scan_pair(const ScanArgs& a, hipStream_t stream) {
    const int64_t nmem = padded_pairs(a);
    if (nmem == 0) return hipSuccess;
    const int S = sides_of(a);
    const bool surp = a.surprise != nullptr;
    if (surp && S != 2) return hipErrorInvalidValue;  // surprise shares: pairs only
    char* ws = static_cast<char*>(a.ws);
    const int64_t area = area_bytes(a);
    clear_pair_flags<<<dim3((unsigned)nmem), 256, 0, stream>>>(
        ws, nmem, area, (int)(S == 4 ? Split<4>::kFlagBytes : Split<2>::kFlagBytes));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nchunks = num_chunks(a);
    const int64_t ntasks = a.B * a.H * nchunks;
    if (ntasks > 0) {
        const int64_t blocks = (ntasks + kWaves - 1) / kWaves;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        pair_coef_kernel<<<dim3((unsigned)blocks), kThreads, 0, stream>>>(a, ws + nmem * area,
                                                                         nchunks);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    ScanArgs args = a;
    void* kargs[] = {&args};
    const bool frozen = a.C != kC;
    const void* fn;
    if (S == 4)
        fn = frozen ? reinterpret_cast<const void*>(&scan_pair_kernel<4, true, false>)
                    : reinterpret_cast<const void*>(&scan_pair_kernel<4, false, false>);
    else if (frozen)
        fn = surp ? reinterpret_cast<const void*>(&scan_pair_kernel<2, true, true>)
                  : reinterpret_cast<const void*>(&scan_pair_kernel<2, true, false>);
    else
        fn = surp ? reinterpret_cast<const void*>(&scan_pair_kernel<2, false, true>)
                  : reinterpret_cast<const void*>(&scan_pair_kernel<2, false, false>);
    e = hipLaunchCooperativeKernel(fn, dim3((unsigned)(S * nmem)), dim3(kThreads), kargs, 0,
                                   stream);
    if (e != hipSuccess || !surp) return e;
    const float* part = reinterpret_cast<const float*>(ws + nmem * area +
                                                       a.B * a.H * nchunks * kCoefBytes);
    const int64_t n = a.B * a.H * a.T;
    if ((n + 15) / 16 > 0xffffffffLL) return hipErrorInvalidConfiguration;
    pair_surprise_kernel<<<dim3((unsigned)((n + 15) / 16)), 256, 0, stream>>>(a, part);
    return hipGetLastError();
}

}  // namespace titans
