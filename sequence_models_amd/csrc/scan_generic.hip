// Generic chunked Titans memory scan and retrieve for gfx950.  With fp32 I/O every
// product is fp32 FMAs; with bf16 I/O the products are bf16 MFMA with fp32 accumulation
// (operands rounded to bf16 as they are staged; state and intermediates stay fp32).
//
// This path serves every supported shape (any L <= 4, widths <= 512, C <= 256,
// fp32 or bf16 I/O).  One 256-thread workgroup owns one (b, h) memory; theta
// and s live in the theta_T / s_T output buffers (L2-resident) and each
// chunk's intermediates live in the caller's workspace.
//
// Per chunk of n <= C tokens (chunk-start weights W_l, momentum S_l), the
// write rule of the Titans pages (momentum s_t = beta_t s_{t-1} + (1-beta_t) g_t,
// write theta_{t+1} = (1-alpha_t) theta_t - eta_t s_t, gradients g_j at the
// chunk-start weights: the summary page's "tensorized mini-batch" form)
// unrolls to
//   theta_t = a_t theta_c - b_t s_in - sum_{j<t} c_{t,j} g_j,
//   s_n     = p s_in + sum_j w_j g_j,
// with a, b, c, p, w products of the chunk's gates (the "associative scan for
// the momentum" of the same page, computed here by a column recurrence: one
// thread per column j, one step per token).  Each g_j is a sum of outer
// products delta_l h_{l-1}^T, so reading token t at its in-chunk weights is
//   U_l = diag(a) Hq W_l^T - diag(b) Hq S_l^T - (Cm o Hq Hk^T) Delta_l
// (rows = tokens; Cm strictly lower triangular), and the chunk-end carry is
//   W_l <- a_n W_l - b_n S_l - Delta_l^T diag(c_n) Hk_{l-1},
//   S_l <- p S_l + Delta_l^T diag(w) Hk_{l-1}.
#include <hip/hip_runtime.h>

#include "generic_util.h"
#include "titans_internal.h"

namespace titans {
namespace {

using namespace generic;

constexpr int kThreads = 256;
constexpr int kTile = 64;   // output tile edge
constexpr int kKStep = 16;  // reduction step
constexpr int kPad = 4;
constexpr int kGemmLdsF32 = 2 * kKStep * (kTile + kPad);  // floats
constexpr int kMK = 32;                                     // MFMA reduction step
constexpr int kMLd = kMK + 8;                               // padded bf16 row of a staged tile
constexpr int kGemmLdsMfma = 2 * kTile * kMLd / 2;          // floats (two bf16 tiles)
constexpr int kGemmLds = kGemmLdsF32 > kGemmLdsMfma ? kGemmLdsF32 : kGemmLdsMfma;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// A(i, k) = p[i*si + k*sk] * (kscale ? kscale[k] : 1)
struct MatA {
    const float* p;
    int64_t si, sk;
    const float* kscale;
};
// B(k, j) = p[k*sk + j*sj]
struct MatB {
    const float* p;
    int64_t sk, sj;
};

// Workgroup GEMM: for every (i < M, j < N) call epi(i, j, sum_k A(i,k) B(k,j)).
// Each output element is owned by exactly one thread.
template <class Epi>
__device__ void block_gemm(int M, int N, int K, MatA A, MatB B, float* lds, Epi epi) {
    float* As = lds;                          // [kKStep][kTile + kPad]
    float* Bs = lds + kKStep * (kTile + kPad);
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    for (int i0 = 0; i0 < M; i0 += kTile) {
        for (int j0 = 0; j0 < N; j0 += kTile) {
            float acc[4][4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;
            for (int k0 = 0; k0 < K; k0 += kKStep) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int e = tid + kThreads * r;
                    int ii, kk;
                    if (A.sk == 1) { kk = e & 15; ii = e >> 4; } else { ii = e & 63; kk = e >> 6; }
                    int gi = i0 + ii, gk = k0 + kk;
                    float val = 0.0f;
                    if (gi < M && gk < K) {
                        val = A.p[gi * A.si + gk * A.sk];
                        if (A.kscale) val *= A.kscale[gk];
                    }
                    As[kk * (kTile + kPad) + ii] = val;
                    int jj;
                    if (B.sj == 1) { jj = e & 63; kk = e >> 6; } else { kk = e & 15; jj = e >> 4; }
                    int gj = j0 + jj;
                    gk = k0 + kk;
                    Bs[kk * (kTile + kPad) + jj] = (gj < N && gk < K) ? B.p[gk * B.sk + gj * B.sj] : 0.0f;
                }
                __syncthreads();
#pragma unroll
                for (int kk = 0; kk < kKStep; ++kk) {
                    float av[4], bv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) av[r] = As[kk * (kTile + kPad) + ty + 16 * r];
#pragma unroll
                    for (int c = 0; c < 4; ++c) bv[c] = Bs[kk * (kTile + kPad) + tx + 16 * c];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(av[r], bv[c], acc[r][c]);
                }
                __syncthreads();
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    int i = i0 + ty + 16 * r, j = j0 + tx + 16 * c;
                    if (i < M && j < N) epi(i, j, acc[r][c]);
                }
        }
    }
    __syncthreads();
}

// The same workgroup GEMM on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
// Per 64 x 64 output tile and 32-wide reduction step, A (64 x 32) and B (32 x 64) are staged
// in LDS as bf16 with the reduction index contiguous ([row i][k], [column j][k]); wave w
// computes output rows 16w .. 16w+15 against the four 16-column tiles.  Operand layouts of
// the MFMA: lane l (g = l / 16, j = l % 16) holds A[j][k] and B[k][j] for k in
// {4g .. 4g+3, 16+4g .. 16+4g+3} and D[4g + r][j], r = 0..3.
template <class Epi>
__device__ void block_gemm_mfma(int M, int N, int K, MatA A, MatB B, float* lds, Epi epi) {
    __bf16* As = reinterpret_cast<__bf16*>(lds);  // [64][kMLd]
    __bf16* Bs = As + kTile * kMLd;                // [64][kMLd]
    const int tid = threadIdx.x;
    const int wv = tid >> 6, g = (tid & 63) >> 4, j = tid & 15;
    for (int i0 = 0; i0 < M; i0 += kTile) {
        for (int j0 = 0; j0 < N; j0 += kTile) {
            f32x4_t acc[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < K; k0 += kMK) {
                // stage: each thread moves two groups of four elements of A and of B
#pragma unroll
                for (int rep = 0; rep < 2; ++rep) {
                    const int e = tid + kThreads * rep;  // 0 .. 511
                    if (A.sk == 1) {                     // four consecutive k of one row
                        const int ii = e >> 3, kq = (e & 7) * 4, gi = i0 + ii;
                        bf16x4_t v;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int gk = k0 + kq + u;
                            float x = 0.f;
                            if (gi < M && gk < K) {
                                x = A.p[gi * A.si + gk];
                                if (A.kscale) x *= A.kscale[gk];
                            }
                            v[u] = (__bf16)x;
                        }
                        *reinterpret_cast<bf16x4_t*>(As + ii * kMLd + kq) = v;
                    } else {                             // four consecutive rows of one k
                        const int kk = e >> 4, iq = (e & 15) * 4, gk = k0 + kk;
                        const float sc = (A.kscale && gk < K) ? A.kscale[gk] : 1.f;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int gi = i0 + iq + u;
                            const float x = (gi < M && gk < K) ? A.p[gi * A.si + gk * A.sk] * sc : 0.f;
                            As[(iq + u) * kMLd + kk] = (__bf16)x;
                        }
                    }
                    if (B.sk == 1) {                     // four consecutive k of one column
                        const int jj = e >> 3, kq = (e & 7) * 4, gj = j0 + jj;
                        bf16x4_t v;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int gk = k0 + kq + u;
                            v[u] = (__bf16)((gj < N && gk < K) ? B.p[gk + gj * B.sj] : 0.f);
                        }
                        *reinterpret_cast<bf16x4_t*>(Bs + jj * kMLd + kq) = v;
                    } else {                             // four consecutive columns of one k
                        const int kk = e >> 4, jq = (e & 15) * 4, gk = k0 + kk;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int gj = j0 + jq + u;
                            const float x = (gj < N && gk < K) ? B.p[gk * B.sk + gj * B.sj] : 0.f;
                            Bs[(jq + u) * kMLd + kk] = (__bf16)x;
                        }
                    }
                }
                __syncthreads();
                const __bf16* ar = As + (16 * wv + j) * kMLd + 4 * g;
                const bf16x8_t af = __builtin_shufflevector(*reinterpret_cast<const bf16x4_t*>(ar),
                                                            *reinterpret_cast<const bf16x4_t*>(ar + 16),
                                                            0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) {
                    const __bf16* br = Bs + (16 * tn + j) * kMLd + 4 * g;
                    const bf16x8_t bf = __builtin_shufflevector(
                        *reinterpret_cast<const bf16x4_t*>(br), *reinterpret_cast<const bf16x4_t*>(br + 16),
                        0, 1, 2, 3, 4, 5, 6, 7);
                    acc[tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[tn], 0, 0, 0);
                }
                __syncthreads();
            }
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = i0 + 16 * wv + 4 * g + r, jc = j0 + 16 * tn + j;
                    if (i < M && jc < N) epi(i, jc, acc[tn][r]);
                }
        }
    }
    __syncthreads();
}

template <bool kMfma, class Epi>
__device__ __forceinline__ void gemm(int M, int N, int K, MatA A, MatB B, float* lds, Epi epi) {
    if constexpr (kMfma)
        block_gemm_mfma(M, N, K, A, B, lds, epi);
    else
        block_gemm(M, N, K, A, B, lds, epi);
}

__device__ __forceinline__ int64_t round64(int64_t x) { return (x + 63) & ~int64_t(63); }

// Float offsets of the per-sequence workspace regions.
struct WsLayout {
    int64_t coef;           // a[C+1], b[C+1], w[C], p
    int64_t cm;             // (C+1) x C
    int64_t hk[TITANS_MAX_LAYERS];      // l = 0..L-1: C x n_l
    int64_t sp[TITANS_MAX_LAYERS];      // l = 1..L-1: C x n_l (SiLU'(Z_l))
    int64_t dl[TITANS_MAX_LAYERS + 1];  // l = 1..L:   C x n_l
    int64_t hq[2];          // ping-pong C x maxw
    int64_t mq;             // C x C
    int64_t per_seq;
};

__host__ __device__ inline WsLayout ws_layout(int C, int L, const int* n) {
    auto r64 = [](int64_t x) { return (x + 63) & ~int64_t(63); };
    WsLayout w{};
    int maxw = 0;
    for (int l = 0; l <= L; ++l) maxw = n[l] > maxw ? n[l] : maxw;
    int64_t o = 0;
    w.coef = o; o += r64(3 * (int64_t)C + 3);
    w.cm = o; o += r64((int64_t)(C + 1) * C);
    for (int l = 0; l < L; ++l) { w.hk[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l < L; ++l) { w.sp[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l <= L; ++l) { w.dl[l] = o; o += r64((int64_t)C * n[l]); }
    w.hq[0] = o; o += r64((int64_t)C * maxw);
    w.hq[1] = o; o += r64((int64_t)C * maxw);
    w.mq = o; o += r64((int64_t)C * C);
    w.per_seq = o;
    return w;
}

// The layout comes in the argument block: it is indexed by layer at run time.
template <bool kMfma>
__global__ void __launch_bounds__(kThreads) scan_generic_kernel(ScanArgs a, WsLayout wl) {
    __shared__ float lds_gemm[kGemmLds];
    __shared__ float s_al[256], s_et[256], s_be[256];

    const int64_t seq = blockIdx.x;
    const int64_t b = seq / a.H, h = seq % a.H;
    const int tid = threadIdx.x;
    const int L = a.L, C = a.C;
    const int64_t P = a.P;
    const int d = a.n[0];

    float* ws = static_cast<float*>(a.ws) + seq * wl.per_seq;
    float* coef_a = ws + wl.coef;
    float* coef_b = coef_a + (C + 1);
    float* coef_w = coef_b + (C + 1);
    float* coef_p = coef_w + C;
    float* Cm = ws + wl.cm;

    float* theta = a.thetaT + b * a.ss[0] + h * a.ss[1];
    float* mom = a.sT + b * a.ss[0] + h * a.ss[1];
    const float* theta0 = a.theta0 + b * a.s0s[0] + h * a.s0s[1];
    const float* mom0 = a.s0 + b * a.s0s[0] + h * a.s0s[1];
    if (theta != theta0)
        for (int64_t i = tid; i < P; i += kThreads) theta[i] = theta0[i];
    if (mom != mom0)
        for (int64_t i = tid; i < P; i += kThreads) mom[i] = mom0[i];
    __syncthreads();

    const int64_t qbase = b * a.qs[0] + h * a.qs[2];
    const int64_t ybase = b * a.ys[0] + h * a.ys[2];
    const int64_t gbase = b * a.gs[0] + h * a.gs[2];

    for (int64_t c0 = 0; c0 < a.T; c0 += C) {
        const int n = (int)((a.T - c0) < C ? (a.T - c0) : C);
        // ---- stage gates, K (as Hk_0) and Q (as Hq_0) in fp32
        for (int t = tid; t < n; t += kThreads) {
            int64_t gi = gbase + (c0 + t) * a.gs[1];
            s_al[t] = a.alpha[gi];
            s_et[t] = a.eta[gi];
            s_be[t] = a.beta[gi];
        }
        float* Hk0 = ws + wl.hk[0];
        float* Hq0 = ws + wl.hq[0];
        for (int e = tid; e < n * d; e += kThreads) {
            int t = e / d, c = e % d;
            int64_t src = qbase + (c0 + t) * a.qs[1] + c;
            Hk0[t * d + c] = load_io(a.k, src, a.io);
            Hq0[t * d + c] = load_io(a.q, src, a.io);
        }
        __syncthreads();

        // ---- gate coefficients: thread j owns column j of Cm
        {
            const int j = tid;
            float Bj = 0.0f, cj = 0.0f, at = 1.0f, bt = 0.0f, pb = 1.0f;
            const float omb_j = (j < n) ? 1.0f - s_be[j] : 0.0f;
            if (j < n) Cm[j] = 0.0f;  // row 0
            if (j == 0) { coef_a[0] = 1.0f; coef_b[0] = 0.0f; }
            for (int t = 0; t < n; ++t) {
                const float al = s_al[t], et = s_et[t], be = s_be[t];
                pb *= be;
                if (j < t) Bj *= be;
                else if (j == t) Bj = 1.0f;
                const float keep = 1.0f - al;
                at *= keep;
                bt = keep * bt + et * pb;
                cj = keep * cj + ((j <= t) ? et * omb_j * Bj : 0.0f);
                if (j < n) Cm[(int64_t)(t + 1) * C + j] = cj;
                if (j == 0) { coef_a[t + 1] = at; coef_b[t + 1] = bt; }
            }
            if (j < n) coef_w[j] = omb_j * Bj;
            if (j == 0) coef_p[0] = pb;
        }
        __syncthreads();

        // ---- key path forward at the chunk-start weights
        for (int l = 1; l <= L; ++l) {
            const float* Hin = ws + wl.hk[l - 1];
            const float* W = theta + a.off[l];
            const int nin = a.n[l - 1], nout = a.n[l];
            MatA A{Hin, nin, 1, nullptr};
            MatB Bm{W, 1, nin};  // B(k, j) = W[j][k]
            if (l < L) {
                float* Hout = ws + wl.hk[l];
                float* Sp = ws + wl.sp[l];
                gemm<kMfma>(n, nout, nin, A, Bm, lds_gemm, [&](int i, int jj, float z) {
                    float sg = sigmoidf_(z);
                    Hout[i * nout + jj] = z * sg;
                    Sp[i * nout + jj] = sg * (1.0f + z * (1.0f - sg));
                });
            } else {
                float* D = ws + wl.dl[L];
                gemm<kMfma>(n, nout, nin, A, Bm, lds_gemm, [&](int i, int jj, float z) {
                    float vv = load_io(a.v, qbase + (c0 + i) * a.qs[1] + jj, a.io);
                    D[i * nout + jj] = bias_grad(z - vv, a.bias, a.bias_param);
                });
            }
        }
        // ---- backward: Delta_{l-1} = (Delta_l W_l) o SiLU'(Z_{l-1})
        for (int l = L; l >= 2; --l) {
            const int nin = a.n[l - 1], nout = a.n[l];
            const float* W = theta + a.off[l];
            const float* Dl = ws + wl.dl[l];
            float* Dp = ws + wl.dl[l - 1];
            const float* Sp = ws + wl.sp[l - 1];
            gemm<kMfma>(n, nin, nout, MatA{Dl, nout, 1, nullptr}, MatB{W, nin, 1}, lds_gemm,
                       [&](int i, int jj, float g) { Dp[i * nin + jj] = g * Sp[i * nin + jj]; });
        }
        // ---- optional: each token's gradient norm; the gradient of layer l is the outer
        // product Delta_l Hk_{l-1}^T, so its squared norm is |Delta_l|^2 |Hk_{l-1}|^2
        if (a.surprise) {
            for (int t = tid; t < n; t += kThreads) {
                float acc = 0.0f;
                // the Delta_l and Hk_l regions are consecutive: walk them by pointer
                const float* Db = ws + wl.dl[1];
                const float* Hb = ws + wl.hk[0];
                for (int l = 1; l <= L; ++l) {
                    const float* Dr = Db + (int64_t)t * a.n[l];
                    const float* Hr = Hb + (int64_t)t * a.n[l - 1];
                    float dd = 0.0f, hh = 0.0f;
                    for (int i = 0; i < a.n[l]; ++i) dd = fmaf(Dr[i], Dr[i], dd);
                    for (int i = 0; i < a.n[l - 1]; ++i) hh = fmaf(Hr[i], Hr[i], hh);
                    acc = fmaf(dd, hh, acc);
                    Db += round64((int64_t)C * a.n[l]);
                    Hb += round64((int64_t)C * a.n[l - 1]);
                }
                a.surprise[gbase + (c0 + t) * a.gs[1]] = sqrtf(acc);
            }
        }
        // ---- retrieval at the in-chunk weights, layer by layer
        int cur = 0;
        for (int l = 1; l <= L; ++l) {
            const int nin = a.n[l - 1], nout = a.n[l];
            const float* Hq = ws + wl.hq[cur];
            float* U = ws + wl.hq[cur ^ 1];
            const float* Hk = ws + wl.hk[l - 1];
            const float* W = theta + a.off[l];
            const float* S = mom + a.off[l];
            const float* Dl = ws + wl.dl[l];
            float* Mq = ws + wl.mq;
            // Mq = Cm o (Hq Hk^T), strictly lower triangular
            gemm<kMfma>(n, n, nin, MatA{Hq, nin, 1, nullptr}, MatB{Hk, 1, nin}, lds_gemm,
                       [&](int i, int jj, float x) {
                           Mq[i * C + jj] = (jj < i) ? Cm[(int64_t)i * C + jj] * x : 0.0f;
                       });
            gemm<kMfma>(n, nout, nin, MatA{Hq, nin, 1, nullptr}, MatB{W, 1, nin}, lds_gemm,
                       [&](int i, int jj, float x) { U[i * nout + jj] = coef_a[i] * x; });
            gemm<kMfma>(n, nout, nin, MatA{Hq, nin, 1, nullptr}, MatB{S, 1, nin}, lds_gemm,
                       [&](int i, int jj, float x) { U[i * nout + jj] -= coef_b[i] * x; });
            if (l < L) {
                gemm<kMfma>(n, nout, n, MatA{Mq, C, 1, nullptr}, MatB{Dl, nout, 1}, lds_gemm,
                           [&](int i, int jj, float x) {
                               float u = U[i * nout + jj] - x;
                               U[i * nout + jj] = u * sigmoidf_(u);
                           });
            } else {
                gemm<kMfma>(n, nout, n, MatA{Mq, C, 1, nullptr}, MatB{Dl, nout, 1}, lds_gemm,
                           [&](int i, int jj, float x) {
                               store_io(a.y, ybase + (c0 + i) * a.ys[1] + jj, a.io,
                                        U[i * nout + jj] - x);
                           });
            }
            cur ^= 1;
        }
        // ---- carry to the next chunk (W first: it needs the chunk-start S)
        const float an = coef_a[n], bn = coef_b[n], pn = coef_p[0];
        const float* crow = Cm + (int64_t)n * C;
        for (int l = 1; l <= L; ++l) {
            const int nin = a.n[l - 1], nout = a.n[l];
            float* W = theta + a.off[l];
            float* S = mom + a.off[l];
            const float* Dl = ws + wl.dl[l];
            const float* Hk = ws + wl.hk[l - 1];
            gemm<kMfma>(nout, nin, n, MatA{Dl, 1, nout, crow}, MatB{Hk, nin, 1}, lds_gemm,
                       [&](int i, int jj, float x) {
                           int64_t o = (int64_t)i * nin + jj;
                           W[o] = an * W[o] - bn * S[o] - x;
                       });
            gemm<kMfma>(nout, nin, n, MatA{Dl, 1, nout, coef_w}, MatB{Hk, nin, 1}, lds_gemm,
                       [&](int i, int jj, float x) {
                           int64_t o = (int64_t)i * nin + jj;
                           S[o] = pn * S[o] + x;
                       });
        }
    }
}

constexpr int kRetrieveTokens = 16;

template <bool kMfma>
__global__ void __launch_bounds__(kThreads) retrieve_generic_kernel(ScanArgs a) {
    extern __shared__ float smem[];
    const int64_t seq = blockIdx.y;
    const int64_t b = seq / a.H, h = seq % a.H;
    const int64_t t0 = (int64_t)blockIdx.x * kRetrieveTokens;
    const int n = (int)((a.T - t0) < kRetrieveTokens ? (a.T - t0) : kRetrieveTokens);
    int maxw = 0;
    for (int l = 0; l <= a.L; ++l) maxw = a.n[l] > maxw ? a.n[l] : maxw;
    float* lds_gemm = smem;
    float* buf[2] = {smem + kGemmLds, smem + kGemmLds + kRetrieveTokens * maxw};
    const float* theta = a.thetaT + b * a.ss[0] + h * a.ss[1];
    const int d = a.n[0];
    const int64_t qbase = b * a.qs[0] + h * a.qs[2] + t0 * a.qs[1];
    const int64_t ybase = b * a.ys[0] + h * a.ys[2] + t0 * a.ys[1];
    for (int e = threadIdx.x; e < n * d; e += kThreads) {
        int t = e / d, c = e % d;
        buf[0][t * d + c] = load_io(a.q, qbase + t * a.qs[1] + c, a.io);
    }
    __syncthreads();
    int cur = 0;
    for (int l = 1; l <= a.L; ++l) {
        const int nin = a.n[l - 1], nout = a.n[l];
        const float* X = buf[cur];
        float* Yb = buf[cur ^ 1];
        const float* W = theta + a.off[l];
        if (l < a.L) {
            gemm<kMfma>(n, nout, nin, MatA{X, nin, 1, nullptr}, MatB{W, 1, nin}, lds_gemm,
                       [&](int i, int jj, float z) { Yb[i * nout + jj] = z * sigmoidf_(z); });
        } else {
            gemm<kMfma>(n, nout, nin, MatA{X, nin, 1, nullptr}, MatB{W, 1, nin}, lds_gemm,
                       [&](int i, int jj, float z) {
                           store_io(a.y, ybase + i * a.ys[1] + jj, a.io, z);
                       });
        }
        cur ^= 1;
    }
}

__global__ void copy_state_kernel(ScanArgs a) {
    const int64_t seq = blockIdx.y;
    const int64_t b = seq / a.H, h = seq % a.H;
    float* th = a.thetaT + b * a.ss[0] + h * a.ss[1];
    float* mo = a.sT + b * a.ss[0] + h * a.ss[1];
    const float* th0 = a.theta0 + b * a.s0s[0] + h * a.s0s[1];
    const float* mo0 = a.s0 + b * a.s0s[0] + h * a.s0s[1];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.P;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (th != th0) th[i] = th0[i];
        if (mo != mo0) mo[i] = mo0[i];
    }
}

}  // namespace

size_t scan_generic_workspace_bytes(const ScanArgs& a) {
    WsLayout w = ws_layout(a.C, a.L, a.n);
    return (size_t)(a.B * a.H) * (size_t)w.per_seq * sizeof(float);
}

hipError_t launch_scan_generic(const ScanArgs& a, hipStream_t stream) {
    const int64_t nseq = a.B * a.H;
    if (nseq == 0) return hipSuccess;
    if (a.T == 0) {
        dim3 grid((unsigned)((a.P + 255) / 256 < 64 ? (a.P + 255) / 256 : 64), (unsigned)nseq);
        copy_state_kernel<<<grid, 256, 0, stream>>>(a);
        return hipGetLastError();
    }
    const WsLayout wl = ws_layout(a.C, a.L, a.n);
    if (a.io == TITANS_BF16)
        scan_generic_kernel<true><<<dim3((unsigned)nseq), kThreads, 0, stream>>>(a, wl);
    else
        scan_generic_kernel<false><<<dim3((unsigned)nseq), kThreads, 0, stream>>>(a, wl);
    return hipGetLastError();
}

hipError_t launch_retrieve_generic(const ScanArgs& a, hipStream_t stream) {
    const int64_t nseq = a.B * a.H;
    if (nseq == 0 || a.T == 0) return hipSuccess;
    int maxw = 0;
    for (int l = 0; l <= a.L; ++l) maxw = a.n[l] > maxw ? a.n[l] : maxw;
    size_t lds = sizeof(float) * (kGemmLds + 2 * kRetrieveTokens * maxw);
    dim3 grid((unsigned)((a.T + kRetrieveTokens - 1) / kRetrieveTokens), (unsigned)nseq);
    if (a.io == TITANS_BF16)
        retrieve_generic_kernel<true><<<grid, kThreads, lds, stream>>>(a);
    else
        retrieve_generic_kernel<false><<<grid, kThreads, lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace titans
