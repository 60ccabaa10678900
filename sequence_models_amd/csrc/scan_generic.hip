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

#include "generic_gemm.h"
#include "generic_util.h"
#include "titans_internal.h"

namespace titans {
namespace {

using namespace generic;

constexpr int kThreads = 256;
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

// Sequence groups of the linear-memory path: group g of a memory runs tokens
// [g span, (g + 1) span) from the state the combine pass left in states (W then S, P
// floats each, per (memory, group)); the last group copies its end state to theta_T, s_T.
struct Groups {
    int G;          // groups per memory; 0: whole sequences from theta0, s0
    int64_t span;   // tokens per group (a multiple of C)
    float* states;  // [B*H][G][2P]
};

// The layout comes in the argument block: it is indexed by layer at run time.
template <bool kMfma>
__global__ void __launch_bounds__(kThreads) scan_generic_kernel(ScanArgs a, WsLayout wl,
                                                                 Groups grp) {
    __shared__ __align__(16) float lds_gemm[kGemmLds];
    __shared__ float s_al[256], s_et[256], s_be[256];

    const int64_t wg = blockIdx.x;  // (memory, group) in group mode, else the memory
    const int64_t seq = grp.G ? wg / grp.G : wg;
    const int64_t grp_i = grp.G ? wg % grp.G : 0;
    const int64_t b = seq / a.H, h = seq % a.H;
    const int tid = threadIdx.x;
    const int L = a.L, C = a.C;
    const int64_t P = a.P;
    const int d = a.n[0];

    float* ws = static_cast<float*>(a.ws) + wg * wl.per_seq;
    float* coef_a = ws + wl.coef;
    float* coef_b = coef_a + (C + 1);
    float* coef_w = coef_b + (C + 1);
    float* coef_p = coef_w + C;
    float* Cm = ws + wl.cm;

    float* thetaT = a.thetaT + b * a.ss[0] + h * a.ss[1];
    float* momT = a.sT + b * a.ss[0] + h * a.ss[1];
    float* theta = thetaT;
    float* mom = momT;
    int64_t t_begin = 0, t_end = a.T;
    if (grp.G) {  // the group's start state was written by the combine pass
        theta = grp.states + wg * 2 * P;
        mom = theta + P;
        t_begin = grp_i * grp.span;
        t_end = t_begin + grp.span < a.T ? t_begin + grp.span : a.T;
    } else {
        const float* theta0 = a.theta0 + b * a.s0s[0] + h * a.s0s[1];
        const float* mom0 = a.s0 + b * a.s0s[0] + h * a.s0s[1];
        if (theta != theta0)
            for (int64_t i = tid; i < P; i += kThreads) theta[i] = theta0[i];
        if (mom != mom0)
            for (int64_t i = tid; i < P; i += kThreads) mom[i] = mom0[i];
    }
    __syncthreads();

    const int64_t qbase = b * a.qs[0] + h * a.qs[2];
    const int64_t ybase = b * a.ys[0] + h * a.ys[2];
    const int64_t gbase = b * a.gs[0] + h * a.gs[2];

    for (int64_t c0 = t_begin; c0 < t_end; c0 += C) {
        const int n = (int)((t_end - c0) < C ? (t_end - c0) : C);
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
    if (grp.G && grp_i == grp.G - 1) {  // the sequence's end state
        __syncthreads();
        for (int64_t i = tid; i < P; i += kThreads) {
            thetaT[i] = theta[i];
            momT[i] = mom[i];
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

// ---------------------------------------------------------------- linear memory (L = 1)
//
// With one layer and the squared-error bias the chunk-end carry is affine in the state
// X = [W | S] (d x 2d): with Delta_j = 2 (W k_j - v_j),
//   W' = a W - b S - sum_j c_j Delta_j k_j^T = W (a I - 2 Gc) - b S + 2 Hc
//   S' = p S + sum_j w_j Delta_j k_j^T      = W (2 Gw) + p S - 2 Hw
// Gc = K^T diag(c) K, Gw = K^T diag(w) K, Hc = V^T diag(c) K, Hw = V^T diag(w) K, i.e.
//   X' = X M + N,  M = [[a I - 2 Gc, 2 Gw], [-b I, p I]],  N = [2 Hc, -2 Hw].
// Affine maps compose associatively (the explainer's "associative scan" applies exactly
// here, and only here: a deeper memory's gradient is not linear in W).  A sequence is cut
// into G groups of chunks: the summary kernel composes each group's maps (P, Q) in
// parallel (P <- P M, Q <- Q M + N from P = I, Q = 0), the combine kernel runs
// X_{g+1} = X_g P_g + Q_g over the groups of a memory, and the generic kernel then runs
// every group's chunks (reads and carry) from its start state in parallel.  fp32
// throughout the summary and combine.

struct LinLayout {  // floats per (memory, group) summary area
    int64_t P11, P12, P21, P22, Q1, Q2;  // the composed map, d x d blocks
    int64_t Gc, Gw, Hc, Hw;             // one chunk's products
    int64_t T[6];                        // P11 Gc, P11 Gw, P21 Gc, P21 Gw, Q1 Gc, Q1 Gw
    int64_t K, V;                        // the chunk's K, V (C x d)
    int64_t c, w;                        // its c_C, w
    int64_t per_group;
};

__host__ __device__ inline LinLayout lin_layout(int C, int d) {
    auto r64 = [](int64_t x) { return (x + 63) & ~int64_t(63); };
    const int64_t dd = r64((int64_t)d * d);
    LinLayout l{};
    int64_t o = 0;
    int64_t* blocks[16] = {&l.P11, &l.P12, &l.P21, &l.P22, &l.Q1, &l.Q2, &l.Gc, &l.Gw,
                           &l.Hc, &l.Hw, &l.T[0], &l.T[1], &l.T[2], &l.T[3], &l.T[4], &l.T[5]};
    for (int i = 0; i < 16; ++i) { *blocks[i] = o; o += dd; }
    l.K = o; o += r64((int64_t)C * d);
    l.V = o; o += r64((int64_t)C * d);
    l.c = o; o += r64(C);
    l.w = o; o += r64(C);
    l.per_group = o;
    return l;
}

__global__ void __launch_bounds__(kThreads) linear_summary_kernel(ScanArgs a, Groups grp,
                                                                   LinLayout ll, float* sums) {
    __shared__ __align__(16) float lds_gemm[kGemmLds];
    __shared__ float s_al[256], s_et[256], s_be[256];
    __shared__ float s_tail[3];  // a_n, b_n, p of the chunk
    const int64_t wg = blockIdx.x;
    const int64_t seq = wg / grp.G, gi = wg % grp.G;
    const int64_t b = seq / a.H, h = seq % a.H;
    const int tid = threadIdx.x, d = a.n[0], C = a.C;
    const int64_t dd = (int64_t)d * d;
    float* z = sums + wg * ll.per_group;
    float *P11 = z + ll.P11, *P12 = z + ll.P12, *P21 = z + ll.P21, *P22 = z + ll.P22;
    float *Q1 = z + ll.Q1, *Q2 = z + ll.Q2;
    float *Gc = z + ll.Gc, *Gw = z + ll.Gw, *Hc = z + ll.Hc, *Hw = z + ll.Hw;
    float* Kst = z + ll.K;
    float* Vst = z + ll.V;
    float* cv = z + ll.c;
    float* wv = z + ll.w;
    for (int64_t e = tid; e < dd; e += kThreads) {
        const int i = (int)(e / d), j = (int)(e % d);
        P11[e] = P22[e] = (i == j) ? 1.0f : 0.0f;
        P12[e] = P21[e] = Q1[e] = Q2[e] = 0.0f;
    }
    const int64_t qbase = b * a.qs[0] + h * a.qs[2];
    const int64_t gbase = b * a.gs[0] + h * a.gs[2];
    const int64_t t_begin = gi * grp.span;
    const int64_t t_end = t_begin + grp.span < a.T ? t_begin + grp.span : a.T;
    for (int64_t c0 = t_begin; c0 < t_end; c0 += C) {
        const int n = (int)((t_end - c0) < C ? (t_end - c0) : C);
        for (int t = tid; t < n; t += kThreads) {
            const int64_t g = gbase + (c0 + t) * a.gs[1];
            s_al[t] = a.alpha[g];
            s_et[t] = a.eta[g];
            s_be[t] = a.beta[g];
        }
        for (int e = tid; e < n * d; e += kThreads) {
            const int t = e / d, c = e % d;
            const int64_t src = qbase + (c0 + t) * a.qs[1] + c;
            Kst[e] = load_io(a.k, src, a.io);
            Vst[e] = load_io(a.v, src, a.io);
        }
        __syncthreads();
        {  // chunk-end coefficients: thread j follows column j of the coefficient recurrence
            const int j = tid;
            float Bj = 0.0f, cj = 0.0f, at = 1.0f, bt = 0.0f, pb = 1.0f;
            const float omb_j = (j < n) ? 1.0f - s_be[j] : 0.0f;
            for (int t = 0; t < n; ++t) {
                const float al = s_al[t], et = s_et[t], be = s_be[t];
                pb *= be;
                if (j < t) Bj *= be;
                else if (j == t) Bj = 1.0f;
                const float keep = 1.0f - al;
                at *= keep;
                bt = keep * bt + et * pb;
                cj = keep * cj + ((j <= t) ? et * omb_j * Bj : 0.0f);
            }
            if (j < n) {
                cv[j] = cj;
                wv[j] = omb_j * Bj;
            }
            if (j == 0) {
                s_tail[0] = at;
                s_tail[1] = bt;
                s_tail[2] = pb;
            }
        }
        __syncthreads();
        // Gc, Gw, Hc, Hw: sums over the chunk's tokens of scaled outer products
        block_gemm_f32(d, d, n, MatA{Kst, 1, d, cv}, MatB{Kst, d, 1}, lds_gemm,
                   [&](int i, int j, float x) { Gc[i * d + j] = x; });
        block_gemm_f32(d, d, n, MatA{Kst, 1, d, wv}, MatB{Kst, d, 1}, lds_gemm,
                   [&](int i, int j, float x) { Gw[i * d + j] = x; });
        block_gemm_f32(d, d, n, MatA{Vst, 1, d, cv}, MatB{Kst, d, 1}, lds_gemm,
                   [&](int i, int j, float x) { Hc[i * d + j] = x; });
        block_gemm_f32(d, d, n, MatA{Vst, 1, d, wv}, MatB{Kst, d, 1}, lds_gemm,
                   [&](int i, int j, float x) { Hw[i * d + j] = x; });
        // the products of the composed map with this chunk's M
        const float* lhs[6] = {P11, P11, P21, P21, Q1, Q1};
        const float* rhs[6] = {Gc, Gw, Gc, Gw, Gc, Gw};
        for (int m = 0; m < 6; ++m) {
            float* Tm = z + ll.T[m];
            block_gemm_f32(d, d, d, MatA{lhs[m], d, 1, nullptr}, MatB{rhs[m], d, 1}, lds_gemm,
                       [&](int i, int j, float x) { Tm[i * d + j] = x; });
        }
        const float an = s_tail[0], bn = s_tail[1], pn = s_tail[2];
        const float *Ta = z + ll.T[0], *Tb = z + ll.T[1], *Tc = z + ll.T[2], *Td = z + ll.T[3],
                    *Te = z + ll.T[4], *Tf = z + ll.T[5];
        for (int64_t e = tid; e < dd; e += kThreads) {  // (P, Q) <- (P M, Q M + N)
            const float p11 = P11[e], p12 = P12[e], p21 = P21[e], p22 = P22[e];
            const float q1 = Q1[e], q2 = Q2[e];
            P11[e] = an * p11 - 2.0f * Ta[e] - bn * p12;
            P12[e] = 2.0f * Tb[e] + pn * p12;
            P21[e] = an * p21 - 2.0f * Tc[e] - bn * p22;
            P22[e] = 2.0f * Td[e] + pn * p22;
            Q1[e] = an * q1 - 2.0f * Te[e] - bn * q2 + 2.0f * Hc[e];
            Q2[e] = 2.0f * Tf[e] + pn * q2 - 2.0f * Hw[e];
        }
        __syncthreads();
    }
}

// X_0 = [theta0 | s0]; X_{g+1} = X_g P_g + Q_g = [W P11 + S P21 + Q1, W P12 + S P22 + Q2]
__global__ void __launch_bounds__(kThreads) linear_combine_kernel(ScanArgs a, Groups grp,
                                                                   LinLayout ll, const float* sums) {
    __shared__ __align__(16) float lds_gemm[kGemmLds];
    const int64_t seq = blockIdx.x;
    const int64_t b = seq / a.H, h = seq % a.H;
    const int tid = threadIdx.x, d = a.n[0];
    const int64_t P = a.P;
    const float* th0 = a.theta0 + b * a.s0s[0] + h * a.s0s[1];
    const float* mo0 = a.s0 + b * a.s0s[0] + h * a.s0s[1];
    float* x0 = grp.states + seq * grp.G * 2 * P;
    for (int64_t i = tid; i < P; i += kThreads) {
        x0[i] = th0[i];
        x0[P + i] = mo0[i];
    }
    __syncthreads();
    for (int g = 0; g + 1 < grp.G; ++g) {
        const float* W = x0 + (int64_t)g * 2 * P;
        const float* S = W + P;
        float* Wn = x0 + (int64_t)(g + 1) * 2 * P;
        float* Sn = Wn + P;
        const float* z = sums + (seq * grp.G + g) * ll.per_group;
        const float *P11 = z + ll.P11, *P12 = z + ll.P12, *P21 = z + ll.P21, *P22 = z + ll.P22;
        const float *Q1 = z + ll.Q1, *Q2 = z + ll.Q2;
        block_gemm_f32(d, d, d, MatA{W, d, 1, nullptr}, MatB{P11, d, 1}, lds_gemm,
                   [&](int i, int j, float x) { Wn[i * d + j] = x + Q1[i * d + j]; });
        block_gemm_f32(d, d, d, MatA{S, d, 1, nullptr}, MatB{P21, d, 1}, lds_gemm,
                   [&](int i, int j, float x) { Wn[i * d + j] += x; });
        block_gemm_f32(d, d, d, MatA{W, d, 1, nullptr}, MatB{P12, d, 1}, lds_gemm,
                   [&](int i, int j, float x) { Sn[i * d + j] = x + Q2[i * d + j]; });
        block_gemm_f32(d, d, d, MatA{S, d, 1, nullptr}, MatB{P22, d, 1}, lds_gemm,
                   [&](int i, int j, float x) { Sn[i * d + j] += x; });
    }
}

// Groups per memory for the linear path: about 512 workgroups over the GPU, at least 8
// chunks per group; 0 if that leaves fewer than two groups.
int64_t linear_groups(const ScanArgs& a, int64_t& span) {
    const int64_t nseq = a.B * a.H;
    const int64_t nch = (a.T + a.C - 1) / a.C;
    if (nseq == 0 || nch < 2) return 0;
    int64_t G = 512 / nseq;
    if (G > nch / 8) G = nch / 8;
    if (G < 2) return 0;
    const int64_t per = (nch + G - 1) / G;  // chunks per group
    G = (nch + per - 1) / per;              // every group non-empty
    span = per * a.C;
    return G;
}

}  // namespace

bool scan_linear_supported(const ScanArgs& a) {
    int64_t span = 0;
    return a.L == 1 && a.bias == TITANS_BIAS_L2 && linear_groups(a, span) >= 2;
}

size_t scan_linear_workspace_bytes(const ScanArgs& a) {
    int64_t span = 0;
    const int64_t G = linear_groups(a, span);
    const int64_t nseq = a.B * a.H;
    const WsLayout w = ws_layout(a.C, a.L, a.n);
    const LinLayout ll = lin_layout(a.C, a.n[0]);
    const int64_t floats = nseq * G * (w.per_seq + ll.per_group + 2 * a.P);
    return (size_t)floats * sizeof(float);
}

hipError_t launch_scan_linear(const ScanArgs& a, hipStream_t stream) {
    int64_t span = 0;
    const int64_t G = linear_groups(a, span);
    const int64_t nseq = a.B * a.H;
    if (G < 2) return hipErrorInvalidValue;  // the caller checked scan_linear_supported
    const WsLayout wl = ws_layout(a.C, a.L, a.n);
    const LinLayout ll = lin_layout(a.C, a.n[0]);
    float* base = static_cast<float*>(a.ws);
    float* sums = base + nseq * G * wl.per_seq;
    Groups grp{(int)G, span, sums + nseq * G * ll.per_group};
    const unsigned nwg = (unsigned)(nseq * G);
    linear_summary_kernel<<<dim3(nwg), kThreads, 0, stream>>>(a, grp, ll, sums);
    linear_combine_kernel<<<dim3((unsigned)nseq), kThreads, 0, stream>>>(a, grp, ll, sums);
    if (a.io == TITANS_BF16)
        scan_generic_kernel<true><<<dim3(nwg), kThreads, 0, stream>>>(a, wl, grp);
    else
        scan_generic_kernel<false><<<dim3(nwg), kThreads, 0, stream>>>(a, wl, grp);
    return hipGetLastError();
}

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
    const Groups whole{0, 0, nullptr};
    if (a.io == TITANS_BF16)
        scan_generic_kernel<true><<<dim3((unsigned)nseq), kThreads, 0, stream>>>(a, wl, whole);
    else
        scan_generic_kernel<false><<<dim3((unsigned)nseq), kThreads, 0, stream>>>(a, wl, whole);
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
