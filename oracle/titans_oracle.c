/*
 * titans_oracle.c -- fp64 CPU oracle for the Titans neural long-term memory scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the cpu_baseline
 * leg of bench.py may load this library.  The product path (the HIP library in
 * sequence_models_amd/) never calls, links or includes anything from here, and
 * this file includes nothing from there.
 *
 * What it computes (plain, sequential, token by token, in double precision):
 *
 *   memory     M_theta = bias-free MLP, widths n_0..n_L, SiLU between layers,
 *              no activation on the output layer.  Titans paper explainer
 *              (0h-n0.github.io, "ニューラル長期メモリモジュール"): the memory is the
 *              weights of an MLP.
 *   read       y_t = M_{theta_t}(q_t), theta_t = weights before token t's write
 *              (same explainer, retrieve formula).
 *   loss       l = || M_theta(k_t) - v_t ||_2^2, no 1/2 factor
 *              (lowest.today Titans summary, "Funzione Obiettivo").
 *              Alternative attentional biases (the MIRAS variants named on the
 *              explainer page, "MIRAS" section, and the ITmedia Titans/MIRAS article:
 *              YAAD uses a Huber loss, MONETA generalized norms), applied to each
 *              component r of r = M_theta(k_t) - v_t and summed:
 *                Huber, threshold delta:  r^2 if |r| <= delta, else 2 delta |r| - delta^2
 *                (the squared loss above with its slope capped at 2 delta);
 *                l_p, p >= 1:             |r|^p
 *              (both reduce to the squared loss: delta -> infinity, p = 2).
 *   surprise   g_t = grad_theta l, taken at the chunk-start weights theta_c
 *              (the chunked "mini-batch" form: lowest.today Titans summary,
 *              "Addestramento Parallelizzato").
 *   momentum   s_t = beta_t s_{t-1} + (1 - beta_t) g_t
 *              (explainer, "モメンタム機構", with a per-token beta).
 *   write      theta_{t+1} = (1 - alpha_t) theta_t - eta_t s_t
 *              (explainer, "適応的重み減衰（忘却ゲート）").
 *
 *   surprise   (optional output) the norm || g_t ||_2 of each token's gradient, the
 *              "momentary surprise" of the explainer ("サプライズ（驚き）メトリクス") that the
 *              momentum accumulates.
 *
 * Chunks of C tokens start at the call's first token; the last chunk may be
 * partial.  Nothing is blocked, fused or reordered: every token does one MLP
 * forward at the current weights (the read), one forward + backward at the
 * frozen chunk-start weights (the gradient), then the two elementwise updates.
 *
 * Parameter layout (shared by theta and s): layers l = 1..L concatenated,
 * W_l row-major with n_l rows and n_{l-1} columns, so z_l = W_l h_{l-1}.
 *
 * Pins: see tests/test_oracle_pins.py (finite differences, a library autograd,
 * closed-form delta rule, orthonormal-key recall, eta = 0, alpha = 1, a scalar
 * closed form with momentum and decay, the alternative letters of the summary
 * page, streaming and permutation invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MAX_LAYERS 8

/* attentional bias kinds */
#define ORACLE_BIAS_L2 0
#define ORACLE_BIAS_HUBER 1
#define ORACLE_BIAS_LP 2

/* loss of one residual component r */
static double bias_loss(int kind, double prm, double r) {
    double a = fabs(r);
    if (kind == ORACLE_BIAS_HUBER) return a <= prm ? r * r : 2.0 * prm * a - prm * prm;
    if (kind == ORACLE_BIAS_LP) return pow(a, prm);
    return r * r;
}

/* its derivative d loss / d r (0 at r = 0 for l_1) */
static double bias_grad(int kind, double prm, double r) {
    double a = fabs(r);
    if (kind == ORACLE_BIAS_HUBER) return a <= prm ? 2.0 * r : (r > 0 ? 2.0 * prm : -2.0 * prm);
    if (kind == ORACLE_BIAS_LP) {
        if (r == 0.0) return 0.0;
        double m = prm * pow(a, prm - 1.0);
        return r > 0 ? m : -m;
    }
    return 2.0 * r;
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }
static double silu(double z) { return z * sigmoid(z); }
/* d/dz [z sigma(z)] = sigma(z) + z sigma(z)(1 - sigma(z)) */
static double silu_prime(double z) {
    double s = sigmoid(z);
    return s * (1.0 + z * (1.0 - s));
}

int64_t oracle_param_count(int L, const int* n) {
    int64_t P = 0;
    for (int l = 1; l <= L; ++l) P += (int64_t)n[l] * n[l - 1];
    return P;
}

static int max_width(int L, const int* n) {
    int m = 0;
    for (int l = 0; l <= L; ++l) if (n[l] > m) m = n[l];
    return m;
}

/* out = M_theta(x).  work must hold 2 * max_width doubles. */
static void mlp_forward(int L, const int* n, const double* theta, const double* x,
                        double* out, double* work) {
    int mw = max_width(L, n);
    double* cur = work;
    double* nxt = work + mw;
    memcpy(cur, x, sizeof(double) * n[0]);
    const double* W = theta;
    for (int l = 1; l <= L; ++l) {
        for (int i = 0; i < n[l]; ++i) {
            double z = 0.0;
            for (int j = 0; j < n[l - 1]; ++j) z += W[(int64_t)i * n[l - 1] + j] * cur[j];
            nxt[i] = (l < L) ? silu(z) : z;
        }
        W += (int64_t)n[l] * n[l - 1];
        double* t = cur; cur = nxt; nxt = t;
    }
    memcpy(out, cur, sizeof(double) * n[L]);
}

/*
 * grad = d/dtheta sum_i loss(M_theta(k)_i - v_i) by explicit backpropagation.
 * Returns the loss.  work must hold (2 * (L + 1) + 2) * max_width doubles.
 *   forward:  h_0 = k, z_l = W_l h_{l-1}, h_l = SiLU(z_l) (l < L), o = z_L
 *   output:   delta_L = loss'(o - v)   (= 2 (o - v) for the squared loss)
 *   backward: delta_{l-1} = (W_l^T delta_l) * SiLU'(z_{l-1})
 *   gradient: dW_l = delta_l h_{l-1}^T
 */
static double mlp_grad(int L, const int* n, const double* theta, const double* k,
                       const double* v, double* grad, double* work, int kind, double prm) {
    int mw = max_width(L, n);
    double* z = work;                    /* z_l at z + l*mw, l = 1..L */
    double* h = work + (int64_t)(L + 1) * mw; /* h_l at h + l*mw, l = 0..L-1 */
    double* delta = h + (int64_t)(L + 1) * mw;
    double* dprev = delta + mw;
    const double* Wl[ORACLE_MAX_LAYERS + 1];
    double* Gl[ORACLE_MAX_LAYERS + 1];
    int64_t off = 0;
    for (int l = 1; l <= L; ++l) {
        Wl[l] = theta + off;
        Gl[l] = grad + off;
        off += (int64_t)n[l] * n[l - 1];
    }
    memcpy(h, k, sizeof(double) * n[0]);
    for (int l = 1; l <= L; ++l) {
        const double* hin = h + (int64_t)(l - 1) * mw;
        double* zl = z + (int64_t)l * mw;
        for (int i = 0; i < n[l]; ++i) {
            double acc = 0.0;
            for (int j = 0; j < n[l - 1]; ++j) acc += Wl[l][(int64_t)i * n[l - 1] + j] * hin[j];
            zl[i] = acc;
        }
        if (l < L) {
            double* hl = h + (int64_t)l * mw;
            for (int i = 0; i < n[l]; ++i) hl[i] = silu(zl[i]);
        }
    }
    double loss = 0.0;
    double* zL = z + (int64_t)L * mw;
    for (int i = 0; i < n[L]; ++i) {
        double e = zL[i] - v[i];
        loss += bias_loss(kind, prm, e);
        delta[i] = bias_grad(kind, prm, e);
    }
    for (int l = L; l >= 1; --l) {
        const double* hin = h + (int64_t)(l - 1) * mw;
        for (int i = 0; i < n[l]; ++i)
            for (int j = 0; j < n[l - 1]; ++j)
                Gl[l][(int64_t)i * n[l - 1] + j] = delta[i] * hin[j];
        if (l > 1) {
            const double* zp = z + (int64_t)(l - 1) * mw;
            for (int j = 0; j < n[l - 1]; ++j) {
                double acc = 0.0;
                for (int i = 0; i < n[l]; ++i) acc += Wl[l][(int64_t)i * n[l - 1] + j] * delta[i];
                dprev[j] = acc * silu_prime(zp[j]);
            }
            memcpy(delta, dprev, sizeof(double) * n[l - 1]);
        }
    }
    return loss;
}

static int64_t grad_work_len(int L, const int* n) {
    return (int64_t)(2 * (L + 1) + 2) * max_width(L, n);
}

/* ---- single-vector entry points (used by the finite-difference pins) ---- */

void oracle_mlp_forward(int L, const int* n, const double* theta, const double* x, double* out) {
    double* work = (double*)malloc(sizeof(double) * 2 * max_width(L, n));
    mlp_forward(L, n, theta, x, out, work);
    free(work);
}

double oracle_mlp_loss_bias(int L, const int* n, const double* theta, const double* k,
                            const double* v, int kind, double prm) {
    double* o = (double*)malloc(sizeof(double) * n[L]);
    oracle_mlp_forward(L, n, theta, k, o);
    double loss = 0.0;
    for (int i = 0; i < n[L]; ++i) loss += bias_loss(kind, prm, o[i] - v[i]);
    free(o);
    return loss;
}

double oracle_mlp_loss(int L, const int* n, const double* theta, const double* k, const double* v) {
    return oracle_mlp_loss_bias(L, n, theta, k, v, ORACLE_BIAS_L2, 0.0);
}

double oracle_mlp_grad_bias(int L, const int* n, const double* theta, const double* k,
                            const double* v, double* grad, int kind, double prm) {
    double* work = (double*)malloc(sizeof(double) * grad_work_len(L, n));
    double loss = mlp_grad(L, n, theta, k, v, grad, work, kind, prm);
    free(work);
    return loss;
}

double oracle_mlp_grad(int L, const int* n, const double* theta, const double* k, const double* v,
                       double* grad) {
    return oracle_mlp_grad_bias(L, n, theta, k, v, grad, ORACLE_BIAS_L2, 0.0);
}

/*
 * One (b, h) sequence.  Inputs are the sequence's own rows: token t of q/k/v
 * at q + t*tok_stride (d contiguous), gates at alpha[t*gate_stride].
 */
static void scan_one(int L, const int* n, int64_t T, int64_t C,
                     const double* q, const double* k, const double* v, int64_t tok_stride,
                     const double* alpha, const double* eta, const double* beta, int64_t gate_stride,
                     const double* theta0, const double* s0,
                     double* y, int64_t y_stride, double* theta, double* s, int kind, double prm,
                     double* surprise, int64_t surprise_stride) {
    int64_t P = oracle_param_count(L, n);
    double* theta_c = (double*)malloc(sizeof(double) * P);
    double* g = (double*)malloc(sizeof(double) * P);
    double* fwork = (double*)malloc(sizeof(double) * 2 * max_width(L, n));
    double* gwork = (double*)malloc(sizeof(double) * grad_work_len(L, n));
    memcpy(theta, theta0, sizeof(double) * P);
    memcpy(s, s0, sizeof(double) * P);
    for (int64_t c0 = 0; c0 < T; c0 += C) {
        memcpy(theta_c, theta, sizeof(double) * P);   /* frozen for this chunk's gradients */
        int64_t c1 = (c0 + C < T) ? c0 + C : T;
        for (int64_t t = c0; t < c1; ++t) {
            /* read with the weights before this token's write */
            mlp_forward(L, n, theta, q + t * tok_stride, y + t * y_stride, fwork);
            /* surprise at the chunk-start weights */
            mlp_grad(L, n, theta_c, k + t * tok_stride, v + t * tok_stride, g, gwork, kind, prm);
            if (surprise) {
                double gg = 0.0;
                for (int64_t i = 0; i < P; ++i) gg += g[i] * g[i];
                surprise[t * surprise_stride] = sqrt(gg);
            }
            double a = alpha[t * gate_stride], e = eta[t * gate_stride], bt = beta[t * gate_stride];
            for (int64_t i = 0; i < P; ++i) {
                s[i] = bt * s[i] + (1.0 - bt) * g[i];
                theta[i] = (1.0 - a) * theta[i] - e * s[i];
            }
        }
    }
    free(theta_c); free(g); free(fwork); free(gwork);
}

/*
 * Full scan over B x H independent sequences, all arrays C-contiguous double:
 *   q, k, v, y : [B, T, H, d]           alpha, eta, beta : [B, T, H]
 *   theta0, s0 : [B, H, P] with batch stride state0_bstride (0 = shared over batch,
 *                H*P = one per batch row); head stride P
 *   theta_T, s_T : [B, H, P]
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
/* surprise: NULL, or [B, T, H] receiving || g_t || of every token */
int oracle_scan_full(int64_t B, int64_t T, int64_t H, int L, const int* n, int64_t C,
                     const double* q, const double* k, const double* v,
                     const double* alpha, const double* eta, const double* beta,
                     const double* theta0, const double* s0, int64_t state0_bstride,
                     double* y, double* theta_T, double* s_T, int nthreads, int kind,
                     double prm, double* surprise) {
    if (L < 1 || L > ORACLE_MAX_LAYERS || C < 1 || B < 0 || T < 0 || H < 0) return -1;
    if (kind < ORACLE_BIAS_L2 || kind > ORACLE_BIAS_LP) return -1;
    if (kind == ORACLE_BIAS_HUBER && !(prm > 0.0)) return -1;
    if (kind == ORACLE_BIAS_LP && !(prm >= 1.0)) return -1;
    if (n[0] != n[L]) return -1;
    int64_t d = n[0];
    int64_t P = oracle_param_count(L, n);
    int64_t nseq = B * H;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t sidx = 0; sidx < nseq; ++sidx) {
        int64_t b = sidx / H, h = sidx % H;
        int64_t tok = H * d;                       /* element stride between tokens */
        int64_t base = b * T * H * d + h * d;
        int64_t gbase = b * T * H + h;
        const double* th0 = theta0 + b * state0_bstride + h * P;
        const double* sg0 = s0 + b * state0_bstride + h * P;
        scan_one(L, n, T, C, q + base, k + base, v + base, tok,
                 alpha + gbase, eta + gbase, beta + gbase, H,
                 th0, sg0, y + base, tok,
                 theta_T + (b * H + h) * P, s_T + (b * H + h) * P, kind, prm,
                 surprise ? surprise + gbase : NULL, H);
    }
    return err;
}

int oracle_scan_bias(int64_t B, int64_t T, int64_t H, int L, const int* n, int64_t C,
                     const double* q, const double* k, const double* v,
                     const double* alpha, const double* eta, const double* beta,
                     const double* theta0, const double* s0, int64_t state0_bstride,
                     double* y, double* theta_T, double* s_T, int nthreads, int kind,
                     double prm) {
    return oracle_scan_full(B, T, H, L, n, C, q, k, v, alpha, eta, beta, theta0, s0,
                            state0_bstride, y, theta_T, s_T, nthreads, kind, prm, NULL);
}

int oracle_scan(int64_t B, int64_t T, int64_t H, int L, const int* n, int64_t C,
                const double* q, const double* k, const double* v,
                const double* alpha, const double* eta, const double* beta,
                const double* theta0, const double* s0, int64_t state0_bstride,
                double* y, double* theta_T, double* s_T, int nthreads) {
    return oracle_scan_bias(B, T, H, L, n, C, q, k, v, alpha, eta, beta, theta0, s0,
                            state0_bstride, y, theta_T, s_T, nthreads, ORACLE_BIAS_L2, 0.0);
}

/*
 * Retrieval with fixed weights (the explainer's read formula with theta held
 * constant): y[b,t,h] = M_{theta[b,h]}(q[b,t,h]).  q, y: [B, T, H, d];
 * theta: [B, H, P] with batch stride theta_bstride (0 = shared over batch).
 */
int oracle_retrieve(int64_t B, int64_t T, int64_t H, int L, const int* n,
                    const double* q, const double* theta, int64_t theta_bstride,
                    double* y, int nthreads) {
    if (L < 1 || L > ORACLE_MAX_LAYERS || n[0] != n[L]) return -1;
    int64_t d = n[0];
    int64_t P = oracle_param_count(L, n);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double* work = (double*)malloc(sizeof(double) * 2 * max_width(L, n));
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t r = 0; r < B * T * H; ++r) {
            int64_t b = r / (T * H), h = r % H;
            mlp_forward(L, n, theta + b * theta_bstride + h * P, q + r * d, y + r * d, work);
        }
        free(work);
    }
    return 0;
}
