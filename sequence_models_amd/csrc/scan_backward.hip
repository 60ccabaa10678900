// Reverse-mode derivatives of the chunked Titans memory scan (the outer loop of the
// two-level optimization: the projections and gates that make q, k, v, alpha, eta, beta
// are trained through the memory's test-time writes; Titans explainer, sections on the
// memory module and its training, and the lowest.today summary, "Addestramento
// Parallelizzato").  Any supported shape, fp32 products (fp32 matrix cores) and state.
//
// Forward (per chunk, start weights W_l, momentum S_l, tokens t = 0..n-1):
//   theta_t = a_t theta_c - b_t s_c - sum_{j<t} c_{t,j} g_j        (read y_t at theta_t)
//   theta_e = a_n theta_c - b_n s_c - sum_j c_{n,j} g_j,   s_e = p_n s_c + sum_j w_{n,j} g_j
// g_j = grad of the loss at theta_c for (k_j, v_j), layer l part Delta_l[j] Hk_{l-1}[j]^T.
// The coefficients follow the token recurrence p_{t+1} = beta_t p_t,
// w_{t+1,j} = beta_t w_{t,j} + (1 - beta_t)[j = t], a_{t+1} = (1 - alpha_t) a_t,
// b_{t+1} = (1 - alpha_t) b_t + eta_t p_{t+1}, c_{t+1,j} = (1 - alpha_t) c_{t,j} + eta_t w_{t+1,j}.
//
// Per chunk, rows = tokens, with the state cotangents (Lt, Ls) = (dtheta_e, ds_e) coming in
// from the later chunks:
//   recompute  key path Hk_l, Zk_l, Delta_l, Gk_l = Delta_{l+1} W_{l+1}; reads at the
//              in-chunk weights Hq_l, Zq_l; A_l = Hq_{l-1} Hk_{l-1}^T, Mq_l = Cm o A_l
//   query adjoint  Dq_L = dY;  Bq_l = Dq_l Delta_l^T, Mb_l = Cm o Bq_l,
//              dHq_{l-1} = diag(a) Dq_l W_l - diag(b) Dq_l S_l - Mb_l Hk_{l-1},
//              Dq_{l-1} = dHq_{l-1} o SiLU'(Zq_{l-1}), dq = dHq_0; coefficient cotangents
//              da_t += <Dq_l W_l, Hq_{l-1}>_row, db_t -= <Dq_l S_l, Hq_{l-1}>_row,
//              dc_{t,j} -= Bq_l[t,j] A_l[t,j]
//   chunk end  da_n = <Lt, theta_c>, db_n = -<Lt, s_c>, dp_n = <Ls, s_c>,
//              dc_{n,j} = -<Delta_l, Hk_{l-1} Lt_l^T>_row, dw_{n,j} = <Delta_l, Hk_{l-1} Ls_l^T>_row
//   second order  the cotangent of g_j is U_j = U_j^e + U_j^y with U_j^e = -c_{n,j} Lt +
//              w_{n,j} Ls and U_j^y = -sum_{t>j} c_{t,j} (Dq Hq^T)_t; pushing it back through
//              g_j = grad loss(theta_c; k_j, v_j) is a Hessian-vector product (Pearlmutter's
//              R-operator): a tangent pass of the key path, RZ_l = RH_{l-1} W_l^T + U_l Hk_{l-1}
//              (U^e_l Hk = -diag(c_n) Hk Lt^T + diag(w_n) Hk Ls^T, U^y_l Hk = -Mq_l^T Dq_l), and
//              of its backward, RDelta_L = loss''(r) RZ_L, RG_l = RDelta_l W_l + U_l^T Delta_l
//              (U^e: -diag(c_n) Delta Lt + diag(w_n) Delta Ls; U^y: -Mb_l^T Hq_{l-1}),
//              RDelta_{l-1} = RG_l o SiLU'(Zk_{l-1}) + Gk_{l-1} o SiLU''(Zk_{l-1}) o RZ_{l-1};
//              dk = RG_1, dv = -loss''(r) RZ_L.  Both passes are linear in U, so they run
//              once for U^y and once for U^e and add.
//   carry      Ls_l <- p_n Ls_l - b_n Lt_l + dLs_l,  dLs_l = -Dq_l^T diag(b) Hq_{l-1}
//              Lt_l <- a_n Lt_l + dLt_l + RDelta^e_l^T Hk_{l-1} + Delta_l^T RH^e_{l-1},
//              dLt_l = Dq_l^T diag(a) Hq_{l-1} + RDelta^y_l^T Hk_{l-1} + Delta_l^T RH^y_{l-1}
//   gates      the coefficient recurrence run backwards.
//
// Everything but the U^e terms, the chunk-end products and the carry's use of (Lt, Ls) is
// independent of the later chunks, so the work is split into three parts over segments of
// chunks:
//   chunk part   one workgroup per (memory, chunk), all chunks of a segment at once:
//                recompute, query adjoint (dq final), the U^y halves of the tangent passes
//                (dk, dv partial), dLt, dLs -> a per-chunk record
//   seq part     one workgroup per memory, the segment's chunks in reverse: the chain
//                through (Lt, Ls) -- chunk-end products, the U^e halves (dk, dv final), the
//                carry
//   gate part    one workgroup per (memory, chunk): the gate cotangents
// after bwd_forward_kernel (one workgroup per memory: the chunk carries forward, storing
// every chunk's start state).  Segments run from the last to the first; one launch of
// bwd_step_kernel runs the seq part of segment s beside the chunk part of segment s - 1 and
// the gate part of segment s + 1 (three record buffers), so the per-chunk work fills the
// compute units the B*H sequential chains leave idle.
#include <hip/hip_runtime.h>

#include "generic_gemm.h"
#include "generic_util.h"
#include "titans_internal.h"

namespace titans {
namespace {

using namespace generic;

constexpr int kThreads = 256;
constexpr int kSegChunks = 32;  // chunks per segment
constexpr int kRecBufs = 3;     // record buffers: the segments of the three parts of a launch

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f2_t;

__host__ __device__ inline int64_t r64(int64_t x) { return (x + 63) & ~int64_t(63); }

// Floats per checkpoint half (theta or s): P rounded up to 16 bytes.
__host__ __device__ inline int64_t ck_half(int64_t P) { return (P + 3) & ~int64_t(3); }

// Float offsets inside one chunk's record (written by bwd_chunk_kernel, completed by
// bwd_seq_kernel, read by bwd_gate_kernel).  The forward sweep uses the head of one record
// per memory (everything before dky) as its working area.
struct RecLayout {
    int64_t ca, cb, cp;                 // a_t, b_t, p_t for t = 0..C
    int64_t cm, wm;                     // c_{t,j}, w_{t,j}: (C + 1) x C
    int64_t gc, gw;                     // their cotangents (rows 0..n-1: U^y part of dc;
                                        // row n: chunk end), (C + 1) x C
    int64_t ga, gb;                     // cotangents of a_t, b_t (t < n: reads; t = n: end)
    int64_t gp;                         // cotangent of p_n
    int64_t hk[TITANS_MAX_LAYERS];      // l = 0..L-1: C x n_l (Hk_0 = K)
    int64_t zk[TITANS_MAX_LAYERS];      // l = 1..L-1
    int64_t gk[TITANS_MAX_LAYERS];      // l = 1..L-1: Delta_{l+1} W_{l+1}
    int64_t dl[TITANS_MAX_LAYERS + 1];  // l = 1..L
    int64_t rr;                         // C x d: M(k) - v
    int64_t dky, dvy;                   // C x d: the U^y parts of dk, dv
    int64_t dlt, dls;                   // ck_half(P) each: dLt, dLs
    int64_t per;
};

__host__ __device__ inline RecLayout rec_layout(int C, int L, const int* n, int64_t P) {
    RecLayout w{};
    const int64_t cc = r64((int64_t)(C + 1) * C), c1 = r64(C + 1);
    int64_t o = 0;
    w.ca = o; o += c1;
    w.cb = o; o += c1;
    w.cp = o; o += c1;
    w.cm = o; o += cc;
    w.wm = o; o += cc;
    w.gc = o; o += cc;
    w.gw = o; o += cc;
    w.ga = o; o += c1;
    w.gb = o; o += c1;
    w.gp = o; o += 64;
    for (int l = 0; l < L; ++l) { w.hk[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l < L; ++l) { w.zk[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l < L; ++l) { w.gk[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l <= L; ++l) { w.dl[l] = o; o += r64((int64_t)C * n[l]); }
    w.rr = o; o += r64((int64_t)C * n[L]);
    w.dky = o; o += r64((int64_t)C * n[0]);
    w.dvy = o; o += r64((int64_t)C * n[0]);
    w.dlt = o; o += r64(ck_half(P));
    w.dls = o; o += r64(ck_half(P));
    w.per = o;
    return w;
}

// Working area of one bwd_chunk_kernel workgroup (per (memory, chunk of the segment)).
struct ChunkScr {
    int64_t hq[TITANS_MAX_LAYERS];      // l = 0..L-1 (Hq_0 = Q)
    int64_t zq[TITANS_MAX_LAYERS];      // l = 1..L-1
    int64_t dq[TITANS_MAX_LAYERS + 1];  // l = 1..L (Dq_L = dY)
    int64_t am[TITANS_MAX_LAYERS + 1];  // l = 1..L: C x C
    int64_t mq[TITANS_MAX_LAYERS + 1];
    int64_t mb[TITANS_MAX_LAYERS + 1];
    int64_t rz[TITANS_MAX_LAYERS + 1];  // l = 1..L
    int64_t rh[TITANS_MAX_LAYERS];      // l = 1..L-1
    int64_t rd[TITANS_MAX_LAYERS + 1];  // l = 1..L
    int64_t tmp;                        // C x max width
    int64_t per;
};

__host__ __device__ inline ChunkScr chunk_scr(int C, int L, const int* n) {
    ChunkScr w{};
    int maxw = 0;
    for (int l = 0; l <= L; ++l) maxw = n[l] > maxw ? n[l] : maxw;
    int64_t o = 0;
    for (int l = 0; l < L; ++l) { w.hq[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l < L; ++l) { w.zq[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l <= L; ++l) { w.dq[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l <= L; ++l) { w.am[l] = o; o += r64((int64_t)C * C); }
    for (int l = 1; l <= L; ++l) { w.mq[l] = o; o += r64((int64_t)C * C); }
    for (int l = 1; l <= L; ++l) { w.mb[l] = o; o += r64((int64_t)C * C); }
    for (int l = 1; l <= L; ++l) { w.rz[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l < L; ++l) { w.rh[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l <= L; ++l) { w.rd[l] = o; o += r64((int64_t)C * n[l]); }
    w.tmp = o; o += r64((int64_t)C * maxw);
    w.per = o;
    return w;
}

// Working area of one bwd_seq_kernel workgroup (per memory).
struct SeqScr {
    int64_t rz[TITANS_MAX_LAYERS + 1];  // l = 1..L
    int64_t rh[TITANS_MAX_LAYERS];      // l = 1..L-1
    int64_t rd[TITANS_MAX_LAYERS + 1];  // l = 1..L
    int64_t tmp;
    int64_t dots;                       // the next chunk's three state products
    int64_t per;
};

__host__ __device__ inline SeqScr seq_scr(int C, int L, const int* n) {
    SeqScr w{};
    int maxw = 0;
    for (int l = 0; l <= L; ++l) maxw = n[l] > maxw ? n[l] : maxw;
    int64_t o = 0;
    for (int l = 1; l <= L; ++l) { w.rz[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l < L; ++l) { w.rh[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l <= L; ++l) { w.rd[l] = o; o += r64((int64_t)C * n[l]); }
    w.tmp = o; o += r64((int64_t)C * maxw);
    w.dots = o; o += 64;
    w.per = o;
    return w;
}

// One part's share of a launch: its segment and the workgroups that run it.
struct Role {
    int64_t first;         // the segment's first chunk
    int count;             // its chunks (0: the part does not run in this launch)
    float* rec;            // its record buffer: [nseq][seg] records
    int64_t blk0;          // first workgroup of the part
};

// Where everything lives in the caller's workspace, and what a launch works on.
struct Plan {
    RecLayout rl;
    ChunkScr cl;
    SeqScr sl;
    int64_t nch, seg;      // chunks per memory, chunks per segment
    float* ckpt;           // [nseq][nch][2 PH]
    float* recs;           // kRecBufs x [nseq][seg] records
    float* cscr;           // [nseq][seg] chunk-part areas
    float* sscr;           // [nseq] seq-part areas
    Role rs, rc, rg;       // seq, chunk and gate parts
    int last_segment;      // the seq part's segment holds the sequence's last chunk
};

inline Plan make_plan(const ScanArgs& a) {
    Plan p{};
    p.rl = rec_layout(a.C, a.L, a.n, a.P);
    p.cl = chunk_scr(a.C, a.L, a.n);
    p.sl = seq_scr(a.C, a.L, a.n);
    p.nch = (a.T + a.C - 1) / a.C;
    p.seg = p.nch < kSegChunks ? p.nch : kSegChunks;
    return p;
}

inline size_t plan_floats(const ScanArgs& a, const Plan& p) {
    const int64_t nseq = a.B * a.H;
    return (size_t)nseq * (size_t)(p.nch * 2 * ck_half(a.P) +
                                   p.seg * (kRecBufs * p.rl.per + p.cl.per) + p.sl.per);
}

inline void place(const ScanArgs& a, Plan& p) {
    const int64_t nseq = a.B * a.H;
    float* base = static_cast<float*>(a.ws);
    p.ckpt = base;
    p.recs = p.ckpt + nseq * p.nch * 2 * ck_half(a.P);
    p.cscr = p.recs + kRecBufs * nseq * p.seg * p.rl.per;
    p.sscr = p.cscr + nseq * p.seg * p.cl.per;
}

__device__ __forceinline__ float silu_prime(float z) {
    const float s = sigmoidf_(z);
    return s * (1.0f + z * (1.0f - s));
}

__device__ __forceinline__ float silu_second(float z) {
    const float s = sigmoidf_(z);
    return s * (1.0f - s) * (2.0f + z * (1.0f - 2.0f * s));
}

// Per-memory bases of every strided buffer.
struct Bases {
    int64_t b, h, q, y, g, st;
};

__device__ __forceinline__ Bases bases_of(const ScanArgs& a, int64_t seq) {
    Bases r;
    r.b = seq / a.H;
    r.h = seq % a.H;
    r.q = r.b * a.qs[0] + r.h * a.qs[2];
    r.y = r.b * a.ys[0] + r.h * a.ys[2];
    r.g = r.b * a.gs[0] + r.h * a.gs[2];
    r.st = r.b * a.ss[0] + r.h * a.ss[1];
    return r;
}

// rows c0 .. c0 + n - 1 of a [T, d] io-dtype operand (row stride rs from base) into
// dst[n][d] as fp32; each thread issues its loads in groups of eight before storing any.
__device__ __forceinline__ void stage_rows(float* dst, const void* src, int64_t base, int64_t rs,
                                           int64_t c0, int n, int d, int io) {
    const int total = n * d;
    for (int e0 = threadIdx.x; e0 < total; e0 += 8 * kThreads) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            int e = e0 + u * kThreads;
            e = e < total ? e : total - 1;
            v[u] = load_io(src, base + (c0 + e / d) * rs + e % d, io);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + u * kThreads;
            if (e < total) dst[e] = v[u];
        }
    }
}

// The chunk's gates into LDS.
__device__ __forceinline__ void stage_gates(const ScanArgs& a, const Bases& bs, int64_t c0, int n,
                                            float* s_al, float* s_et, float* s_be) {
    for (int t = threadIdx.x; t < n; t += kThreads) {
        const int64_t gi = bs.g + (c0 + t) * a.gs[1];
        s_al[t] = a.alpha[gi];
        s_et[t] = a.eta[gi];
        s_be[t] = a.beta[gi];
    }
}

// Coefficients of the chunk into the record: thread j follows column j of c and w;
// thread 0 also writes a_t, b_t, p_t.  Rows t = 0..n of every array.
__device__ __forceinline__ void coefficients(const RecLayout& rl, float* rec, int C, int n,
                                             const float* s_al, const float* s_et,
                                             const float* s_be) {
    const int j = threadIdx.x;
    float* ca = rec + rl.ca;
    float* cb = rec + rl.cb;
    float* cp = rec + rl.cp;
    float* cm = rec + rl.cm;
    float* wm = rec + rl.wm;
    float wj = 0.0f, cj = 0.0f, at = 1.0f, bt = 0.0f, pt = 1.0f;
    if (j < C) { cm[j] = 0.0f; wm[j] = 0.0f; }
    if (j == 0) { ca[0] = 1.0f; cb[0] = 0.0f; cp[0] = 1.0f; }
    for (int t = 0; t < n; ++t) {
        const float al = s_al[t], et = s_et[t], be = s_be[t];
        const float keep = 1.0f - al;
        pt *= be;
        wj = be * wj + ((j == t) ? 1.0f - be : 0.0f);
        at *= keep;
        bt = keep * bt + et * pt;
        cj = keep * cj + et * wj;
        if (j < C) {
            cm[(int64_t)(t + 1) * C + j] = cj;
            wm[(int64_t)(t + 1) * C + j] = wj;
        }
        if (j == 0) { ca[t + 1] = at; cb[t + 1] = bt; cp[t + 1] = pt; }
    }
}

// Key path at the chunk-start weights into the record: Zk, Hk, the residual r = M(k) - v,
// the output error loss'(r) and the errors Delta_l, Gk_l of every layer (Hk_0 staged).
template <bool kMfma>
__device__ __forceinline__ void key_path(const ScanArgs& a, const RecLayout& rl, float* rec,
                                         const float* theta, const Bases& bs, int64_t c0, int n,
                                         float* lds) {
    const int L = a.L;
    for (int l = 1; l <= L; ++l) {
        const int nin = a.n[l - 1], nout = a.n[l];
        const float* W = theta + a.off[l];
        const MatA A{rec + rl.hk[l - 1], nin, 1, nullptr};
        const MatB Bm{W, 1, nin};
        if (l < L) {
            float* Hout = rec + rl.hk[l];
            float* Z = rec + rl.zk[l];
            gemm<kMfma>(n, nout, nin, A, Bm, lds, [&](int i, int j, float z) {
                Z[i * nout + j] = z;
                Hout[i * nout + j] = z * sigmoidf_(z);
            });
        } else {
            float* R = rec + rl.rr;
            float* D = rec + rl.dl[L];
            gemm2<kMfma>(
                n, nout, nin, A, Bm, lds,
                [&](int i, int j) { return load_io(a.v, bs.q + (c0 + i) * a.qs[1] + j, a.io); },
                [&](int i, int j, float z, float v) {
                    const float r = z - v;
                    R[i * nout + j] = r;
                    D[i * nout + j] = bias_grad(r, a.bias, a.bias_param);
                });
        }
    }
    for (int l = L; l >= 2; --l) {
        const int nin = a.n[l - 1], nout = a.n[l];
        const float* Z = rec + rl.zk[l - 1];
        float* G = rec + rl.gk[l - 1];
        float* Dp = rec + rl.dl[l - 1];
        gemm2<kMfma>(n, nin, nout, MatA{rec + rl.dl[l], nout, 1, nullptr},
                     MatB{theta + a.off[l], nin, 1}, lds,
                     [&](int i, int j) { return Z[i * nin + j]; },
                     [&](int i, int j, float g, float z) {
                         G[i * nin + j] = g;
                         Dp[i * nin + j] = g * silu_prime(z);
                     });
    }
}

// Sum of x, y, z over the workgroup (every thread gets the sums).
__device__ __forceinline__ void block_sum3(float& x, float& y, float& z, float* red) {
    for (int o = 32; o > 0; o >>= 1) {
        x += __shfl_xor(x, o);
        y += __shfl_xor(y, o);
        z += __shfl_xor(z, o);
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { red[w] = x; red[4 + w] = y; red[8 + w] = z; }
    __syncthreads();
    x = red[0] + red[1] + red[2] + red[3];
    y = red[4] + red[5] + red[6] + red[7];
    z = red[8] + red[9] + red[10] + red[11];
    __syncthreads();
}

// ---------------------------------------------------------------- forward sweep

template <bool kMfma>
__global__ void __launch_bounds__(kThreads) bwd_forward_kernel(BwdArgs A, Plan pl) {
    __shared__ __align__(16) float lds_gemm[kGemmLds];
    __shared__ float s_al[256], s_et[256], s_be[256];
    const ScanArgs& a = A.a;
    const RecLayout& rl = pl.rl;
    const int64_t seq = blockIdx.x;
    const Bases bs = bases_of(a, seq);
    const int C = a.C, L = a.L, d = a.n[0];
    const int64_t P = a.P, nch = pl.nch, PH = ck_half(P);
    float* ws = pl.recs + seq * pl.seg * rl.per;  // a record of this memory as working area
    float* ck = pl.ckpt + seq * nch * 2 * PH;
    {
        const float* th0 = a.theta0 + bs.b * a.s0s[0] + bs.h * a.s0s[1];
        const float* mo0 = a.s0 + bs.b * a.s0s[0] + bs.h * a.s0s[1];
        for (int64_t i = threadIdx.x; i < P; i += kThreads) {
            ck[i] = th0[i];
            ck[PH + i] = mo0[i];
        }
    }
    __syncthreads();
    for (int64_t ci = 0; ci + 1 < nch; ++ci) {
        const int64_t c0 = ci * C;
        const int n = C;  // every chunk but the last is full
        const float* th = ck + ci * 2 * PH;
        const float* mo = th + PH;
        float* thn = ck + (ci + 1) * 2 * PH;
        float* mon = thn + PH;
        stage_gates(a, bs, c0, n, s_al, s_et, s_be);
        stage_rows(ws + rl.hk[0], a.k, bs.q, a.qs[1], c0, n, d, a.io);
        __syncthreads();
        coefficients(rl, ws, C, n, s_al, s_et, s_be);
        __syncthreads();
        key_path<kMfma>(a, rl, ws, th, bs, c0, n, lds_gemm);
        const float an = ws[rl.ca + n], bn = ws[rl.cb + n], pn = ws[rl.cp + n];
        const float* crow = ws + rl.cm + (int64_t)n * C;
        const float* wrow = ws + rl.wm + (int64_t)n * C;
        for (int l = 1; l <= L; ++l) {
            const int nin = a.n[l - 1], nout = a.n[l];
            const int64_t off = a.off[l];
            const MatB Hk{ws + rl.hk[l - 1], nin, 1};
            gemm2<kMfma>(
                nout, nin, n, MatA{ws + rl.dl[l], 1, nout, crow}, Hk, lds_gemm,
                [&](int i, int j) {
                    const int64_t o = off + (int64_t)i * nin + j;
                    return f2_t{th[o], mo[o]};
                },
                [&](int i, int j, float x, f2_t t) {
                    thn[off + (int64_t)i * nin + j] = an * t[0] - bn * t[1] - x;
                });
            gemm2<kMfma>(
                nout, nin, n, MatA{ws + rl.dl[l], 1, nout, wrow}, Hk, lds_gemm,
                [&](int i, int j) { return mo[off + (int64_t)i * nin + j]; },
                [&](int i, int j, float x, float m) { mon[off + (int64_t)i * nin + j] = pn * m + x; });
        }
    }
}

// ---------------------------------------------------------------- per-chunk part

template <bool kMfma>
__device__ __forceinline__ void chunk_part(const BwdArgs& A, const Plan& pl, int64_t blk,
                                           float* lds_gemm) {
    __shared__ float s_al[256], s_et[256], s_be[256];
    __shared__ float s_ga[257], s_gb[257];  // U^y-path cotangents of a_t, b_t
    __shared__ float s_ca[257], s_cb[257];
    const ScanArgs& a = A.a;
    const RecLayout& rl = pl.rl;
    const ChunkScr& cl = pl.cl;
    const int64_t seq = blk / pl.rc.count;
    const int cs = (int)(blk - seq * pl.rc.count);  // chunk within the segment
    const int64_t ci = pl.rc.first + cs;
    const Bases bs = bases_of(a, seq);
    const int tid = threadIdx.x;
    const int C = a.C, L = a.L, d = a.n[0];
    const int64_t PH = ck_half(a.P);
    const int64_t c0 = ci * C;
    const int n = (int)((a.T - c0) < C ? (a.T - c0) : C);
    const float* th = pl.ckpt + (seq * pl.nch + ci) * 2 * PH;
    const float* mo = th + PH;
    float* rec = pl.rc.rec + (seq * pl.seg + cs) * rl.per;
    float* ws = pl.cscr + (seq * pl.seg + cs) * cl.per;
    float* cm = rec + rl.cm;
    float* gc = rec + rl.gc;
    float* tmp = ws + cl.tmp;

    // ---- stage: gates, K, Q, dY; coefficients
    stage_gates(a, bs, c0, n, s_al, s_et, s_be);
    stage_rows(rec + rl.hk[0], a.k, bs.q, a.qs[1], c0, n, d, a.io);
    stage_rows(ws + cl.hq[0], a.q, bs.q, a.qs[1], c0, n, d, a.io);
    stage_rows(ws + cl.dq[L], A.dy, bs.y, a.ys[1], c0, n, d, a.io);
    for (int t = tid; t <= n; t += kThreads) { s_ga[t] = 0.0f; s_gb[t] = 0.0f; }
    __syncthreads();
    coefficients(rl, rec, C, n, s_al, s_et, s_be);
    __syncthreads();
    for (int t = tid; t <= n; t += kThreads) {
        s_ca[t] = rec[rl.ca + t];
        s_cb[t] = rec[rl.cb + t];
    }
    __syncthreads();

    // ---- recompute: key path, then the reads at the in-chunk weights
    key_path<kMfma>(a, rl, rec, th, bs, c0, n, lds_gemm);
    for (int l = 1; l <= L; ++l) {
        const int nin = a.n[l - 1], nout = a.n[l];
        const float* Hq = ws + cl.hq[l - 1];
        float* Am = ws + cl.am[l];
        float* Mq = ws + cl.mq[l];
        gemm2<kMfma>(n, n, nin, MatA{Hq, nin, 1, nullptr}, MatB{rec + rl.hk[l - 1], 1, nin},
                     lds_gemm,
                     [&](int i, int j) { return (j < i) ? cm[(int64_t)i * C + j] : 0.0f; },
                     [&](int i, int j, float x, float c) {
                         Am[i * C + j] = x;
                         Mq[i * C + j] = c * x;
                     });
        if (l == L) break;  // the output itself is not needed
        float* Z = ws + cl.zq[l];
        float* Hn = ws + cl.hq[l];
        gemm<kMfma>(n, nout, nin, MatA{Hq, nin, 1, nullptr}, MatB{th + a.off[l], 1, nin},
                    lds_gemm, [&](int i, int j, float x) { Z[i * nout + j] = s_ca[i] * x; });
        gemm2<kMfma>(n, nout, nin, MatA{Hq, nin, 1, nullptr}, MatB{mo + a.off[l], 1, nin},
                     lds_gemm, [&](int i, int j) { return Z[i * nout + j]; },
                     [&](int i, int j, float x, float z) { Z[i * nout + j] = z - s_cb[i] * x; });
        gemm2<kMfma>(n, nout, n, MatA{Mq, C, 1, nullptr}, MatB{rec + rl.dl[l], nout, 1},
                     lds_gemm, [&](int i, int j) { return Z[i * nout + j]; },
                     [&](int i, int j, float x, float z0) {
                         const float z = z0 - x;
                         Z[i * nout + j] = z;
                         Hn[i * nout + j] = z * sigmoidf_(z);
                     });
    }

    // ---- query adjoint, layer L down to 1 (dq is final here)
    for (int l = L; l >= 1; --l) {
        const int nin = a.n[l - 1], nout = a.n[l];
        const float* Dq = ws + cl.dq[l];
        const float* Hq = ws + cl.hq[l - 1];
        const float* Am = ws + cl.am[l];
        float* Mb = ws + cl.mb[l];
        const bool first = (l == L);
        gemm2<kMfma>(n, n, nout, MatA{Dq, nout, 1, nullptr}, MatB{rec + rl.dl[l], 1, nout},
                     lds_gemm,
                     [&](int i, int j) {
                         const bool low = j < i;
                         const int64_t o = (int64_t)i * C + j;
                         return f32x4_t{low ? cm[o] : 0.0f, low ? Am[o] : 0.0f,
                                        first ? 0.0f : gc[o], 0.0f};
                     },
                     [&](int i, int j, float x, f32x4_t u) {
                         Mb[i * C + j] = u[0] * x;
                         gc[(int64_t)i * C + j] = u[2] - x * u[1];
                     });
        gemm2<kMfma>(n, nin, nout, MatA{Dq, nout, 1, nullptr}, MatB{th + a.off[l], nin, 1},
                     lds_gemm, [&](int i, int j) { return Hq[i * nin + j]; },
                     [&](int i, int j, float x, float h) {
                         tmp[i * nin + j] = s_ca[i] * x;
                         atomicAdd(&s_ga[i], x * h);
                     });
        gemm2<kMfma>(n, nin, nout, MatA{Dq, nout, 1, nullptr}, MatB{mo + a.off[l], nin, 1},
                     lds_gemm,
                     [&](int i, int j) { return f2_t{tmp[i * nin + j], Hq[i * nin + j]}; },
                     [&](int i, int j, float x, f2_t u) {
                         tmp[i * nin + j] = u[0] - s_cb[i] * x;
                         atomicAdd(&s_gb[i], -x * u[1]);
                     });
        if (l > 1) {
            const float* Zq = ws + cl.zq[l - 1];
            float* Dn = ws + cl.dq[l - 1];
            gemm2<kMfma>(n, nin, n, MatA{Mb, C, 1, nullptr}, MatB{rec + rl.hk[l - 1], nin, 1},
                         lds_gemm,
                         [&](int i, int j) { return f2_t{tmp[i * nin + j], Zq[i * nin + j]}; },
                         [&](int i, int j, float x, f2_t u) {
                             Dn[i * nin + j] = (u[0] - x) * silu_prime(u[1]);
                         });
        } else {
            gemm2<kMfma>(n, nin, n, MatA{Mb, C, 1, nullptr}, MatB{rec + rl.hk[0], nin, 1},
                         lds_gemm, [&](int i, int j) { return tmp[i * nin + j]; },
                         [&](int i, int j, float x, float t) {
                             store_io(A.dq, bs.q + (c0 + i) * a.qs[1] + j, a.io, t - x);
                         });
        }
    }
    for (int t = tid; t < n; t += kThreads) {
        rec[rl.ga + t] = s_ga[t];
        rec[rl.gb + t] = s_gb[t];
    }

    // ---- U^y half of the key tangent pass: RZ_l = RH_{l-1} W_l^T - Mq_l^T Dq_l
    for (int l = 1; l <= L; ++l) {
        const int nin = a.n[l - 1], nout = a.n[l];
        float* RZ = ws + cl.rz[l];
        const float* Zk = l < L ? rec + rl.zk[l] : nullptr;
        float* RH = l < L ? ws + cl.rh[l] : nullptr;
        if (l > 1)
            gemm<kMfma>(n, nout, nin, MatA{ws + cl.rh[l - 1], nin, 1, nullptr},
                        MatB{th + a.off[l], 1, nin}, lds_gemm,
                        [&](int i, int j, float x) { RZ[i * nout + j] = x; });
        gemm2<kMfma>(n, nout, n, MatA{ws + cl.mq[l], 1, C, nullptr}, MatB{ws + cl.dq[l], nout, 1},
                     lds_gemm,
                     [&](int i, int j) {
                         return f2_t{l > 1 ? RZ[i * nout + j] : 0.0f, Zk ? Zk[i * nout + j] : 0.0f};
                     },
                     [&](int i, int j, float x, f2_t u) {
                         const float rz = u[0] - x;
                         RZ[i * nout + j] = rz;
                         if (RH) RH[i * nout + j] = rz * silu_prime(u[1]);
                     });
    }

    // ---- U^y half of its backward: dk, dv partials into the record
    {
        const float* R = rec + rl.rr;
        const float* RZ = ws + cl.rz[L];
        float* RD = ws + cl.rd[L];
        float* dvy = rec + rl.dvy;
        for (int e = tid; e < n * d; e += kThreads) {
            const float s = bias_grad_prime(R[e], a.bias, a.bias_param) * RZ[e];
            RD[e] = s;
            dvy[e] = -s;
        }
    }
    __syncthreads();
    for (int l = L; l >= 1; --l) {
        const int nin = a.n[l - 1], nout = a.n[l];
        gemm<kMfma>(n, nin, n, MatA{ws + cl.mb[l], 1, C, nullptr}, MatB{ws + cl.hq[l - 1], nin, 1},
                    lds_gemm, [&](int i, int j, float x) { tmp[i * nin + j] = -x; });
        if (l > 1) {
            const float* Zk = rec + rl.zk[l - 1];
            const float* Gk = rec + rl.gk[l - 1];
            const float* RZp = ws + cl.rz[l - 1];
            float* RDp = ws + cl.rd[l - 1];
            gemm2<kMfma>(n, nin, nout, MatA{ws + cl.rd[l], nout, 1, nullptr},
                         MatB{th + a.off[l], nin, 1}, lds_gemm,
                         [&](int i, int j) {
                             const int o = i * nin + j;
                             return f32x4_t{tmp[o], Zk[o], Gk[o], RZp[o]};
                         },
                         [&](int i, int j, float x, f32x4_t u) {
                             RDp[i * nin + j] =
                                 (u[0] + x) * silu_prime(u[1]) + u[2] * silu_second(u[1]) * u[3];
                         });
        } else {
            float* dky = rec + rl.dky;
            gemm2<kMfma>(n, nin, nout, MatA{ws + cl.rd[1], nout, 1, nullptr},
                         MatB{th + a.off[1], nin, 1}, lds_gemm,
                         [&](int i, int j) { return tmp[i * nin + j]; },
                         [&](int i, int j, float x, float t) { dky[i * nin + j] = t + x; });
        }
    }

    // ---- the carry's increments that do not involve (Lt, Ls)
    for (int l = 1; l <= L; ++l) {
        const int nin = a.n[l - 1], nout = a.n[l];
        float* dLt = rec + rl.dlt + a.off[l];
        float* dLs = rec + rl.dls + a.off[l];
        const MatB Hq{ws + cl.hq[l - 1], nin, 1};
        gemm<kMfma>(nout, nin, n, MatA{ws + cl.dq[l], 1, nout, rec + rl.cb}, Hq, lds_gemm,
                    [&](int i, int j, float x) { dLs[(int64_t)i * nin + j] = -x; });
        gemm<kMfma>(nout, nin, n, MatA{ws + cl.dq[l], 1, nout, rec + rl.ca}, Hq, lds_gemm,
                    [&](int i, int j, float x) { dLt[(int64_t)i * nin + j] = x; });
        gemm2<kMfma>(nout, nin, n, MatA{ws + cl.rd[l], 1, nout, nullptr},
                     MatB{rec + rl.hk[l - 1], nin, 1}, lds_gemm,
                     [&](int i, int j) { return dLt[(int64_t)i * nin + j]; },
                     [&](int i, int j, float x, float t) { dLt[(int64_t)i * nin + j] = t + x; });
        if (l > 1)
            gemm2<kMfma>(nout, nin, n, MatA{rec + rl.dl[l], 1, nout, nullptr},
                         MatB{ws + cl.rh[l - 1], nin, 1}, lds_gemm,
                         [&](int i, int j) { return dLt[(int64_t)i * nin + j]; },
                         [&](int i, int j, float x, float t) { dLt[(int64_t)i * nin + j] = t + x; });
    }
}

// ---------------------------------------------------------------- the chain through (Lt, Ls)

template <bool kMfma>
__device__ __forceinline__ void seq_part(const BwdArgs& A, const Plan& pl, int64_t seq,
                                         float* lds_gemm) {
    __shared__ float s_gcn[256], s_gwn[256];     // cotangents of c_{n,j}, w_{n,j}
    __shared__ float s_crow[256], s_wrow[256];   // c_{n,j}, w_{n,j}
    __shared__ float s_red[12];
    __shared__ float s_dot[3];  // <Lt, theta_c>, <Lt, s_c>, <Ls, s_c> of the current chunk
    const ScanArgs& a = A.a;
    const RecLayout& rl = pl.rl;
    const SeqScr& sl = pl.sl;
    const Bases bs = bases_of(a, seq);
    const int tid = threadIdx.x;
    const int C = a.C, L = a.L, d = a.n[0];
    const int64_t P = a.P, PH = ck_half(P);
    const float* ck = pl.ckpt + seq * pl.nch * 2 * PH;
    float* ws = pl.sscr + seq * sl.per;
    float* tmp = ws + sl.tmp;
    float* Lt = A.dtheta0 + bs.st;
    float* Ls = A.ds0 + bs.st;
    if (pl.last_segment) {  // (Lt, Ls) start as (dtheta_T, ds_T); products for the last chunk
        const float* dT = A.dthetaT ? A.dthetaT + bs.st : nullptr;
        const float* dS = A.dsT ? A.dsT + bs.st : nullptr;
        for (int64_t i = tid; i < P; i += kThreads) {
            if (dT != Lt) Lt[i] = dT ? dT[i] : 0.0f;
            if (dS != Ls) Ls[i] = dS ? dS[i] : 0.0f;
        }
        __syncthreads();
        const float* th = ck + (pl.nch - 1) * 2 * PH;
        const float* mo = th + PH;
        float x = 0.0f, y = 0.0f, z = 0.0f;
        for (int64_t i = tid; i < P; i += kThreads) {
            x = fmaf(Lt[i], th[i], x);
            y = fmaf(Lt[i], mo[i], y);
            z = fmaf(Ls[i], mo[i], z);
        }
        block_sum3(x, y, z, s_red);
        if (tid == 0) { s_dot[0] = x; s_dot[1] = y; s_dot[2] = z; }
    } else if (tid < 3) {
        s_dot[tid] = ws[sl.dots + tid];
    }
    __syncthreads();

    for (int cs = pl.rs.count - 1; cs >= 0; --cs) {
        const int64_t ci = pl.rs.first + cs;
        const int64_t c0 = ci * C;
        const int n = (int)((a.T - c0) < C ? (a.T - c0) : C);
        const float* th = ck + ci * 2 * PH;
        float* rec = pl.rs.rec + (seq * pl.seg + cs) * rl.per;
        for (int t = tid; t < n; t += kThreads) {
            s_gcn[t] = 0.0f;
            s_gwn[t] = 0.0f;
            s_crow[t] = rec[rl.cm + (int64_t)n * C + t];
            s_wrow[t] = rec[rl.wm + (int64_t)n * C + t];
        }
        if (tid == 0) {
            rec[rl.ga + n] = s_dot[0];
            rec[rl.gb + n] = -s_dot[1];
            rec[rl.gp] = s_dot[2];
        }
        __syncthreads();

        // ---- chunk-end products: U^e_l Hk_{l-1} starts RZ_l; dc_n, dw_n
        for (int l = 1; l <= L; ++l) {
            const int nin = a.n[l - 1], nout = a.n[l];
            const float* Dl = rec + rl.dl[l];
            float* RZ = ws + sl.rz[l];
            const MatA Hk{rec + rl.hk[l - 1], nin, 1, nullptr};
            gemm2<kMfma>(n, nout, nin, Hk, MatB{Lt + a.off[l], 1, nin}, lds_gemm,
                         [&](int i, int j) { return Dl[i * nout + j]; },
                         [&](int i, int j, float x, float dl) {
                             RZ[i * nout + j] = -s_crow[i] * x;
                             atomicAdd(&s_gcn[i], -x * dl);
                         });
            gemm2<kMfma>(n, nout, nin, Hk, MatB{Ls + a.off[l], 1, nin}, lds_gemm,
                         [&](int i, int j) { return f2_t{RZ[i * nout + j], Dl[i * nout + j]}; },
                         [&](int i, int j, float x, f2_t u) {
                             RZ[i * nout + j] = u[0] + s_wrow[i] * x;
                             atomicAdd(&s_gwn[i], x * u[1]);
                         });
        }

        // ---- U^e half of the key tangent pass
        for (int l = 1; l <= L; ++l) {
            const int nin = a.n[l - 1], nout = a.n[l];
            float* RZ = ws + sl.rz[l];
            const float* Zk = l < L ? rec + rl.zk[l] : nullptr;
            float* RH = l < L ? ws + sl.rh[l] : nullptr;
            if (l > 1) {
                gemm2<kMfma>(n, nout, nin, MatA{ws + sl.rh[l - 1], nin, 1, nullptr},
                             MatB{th + a.off[l], 1, nin}, lds_gemm,
                             [&](int i, int j) {
                                 return f2_t{RZ[i * nout + j], Zk ? Zk[i * nout + j] : 0.0f};
                             },
                             [&](int i, int j, float x, f2_t u) {
                                 const float rz = u[0] + x;
                                 RZ[i * nout + j] = rz;
                                 if (RH) RH[i * nout + j] = rz * silu_prime(u[1]);
                             });
            } else if (RH) {
                for (int e = tid; e < n * nout; e += kThreads) RH[e] = RZ[e] * silu_prime(Zk[e]);
                __syncthreads();
            }
        }

        // ---- U^e half of its backward; dk, dv final
        {
            const float* R = rec + rl.rr;
            const float* RZ = ws + sl.rz[L];
            const float* dvy = rec + rl.dvy;
            float* RD = ws + sl.rd[L];
            for (int e = tid; e < n * d; e += kThreads) {
                const int t = e / d, c = e % d;
                const float s = bias_grad_prime(R[e], a.bias, a.bias_param) * RZ[e];
                RD[e] = s;
                store_io(A.dv, bs.q + (c0 + t) * a.qs[1] + c, a.io, dvy[e] - s);
            }
        }
        __syncthreads();
        for (int l = L; l >= 1; --l) {
            const int nin = a.n[l - 1], nout = a.n[l];
            const float* Dl = rec + rl.dl[l];
            gemm<kMfma>(n, nin, nout, MatA{Dl, nout, 1, nullptr}, MatB{Lt + a.off[l], nin, 1},
                        lds_gemm, [&](int i, int j, float x) { tmp[i * nin + j] = -s_crow[i] * x; });
            gemm2<kMfma>(n, nin, nout, MatA{Dl, nout, 1, nullptr}, MatB{Ls + a.off[l], nin, 1},
                         lds_gemm, [&](int i, int j) { return tmp[i * nin + j]; },
                         [&](int i, int j, float x, float t) { tmp[i * nin + j] = t + s_wrow[i] * x; });
            if (l > 1) {
                const float* Zk = rec + rl.zk[l - 1];
                const float* Gk = rec + rl.gk[l - 1];
                const float* RZp = ws + sl.rz[l - 1];
                float* RDp = ws + sl.rd[l - 1];
                gemm2<kMfma>(n, nin, nout, MatA{ws + sl.rd[l], nout, 1, nullptr},
                             MatB{th + a.off[l], nin, 1}, lds_gemm,
                             [&](int i, int j) {
                                 const int o = i * nin + j;
                                 return f32x4_t{tmp[o], Zk[o], Gk[o], RZp[o]};
                             },
                             [&](int i, int j, float x, f32x4_t u) {
                                 RDp[i * nin + j] =
                                     (u[0] + x) * silu_prime(u[1]) + u[2] * silu_second(u[1]) * u[3];
                             });
            } else {
                const float* dky = rec + rl.dky;
                gemm2<kMfma>(n, nin, nout, MatA{ws + sl.rd[1], nout, 1, nullptr},
                             MatB{th + a.off[1], nin, 1}, lds_gemm,
                             [&](int i, int j) { return f2_t{tmp[i * nin + j], dky[i * nin + j]}; },
                             [&](int i, int j, float x, f2_t u) {
                                 store_io(A.dk, bs.q + (c0 + i) * a.qs[1] + j, a.io, u[1] + u[0] + x);
                             });
            }
        }

        // ---- carry (Lt, Ls) to the chunk start; the next chunk's state products ride along
        // in the epilogues that write the final values (its checkpoint is chunk ci - 1's)
        {
            const float an = rec[rl.ca + n], bn = rec[rl.cb + n], pn = rec[rl.cp + n];
            const bool dots = ci > 0;
            const float* thp = dots ? ck + (ci - 1) * 2 * PH : ck;
            const float* mop = thp + PH;
            const float* dLt0 = rec + rl.dlt;
            const float* dLs0 = rec + rl.dls;
            float dx = 0.0f, dy = 0.0f, dz = 0.0f;
            for (int l = 1; l <= L; ++l) {
                const int nin = a.n[l - 1], nout = a.n[l];
                const int64_t off = a.off[l];
                const bool fin = l == 1;  // this product writes the layer's final Lt
                // Ls is elementwise; it rides in the first product's epilogue
                gemm2<kMfma>(
                    nout, nin, n, MatA{ws + sl.rd[l], 1, nout, nullptr},
                    MatB{rec + rl.hk[l - 1], nin, 1}, lds_gemm,
                    [&](int i, int j) {
                        const int64_t o = off + (int64_t)i * nin + j;
                        return f32x4_t{Lt[o], Ls[o], dLt0[o], dLs0[o]};
                    },
                    [&](int i, int j, float x, f32x4_t u) {
                        const int64_t o = off + (int64_t)i * nin + j;
                        const float ls = pn * u[1] - bn * u[0] + u[3];
                        const float lt = an * u[0] + u[2] + x;
                        Ls[o] = ls;
                        Lt[o] = lt;
                        if (dots) {
                            const float tp = thp[o], sp = mop[o];
                            dz = fmaf(ls, sp, dz);
                            if (fin) {
                                dx = fmaf(lt, tp, dx);
                                dy = fmaf(lt, sp, dy);
                            }
                        }
                    });
                if (!fin)
                    gemm2<kMfma>(nout, nin, n, MatA{rec + rl.dl[l], 1, nout, nullptr},
                                 MatB{ws + sl.rh[l - 1], nin, 1}, lds_gemm,
                                 [&](int i, int j) {
                                     const int64_t o = off + (int64_t)i * nin + j;
                                     return f32x4_t{Lt[o], dots ? thp[o] : 0.0f,
                                                    dots ? mop[o] : 0.0f, 0.0f};
                                 },
                                 [&](int i, int j, float x, f32x4_t u) {
                                     const float lt = u[0] + x;
                                     Lt[off + (int64_t)i * nin + j] = lt;
                                     dx = fmaf(lt, u[1], dx);
                                     dy = fmaf(lt, u[2], dy);
                                 });
            }
            if (dots) {
                block_sum3(dx, dy, dz, s_red);
                if (tid == 0) { s_dot[0] = dx; s_dot[1] = dy; s_dot[2] = dz; }
            }
        }
        for (int t = tid; t < n; t += kThreads) {
            rec[rl.gc + (int64_t)n * C + t] = s_gcn[t];
            rec[rl.gw + (int64_t)n * C + t] = s_gwn[t];
        }
        __syncthreads();
    }
    if (tid < 3) ws[sl.dots + tid] = s_dot[tid];
}

// ---------------------------------------------------------------- gate cotangents

__device__ __forceinline__ void gate_part(const BwdArgs& A, const Plan& pl, int64_t blk) {
    __shared__ float s_al[256], s_et[256], s_be[256];
    __shared__ float s_abar[257], s_bbar[257], s_pbar[257];
    const ScanArgs& a = A.a;
    const RecLayout& rl = pl.rl;
    const int64_t seq = blk / pl.rg.count;
    const int cs = (int)(blk - seq * pl.rg.count);
    const int64_t ci = pl.rg.first + cs;
    const Bases bs = bases_of(a, seq);
    const int tid = threadIdx.x;
    const int C = a.C;
    const int64_t c0 = ci * C;
    const int n = (int)((a.T - c0) < C ? (a.T - c0) : C);
    float* rec = pl.rg.rec + (seq * pl.seg + cs) * rl.per;
    const float* ca = rec + rl.ca;
    const float* cb = rec + rl.cb;
    const float* cp = rec + rl.cp;
    const float* cm = rec + rl.cm;
    const float* wm = rec + rl.wm;
    float* gc = rec + rl.gc;
    float* gw = rec + rl.gw;
    stage_gates(a, bs, c0, n, s_al, s_et, s_be);
    __syncthreads();
    if (tid < n) {  // column j: cotangents of c_{t,j} (in place in gc) and w_{t,j} (into gw)
        const int j = tid;
        float cr = gc[(int64_t)n * C + j], wr = gw[(int64_t)n * C + j];
        for (int t0 = n - 1; t0 >= 0; t0 -= 8) {
            float yv[8];  // the U^y terms of eight rows, loaded before any store
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 - u;
                yv[u] = gc[(int64_t)(t >= 0 ? t : 0) * C + j];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 - u;
                if (t < 0) break;
                wr = fmaf(s_et[t], cr, wr);                   // of w_{t+1,j}, complete
                gw[(int64_t)(t + 1) * C + j] = wr;
                cr = yv[u] + (1.0f - s_al[t]) * cr;           // of c_{t,j}
                gc[(int64_t)t * C + j] = cr;
                wr *= s_be[t];
            }
        }
    }
    if (tid == kThreads - 1) {  // cotangents of a_t, b_t, p_t
        float ab = rec[rl.ga + n], bb = rec[rl.gb + n], pb = rec[rl.gp];
        for (int t = n - 1; t >= 0; --t) {
            pb = fmaf(s_et[t], bb, pb);
            s_abar[t + 1] = ab;
            s_bbar[t + 1] = bb;
            s_pbar[t + 1] = pb;
            const float keep = 1.0f - s_al[t];
            ab = rec[rl.ga + t] + keep * ab;
            bb = rec[rl.gb + t] + keep * bb;
            pb *= s_be[t];
        }
    }
    __syncthreads();
    if (tid < n) {
        const int t = tid;
        const float* cn = gc + (int64_t)(t + 1) * C;
        const float* wn = gw + (int64_t)(t + 1) * C;
        const float* ct = cm + (int64_t)t * C;
        const float* w1 = wm + (int64_t)(t + 1) * C;
        const float* w0 = wm + (int64_t)t * C;
        float sa = 0.0f, se = 0.0f, sb = 0.0f;
        for (int j = 0; j < t; ++j) {
            sa = fmaf(cn[j], ct[j], sa);
            sb = fmaf(wn[j], w0[j], sb);
        }
        for (int j = 0; j <= t; ++j) se = fmaf(cn[j], w1[j], se);
        const int64_t gi = bs.g + (c0 + t) * a.gs[1];
        A.dalpha[gi] = -s_abar[t + 1] * ca[t] - s_bbar[t + 1] * cb[t] - sa;
        A.deta[gi] = s_bbar[t + 1] * cp[t + 1] + se;
        A.dbeta[gi] = s_pbar[t + 1] * cp[t] + sb - wn[t];
    }
}

// One launch: the seq part (workgroups 0 .. B*H - 1 when it runs) beside the chunk and gate
// parts of other segments.  Each workgroup takes exactly one role and every role ends.
template <bool kMfma>
__global__ void __launch_bounds__(kThreads, 2) bwd_step_kernel(BwdArgs A, Plan pl) {
    __shared__ __align__(16) float lds_gemm[kGemmLds];
    const int64_t blk = blockIdx.x;
    if (pl.rs.count > 0 && blk >= pl.rs.blk0 && blk < pl.rc.blk0)
        seq_part<kMfma>(A, pl, blk - pl.rs.blk0, lds_gemm);
    else if (pl.rc.count > 0 && blk >= pl.rc.blk0 && blk < pl.rg.blk0)
        chunk_part<kMfma>(A, pl, blk - pl.rc.blk0, lds_gemm);
    else if (pl.rg.count > 0 && blk >= pl.rg.blk0)
        gate_part(A, pl, blk - pl.rg.blk0);
}

// T = 0: the state cotangents pass through.
__global__ void bwd_copy_kernel(BwdArgs A) {
    const ScanArgs& a = A.a;
    const int64_t seq = blockIdx.y;
    const int64_t b = seq / a.H, h = seq % a.H;
    const int64_t o = b * a.ss[0] + h * a.ss[1];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.P;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float* dT = A.dthetaT ? A.dthetaT + o : nullptr;
        const float* dS = A.dsT ? A.dsT + o : nullptr;
        if (A.dtheta0 + o != dT) A.dtheta0[o + i] = dT ? dT[i] : 0.0f;
        if (A.ds0 + o != dS) A.ds0[o + i] = dS ? dS[i] : 0.0f;
    }
}

}  // namespace

size_t scan_backward_workspace_bytes(const ScanArgs& a) {
    const Plan p = make_plan(a);
    return plan_floats(a, p) * sizeof(float);
}

hipError_t launch_scan_backward(const BwdArgs& A, hipStream_t stream) {
    const ScanArgs& a = A.a;
    const int64_t nseq = a.B * a.H;
    if (nseq == 0) return hipSuccess;
    if (a.T == 0) {
        dim3 grid((unsigned)((a.P + 255) / 256 < 64 ? (a.P + 255) / 256 : 64), (unsigned)nseq);
        bwd_copy_kernel<<<grid, 256, 0, stream>>>(A);
        return hipGetLastError();
    }
    Plan p = make_plan(a);
    place(a, p);
    bwd_forward_kernel<false><<<dim3((unsigned)nseq), kThreads, 0, stream>>>(A, p);
    const int64_t nseg = (p.nch + p.seg - 1) / p.seg;
    // role of segment s (count 0 outside 0 .. nseg-1); segment s keeps record buffer s % 3
    auto role = [&](int64_t s) {
        Role r{};
        if (s < 0 || s >= nseg) return r;
        r.first = s * p.seg;
        r.count = (int)((p.nch - r.first) < p.seg ? (p.nch - r.first) : p.seg);
        r.rec = p.recs + (s % kRecBufs) * nseq * p.seg * p.rl.per;
        return r;
    };
    // launch i (i = 0 .. nseg + 1): seq part of segment nseg - i, chunk part of segment
    // nseg - 1 - i, gate part of segment nseg + 1 - i
    for (int64_t i = 0; i <= nseg + 1; ++i) {
        const int64_t s = nseg - i;
        p.rs = role(s);
        p.rc = role(s - 1);
        p.rg = role(s + 1);
        p.last_segment = s == nseg - 1;
        const int64_t ns = p.rs.count ? nseq : 0;
        p.rs.blk0 = 0;
        p.rc.blk0 = ns;
        p.rg.blk0 = ns + nseq * p.rc.count;
        const int64_t blocks = p.rg.blk0 + nseq * p.rg.count;
        if (blocks == 0) continue;
        bwd_step_kernel<false><<<dim3((unsigned)blocks), kThreads, 0, stream>>>(A, p);
    }
    return hipGetLastError();
}

}  // namespace titans
