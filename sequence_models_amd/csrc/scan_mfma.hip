// Fused chunked Titans memory scan on gfx950 MFMA, for the 64 -> 256 -> 64 SiLU
// memory with chunks of 64 tokens and bf16 q/k/v/y (fp32 gates and state).
//
// One 256-thread workgroup owns one (b, h) memory for the whole sequence.  Wave
// w (0..3) owns hidden units 64w .. 64w+63: rows 64w.. of W1 / S1 and columns
// 64w.. of W2 / S2.  Those fp32 weights and momenta stay in registers as MFMA
// accumulators from the first token to the last; nothing of the state goes
// back to HBM until the sequence ends.
//
// Per chunk (chunk-start weights W, momenta S; rows of the C x . matrices are
// tokens; the algebra is the unrolled momentum / forget-gated write rule of the
// Titans pages with gradients frozen at the chunk start, each gradient being
// an outer product delta h^T):
//   coefficients  a_t, b_t, c_{t,j} (strictly lower), p, w_j from the gates
//                 (column recurrence, one lane per column)
//   key forward   Z = K W1^T, Hk = SiLU(Z), O = Hk W2^T
//   backward      E2 = 2 (O - V), D1 = (E2 W2) o SiLU'(Z)
//   reads         Zq = diag(a) Q W1^T - diag(b) Q S1^T - (Cm o Q K^T) D1
//                 Hq = SiLU(Zq)
//                 Y  = diag(a) Hq W2^T - diag(b) Hq S2^T - (Cm o Hq Hk^T) E2
//   carry         W1 <- a_C W1 - b_C S1 - D1^T diag(c_C) K,  S1 <- p S1 + D1^T diag(w) K
//                 W2 <- a_C W2 - b_C S2 - E2^T diag(c_C) Hk, S2 <- p S2 + E2^T diag(w) Hk
// Every product is a bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation.
// O and Y are sums over the four waves' hidden slices; they are reduced through
// LDS in a fixed order ((w0 + w2) + (w1 + w3) for O, (w0 + w1) + (w2 + w3) for Y),
// so the result is bitwise reproducible.
//
// Operand layouts.  For the 16x16x32 MFMA lane l (g = l / 16, j = l % 16) holds
// A[j][k], B[k][j] for eight k of a 32-wide block and D[4g + r][j], r = 0..3.
// An accumulator block is reused as an operand without leaving registers when
// its row index is the next product's reduction index: the eight k-slots of
// lane (g, j) are then rows {4g .. 4g+3} of the block's first 16-row tile and
// {16+4g .. 16+4g+3} of its second.  Every product uses that k order, so LDS
// fragments are read as two 8-byte pieces at columns 4g and 16 + 4g of a
// k-contiguous row.  LDS matrices are 64 x 64 with rows padded to 68 elements:
// the 16 rows a fragment read touches then start in distinct banks, and every
// LDS address is one per-lane base register plus an immediate offset.
#include <hip/hip_runtime.h>

#include "mfma_util.h"
#include "titans_internal.h"

namespace titans {
namespace {

using namespace fused;

constexpr int kD = 64;       // key / value / query width
constexpr int kHid = 256;    // hidden width of the memory MLP
constexpr int kC = 64;       // chunk length
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

constexpr int kMat = kC * kLd;  // elements of one padded 64 x 64 matrix

struct __attribute__((aligned(16))) Smem {
    // Regions are reused within a chunk; the comment gives each region's lives in order.
    float r[2][kMat];          // O partials (pairwise reduction) -> the waves' bf16 W2 slices
                               //   -> Y^T partial slots 0, 1   ([c][dd] fp32)
    __bf16 qa[kMat];           // raw Q -> diag(a) Q [c][d]     } Y^T partial slot 2
    __bf16 qb[kMat];           // -diag(b) Q [c][d]             }
    __bf16 mq[kMat];           // -(Cm o Q K^T) [c][c']         } Y^T partial slot 3
    __bf16 e2l[kMat];          // K [c][d] -> E2 [c][dd]        }
    __bf16 e2t[kMat];          // E2^T [dd][c]
    __bf16 e2c[kMat];          // -(diag(c_C) E2)^T [dd][c]
    __bf16 e2w[kMat];          // (diag(w) E2)^T [dd][c]
    __bf16 kc[kMat];           // -(diag(c_C) K)^T [d][c]
    __bf16 kw[kMat];           // (diag(w) K)^T    [d][c]
    __bf16 hk[kWaves][kMat];   // each wave's Hk slice [c][h]
    __bf16 cm[kMat];           // c_{t,j}, t, j < 64 (rows t)
    float a[kC + 4], b[kC + 4];
    float cc[kC], w[kC], inva[kC];
    float et[kC], omb[kC];
    float la2[kC + 4];         // sum_{m<t} log2(1 - alpha_m), t = 0..64
    float la2i[kC];            // sum_{m<=t} log2(1 - alpha_m)
    float lb2[kC];             // sum_{m<=t} log2(beta_m)
    float p;
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");

// The four private Y^T partial slots (64 x 64 fp32 each).
__device__ __forceinline__ float* yslot(Smem& sm, int w) {
    switch (w) {
        case 0: return sm.r[0];
        case 1: return sm.r[1];
        case 2: return reinterpret_cast<float*>(sm.qa);
        default: return reinterpret_cast<float*>(sm.mq);
    }
}

__global__ void __launch_bounds__(kThreads, 1) scan_mfma_kernel(ScanArgs A) {
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int wv = tid >> 6, l = tid & 63, g = l >> 4, j = l & 15;
    const int64_t seq = blockIdx.x;
    const int64_t bi = seq / A.H, hi = seq % A.H;

    const float* th0 = A.theta0 + bi * A.s0s[0] + hi * A.s0s[1];
    const float* mo0 = A.s0 + bi * A.s0s[0] + hi * A.s0s[1];
    float* thT = A.thetaT + bi * A.ss[0] + hi * A.ss[1];
    float* moT = A.sT + bi * A.ss[0] + hi * A.ss[1];
    constexpr int kOff2 = kHid * kD;  // W2 follows W1 (256 x 64) in a memory

    // ---- state: W1T[dt][ht] = W1[h][d] (rows d = 16dt+4g+r, cols h = 64wv+16ht+j),
    //             W2T[ht][dt] = W2[dd][h] (rows h = 64wv+16ht+4g+r, cols dd = 16dt+j)
    f32x4 W1T[4][4], S1T[4][4], W2T[4][4], S2T[4][4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
            const int h = 64 * wv + 16 * ht + j;
            const int d = 16 * dt + 4 * g;
            W1T[dt][ht] = *reinterpret_cast<const f32x4*>(th0 + h * kD + d);
            S1T[dt][ht] = *reinterpret_cast<const f32x4*>(mo0 + h * kD + d);
            const int h2 = 64 * wv + 16 * ht + 4 * g;
            const int dd = 16 * dt + j;
            W2T[ht][dt] = *reinterpret_cast<const f32x4*>(th0 + kOff2 + dd * kHid + h2);
            S2T[ht][dt] = *reinterpret_cast<const f32x4*>(mo0 + kOff2 + dd * kHid + h2);
            tile_fence();
        }

    const __bf16* qg = static_cast<const __bf16*>(A.q);
    const __bf16* kg = static_cast<const __bf16*>(A.k);
    const __bf16* vg = static_cast<const __bf16*>(A.v);
    __bf16* yg = static_cast<__bf16*>(A.y);
    const int64_t qbase = bi * A.qs[0] + hi * A.qs[2];
    const int64_t ybase = bi * A.ys[0] + hi * A.ys[2];
    const int64_t gbase = bi * A.gs[0] + hi * A.gs[2];
    // this thread's slice of a chunk's 64 x 64 token tiles: row rc, columns cl0 .. cl0+15
    const int rc = tid >> 2, cl0 = 16 * (tid & 3);

    // prefetch registers (the next chunk's K, Q rows and gates)
    bf16x8 kpre[2], qpre[2];
    float gpre[3] = {0.f, 0.f, 1.f};
    auto prefetch = [&](int64_t t0) {
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
        {
            const int64_t tt = t0 + l;
            if (tt < A.T) {
                const int64_t go = gbase + tt * A.gs[1];
                gpre[0] = A.alpha[go];
                gpre[1] = A.eta[go];
                gpre[2] = A.beta[go];
            } else {  // padding tokens: no decay, no write, momentum kept
                gpre[0] = 0.f;
                gpre[1] = 0.f;
                gpre[2] = 1.f;
            }
        }
    };
    prefetch(0);

    for (int64_t c0 = 0; c0 < A.T; c0 += kC) {
        const int n = (int)((A.T - c0) < kC ? (A.T - c0) : kC);
        // ================= P0: commit the prefetched chunk; load V
        {
            const int xb = opq(rc * kLd + cl0);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                *reinterpret_cast<bf16x4*>(sm.e2l + xb + 4 * q4) = half4(kpre[q4 >> 1], q4 & 1);
                *reinterpret_cast<bf16x4*>(sm.qa + xb + 4 * q4) = half4(qpre[q4 >> 1], q4 & 1);
            }
        }
        {
            // Gate prefixes over the chunk's tokens (lane l = token l; every wave holds the
            // gates, each wave runs its share of the lane-parallel DPP scans):
            //   a_t = prod_{m<t} (1 - alpha_m),  p = prod_m beta_m,
            //   b_{t+1} = (1 - alpha_t) b_t + eta_t prod_{m<=t} beta_m,
            //   la2 / lb2: log2 prefix sums of (1 - alpha) and beta for the coefficient matrix
            //   (a zero factor stays exactly zero through exp2 of a very negative exponent).
            const float keep = 1.f - gpre[0], et_l = gpre[1], be_l = gpre[2];
            if (wv == 0) {
                const float pa = wave_scan_mul(keep);
                const float a_l = lane_prev(pa, 1.f);
                sm.a[l] = a_l;
                sm.inva[l] = 1.f / a_l;
                if (l == 63) sm.a[kC] = pa;
            } else if (wv == 1) {
                const float pbl = wave_scan_mul(be_l);
                sm.lb2[l] = wave_scan_add(be_l > 0.f ? __log2f(be_l) : -1024.f);
                if (l == 63) sm.p = pbl;
            } else if (wv == 2) {
                const float lk = wave_scan_add(keep > 0.f ? __log2f(keep) : -1024.f);
                sm.la2[l] = lane_prev(lk, 0.f);
                sm.la2i[l] = lk;
                if (l == 63) sm.la2[kC] = lk;
            } else {
                float mk = keep, mc = et_l * wave_scan_mul(be_l);
                wave_scan_affine(mk, mc);  // affine maps x -> keep_t x + eta_t p_t, composed
                sm.b[l] = lane_prev(mc, 0.f);
                sm.et[l] = et_l;
                sm.omb[l] = 1.f - be_l;
                if (l == 63) sm.b[kC] = mc;
            }
        }
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

        // ================= P1: coefficients (wave 0); key forward and O partials (all)
        // Coefficient matrix c_{t,j} = sum_{j<=i<t} L1[t][i] L2[i][j] with
        //   L1[t][i] = prod_{i<m<t} (1 - alpha_m),  L2[i][j] = eta_i (1 - beta_j) prod_{j<m<=i} beta_m,
        // every entry an exp2 of a difference of log2 prefix sums (positive terms only),
        // the sum one bf16 MFMA product.  Row C of L1 gives the chunk-end row c_C.
        __bf16* l1m = sm.e2t;   // L1 [t][i]
        __bf16* l2t = sm.e2c;   // L2^T [j][i]
        __bf16* l1c = sm.e2w;   // row 0: L1[C][i] (rows 1..15 unused)
        {
            const int xb = opq(rc * kLd + cl0);
            const float lat = sm.la2[rc], lbj = sm.lb2[rc], ombj = sm.omb[rc];
            bf16x8 v1[2], v2[2];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 la = *reinterpret_cast<const f32x4*>(sm.la2i + cl0 + 4 * q4);
                const f32x4 lbv = *reinterpret_cast<const f32x4*>(sm.lb2 + cl0 + 4 * q4);
                const f32x4 etv = *reinterpret_cast<const f32x4*>(sm.et + cl0 + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = cl0 + 4 * q4 + e;
                    // out-of-triangle exponents may be +inf; the select discards them
                    const float x1 = __builtin_amdgcn_exp2f(lat - la[e]);
                    const float x2 = etv[e] * __builtin_amdgcn_exp2f(lbv[e] - lbj) * ombj;
                    v1[q4 >> 1][(q4 & 1) * 4 + e] = (__bf16)(i < rc ? x1 : 0.f);
                    v2[q4 >> 1][(q4 & 1) * 4 + e] = (__bf16)(i >= rc ? x2 : 0.f);
                }
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                *reinterpret_cast<bf16x8*>(l1m + xb + 8 * q) = v1[q];
                *reinterpret_cast<bf16x8*>(l2t + xb + 8 * q) = v2[q];
            }
            if (wv == 0) {
                l1c[l] = (__bf16)__builtin_amdgcn_exp2f(sm.la2[kC] - sm.la2i[l]);
                sm.w[l] = sm.omb[l] * __builtin_amdgcn_exp2f(sm.lb2[kC - 1] - sm.lb2[l]);
            }
        }
        __syncthreads();  // B1b
        {
            // Cm^T[j][t] = sum_i L2^T[j][i] L1^T[i][t]: wave w owns column tile t in 16w..16w+15
            const int rb = opq(j * kLd + 4 * g);
            const __bf16* l2r = l2t + rb;
            const __bf16* l1r = l1m + rb;
            __bf16* cmw = sm.cm + rb + 16 * wv * kLd;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                f32x4 x = zero4();
                if (jt <= wv) {
                    x = mfma(frag(l2r, fo(jt, 0)), frag(l1r, fo(wv, 0)), x);
                    x = mfma(frag(l2r, fo(jt, 1)), frag(l1r, fo(wv, 1)), x);
                }
                *reinterpret_cast<bf16x4*>(cmw + 16 * jt) = bf4(x);
            }
            if (wv == 0) {
                const __bf16* l1cr = l1c + rb;
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    f32x4 x = mfma(frag(l2r, fo(jt, 0)), frag(l1cr, 0), zero4());
                    x = mfma(frag(l2r, fo(jt, 1)), frag(l1cr, 32), x);
                    if (j == 0) *reinterpret_cast<f32x4*>(sm.cc + 16 * jt + 4 * g) = x;
                }
            }
        }
        // Z = K W1^T (rows c, cols h), one column tile of hidden units at a time
        bf16x4 Hk[4][4], Sp[4][4];
        {
            const int rb = opq(j * kLd + 4 * g), wb = opq(4 * g * kLd + j);
            const __bf16* ks = sm.e2l + rb;
            __bf16* hkw = sm.hk[wv] + wb;
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
                const bf16x8 bw0 = state_frag(W1T[0][ht], W1T[1][ht]);
                const bf16x8 bw1 = state_frag(W1T[2][ht], W1T[3][ht]);
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
                    }
                    Hk[ct][ht] = bf4(hk);
                    Sp[ct][ht] = bf4(sp);
#pragma unroll
                    for (int r = 0; r < 4; ++r) hkw[(16 * ct + r) * kLd + 16 * ht] = Hk[ct][ht][r];
                    tile_fence();
                }
            }
        }
        wave_lds_sync();
        // O^T partial over this wave's hidden slice: O^T[dd][c] = sum_h W2[dd][h] Hk[c][h]
        f32x4 Ot[4][4];
        {
            const int rb = opq(j * kLd + 4 * g);
            const __bf16* hkr = sm.hk[wv] + rb;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x8 a0 = state_frag(W2T[0][dt], W2T[1][dt]);
                const bf16x8 a1 = state_frag(W2T[2][dt], W2T[3][dt]);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    Ot[dt][ct] = mfma(a0, frag(hkr, fo(ct, 0)), zero4());
                    Ot[dt][ct] = mfma(a1, frag(hkr, fo(ct, 1)), Ot[dt][ct]);
                    tile_fence();
                }
            }
            // deterministic pairwise reduction, stage 1: waves 2, 3 store their partials
            if (wv >= 2) {
                float* slot = sm.r[wv - 2] + rb;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        *reinterpret_cast<f32x4*>(slot + 16 * ct * kLd + 16 * dt) = Ot[dt][ct];
            }
        }
        __syncthreads();  // B2: coefficients, O stage 1

        // ================= P2: stage 2 of O; scaled Q and K copies; Mq
        if (wv < 2) {
            float* slot = sm.r[wv] + opq(j * kLd + 4 * g);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    f32x4* p = reinterpret_cast<f32x4*>(slot + 16 * ct * kLd + 16 * dt);
                    *p = Ot[dt][ct] + *p;
                }
        }
        {
            const float ar = sm.a[rc], br = -sm.b[rc];
            const float ccr = -sm.cc[rc], wr = sm.w[rc];
            const int xb = opq(rc * kLd + cl0), xt = opq(cl0 * kLd + rc);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 qv = f4(*reinterpret_cast<const bf16x4*>(sm.qa + xb + 4 * q4));
                *reinterpret_cast<bf16x4*>(sm.qa + xb + 4 * q4) = bf4(qv * ar);
                *reinterpret_cast<bf16x4*>(sm.qb + xb + 4 * q4) = bf4(qv * br);
                const f32x4 kv = f4(*reinterpret_cast<const bf16x4*>(sm.e2l + xb + 4 * q4));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sm.kc[xt + (4 * q4 + e) * kLd] = (__bf16)(kv[e] * ccr);
                    sm.kw[xt + (4 * q4 + e) * kLd] = (__bf16)(kv[e] * wr);
                }
            }
        }
        wave_lds_sync();  // this wave's rows of diag(a) Q are the ones its Mq tile reads
        {
            // Mq[c][c'] = -(c_{c,c'} / a_c) (Qa K^T)[c][c'] for column tile c = 16 wv + j
            const int rb = opq(j * kLd + 4 * g);
            const __bf16* ks = sm.e2l + rb;
            const __bf16* qr = sm.qa + rb + 16 * wv * kLd;
            const __bf16* cmr = sm.cm + rb + 16 * wv * kLd;
            __bf16* mqw = sm.mq + rb + 16 * wv * kLd;
            const float ia = sm.inva[16 * wv + j];
#pragma unroll
            for (int ctp = 0; ctp < 4; ++ctp) {
                f32x4 x = zero4();
                if (ctp <= wv) {
                    x = mfma(frag(ks, fo(ctp, 0)), frag(qr, 0), x);
                    x = mfma(frag(ks, fo(ctp, 1)), frag(qr, 32), x);
                    const f32x4 cmv = f4(*reinterpret_cast<const bf16x4*>(cmr + 16 * ctp));
                    x = x * cmv * (-ia);
                }
                *reinterpret_cast<bf16x4*>(mqw + 16 * ctp) = bf4(x);
            }
        }
        __syncthreads();  // B3

        // ================= P3: E2 = loss'(O - V) (2 (O - V) for the squared error) in its
        // four layouts
        {
            const int xb = opq(rc * kLd + cl0), xt = opq(cl0 * kLd + rc);
            const float ccr = -sm.cc[rc], wr = sm.w[rc];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 o = *reinterpret_cast<const f32x4*>(sm.r[0] + xb + 4 * q4) +
                                *reinterpret_cast<const f32x4*>(sm.r[1] + xb + 4 * q4);
                const f32x4 v4 = f4(half4(vr[q4 >> 1], q4 & 1));
                const f32x4 e = bias_grad4(o - v4, A.bias, A.bias_param);
                *reinterpret_cast<bf16x4*>(sm.e2l + xb + 4 * q4) = bf4(e);
#pragma unroll
                for (int ee = 0; ee < 4; ++ee) {
                    const int o2 = xt + (4 * q4 + ee) * kLd;
                    sm.e2t[o2] = (__bf16)e[ee];
                    sm.e2c[o2] = (__bf16)(e[ee] * ccr);
                    sm.e2w[o2] = (__bf16)(e[ee] * wr);
                }
            }
        }
        __syncthreads();  // B4

        // ================= P4: backward, reads at the in-chunk weights
        // this wave's W2 slice as bf16 [h][dd] (B operand of G = E2 W2)
        __bf16* w2c = reinterpret_cast<__bf16*>(&sm.r[0][0]) + wv * kMat;
        {
            __bf16* w2w = w2c + opq(4 * g * kLd + j);
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x4 v = bf4(opaque(W2T[ht][dt]));
#pragma unroll
                    for (int r = 0; r < 4; ++r) w2w[(16 * ht + r) * kLd + 16 * dt] = v[r];
                    tile_fence();
                }
        }
        wave_lds_sync();
        // G = E2 W2 (rows c, cols h); D1 = G o SiLU'(Z)
        bf16x4 D1[4][4];
        {
            const int rb = opq(j * kLd + 4 * g);
            const __bf16* w2r = w2c + rb;
            const __bf16* er = sm.e2l + rb;
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
                const bf16x8 b0 = frag(w2r, fo(ht, 0));
                const bf16x8 b1 = frag(w2r, fo(ht, 1));
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    f32x4 gg = mfma(frag(er, fo(ct, 0)), b0, zero4());
                    gg = mfma(frag(er, fo(ct, 1)), b1, gg);
                    D1[ct][ht] = bf4(gg * f4(Sp[ct][ht]));
                }
            }
        }
        // Zq^T (rows h, cols c) = W1 (diag(a) Q)^T + S1 (-diag(b) Q)^T + D1^T Mq^T; Hq = SiLU
        bf16x4 Hq[4][4];
        {
            const int rb = opq(j * kLd + 4 * g);
            const __bf16* qar = sm.qa + rb;
            const __bf16* qbr = sm.qb + rb;
            const __bf16* mqr = sm.mq + rb;
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
                const bf16x8 aw0 = state_frag(W1T[0][ht], W1T[1][ht]);
                const bf16x8 aw1 = state_frag(W1T[2][ht], W1T[3][ht]);
                const bf16x8 as0 = state_frag(S1T[0][ht], S1T[1][ht]);
                const bf16x8 as1 = state_frag(S1T[2][ht], S1T[3][ht]);
                const bf16x8 ad0 = cat(D1[0][ht], D1[1][ht]);
                const bf16x8 ad1 = cat(D1[2][ht], D1[3][ht]);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    f32x4 zq = mfma(aw0, frag(qar, fo(ct, 0)), zero4());
                    zq = mfma(aw1, frag(qar, fo(ct, 1)), zq);
                    zq = mfma(as0, frag(qbr, fo(ct, 0)), zq);
                    zq = mfma(as1, frag(qbr, fo(ct, 1)), zq);
                    zq = mfma(ad0, frag(mqr, fo(ct, 0)), zq);
                    if (ct >= 2) zq = mfma(ad1, frag(mqr, fo(ct, 1)), zq);
                    f32x4 hq;
#pragma unroll
                    for (int r = 0; r < 4; ++r) hq[r] = zq[r] * sigmoid(zq[r]);
                    Hq[ht][ct] = bf4(hq);
                }
            }
        }
        __syncthreads();  // B5: Q, Mq, E2 [c][dd] and the W2 slices are dead -> Y slots
        // Y^T (rows dd, cols c) = a_c (W2 Hq^T) - b_c (S2 Hq^T) + E2^T Pm^T,
        // Pm^T[c'][c] = -c_{c,c'} (Hk Hq^T)[c'][c]; each wave stores its partial in its slot
        {
            const int rb = opq(j * kLd + 4 * g);
            bf16x4 pm[4][4];  // [ct][ctp]
            {
                const __bf16* hkr = sm.hk[wv] + rb;
                const __bf16* cmr = sm.cm + rb;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const bf16x8 bq0 = cat(Hq[0][ct], Hq[1][ct]);
                    const bf16x8 bq1 = cat(Hq[2][ct], Hq[3][ct]);
#pragma unroll
                    for (int ctp = 0; ctp < 4; ++ctp) {
                        f32x4 pt = zero4();
                        if (ctp <= ct) {
                            pt = mfma(frag(hkr, fo(ctp, 0)), bq0, pt);
                            pt = mfma(frag(hkr, fo(ctp, 1)), bq1, pt);
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
                const bf16x8 aw0 = state_frag(W2T[0][dt], W2T[1][dt]);
                const bf16x8 aw1 = state_frag(W2T[2][dt], W2T[3][dt]);
                const bf16x8 as0 = state_frag(S2T[0][dt], S2T[1][dt]);
                const bf16x8 as1 = state_frag(S2T[2][dt], S2T[3][dt]);
                const bf16x8 e0 = frag(etr, fo(dt, 0));
                const bf16x8 e1 = frag(etr, fo(dt, 1));
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const bf16x8 bq0 = cat(Hq[0][ct], Hq[1][ct]);
                    const bf16x8 bq1 = cat(Hq[2][ct], Hq[3][ct]);
                    const float ac = sm.a[16 * ct + j], bc = sm.b[16 * ct + j];
                    f32x4 u1 = mfma(aw0, bq0, zero4());
                    u1 = mfma(aw1, bq1, u1);
                    f32x4 u2 = mfma(as0, bq0, zero4());
                    u2 = mfma(as1, bq1, u2);
                    f32x4 yt = ac * u1 - bc * u2;
                    yt = mfma(e0, cat(pm[ct][0], pm[ct][1]), yt);
                    if (ct >= 2) yt = mfma(e1, cat(pm[ct][2], pm[ct][3]), yt);
                    *reinterpret_cast<f32x4*>(slot + 16 * ct * kLd + 16 * dt) = yt;
                }
            }
        }
        __syncthreads();  // B6: all Y partials stored

        // ================= P5: y out; carry the state to the next chunk
        if (rc < n) {
            const int xb = opq(rc * kLd + cl0);
            bf16x8 out[2];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int e = xb + 4 * q4;
                const f32x4 yv = (*reinterpret_cast<const f32x4*>(yslot(sm, 0) + e) +
                                  *reinterpret_cast<const f32x4*>(yslot(sm, 1) + e)) +
                                 (*reinterpret_cast<const f32x4*>(yslot(sm, 2) + e) +
                                  *reinterpret_cast<const f32x4*>(yslot(sm, 3) + e));
                const bf16x4 yb = bf4(yv);
#pragma unroll
                for (int k = 0; k < 4; ++k) out[q4 >> 1][(q4 & 1) * 4 + k] = yb[k];
            }
            const int64_t o = ybase + (c0 + rc) * A.ys[1] + cl0;
            *reinterpret_cast<bf16x8*>(yg + o) = out[0];
            *reinterpret_cast<bf16x8*>(yg + o + 8) = out[1];
        }
        __syncthreads();  // B7: the Y slots are read before the next chunk reuses them
        if (c0 + kC < A.T) prefetch(c0 + kC);
        {
            const float aC = sm.a[kC], bC = sm.b[kC], pC = sm.p;
            const int rb = opq(j * kLd + 4 * g);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x8 kc0 = frag(sm.kc + rb, fo(dt, 0));
                const bf16x8 kc1 = frag(sm.kc + rb, fo(dt, 1));
                const bf16x8 kw0 = frag(sm.kw + rb, fo(dt, 0));
                const bf16x8 kw1 = frag(sm.kw + rb, fo(dt, 1));
                const bf16x8 ec0 = frag(sm.e2c + rb, fo(dt, 0));
                const bf16x8 ec1 = frag(sm.e2c + rb, fo(dt, 1));
                const bf16x8 ew0 = frag(sm.e2w + rb, fo(dt, 0));
                const bf16x8 ew1 = frag(sm.e2w + rb, fo(dt, 1));
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) {
                    const bf16x8 bd0 = cat(D1[0][ht], D1[1][ht]);  // B: D1 [c][h]
                    const bf16x8 bd1 = cat(D1[2][ht], D1[3][ht]);
                    const bf16x8 ah0 = cat(Hk[0][ht], Hk[1][ht]);  // A: Hk^T [h][c]
                    const bf16x8 ah1 = cat(Hk[2][ht], Hk[3][ht]);
                    // chunk-end rescale (a_C W - b_C S, p S) fused into the accumulator input
                    const f32x4 tw1 = aC * W1T[dt][ht] - bC * S1T[dt][ht];
                    const f32x4 ts1 = pC * S1T[dt][ht];
                    W1T[dt][ht] = mfma(kc1, bd1, mfma(kc0, bd0, tw1));
                    S1T[dt][ht] = mfma(kw1, bd1, mfma(kw0, bd0, ts1));
                    const f32x4 tw2 = aC * W2T[ht][dt] - bC * S2T[ht][dt];
                    const f32x4 ts2 = pC * S2T[ht][dt];
                    W2T[ht][dt] = mfma(ah1, ec1, mfma(ah0, ec0, tw2));
                    S2T[ht][dt] = mfma(ah1, ew1, mfma(ah0, ew0, ts2));
                    tile_fence();
                }
            }
        }
    }

    // ---- final memory and momentum
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
            const int h = 64 * wv + 16 * ht + j;
            const int d = 16 * dt + 4 * g;
            *reinterpret_cast<f32x4*>(thT + h * kD + d) = W1T[dt][ht];
            *reinterpret_cast<f32x4*>(moT + h * kD + d) = S1T[dt][ht];
            const int h2 = 64 * wv + 16 * ht + 4 * g;
            const int dd = 16 * dt + j;
            *reinterpret_cast<f32x4*>(thT + kOff2 + dd * kHid + h2) = W2T[ht][dt];
            *reinterpret_cast<f32x4*>(moT + kOff2 + dd * kHid + h2) = S2T[ht][dt];
            tile_fence();
        }
}

}  // namespace

bool scan_mfma_supported(const ScanArgs& a) {
    return a.L == 2 && a.n[0] == kD && a.n[1] == kHid && a.n[2] == kD && a.C == kC &&
           a.io == TITANS_BF16;
}

hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t stream) {
    const int64_t nseq = a.B * a.H;
    if (nseq == 0) return hipSuccess;
    scan_mfma_kernel<<<dim3((unsigned)nseq), kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace titans
