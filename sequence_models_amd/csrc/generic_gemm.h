// Workgroup matrix products of the generic (any-shape) kernels: a 256-thread workgroup
// computes C = A B tile by tile and hands every output element to an epilogue functor.
// fp32 FMAs (block_gemm_f32) or bf16 MFMA with fp32 accumulation (block_gemm_mfma).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace titans {
namespace generic {

constexpr int kGemmThreads = 256;
constexpr int kTile = 64;   // output tile edge
constexpr int kMK = 32;                                     // MFMA reduction step
constexpr int kMLd = kMK + 8;                               // padded bf16 row of a staged tile
constexpr int kGemmLdsMfma = 2 * kTile * kMLd / 2;          // floats (two bf16 tiles)
constexpr int kK2 = 32;                                     // fp32 reduction step
constexpr int kLd2 = kTile + 4;                             // padded row of a staged fp32 tile
constexpr int kGemmLdsF32v2 = 2 * 2 * kK2 * kLd2;           // floats (A and B, two buffers)
// LDS floats a caller provides (16-byte aligned) for either product below
constexpr int kGemmLds = kGemmLdsMfma > kGemmLdsF32v2 ? kGemmLdsMfma : kGemmLdsF32v2;

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

// Workgroup GEMM on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation): for every
// (i < M, j < N) call epi(i, j, sum_k A(i,k) B(k,j)), each output element from one thread.
// Per 64 x 64 output tile and 32-wide reduction step, A (64 x 32) and B (32 x 64) are staged
// in LDS as bf16 with the reduction index contiguous ([row i][k], [column j][k]); wave w
// computes output rows 16w .. 16w+15 against the four 16-column tiles.  Operand layouts of
// the MFMA: lane l (g = l / 16, j = l % 16) holds A[j][k] and B[k][j] for k in
// {4g .. 4g+3, 16+4g .. 16+4g+3} and D[4g + r][j], r = 0..3.
template <class Pre, class Epi>
__device__ void block_gemm_mfma(int M, int N, int K, MatA A, MatB B, float* lds, Pre pre, Epi epi) {
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
                    const int e = tid + kGemmThreads * rep;  // 0 .. 511
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
            decltype(pre(0, 0)) pv[4][4];
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = i0 + 16 * wv + 4 * g + r, jc = j0 + 16 * tn + j;
                    if (i < M && jc < N) pv[tn][r] = pre(i, jc);
                }
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = i0 + 16 * wv + 4 * g + r, jc = j0 + 16 * tn + j;
                    if (i < M && jc < N) epi(i, jc, acc[tn][r], pv[tn][r]);
                }
        }
    }
    __syncthreads();
}

// fp32 workgroup GEMM, same contract.  The product is one stream of steps -- every 64 x 64
// output tile times every 32-deep slice of the reduction, tile by tile -- and each step's
// operands are loaded two steps ahead, across tile boundaries, into registers, then written
// to one of two LDS buffers after the current step's FMAs (one barrier per step).  An
// output tile's epilogue operands (pre) are requested before its last step's products.  The
// products run on the fp32 matrix cores (v_mfma_f32_16x16x4f32: fp32 operands, fp32
// accumulation, the same precision as FMAs): wave w computes rows 16 w .. 16 w + 15 of the
// tile against its four 16-column tiles, each lane reading one A and four B values from
// LDS per 4-deep slice (lane l: row / column l % 16, reduction index l / 16; result rows
// 4 (l / 16) .. + 3).  Staging: eight elements of A and eight of B per thread, consecutive
// threads on the operand's contiguous dimension; out-of-range elements load a clamped
// in-range address and are zeroed when written to LDS, so the loads carry no branches.
template <class Pre, class Epi>
__device__ void block_gemm_f32(int M, int N, int K, MatA A, MatB B, float* lds, Pre pre, Epi epi) {
    const int tid = threadIdx.x;
    const int wv = tid >> 6, lr = tid & 15, lk = (tid & 63) >> 4;
    const bool a_kc = A.sk == 1, b_jc = B.sj == 1;
    const bool scaled = A.kscale != nullptr;
    // element offsets inside one operand (a per-memory slice, far below 2^32 elements):
    // 32-bit arithmetic from the uniform base pointer
    const unsigned asi = (unsigned)A.si, ask = (unsigned)A.sk, bsk = (unsigned)B.sk,
                   bsj = (unsigned)B.sj;
    const int tiles_n = (N + kTile - 1) / kTile;
    const int steps = (K + kK2 - 1) / kK2;
    const int total = ((M + kTile - 1) / kTile) * tiles_n * steps;
    if (total == 0 || M <= 0 || N <= 0) {
        __syncthreads();
        return;
    }
    struct Stage {
        float a[8], b[8], s[8];
    };
    auto origin = [&](int st, int& i0, int& j0, int& k0) {
        const int t = st / steps;
        k0 = (st - t * steps) * kK2;
        i0 = (t / tiles_n) * kTile;
        j0 = (t - (t / tiles_n) * tiles_n) * kTile;
    };
    // staging element r of this thread: A (ii, ka) and B (kb, jj), linear in r
    const int a_ii0 = a_kc ? tid >> 5 : tid & 63, a_ka0 = a_kc ? tid & 31 : tid >> 6;
    const int b_jj0 = b_jc ? tid & 63 : tid >> 5, b_kb0 = b_jc ? tid >> 6 : tid & 31;
    const unsigned a_off0 = a_ii0 * asi + a_ka0 * ask, b_off0 = b_kb0 * bsk + b_jj0 * bsj;
    const unsigned a_dr = a_kc ? 8 * asi : 4 * ask, b_dr = b_jc ? 4 * bsk : 8 * bsj;
    auto interior = [&](int i0, int j0, int k0) {
        return i0 + kTile <= M && j0 + kTile <= N && k0 + kK2 <= K;
    };
    auto load = [&](Stage& g, int st) {
        int i0, j0, k0;
        origin(st, i0, j0, k0);
        if (interior(i0, j0, k0)) {  // uniform: no clamps, offsets linear in r
            const float* pa = A.p + (i0 * asi + k0 * ask + a_off0);
            const float* pb = B.p + (k0 * bsk + j0 * bsj + b_off0);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                g.a[r] = pa[r * a_dr];
                g.b[r] = pb[r * b_dr];
                if (scaled) g.s[r] = A.kscale[k0 + a_ka0 + (a_kc ? 0 : 4 * r)];
            }
            return;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int e = tid + kGemmThreads * r;
            const int ii = a_kc ? e >> 5 : e & 63, ka = a_kc ? e & 31 : e >> 6;
            const int gi = i0 + ii, gka = k0 + ka;
            const unsigned ci = gi < M ? gi : M - 1, cka = gka < K ? gka : K - 1;
            g.a[r] = A.p[ci * asi + cka * ask];
            if (scaled) g.s[r] = A.kscale[cka];
            const int jj = b_jc ? e & 63 : e >> 5, kb = b_jc ? e >> 6 : e & 31;
            const int gj = j0 + jj, gkb = k0 + kb;
            const unsigned cj = gj < N ? gj : N - 1, ckb = gkb < K ? gkb : K - 1;
            g.b[r] = B.p[ckb * bsk + cj * bsj];
        }
    };
    auto store = [&](const Stage& g, int st) {
        int i0, j0, k0;
        origin(st, i0, j0, k0);
        float* As = lds + (st & 1) * kK2 * kLd2;
        float* Bs = lds + (2 + (st & 1)) * kK2 * kLd2;
        if (interior(i0, j0, k0)) {
            float* pa = As + a_ka0 * kLd2 + a_ii0;
            float* pb = Bs + b_kb0 * kLd2 + b_jj0;
            const int sa = a_kc ? 8 : 4 * kLd2, sb = b_jc ? 4 * kLd2 : 8;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                pa[r * sa] = scaled ? g.a[r] * g.s[r] : g.a[r];
                pb[r * sb] = g.b[r];
            }
            return;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int e = tid + kGemmThreads * r;
            const int ii = a_kc ? e >> 5 : e & 63, ka = a_kc ? e & 31 : e >> 6;
            const float x = scaled ? g.a[r] * g.s[r] : g.a[r];
            As[ka * kLd2 + ii] = (i0 + ii < M && k0 + ka < K) ? x : 0.0f;
            const int jj = b_jc ? e & 63 : e >> 5, kb = b_jc ? e >> 6 : e & 31;
            Bs[kb * kLd2 + jj] = (j0 + jj < N && k0 + kb < K) ? g.b[r] : 0.0f;
        }
    };
    f32x4_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    decltype(pre(0, 0)) pv[4][4];
    // step st: its operands are in LDS buffer st & 1; `freed` held them and now takes
    // step st + 2's loads; `pending` holds step st + 1's, written to LDS after the FMAs
    auto step = [&](int st, Stage& freed, Stage& pending) {
        if (st + 2 < total) load(freed, st + 2);
        int i0, j0, k0;
        origin(st, i0, j0, k0);
        const bool last = k0 + kK2 >= K;
        if (last) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = i0 + 16 * wv + 4 * lk + r, j = j0 + 16 * t + lr;
                    pv[t][r] = pre(i < M ? i : M - 1, j < N ? j : N - 1);
                }
        }
        // fp32 MFMA (v_mfma_f32_16x16x4f32): wave w owns output rows 16 w .. 16 w + 15 of the
        // tile against four 16-column tiles; per 4-deep slice lane (lr, lk) feeds
        // A[16 w + lr][k] and B[k][16 t + lr] with k = 4 kg + lk
        const float* As = lds + (st & 1) * kK2 * kLd2 + lk * kLd2 + 16 * wv + lr;
        const float* Bs = lds + (2 + (st & 1)) * kK2 * kLd2 + lk * kLd2 + lr;
        float fa[kK2 / 4], fb[kK2 / 4][4];  // the whole step's operands first: one LDS wait
#pragma unroll
        for (int kg = 0; kg < kK2 / 4; ++kg) {
            fa[kg] = As[4 * kg * kLd2];
#pragma unroll
            for (int t = 0; t < 4; ++t) fb[kg][t] = Bs[4 * kg * kLd2 + 16 * t];
        }
#pragma unroll
        for (int kg = 0; kg < kK2 / 4; ++kg)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[kg], fb[kg][t], acc[t], 0, 0, 0);
        if (last) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = i0 + 16 * wv + 4 * lk + r, j = j0 + 16 * t + lr;
                    if (i < M && j < N) epi(i, j, acc[t][r], pv[t][r]);
                }
                acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (st + 1 < total) store(pending, st + 1);
        __syncthreads();
    };
    Stage g0, g1;
    load(g0, 0);
    if (total > 1) load(g1, 1);
    store(g0, 0);
    __syncthreads();
    for (int st = 0; st < total; st += 2) {
        step(st, g0, g1);
        if (st + 1 < total) step(st + 1, g1, g0);
    }
}

// Epilogues in two parts: pre(i, j) loads what element (i, j) needs (any value type) and
// runs for all of a thread's elements before any epi(i, j, sum, pre value) writes, so the
// loads are in flight together rather than each waiting behind the previous element's
// stores (which the compiler cannot prove do not alias them).
template <bool kMfma, class Pre, class Epi>
__device__ __forceinline__ void gemm2(int M, int N, int K, MatA A, MatB B, float* lds, Pre pre,
                                      Epi epi) {
    if constexpr (kMfma)
        block_gemm_mfma(M, N, K, A, B, lds, pre, epi);
    else
        block_gemm_f32(M, N, K, A, B, lds, pre, epi);
}

struct NoPre {
    __device__ int operator()(int, int) const { return 0; }
};

// An epilogue that loads nothing.
template <bool kMfma, class Epi>
__device__ __forceinline__ void gemm(int M, int N, int K, MatA A, MatB B, float* lds, Epi epi) {
    gemm2<kMfma>(M, N, K, A, B, lds, NoPre{}, [&](int i, int j, float x, int) { epi(i, j, x); });
}

// For the linear path's fixed-size products.
template <class Epi>
__device__ __forceinline__ void block_gemm_f32(int M, int N, int K, MatA A, MatB B, float* lds,
                                               Epi epi) {
    gemm2<false>(M, N, K, A, B, lds, NoPre{}, [&](int i, int j, float x, int) { epi(i, j, x); });
}

}  // namespace generic
}  // namespace titans
