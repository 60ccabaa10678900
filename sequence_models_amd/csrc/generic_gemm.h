// Workgroup matrix products of the generic (any-shape) kernels: a 256-thread workgroup
// computes C = A B tile by tile and hands every output element to an epilogue functor.
// fp32 FMAs (block_gemm) or bf16 MFMA with fp32 accumulation (block_gemm_mfma).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace titans {
namespace generic {

constexpr int kGemmThreads = 256;
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
                    int e = tid + kGemmThreads * r;
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

}  // namespace generic
}  // namespace titans
