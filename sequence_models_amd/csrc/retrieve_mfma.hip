// Read with fixed weights, y = M_theta(q), on gfx950 MFMA for the 64 -> 256 -> 64 SiLU
// memory with bf16 q / y (the explainer's retrieve formula with theta held constant).
//
// A workgroup (eight waves) serves one (b, h) memory and a block of kTokens tokens.  It
// converts that memory's fp32 W1 (256 x 64) and W2 (64 x 256) to bf16 in LDS once (W1
// times -log2(e) and W2 times -ln(2), which saves the sigmoid's scaling multiply); each
// wave then takes 32-token tiles (at most 128 registers: two workgroups, four waves per
// SIMD, share each compute unit):
//   Z^T = W1 Q^T            (rows h, cols tokens), 32 hidden units at a time
//   H^T = SiLU(Z^T)         registers only
//   Y^T += W2[:, block] H^T[block]   accumulated over the eight 32-unit blocks
// Q fragments come straight from global memory in the operand layout (each token row is
// read whole across a tile's loads); Y^T tiles go out as 8-byte rows of 4 bf16.  The
// per-element cost is the SiLU (two transcendental ops per hidden unit and token), which
// bounds this kernel on the vector ALUs rather than on MFMA or HBM.
#include <hip/hip_runtime.h>

#include "mfma_util.h"
#include "titans_internal.h"

namespace titans {
namespace {

using namespace fused;

constexpr int kD = 64;
constexpr int kHid = 256;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCt = 2;                          // 16-token column tiles per wave tile
constexpr int kTile = 16 * kCt;                 // tokens per wave tile
constexpr int kTiles = 8;                       // wave tiles per wave
constexpr int kTokens = kTile * kWaves * kTiles;  // tokens per workgroup
constexpr int kLd1 = kD + 4;                    // W1 rows (k = d), padded
constexpr int kLd2 = kHid + 8;                  // W2 rows (k = h), padded
constexpr float kLn2 = 0.69314718055994531f;

struct __attribute__((aligned(16))) RSmem {
    __bf16 w1[kHid * kLd1];  // W1 [h][d]
    __bf16 w2[kD * kLd2];    // W2 [dd][h]
};

__global__ void __launch_bounds__(kThreads, 4) retrieve_mfma_kernel(ScanArgs A) {
    __shared__ RSmem sm;
    const int tid = threadIdx.x;
    const int wv = tid >> 6, l = tid & 63, g = l >> 4, j = l & 15;
    const int64_t seq = blockIdx.y;
    const int64_t bi = seq / A.H, hi = seq % A.H;
    const float* th = A.thetaT + bi * A.ss[0] + hi * A.ss[1];

    // weights to bf16 in LDS: W1 rows h (64 floats each), W2 rows dd (256 floats each)
#pragma unroll 4
    for (int i = tid; i < kHid * kD / 4; i += kThreads) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(th + 4 * i);
        const int h = (4 * i) / kD, d = (4 * i) % kD;
        *reinterpret_cast<bf16x4*>(sm.w1 + h * kLd1 + d) = bf4(v * -kLog2e);
    }
#pragma unroll 4
    for (int i = tid; i < kD * kHid / 4; i += kThreads) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(th + kHid * kD + 4 * i);
        const int dd = (4 * i) / kHid, h = (4 * i) % kHid;
        *reinterpret_cast<bf16x4*>(sm.w2 + dd * kLd2 + h) = bf4(v * -kLn2);
    }
    __syncthreads();

    const __bf16* qg = static_cast<const __bf16*>(A.q);
    __bf16* yg = static_cast<__bf16*>(A.y);
    const int64_t qbase = bi * A.qs[0] + hi * A.qs[2];
    const int64_t ybase = bi * A.ys[0] + hi * A.ys[2];
    const __bf16* w1r = sm.w1 + j * kLd1 + 4 * g;
    const __bf16* w2r = sm.w2 + j * kLd2 + 4 * g;

    for (int tile = 0; tile < kTiles; ++tile) {
        const int64_t t0 = (int64_t)blockIdx.x * kTokens + kTile * (kWaves * tile + wv);
        if (t0 >= A.T) break;
        // Q^T as B operands: token 16 ct + j, columns 32 kb + {4g .. 4g+3, 16+4g .. 16+4g+3}
        bf16x8 qf[kCt][2];
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) {
            const int64_t t = t0 + 16 * ct + j;
            if (t < A.T) {
                const __bf16* p = qg + qbase + t * A.qs[1] + 4 * g;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    qf[ct][kb] = cat(*reinterpret_cast<const bf16x4*>(p + 32 * kb),
                                     *reinterpret_cast<const bf16x4*>(p + 32 * kb + 16));
            } else {
                qf[ct][0] = qf[ct][1] = bf16x8{};
            }
        }
        f32x4 yt[4][kCt];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int ct = 0; ct < kCt; ++ct) yt[dt][ct] = zero4();
#pragma unroll 2
        for (int hb = 0; hb < kHid / 32; ++hb) {
            bf16x4 hT[2][kCt];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int ht = 2 * hb + hh;
                const bf16x8 wa = frag(w1r, 16 * ht * kLd1);
                const bf16x8 wb = frag(w1r, 16 * ht * kLd1 + 32);
#pragma unroll
                for (int ct = 0; ct < kCt; ++ct) {
                    // W1 was staged times -log2(e): z' = -log2(e) z, sigma(z) = 1 / (1 + 2^z'),
                    // and the factor -ln(2) that turns z' sigma back into SiLU(z) is in W2
                    f32x4 z = mfma(wa, qf[ct][0], zero4());
                    z = mfma(wb, qf[ct][1], z);
                    f32x4 hv;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        hv[r] = z[r] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z[r]));
                    hT[hh][ct] = bf4(hv);
                }
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x8 w = frag(w2r, 16 * dt * kLd2 + 32 * hb);
#pragma unroll
                for (int ct = 0; ct < kCt; ++ct)
                    yt[dt][ct] = mfma(w, cat(hT[0][ct], hT[1][ct]), yt[dt][ct]);
            }
        }
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) {
            const int64_t t = t0 + 16 * ct + j;
            if (t < A.T) {
                __bf16* p = yg + ybase + t * A.ys[1] + 4 * g;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    *reinterpret_cast<bf16x4*>(p + 16 * dt) = bf4(yt[dt][ct]);
            }
        }
    }
}

}  // namespace

bool retrieve_mfma_supported(const ScanArgs& a) {
    return a.L == 2 && a.n[0] == kD && a.n[1] == kHid && a.n[2] == kD && a.io == TITANS_BF16;
}

hipError_t launch_retrieve_mfma(const ScanArgs& a, hipStream_t stream) {
    const int64_t nseq = a.B * a.H;
    if (nseq == 0 || a.T == 0) return hipSuccess;
    const dim3 grid((unsigned)((a.T + kTokens - 1) / kTokens), (unsigned)nseq);
    retrieve_mfma_kernel<<<grid, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace titans
