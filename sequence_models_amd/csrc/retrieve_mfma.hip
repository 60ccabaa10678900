// Read with fixed weights, y = M_theta(q), on gfx950 MFMA for the 64 -> 256 -> 64 SiLU
// memory with bf16 q / y (the explainer's retrieve formula with theta held constant).
//
// A workgroup (sixteen waves, one per compute unit: four waves per SIMD at most 128
// registers each) serves one (b, h) memory and a block of tokens.  It converts that
// memory's fp32 W1 (256 x 64) and W2 (64 x 256) to bf16 in LDS once (W1 times -log2(e)
// and W2 times -ln(2), which saves the sigmoid's scaling multiply); its waves then take
// the block's 32-token tiles from an LDS counter, in order, as each finishes its last
// (waves that share a SIMD do not progress at equal rates, and fixed shares left the
// slowest wave of a workgroup 20 % behind the fastest):
//   Z^T = W1 Q^T            (rows h, cols tokens), 32 hidden units at a time
//   H^T = SiLU(Z^T)         registers only
//   Y^T += W2[:, block] H^T[block]   accumulated over the eight 32-unit blocks
//
// Layouts (v_mfma_f32_16x16x32_bf16: lane l, g = l / 16, j = l % 16, holds A[j][8g..8g+7],
// B[8g..8g+7][j] and D[4g..4g+3][j]).  Every operand is one 16-byte access:
//   * Z's reduction index is d in natural order, so lane (g, j) of k-block kb holds
//     d = 32 kb + 8 g .. +7 of token j (Q, straight from global memory) and of hidden row j
//     (W1, from LDS);
//   * Y's reduction index is h in the order Z's accumulators leave it: the eight k-slots
//     of lane (g, j) in block hb are h = 32 hb + 4g .. +3 and 32 hb + 16 + 4g .. +3 (two
//     Z row tiles).  W2 is stored in LDS with each 32-column block permuted to that order;
//   * Y's output rows are W2's rows permuted so that lane (g, j) of the four output tiles
//     dt holds d = 32 (dt / 2) + 8 g + 4 (dt % 2) .. +3: two 16-byte stores per token, and
//     the four lanes of a token write 64 contiguous bytes per store.
// Padded LDS rows (72 and 264 bf16) make the sixteen 16-byte reads of a quarter-wave hit
// distinct banks.  y is written with non-temporal stores (streamed, not read back here).
#include <hip/hip_runtime.h>

#include "mfma_util.h"
#include "titans_internal.h"

namespace titans {
namespace {

using namespace fused;

constexpr int kD = 64;
constexpr int kHid = 256;
constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kCt = 2;                          // 16-token column tiles per wave tile
constexpr int kTile = 16 * kCt;                 // tokens per wave tile
constexpr int kMaxTiles = 16;                   // wave tiles per wave (launch picks <=)
constexpr int kLd1 = kD + 8;                    // W1 rows (k = d)
constexpr int kLd2 = kHid + 8;                  // W2 rows (k = h, permuted)
constexpr float kLn2 = 0.69314718055994531f;

struct __attribute__((aligned(16))) RSmem {
    __bf16 w1[kHid * kLd1];  // W1 [h][d]
    __bf16 w2[kD * kLd2];    // W2, rows and columns permuted as above
    int next;                // next wave tile of the workgroup's block
};

// LDS row of W2's output row d, and LDS column of the first of four consecutive hidden
// units h = 4m .. 4m+3 (the permutations of the header).
__device__ __forceinline__ int w2_row(int d) {
    return 16 * (2 * (d / 32) + (d % 8) / 4) + 4 * ((d % 32) / 8) + d % 4;
}
__device__ __forceinline__ int w2_col(int m) { return 32 * (m / 8) + 8 * (m % 4) + 4 * ((m % 8) / 4); }

// tiles: wave tiles per wave on average (1 .. kMaxTiles); a workgroup covers
// kTile * kWaves * tiles tokens of memory blockIdx.y.
__global__ void __launch_bounds__(kThreads, 4) retrieve_mfma_kernel(ScanArgs A, int tiles) {
    __shared__ RSmem sm;
    const int tid = threadIdx.x;
    const int wv = tid >> 6, l = tid & 63, g = l >> 4, j = l & 15;
    const int64_t seq = blockIdx.y;
    const int64_t bi = seq / A.H, hi = seq % A.H;
    const float* th = A.thetaT + bi * A.ss[0] + hi * A.ss[1];
    if (tid == 0) sm.next = kWaves;

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
        const int dd = (4 * i) / kHid, m = i % (kHid / 4);
        *reinterpret_cast<bf16x4*>(sm.w2 + w2_row(dd) * kLd2 + w2_col(m)) = bf4(v * -kLn2);
    }
    __syncthreads();

    const __bf16* qg = static_cast<const __bf16*>(A.q);
    __bf16* yg = static_cast<__bf16*>(A.y);
    const int64_t qbase = bi * A.qs[0] + hi * A.qs[2];
    const int64_t ybase = bi * A.ys[0] + hi * A.ys[2];
    const __bf16* w1r = sm.w1 + j * kLd1 + 8 * g;
    const __bf16* w2r = sm.w2 + j * kLd2 + 8 * g;
    const int64_t block0 = (int64_t)blockIdx.x * kTile * kWaves * tiles;

    // wave tiles are handed out in order as waves finish their previous one (the first is
    // the wave's own), so the waves of a workgroup end within about one tile of each other
    for (int tile = wv; tile < kWaves * tiles;) {
        const int64_t t0 = block0 + kTile * tile;
        if (t0 >= A.T) break;
        // Q^T as B operands: token 16 ct + j, d = 32 kb + 8 g .. +7
        bf16x8 qf[kCt][2];
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) {
            const int64_t t = t0 + 16 * ct + j;
            if (t < A.T) {
                const __bf16* p = qg + qbase + t * A.qs[1] + 8 * g;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) qf[ct][kb] = *reinterpret_cast<const bf16x8*>(p + 32 * kb);
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
                const bf16x8 wa = *reinterpret_cast<const bf16x8*>(w1r + 16 * ht * kLd1);
                const bf16x8 wb = *reinterpret_cast<const bf16x8*>(w1r + 16 * ht * kLd1 + 32);
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
                const bf16x8 w = *reinterpret_cast<const bf16x8*>(w2r + 16 * dt * kLd2 + 32 * hb);
#pragma unroll
                for (int ct = 0; ct < kCt; ++ct)
                    yt[dt][ct] = mfma(w, cat(hT[0][ct], hT[1][ct]), yt[dt][ct]);
            }
        }
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) {
            const int64_t t = t0 + 16 * ct + j;
            if (t < A.T) {
                __bf16* p = yg + ybase + t * A.ys[1] + 8 * g;
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    __builtin_nontemporal_store(cat(bf4(yt[2 * s][ct]), bf4(yt[2 * s + 1][ct])),
                                                reinterpret_cast<bf16x8*>(p + 32 * s));
            }
        }
        int nt = 0;
        if (l == 0) nt = atomicAdd(&sm.next, 1);
        tile = __builtin_amdgcn_readfirstlane(nt);
    }
}

}  // namespace

bool retrieve_mfma_supported(const ScanArgs& a) {
    return a.L == 2 && a.n[0] == kD && a.n[1] == kHid && a.n[2] == kD && a.io == TITANS_BF16;
}

// Tiles per wave: the most (fewest weight conversions per token) that still gives one
// workgroup per compute unit.
int retrieve_mfma_tiles(const ScanArgs& a, int64_t cus) {
    int tiles = kMaxTiles;
    while (tiles > 1 && a.B * a.H * ((a.T + kTile * kWaves * tiles - 1) / (kTile * kWaves * tiles)) < cus)
        tiles /= 2;
    return tiles;
}

hipError_t launch_retrieve_mfma(const ScanArgs& a, int64_t cus, hipStream_t stream) {
    const int64_t nseq = a.B * a.H;
    if (nseq == 0 || a.T == 0) return hipSuccess;
    const int tiles = retrieve_mfma_tiles(a, cus);
    const int64_t block = (int64_t)kTile * kWaves * tiles;
    const dim3 grid((unsigned)((a.T + block - 1) / block), (unsigned)nseq);
    retrieve_mfma_kernel<<<grid, kThreads, 0, stream>>>(a, tiles);
    return hipGetLastError();
}

}  // namespace titans
