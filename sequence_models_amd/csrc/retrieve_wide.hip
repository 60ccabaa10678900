// Read with fixed weights, y = M_theta(q), on gfx950 MFMA for any memory whose widths are
// multiples of 16 (up to 512, L <= 4) with bf16 q / y (the explainer's retrieve formula
// with theta held constant).  The 64 -> 256 -> 64 memory has its own kernel
// (retrieve_mfma.hip) that keeps both weight matrices in LDS; wider memories (the deep
// 128-512-512-512-128 one holds 2.6 MB of weights) do not fit, so here the weights stream.
//
// A workgroup (eight waves, two per SIMD) serves one (b, h) memory and 128 tokens: every
// weight window that streams through LDS is used by 128 tokens.  The tokens' activations
// stay in one LDS buffer as bf16 across all layers (128 x 512, 133 KB); each layer's
// weights pass through one LDS window of 256 outputs x 32 inputs while the next window's
// 16-byte loads are in flight in registers (stored after a barrier).  Per window, wave
// (o, q) computes outputs 128 o .. 128 o + 127 of the window's 256 for tokens
// 32 q .. 32 q + 31 (v_mfma_f32_16x16x32_bf16, A = weight rows, B = activation rows, fp32
// accumulation): of the splits of a window over eight waves, the one that reads the least
// from LDS (80 KB per window; LDS reads, not the matrix cores, set the pace here).  An
// output tile's epilogue applies SiLU and keeps the bf16 result in registers until the
// layer's last window is done (its inputs are still being read); then every wave writes
// its outputs over the inputs.  The last layer writes y.
// Workgroups are numbered so that each XCD holds whole memories: all token tiles of a
// memory then read its weights through one L2.
#include <hip/hip_runtime.h>

#include "mfma_util.h"
#include "titans_internal.h"

namespace titans {
namespace {

using namespace fused;

constexpr int kThreads = 512;
constexpr int kTok = 128;         // tokens per workgroup
constexpr int kQuarters = 4;      // token quarters: waves 2q, 2q+1 take quarter q
constexpr int kCt = kTok / 16 / kQuarters;  // 16-token tiles per wave
constexpr int kTw = 8;            // 16-output tiles per wave (of a window's sixteen)
constexpr int kMaxTiles = 2;      // 256-output tiles of a 512-wide layer
constexpr int kOut = 256;         // outputs per tile
constexpr int kWin = 32;          // inputs per weight window (one MFMA step)
constexpr int kMaxW = 512;
constexpr int kActLd = kMaxW + 8; // padded activation row (bf16)
constexpr int kWLd = kWin + 8;    // padded weight row (bf16)
constexpr int kGroups = kOut * kWin / 4 / kThreads;  // 16-byte groups per thread per window

struct __attribute__((aligned(16))) WSmem {
    __bf16 act[kTok * kActLd];     // [token][feature]
    __bf16 w[kOut * kWLd];         // [output][input - k0]
};

// One weight window: rows o0 .. o0+255 (< nout) and columns k0 .. k0+31 (< nin) of W
// (row-major nout x nin, fp32; zero outside).  Thread t loads columns 4 (t % 8) .. +3 of
// rows t / 8 + 64 m, m < 4: four 16-byte loads (a row's 32 floats from 8 threads).
struct Window {
    f32x4 v[kGroups];
};

__device__ __forceinline__ void load_window(Window& x, const float* W, int nout, int nin, int o0,
                                            int k0) {
    const int tid = threadIdx.x;
    const int k = k0 + 4 * (tid % (kWin / 4));
#pragma unroll
    for (int m = 0; m < kGroups; ++m) {
        const int r = o0 + tid / (kWin / 4) + (kThreads / (kWin / 4)) * m;
        x.v[m] = (r < nout && k < nin) ? *reinterpret_cast<const f32x4*>(W + (int64_t)r * nin + k)
                                       : zero4();
    }
}

__device__ __forceinline__ void store_window(const Window& x, __bf16* dst) {
    const int tid = threadIdx.x;
    const int kk = 4 * (tid % (kWin / 4));
#pragma unroll
    for (int m = 0; m < kGroups; ++m)
        *reinterpret_cast<bf16x4*>(dst + (tid / (kWin / 4) + (kThreads / (kWin / 4)) * m) * kWLd + kk) =
            bf4(x.v[m]);
}

__global__ void __launch_bounds__(kThreads, 2) retrieve_wide_kernel(ScanArgs A) {
    __shared__ WSmem sm;
    const int tid = threadIdx.x;
    const int wo2 = (tid >> 6) & 1, quarter = tid >> 7, g = (tid & 63) >> 4, j = tid & 15;
    const int tb = 32 * quarter;  // the wave's first token in the block

    // XCD-contiguous numbering of (memory, token tile)
    const int64_t ntiles = (A.T + kTok - 1) / kTok;
    const int64_t nblk = gridDim.x;
    const int64_t w = blockIdx.x;
    const int64_t full = nblk & ~int64_t(7);
    const int64_t lid = w < full ? (w & 7) * (full >> 3) + (w >> 3) : w;
    const int64_t seq = lid / ntiles;
    const int64_t t0 = (lid % ntiles) * kTok;
    const int64_t bi = seq / A.H, hi = seq % A.H;
    const float* th = A.thetaT + bi * A.ss[0] + hi * A.ss[1];
    const __bf16* qg = static_cast<const __bf16*>(A.q);
    __bf16* yg = static_cast<__bf16*>(A.y);
    const int64_t qbase = bi * A.qs[0] + hi * A.qs[2];
    const int64_t ybase = bi * A.ys[0] + hi * A.ys[2];
    const int d = A.n[0];

    // the window sequence: layer l, output tile o0, input window k0
    int wl = 1, wo = 0, wk = 0;
    auto advance = [&](int& L_, int& o_, int& k_) {
        k_ += kWin;
        if (k_ >= A.n[L_ - 1]) {
            k_ = 0;
            o_ += kOut;
            if (o_ >= A.n[L_]) {
                o_ = 0;
                ++L_;
            }
        }
    };

    // first window in flight while q lands in LDS.  The activation buffer starts at zero:
    // a 32-wide MFMA step over a width that is a multiple of 16 only reads up to 16
    // columns past it, against zero weights, and those columns must be finite.
    Window nx;
    load_window(nx, th + A.off[1], A.n[1], A.n[0], 0, 0);
    for (int i = tid; i < kTok * kActLd / 8; i += kThreads)
        reinterpret_cast<bf16x8*>(&sm.act[0])[i] = bf16x8{};
    __syncthreads();
    for (int i = tid; i < kTok * (d / 4); i += kThreads) {
        const int t = i / (d / 4), c = 4 * (i % (d / 4));
        bf16x4 v{};
        if (t0 + t < A.T)
            v = *reinterpret_cast<const bf16x4*>(qg + qbase + (t0 + t) * A.qs[1] + c);
        *reinterpret_cast<bf16x4*>(sm.act + t * kActLd + c) = v;
    }
    store_window(nx, sm.w);
    __syncthreads();

    f32x4 acc[kTw][kCt];
#pragma unroll
    for (int tw = 0; tw < kTw; ++tw)
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) acc[tw][ct] = zero4();
    // SiLU outputs of the current hidden layer: window ot, the wave's output tile tw, token
    // tile ct (outputs f0 .. f0+3 of the lane's token)
    bf16x4 stash[kMaxTiles][kTw][kCt];
    while (wl <= A.L) {
        const int nin = A.n[wl - 1], nout = A.n[wl];
        // the following window's loads go out before this one's MFMAs
        int L2 = wl, o2 = wo, k2 = wk;
        advance(L2, o2, k2);
        const bool more = L2 <= A.L;
        if (more) load_window(nx, th + A.off[L2], A.n[L2], A.n[L2 - 1], o2, k2);

        // every operand of the window's products is read before the first of them (one
        // LDS wait); past a width that is a multiple of 16 the step reads zero weights
        const __bf16* ar = sm.w + (128 * wo2 + j) * kWLd + 4 * g;
        bf16x8 a[kTw], b[kCt];
#pragma unroll
        for (int tw = 0; tw < kTw; ++tw) a[tw] = frag(ar + 16 * tw * kWLd, 0);
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) b[ct] = frag(sm.act + (tb + 16 * ct + j) * kActLd + wk + 4 * g, 0);
#pragma unroll
        for (int tw = 0; tw < kTw; ++tw)
#pragma unroll
            for (int ct = 0; ct < kCt; ++ct) acc[tw][ct] = mfma(a[tw], b[ct], acc[tw][ct]);
        if (wk + kWin >= nin) {  // last window of this output tile: epilogue
#pragma unroll
            for (int tw = 0; tw < kTw; ++tw) {
                const int f0 = wo + 128 * wo2 + 16 * tw + 4 * g;  // outputs f0 .. f0+3 of token tb + 16 ct + j
                if (wl < A.L) {
                    bf16x4 h[kCt];
#pragma unroll
                    for (int ct = 0; ct < kCt; ++ct) {
                        f32x4 x;
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[r] = acc[tw][ct][r] * sigmoid(acc[tw][ct][r]);
                        h[ct] = bf4(x);
                    }
                    // constant indices only (a switch, not a dynamic register index)
                    switch (wo / kOut) {
#define TITANS_STASH(i) \
    case i:             \
        _Pragma("unroll") for (int ct = 0; ct < kCt; ++ct) stash[i][tw][ct] = h[ct]; break;
                        TITANS_STASH(0) TITANS_STASH(1)
#undef TITANS_STASH
                        default: break;
                    }
                } else {
#pragma unroll
                    for (int ct = 0; ct < kCt; ++ct) {
                        const int64_t t = t0 + tb + 16 * ct + j;
                        if (f0 < nout && t < A.T)
                            *reinterpret_cast<bf16x4*>(yg + ybase + t * A.ys[1] + f0) = bf4(acc[tw][ct]);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < kCt; ++ct) acc[tw][ct] = zero4();
            }
        }
        __syncthreads();  // this window and, at a layer's end, the layer's inputs are read
        if (more) store_window(nx, sm.w);
        if (more && L2 != wl) {
            // hidden layer wl is done: its outputs replace its inputs
#pragma unroll
            for (int ot = 0; ot < kMaxTiles; ++ot)
#pragma unroll
                for (int tw = 0; tw < kTw; ++tw) {
                    const int f0 = kOut * ot + 128 * wo2 + 16 * tw + 4 * g;
                    if (kOut * ot < nout && f0 < nout)
#pragma unroll
                        for (int ct = 0; ct < kCt; ++ct)
                            *reinterpret_cast<bf16x4*>(sm.act + (tb + 16 * ct + j) * kActLd + f0) = stash[ot][tw][ct];
                }
        }
        __syncthreads();  // the next window (and a finished layer's outputs) are in LDS
        wl = L2;
        wo = o2;
        wk = k2;
    }
}

}  // namespace

bool retrieve_wide_supported(const ScanArgs& a) {
    if (a.io != TITANS_BF16 || a.L < 1 || a.L > TITANS_MAX_LAYERS) return false;
    for (int l = 0; l <= a.L; ++l)
        if (a.n[l] % 16 != 0 || a.n[l] > kMaxW) return false;
    return true;
}

hipError_t launch_retrieve_wide(const ScanArgs& a, hipStream_t stream) {
    const int64_t nseq = a.B * a.H;
    if (nseq == 0 || a.T == 0) return hipSuccess;
    const int64_t blocks = (a.T + kTok - 1) / kTok * nseq;
    retrieve_wide_kernel<<<dim3((unsigned)blocks), kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace titans
