// Chunked Titans memory scan as a chain of GPU-wide phases, for memories whose chunk work
// is too large for one compute unit (the deep 128-512-512-512-128 memory holds 2.6 MB of
// weights and 2.6 MB of momentum per head, and a few such heads leave most of the GPU
// idle when each runs on one workgroup).
//
// The algebra is the generic kernel's (gradients at the chunk-start weights, the
// summary page's "tensorized mini-batch" form; the momentum / forget recurrence unrolled
// into per-chunk coefficients a, b, c, w, p; reads at the in-chunk weights
//   U_l = diag(a) Hq W_l^T - diag(b) Hq S_l^T - (Cm o Hq Hk^T) Delta_l,
// chunk-end carry W_l <- a_n W_l - b_n S_l - Delta_l^T diag(c_n) Hk, S_l <- p S_l +
// Delta_l^T diag(w) Hk).  What changes is how a chunk's work is spread: each matrix
// product of the chunk is cut into 64 x 64 output tiles, the tiles of every memory form
// one kernel launch, and consecutive launches on the stream are the barriers between
// dependent products.  Products that depend on the same inputs share a launch:
//   launch 1          key forward of layer 1, the layer-1 read products (Cm o Q K^T and
//                     a Q W1^T - b Q S1^T; q and k are read from the caller's tensors),
//                     and the next chunk's coefficients (double-buffered by chunk parity);
//   launches 2..L     key forward of layers 2..L (SiLU and SiLU' in the epilogue; the last
//                     layer's epilogue forms Delta_L = 2 (O - V));
//   L - 1 launches    backward Delta_{l-1} = (Delta_l W_l) o SiLU'(Z_{l-1});
//   2L - 1 launches   reads: U_l -= (Cm o Hq Hk^T) Delta_l then SiLU (or y for l = L),
//                     then the next layer's read products; the last one also carries every
//                     layer's W_l and S_l to the chunk end (all of their readers are done).
// That is 4L - 2 launches per chunk.  With bf16 I/O a tile stages its whole reduction
// extent (<= 512) of both operands in LDS as bf16 (one load latency per tile) and runs
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation; with fp32 I/O it runs 16-wide fp32 FMA
// steps.  State and intermediates are fp32 in HBM (theta_T / s_T and the workspace).
#include <hip/hip_runtime.h>

#include "generic_util.h"
#include "titans_internal.h"

namespace titans {
namespace {

using namespace generic;

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kKStep = 16;  // fp32 reduction step
constexpr int kPad = 4;
constexpr int kMaxSeg = 6;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// Operand of a tile product: element (r, k) = p[r * sr + k * sk] * (ks ? ks[k] : 1), read
// from fp32 p or, when pb is set, from bf16 pb (q and k straight from a bf16 input).
// Every operand here has sk == 1 or sr == 1.
struct Opnd {
    const float* p;
    int64_t sr, sk;
    const float* ks;
    const __bf16* pb = nullptr;
};

// Vector loads (16 bytes of fp32, 8 of bf16) are used when the operand's base and its
// stride across the vector direction keep every group of four aligned.
__device__ __forceinline__ bool vec_ok(const Opnd& X) {
    const int64_t s = X.sk == 1 ? X.sr : X.sk;
    const uintptr_t base = X.pb ? reinterpret_cast<uintptr_t>(X.pb) : reinterpret_cast<uintptr_t>(X.p);
    return (base & (X.pb ? 7u : 15u)) == 0 && (s & 3) == 0;
}

__device__ __forceinline__ f32x4_t widen(bf16x4_t t) {
    return f32x4_t{(float)t[0], (float)t[1], (float)t[2], (float)t[3]};
}

// Four consecutive elements along the contiguous index starting at (r, k): k .. k+3 of
// row r when sk == 1, rows r .. r+3 of column k otherwise; zero outside R x K.
__device__ __forceinline__ f32x4_t load4(const Opnd& X, bool vec, int r, int R, int k, int K) {
    if (X.pb) {
        const int64_t o = X.sk == 1 ? (int64_t)r * X.sr + k : r + (int64_t)k * X.sk;
        const bool in = X.sk == 1 ? (r < R && k + 3 < K) : (r + 3 < R && k < K);
        if (vec && in) return widen(*reinterpret_cast<const bf16x4_t*>(X.pb + o));
        f32x4_t v;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool ok = X.sk == 1 ? (r < R && k + u < K) : (r + u < R && k < K);
            v[u] = ok ? (float)X.pb[o + u] : 0.f;  // the unit-stride index advances
        }
        return v;
    }
    if (X.sk == 1) {
        const float* q = X.p + (int64_t)r * X.sr + k;
        if (vec && r < R && k + 3 < K) return *reinterpret_cast<const f32x4_t*>(q);
        f32x4_t v;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = (r < R && k + u < K) ? q[u] : 0.f;
        return v;
    }
    const float* q = X.p + r + (int64_t)k * X.sk;
    if (vec && r + 3 < R && k < K) return *reinterpret_cast<const f32x4_t*>(q);
    f32x4_t v;
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = (r + u < R && k < K) ? q[u] : 0.f;
    return v;
}

// Where thread tid's two groups of a 32-wide k slice sit in the 64-row tile: with
// sk == 1, rows (tid >> 3) + 32 p and k = 4 (tid & 7) .. +3 (eight lanes read 128
// contiguous bytes of a row); with sr == 1, rows 4 (tid & 15) .. +3 and k = (tid >> 4) +
// 16 p (sixteen lanes read 256 contiguous bytes of a column).
__device__ __forceinline__ void grp_pos(const Opnd& X, int tid, int p, int& rr, int& kk) {
    if (X.sk == 1) { rr = (tid >> 3) + 32 * p; kk = 4 * (tid & 7); }
    else { rr = 4 * (tid & 15); kk = (tid >> 4) + 16 * p; }
}

__device__ __forceinline__ void store4(__bf16* dst, int ld, const Opnd& X, int rr, int k, int K,
                                       f32x4_t v, int kl) {
    // k: the operand's column (scale, range); kl: the LDS column
    if (X.sk == 1) {
        bf16x4_t o;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float x = v[u];
            if (X.ks && k + u < K) x *= X.ks[k + u];
            o[u] = (__bf16)x;
        }
        *reinterpret_cast<bf16x4_t*>(dst + rr * ld + kl) = o;
    } else {
        const float ksc = (X.ks && k < K) ? X.ks[k] : 1.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[(rr + u) * ld + kl] = (__bf16)(v[u] * ksc);
    }
}

// Stage rows r0 .. r0+63 (< R) x columns kb .. kb+Kw-1 (< K) of each operand X[o] into
// dst[o][r][k - kb] as bf16 (row length ld, zero-filled up to Kwp = Kw rounded up to 32).
// Each batch of kSl 32-wide slices issues every 16-byte load before its first LDS store,
// so the tile waits for one load latency per batch.  With kShare01, operand 1 is operand
// 0's data under other scales and reuses its loads.
// Interior tiles (every row and column of the window in range, vector-aligned, no
// per-k scale on a k-contiguous operand) take an unchecked copy of the loop with the
// operand's layout and source type decided once per batch: plain vector loads at
// r * sr + k * sk, packed conversion to bf16.
template <int kN, int kSl, bool kShare01>
__device__ __forceinline__ void stage_fast(__bf16* const* dst, const Opnd* X, const int* r0,
                                           int kb, int Kwp, int ld) {
    const int tid = threadIdx.x;
    for (int s0 = 0; s0 < Kwp; s0 += 32 * kSl) {
        const int nsl = (Kwp - s0) / 32 < kSl ? (Kwp - s0) / 32 : kSl;
        f32x4_t v[kN][kSl][2];
#pragma unroll
        for (int o = 0; o < kN; ++o) {
            if (kShare01 && o == 1) continue;
            const Opnd& Y = X[o];
            int64_t base[2];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                int rr, kk;
                grp_pos(Y, tid, p, rr, kk);
                base[p] = (int64_t)(r0[o] + rr) * Y.sr + (int64_t)(kb + s0 + kk) * Y.sk;
            }
            const int64_t step = 32 * Y.sk;
            if (Y.pb) {
#pragma unroll
                for (int sl = 0; sl < kSl; ++sl)
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        v[o][sl][p] = sl < nsl ? widen(*reinterpret_cast<const bf16x4_t*>(
                                                     Y.pb + base[p] + sl * step))
                                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
            } else {
#pragma unroll
                for (int sl = 0; sl < kSl; ++sl)
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        v[o][sl][p] = sl < nsl ? *reinterpret_cast<const f32x4_t*>(
                                                     Y.p + base[p] + sl * step)
                                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int o = 0; o < kN; ++o) {
            const Opnd& Y = X[o];
            const int ov = (kShare01 && o == 1) ? 0 : o;
            if (Y.sk == 1) {  // four consecutive k of one row: one 8-byte store
                const int rr = tid >> 3, kk = 4 * (tid & 7);
#pragma unroll
                for (int sl = 0; sl < kSl; ++sl)
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        if (sl < nsl)
                            *reinterpret_cast<bf16x4_t*>(dst[o] + (rr + 32 * p) * ld + s0 + 32 * sl + kk) =
                                __builtin_convertvector(v[ov][sl][p], bf16x4_t);
            } else {  // four consecutive rows of one k: four 2-byte stores
                const int rr = 4 * (tid & 15), kk = tid >> 4;
#pragma unroll
                for (int sl = 0; sl < kSl; ++sl)
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        if (sl >= nsl) continue;
                        const int kl = s0 + 32 * sl + kk + 16 * p;
                        f32x4_t x = v[ov][sl][p];
                        if (Y.ks) x = x * Y.ks[kb + kl];
                        const bf16x4_t b = __builtin_convertvector(x, bf16x4_t);
#pragma unroll
                        for (int u = 0; u < 4; ++u) dst[o][(rr + u) * ld + kl] = b[u];
                    }
            }
        }
    }
}

template <int kN, int kSl, bool kShare01>
__device__ __forceinline__ void stage_checked(__bf16* const* dst, const Opnd* X, const int* r0,
                                              const int* R, int kb, int Kwp, int K, int ld,
                                              const bool* vec) {
    const int tid = threadIdx.x;
    for (int s0 = 0; s0 < Kwp; s0 += 32 * kSl) {
        f32x4_t v[kN][kSl][2];
#pragma unroll
        for (int o = 0; o < kN; ++o) {
            if (kShare01 && o == 1) continue;
#pragma unroll
            for (int sl = 0; sl < kSl; ++sl)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    int rr, kk;
                    grp_pos(X[o], tid, p, rr, kk);
                    const int k = kb + s0 + 32 * sl + kk;
                    v[o][sl][p] = (s0 + 32 * sl < Kwp)
                                      ? load4(X[o], vec[o], r0[o] + rr, R[o], k, K)
                                      : f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
        }
#pragma unroll
        for (int o = 0; o < kN; ++o)
#pragma unroll
            for (int sl = 0; sl < kSl; ++sl)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    if (s0 + 32 * sl >= Kwp) continue;
                    const int ov = (kShare01 && o == 1) ? 0 : o;
                    int rr, kk;
                    grp_pos(X[o], tid, p, rr, kk);
                    const int kl = s0 + 32 * sl + kk;
                    store4(dst[o], ld, X[o], rr, kb + kl, K, v[ov][sl][p], kl);
                }
    }
}

template <int kN, int kSl, bool kShare01 = false>
__device__ __forceinline__ void stage(__bf16* const* dst, const Opnd* X, const int* r0,
                                      const int* R, int kb, int Kwp, int K, int ld) {
    bool vec[kN];
    bool full = kb + Kwp <= K;
#pragma unroll
    for (int o = 0; o < kN; ++o) {
        vec[o] = vec_ok(X[o]);
        full = full && vec[o] && r0[o] + kTile <= R[o] && !(X[o].sk == 1 && X[o].ks);
    }
    if (full)
        stage_fast<kN, kSl, kShare01>(dst, X, r0, kb, Kwp, ld);
    else  // edge tiles: one slice per batch keeps this copy of the loop small
        stage_checked<kN, 1, kShare01>(dst, X, r0, R, kb, Kwp, K, ld, vec);
}

// Logistic function: on the bf16 MFMA path the hardware exp2 / reciprocal (about one ulp
// each, far inside bf16 rounding); on the fp32 path the accurate library forms.
template <bool kFast>
__device__ __forceinline__ float sigm(float z) {
    if constexpr (kFast)
        return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
    else
        return sigmoidf_(z);
}

// LDS bytes of a bf16 tile product with reduction extent K and n staged operands.
__host__ __device__ constexpr int mfma_lds_bytes(int K, int n = 2) {
    return n * kTile * (((K + 31) & ~31) + 8) * 2;
}

// acc[tn] += A B^T over the staged k range for wave w's rows 16w .. 16w+15 of the tile.
// Operand layouts of v_mfma_f32_16x16x32_bf16: lane l (g = l / 16, j = l % 16) holds
// A[j][k] and B[k][j] for k in {4g .. 4g+3, 16+4g .. 16+4g+3}; the result D[4g + r][j].
__device__ __forceinline__ void mfma_tile(const __bf16* As, const __bf16* Bs, int Kp, int ld,
                                          f32x4_t* acc) {
    const int tid = threadIdx.x;
    const int wv = tid >> 6, g = (tid & 63) >> 4, j = tid & 15;
    const __bf16* ar = As + (16 * wv + j) * ld + 4 * g;
    const __bf16* br = Bs + j * ld + 4 * g;
    for (int k0 = 0; k0 < Kp; k0 += 32) {
        const bf16x8_t af = __builtin_shufflevector(*reinterpret_cast<const bf16x4_t*>(ar + k0),
                                                    *reinterpret_cast<const bf16x4_t*>(ar + k0 + 16),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            const __bf16* b = br + 16 * tn * ld + k0;
            const bf16x8_t bf = __builtin_shufflevector(*reinterpret_cast<const bf16x4_t*>(b),
                                                        *reinterpret_cast<const bf16x4_t*>(b + 16),
                                                        0, 1, 2, 3, 4, 5, 6, 7);
            acc[tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[tn], 0, 0, 0);
        }
    }
}

// epi(i, j, v) for every in-range element of the tile, each by exactly one thread (the
// same thread for the same (i, j) in every tile call).
template <class Epi>
__device__ __forceinline__ void tile_epilogue(int i0, int j0, int M, int N, const f32x4_t* acc,
                                              Epi epi) {
    const int tid = threadIdx.x;
    const int wv = tid >> 6, g = (tid & 63) >> 4, j = tid & 15;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 16 * wv + 4 * g + r, jc = j0 + 16 * tn + j;
            if (i < M && jc < N) epi(i, jc, acc[tn][r]);
        }
}

__device__ __forceinline__ void zero_acc(f32x4_t* acc) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// out(i, j) = sum_{k < K} A(i, k) B(j, k) for the 64 x 64 tile at (i0, j0) of an M x N
// result (K <= 512), bf16 operands, fp32 accumulation; epi(i, j, out).  kSl 32-wide
// slices per staging batch.
template <int kSl = 8, class Epi>
__device__ __forceinline__ void tile_mfma(int i0, int j0, int M, int N, int K, Opnd A, Opnd B,
                                          __bf16* lds, Epi epi) {
    const int Kp = (K + 31) & ~31, ld = Kp + 8;
    __bf16* const dst[2] = {lds, lds + kTile * ld};
    const Opnd X[2] = {A, B};
    const int r0[2] = {i0, j0}, R[2] = {M, N};
    stage<2, kSl>(dst, X, r0, R, 0, Kp, K, ld);
    __syncthreads();
    f32x4_t acc[4];
    zero_acc(acc);
    mfma_tile(dst[0], dst[1], Kp, ld, acc);
    tile_epilogue(i0, j0, M, N, acc, epi);
    __syncthreads();  // the LDS tiles may be restaged by the next product
}

// The same product for an epilogue that also reads one value per element from global
// memory: pre(i, j) for each of the thread's sixteen elements is loaded before the
// operands are staged, so those loads overlap the staging instead of following the
// products one element at a time; epi(i, j, out, pre(i, j)).
template <int kSl = 8, class Pre, class Epi>
__device__ __forceinline__ void tile_mfma_pre(int i0, int j0, int M, int N, int K, Opnd A, Opnd B,
                                              __bf16* lds, Pre pre, Epi epi) {
    const int tid = threadIdx.x;
    const int wv = tid >> 6, g = (tid & 63) >> 4, j = tid & 15;
    float pv[4][4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 16 * wv + 4 * g + r, jc = j0 + 16 * tn + j;
            pv[tn][r] = (i < M && jc < N) ? pre(i, jc) : 0.f;
        }
    const int Kp = (K + 31) & ~31, ld = Kp + 8;
    __bf16* const dst[2] = {lds, lds + kTile * ld};
    const Opnd X[2] = {A, B};
    const int r0[2] = {i0, j0}, R[2] = {M, N};
    stage<2, kSl>(dst, X, r0, R, 0, Kp, K, ld);
    __syncthreads();
    f32x4_t acc[4];
    zero_acc(acc);
    mfma_tile(dst[0], dst[1], Kp, ld, acc);
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 16 * wv + 4 * g + r, jc = j0 + 16 * tn + j;
            if (i < M && jc < N) epi(i, jc, acc[tn][r], pv[tn][r]);
        }
    __syncthreads();  // the LDS tiles may be restaged by the next product
}

constexpr int kWin3 = 128;  // k window of a three-operand staging round (52 KB of LDS)

// out1 = A B1^T and out2 = A B2^T: A, B1, B2 staged together in k windows of 128 (A is
// loaded once); epi(i, j, out1, out2, pre(i)), with pre(i) (two floats of row i) loaded
// before the staging.
template <class Pre, class Epi>
__device__ __forceinline__ void tile_mfma_shared_a(int i0, int j0, int M, int N, int K, Opnd A,
                                                   Opnd B1, Opnd B2, __bf16* lds, Pre pre, Epi epi) {
    float2 pr[4];
    {
        const int wv0 = threadIdx.x >> 6, g0 = (threadIdx.x & 63) >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 16 * wv0 + 4 * g0 + r;
            pr[r] = i < M ? pre(i) : float2{0.f, 0.f};
        }
    }
    const int Kw = K < kWin3 ? K : kWin3;
    const int Kwp = (Kw + 31) & ~31, ld = Kwp + 8;
    __bf16* const dst[3] = {lds, lds + kTile * ld, lds + 2 * kTile * ld};
    const Opnd X[3] = {A, B1, B2};
    const int r0[3] = {i0, j0, j0}, R[3] = {M, N, N};
    f32x4_t acc1[4], acc2[4];
    zero_acc(acc1);
    zero_acc(acc2);
    for (int kb = 0; kb < K; kb += kWin3) {
        const int kw = (K - kb) < kWin3 ? (K - kb) : kWin3;
        const int kwp = (kw + 31) & ~31;
        stage<3, 4>(dst, X, r0, R, kb, kwp, K, ld);
        __syncthreads();
        mfma_tile(dst[0], dst[1], kwp, ld, acc1);
        mfma_tile(dst[0], dst[2], kwp, ld, acc2);
        __syncthreads();
    }
    const int tid = threadIdx.x;
    const int wv = tid >> 6, g = (tid & 63) >> 4, j = tid & 15;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 16 * wv + 4 * g + r, jc = j0 + 16 * tn + j;
            if (i < M && jc < N) epi(i, jc, acc1[tn][r], acc2[tn][r], pr[r]);
        }
}

// The chunk-end carry of one 64 x 64 tile of W_l and S_l (M = n_l rows, N = n_{l-1}
// columns, K = n tokens):
//   W <- a_n W - b_n S - (c_n o Delta)^T Hk,   S <- p S + (w o Delta)^T Hk,
// with A1 = c_n-scaled Delta^T and A2 = w-scaled Delta^T sharing their loads and both
// products sharing B = Hk.  The tile's old W and S values are loaded first, so their
// latency overlaps the staging.
__device__ __forceinline__ void tile_carry(int i0, int j0, int M, int N, int K, Opnd A1, Opnd A2,
                                           Opnd B, float* W, float* S, int64_t ldw, float an,
                                           float bn, float pn, __bf16* lds) {
    const int tid = threadIdx.x;
    const int wv = tid >> 6, g = (tid & 63) >> 4, j = tid & 15;
    float w_old[4][4], s_old[4][4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 16 * wv + 4 * g + r, jc = j0 + 16 * tn + j;
            const bool in = i < M && jc < N;
            const int64_t o = (int64_t)i * ldw + jc;
            w_old[tn][r] = in ? W[o] : 0.f;
            s_old[tn][r] = in ? S[o] : 0.f;
        }
    const int Kw = K < kWin3 ? K : kWin3;
    const int ld = ((Kw + 31) & ~31) + 8;
    __bf16* const dst[3] = {lds, lds + kTile * ld, lds + 2 * kTile * ld};
    const Opnd X[3] = {A1, A2, B};
    const int r0[3] = {i0, i0, j0}, R[3] = {M, M, N};
    f32x4_t acc1[4], acc2[4];
    zero_acc(acc1);
    zero_acc(acc2);
    for (int kb = 0; kb < K; kb += kWin3) {
        const int kw = (K - kb) < kWin3 ? (K - kb) : kWin3;
        const int kwp = (kw + 31) & ~31;
        stage<3, 2, true>(dst, X, r0, R, kb, kwp, K, ld);
        __syncthreads();
        mfma_tile(dst[0], dst[2], kwp, ld, acc1);
        mfma_tile(dst[1], dst[2], kwp, ld, acc2);
        __syncthreads();
    }
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 16 * wv + 4 * g + r, jc = j0 + 16 * tn + j;
            if (i < M && jc < N) {
                const int64_t o = (int64_t)i * ldw + jc;
                W[o] = an * w_old[tn][r] - bn * s_old[tn][r] - acc1[tn][r];
                S[o] = pn * s_old[tn][r] + acc2[tn][r];
            }
        }
}

// The same contract in fp32 FMAs: 16-wide reduction steps staged in LDS, 4 x 4 outputs
// per thread.
template <class Epi>
__device__ __forceinline__ void tile_f32(int i0, int j0, int M, int N, int K, Opnd A, Opnd B, float* lds,
                         Epi epi) {
    float* As = lds;  // [kKStep][kTile + kPad]
    float* Bs = lds + kKStep * (kTile + kPad);
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    float acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += kKStep) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = tid + kThreads * r;
            int ii, kk;
            if (A.sk == 1) { kk = e & 15; ii = e >> 4; } else { ii = e & 63; kk = e >> 6; }
            int gi = i0 + ii, gk = k0 + kk;
            float val = 0.0f;
            if (gi < M && gk < K) {
                val = A.p[(int64_t)gi * A.sr + (int64_t)gk * A.sk];
                if (A.ks) val *= A.ks[gk];
            }
            As[kk * (kTile + kPad) + ii] = val;
            if (B.sk == 1) { kk = e & 15; ii = e >> 4; } else { ii = e & 63; kk = e >> 6; }
            gi = j0 + ii;
            gk = k0 + kk;
            val = 0.0f;
            if (gi < N && gk < K) {
                val = B.p[(int64_t)gi * B.sr + (int64_t)gk * B.sk];
                if (B.ks) val *= B.ks[gk];
            }
            Bs[kk * (kTile + kPad) + ii] = val;
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
            const int i = i0 + ty + 16 * r, j = j0 + tx + 16 * c;
            if (i < M && j < N) epi(i, j, acc[r][c]);
        }
}

constexpr int kF32Lds = 2 * kKStep * (kTile + kPad) * 4;  // bytes

template <bool kMfma, int kSl = 8, class Epi>
__device__ __forceinline__ void tile(int i0, int j0, int M, int N, int K, Opnd A, Opnd B,
                                     void* lds, Epi epi) {
    if constexpr (kMfma)
        tile_mfma<kSl>(i0, j0, M, N, K, A, B, static_cast<__bf16*>(lds), epi);
    else
        tile_f32(i0, j0, M, N, K, A, B, static_cast<float*>(lds), epi);
}

// tile() for an epilogue epi(i, j, out, pre(i, j)) that reads one global value per element.
template <bool kMfma, int kSl = 8, class Pre, class Epi>
__device__ __forceinline__ void tile_pre(int i0, int j0, int M, int N, int K, Opnd A, Opnd B,
                                         void* lds, Pre pre, Epi epi) {
    if constexpr (kMfma)
        tile_mfma_pre<kSl>(i0, j0, M, N, K, A, B, static_cast<__bf16*>(lds), pre, epi);
    else
        tile_f32(i0, j0, M, N, K, A, B, static_cast<float*>(lds),
                 [&](int i, int jj, float x) { epi(i, jj, x, pre(i, jj)); });
}

// Float offsets of the per-memory workspace regions.
struct PhLayout {
    int64_t coef[2];   // by chunk parity: a[C+1], b[C+1], w[C], p
    int64_t cm[2];     // by chunk parity: (C+1) x C, row t = c_{t, j}
    int64_t hk[TITANS_MAX_LAYERS];      // l = 1..L-1: C x n_l
    int64_t sp[TITANS_MAX_LAYERS];      // l = 1..L-1: C x n_l, SiLU'(Z_l)
    int64_t dl[TITANS_MAX_LAYERS + 1];  // l = 1..L:   C x n_l
    int64_t hq[2];     // U_l / Hq_l in buffer l & 1: C x maxw
    int64_t mq;        // C x C
    int64_t per_seq;
};

__host__ __device__ inline PhLayout ph_layout(int C, int L, const int* n) {
    auto r64 = [](int64_t x) { return (x + 63) & ~int64_t(63); };
    PhLayout w{};
    int maxw = 0;
    for (int l = 0; l <= L; ++l) maxw = n[l] > maxw ? n[l] : maxw;
    int64_t o = 0;
    for (int p = 0; p < 2; ++p) {
        w.coef[p] = o; o += r64(3 * (int64_t)C + 3);
        w.cm[p] = o; o += r64((int64_t)(C + 1) * C);
    }
    for (int l = 1; l < L; ++l) { w.hk[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l < L; ++l) { w.sp[l] = o; o += r64((int64_t)C * n[l]); }
    for (int l = 1; l <= L; ++l) { w.dl[l] = o; o += r64((int64_t)C * n[l]); }
    w.hq[0] = o; o += r64((int64_t)C * maxw);
    w.hq[1] = o; o += r64((int64_t)C * maxw);
    w.mq = o; o += r64((int64_t)C * C);
    w.per_seq = o;
    return w;
}

enum Task : int { kPrep = 0, kFwd, kBwd, kMq, kU, kQb, kCarry, kNorm };

// One segment of a launch: `count` blocks of one task on layer l; tiles are numbered
// row-major over ceil(M/64) x tj tiles.
struct Seg {
    int task, l, tj, count;
};

struct Phase {
    PhLayout wl;  // workspace layout (in the argument block: indexed by layer at run time)
    int gx;       // blocks per memory
    int nseg;
    Seg seg[kMaxSeg];
    int64_t c0;  // first token of the chunk the products serve
    int n;       // its length
    int par;     // its parity buffer
    int64_t c0p; // chunk a kPrep task stages (into parity buffer ppar)
    int np;
    int ppar;
};

constexpr unsigned bit(int task) { return 1u << task; }
// The task sets one launch can hold; each is its own kernel instance, so the register
// allocation of one step's tiles does not pay for another's.
constexpr unsigned kSetFirst = bit(kFwd) | bit(kMq) | bit(kU) | bit(kPrep);
constexpr unsigned kSetFwd = bit(kFwd);
constexpr unsigned kSetBwd = bit(kBwd);
constexpr unsigned kSetRead = bit(kMq) | bit(kU);
constexpr unsigned kSetLast = bit(kQb) | bit(kCarry);
constexpr unsigned kSetNorm = bit(kNorm);

template <bool kMfma, unsigned kTasks>
__global__ void __launch_bounds__(kThreads, kTasks == kSetLast ? 2 : 1) phase_kernel(ScanArgs a, Phase ph) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ float s_al[256], s_et[256], s_be[256];

    // Workgroup w runs on XCD w % 8; renumber so that each XCD holds a contiguous range of
    // (memory, task) ids -- the tiles of one memory share operands through that XCD's L2.
    const int64_t nblk = gridDim.x;
    const int64_t w = blockIdx.x;
    const int64_t full = nblk & ~int64_t(7);
    const int64_t lid = w < full ? (w & 7) * (full >> 3) + (w >> 3) : w;
    const int64_t seq = lid / ph.gx;

    // find this block's segment (unrolled: no dynamic indexing of the argument block)
    int t = (int)(lid % ph.gx);
    Seg sg = ph.seg[0];
#pragma unroll
    for (int s = 1; s < kMaxSeg; ++s) {
        if (s < ph.nseg && t >= sg.count) {
            t -= sg.count;
            sg = ph.seg[s];
        }
    }
    const int i0 = (t / sg.tj) * kTile, j0 = (t % sg.tj) * kTile;

    const int64_t b = seq / a.H, h = seq % a.H;
    const int tid = threadIdx.x;
    const int L = a.L, C = a.C;
    const PhLayout& wl = ph.wl;
    float* ws = static_cast<float*>(a.ws) + seq * wl.per_seq;
    float* theta = a.thetaT + b * a.ss[0] + h * a.ss[1];
    float* mom = a.sT + b * a.ss[0] + h * a.ss[1];
    const int64_t qbase = b * a.qs[0] + h * a.qs[2];
    const int64_t ybase = b * a.ys[0] + h * a.ys[2];
    const int64_t gbase = b * a.gs[0] + h * a.gs[2];

    if (kTasks & bit(kPrep) && sg.task == kPrep) {
        // gates of chunk (c0p, np) -> its coefficients in parity buffer ppar
        const int n = ph.np, pp = ph.ppar;
        const int64_t c0 = ph.c0p;
        for (int i = tid; i < n; i += kThreads) {
            const int64_t gi = gbase + (c0 + i) * a.gs[1];
            s_al[i] = a.alpha[gi];
            s_et[i] = a.eta[gi];
            s_be[i] = a.beta[gi];
        }
        __syncthreads();
        // thread j owns column j of Cm: c_{t,j} for t = 0..n (the generic kernel's recurrence)
        float* ca = ws + wl.coef[pp];
        float* cb = ca + (C + 1);
        float* cw = cb + (C + 1);
        float* cp = cw + C;
        float* Cm = ws + wl.cm[pp];
        const int j = tid;
        float Bj = 0.0f, cj = 0.0f, at = 1.0f, bt = 0.0f, pb = 1.0f;
        const float omb_j = (j < n) ? 1.0f - s_be[j] : 0.0f;
        if (j < n) Cm[j] = 0.0f;
        if (j == 0) { ca[0] = 1.0f; cb[0] = 0.0f; }
        for (int tt = 0; tt < n; ++tt) {
            const float al = s_al[tt], et = s_et[tt], be = s_be[tt];
            pb *= be;
            if (j < tt) Bj *= be;
            else if (j == tt) Bj = 1.0f;
            const float keep = 1.0f - al;
            at *= keep;
            bt = keep * bt + et * pb;
            cj = keep * cj + ((j <= tt) ? et * omb_j * Bj : 0.0f);
            if (j < n) Cm[(int64_t)(tt + 1) * C + j] = cj;
            if (j == 0) { ca[tt + 1] = at; cb[tt + 1] = bt; }
        }
        if (j < n) cw[j] = omb_j * Bj;
        if (j == 0) cp[0] = pb;

        return;
    }

    const int n = ph.n, par = ph.par, l = sg.l;
    const int64_t c0 = ph.c0;
    const float* coef_a = ws + wl.coef[par];
    const float* coef_b = coef_a + (C + 1);
    const float* coef_w = coef_b + (C + 1);
    const float* coef_p = coef_w + C;
    const float* Cm = ws + wl.cm[par];
    const int nin = a.n[l - 1], nout = a.n[l];
    // Hk_{l-1} and Hq_{l-1} as (token, unit) or (unit, token) operands; for l = 1 these
    // are k and q themselves, read from the caller's tensors
    const int64_t in_off = qbase + c0 * a.qs[1];
    auto input = [&](const void* p, int64_t sr, int64_t sk) {
        Opnd o{nullptr, sr, sk, nullptr};
        if (a.io == TITANS_BF16)
            o.pb = static_cast<const __bf16*>(p) + in_off;
        else
            o.p = static_cast<const float*>(p) + in_off;
        return o;
    };
    const Opnd hk_rows = l == 1 ? input(a.k, a.qs[1], 1) : Opnd{ws + wl.hk[l - 1], nin, 1, nullptr};
    const Opnd hk_cols = l == 1 ? input(a.k, 1, a.qs[1]) : Opnd{ws + wl.hk[l - 1], 1, nin, nullptr};
    const Opnd hq_rows = l == 1 ? input(a.q, a.qs[1], 1) : Opnd{ws + wl.hq[(l - 1) & 1], nin, 1, nullptr};
    float* U = ws + wl.hq[l & 1];
    float* Dl = ws + wl.dl[l];
    float* Mq = ws + wl.mq;
    float* W = theta + a.off[l];
    float* S = mom + a.off[l];
    void* lds = smem;

    if (kTasks & bit(kNorm) && sg.task == kNorm) {
        // each token's gradient norm: the gradient of layer l is Delta_l Hk_{l-1}^T, so its
        // squared norm is |Delta_l|^2 |Hk_{l-1}|^2 (Hk_0 = k, read from the caller's tensor)
        for (int t = tid; t < n; t += kThreads) {
            float acc = 0.0f;
            for (int m = 1; m <= L; ++m) {
                const float* Dr = ws + wl.dl[m] + (int64_t)t * a.n[m];
                float dd = 0.0f, hh = 0.0f;
                for (int i = 0; i < a.n[m]; ++i) dd = fmaf(Dr[i], Dr[i], dd);
                if (m == 1) {
                    for (int i = 0; i < a.n[0]; ++i) {
                        const float x = load_io(a.k, in_off + (int64_t)t * a.qs[1] + i, a.io);
                        hh = fmaf(x, x, hh);
                    }
                } else {
                    const float* Hr = ws + wl.hk[m - 1] + (int64_t)t * a.n[m - 1];
                    for (int i = 0; i < a.n[m - 1]; ++i) hh = fmaf(Hr[i], Hr[i], hh);
                }
                acc = fmaf(dd, hh, acc);
            }
            a.surprise[gbase + (c0 + t) * a.gs[1]] = sqrtf(acc);
        }
        return;
    }

    switch (sg.task) {
        case kFwd: {  // Z_l = Hk_{l-1} W_l^T
            if constexpr (!(kTasks & bit(kFwd))) break;
            const Opnd A = hk_rows, Bo{W, nin, 1, nullptr};
            if (l < L) {
                float* Hout = ws + wl.hk[l];
                float* Sp = ws + wl.sp[l];
                tile<kMfma>(i0, j0, n, nout, nin, A, Bo, lds, [&](int i, int jj, float z) {
                    const float sg_ = sigm<kMfma>(z);
                    Hout[i * nout + jj] = z * sg_;
                    Sp[i * nout + jj] = sg_ * (1.0f + z * (1.0f - sg_));
                });
            } else {
                tile_pre<kMfma>(
                    i0, j0, n, nout, nin, A, Bo, lds,
                    [&](int i, int jj) { return load_io(a.v, qbase + (c0 + i) * a.qs[1] + jj, a.io); },
                    [&](int i, int jj, float z, float vv) {
                        Dl[i * nout + jj] = bias_grad(z - vv, a.bias, a.bias_param);
                    });
            }
            break;
        }
        case kBwd: {  // Delta_{l-1} = (Delta_l W_l) o SiLU'(Z_{l-1})
            if constexpr (!(kTasks & bit(kBwd))) break;
            float* Dp = ws + wl.dl[l - 1];
            const float* Sp = ws + wl.sp[l - 1];
            tile_pre<kMfma>(i0, j0, n, nin, nout, Opnd{Dl, nout, 1, nullptr}, Opnd{W, 1, nin, nullptr},
                            lds, [&](int i, int jj) { return Sp[i * nin + jj]; },
                            [&](int i, int jj, float x, float sp) { Dp[i * nin + jj] = x * sp; });
            break;
        }
        case kMq: {  // Mq = Cm o (Hq_{l-1} Hk_{l-1}^T), strictly lower triangular
            if constexpr (!(kTasks & bit(kMq))) break;
            tile_pre<kMfma>(i0, j0, n, n, nin, hq_rows, hk_rows, lds,
                            [&](int i, int jj) { return (jj < i) ? Cm[(int64_t)i * C + jj] : 0.0f; },
                            [&](int i, int jj, float x, float cm) { Mq[i * C + jj] = (jj < i) ? cm * x : 0.0f; });
            break;
        }
        case kU: {  // U_l = diag(a) Hq W_l^T - diag(b) Hq S_l^T
            if constexpr (!(kTasks & bit(kU))) break;
            if constexpr (kMfma) {  // both products from one staging of Hq, W, S
                tile_mfma_shared_a(i0, j0, n, nout, nin, hq_rows,
                                   Opnd{W, nin, 1, nullptr}, Opnd{S, nin, 1, nullptr},
                                   static_cast<__bf16*>(lds),
                                   [&](int i) { return float2{coef_a[i], coef_b[i]}; },
                                   [&](int i, int jj, float xw, float xs, float2 ab) {
                                       U[i * nout + jj] = ab.x * xw - ab.y * xs;
                                   });
            } else {
                const Opnd A = hq_rows;
                tile<kMfma>(i0, j0, n, nout, nin, A, Opnd{W, nin, 1, nullptr}, lds,
                            [&](int i, int jj, float x) { U[i * nout + jj] = coef_a[i] * x; });
                tile<kMfma>(i0, j0, n, nout, nin, A, Opnd{S, nin, 1, nullptr}, lds,
                            [&](int i, int jj, float x) { U[i * nout + jj] -= coef_b[i] * x; });
            }
            break;
        }
        case kQb: {  // U_l -= Mq Delta_l; then Hq_l = SiLU(U_l) in place, or y
            if constexpr (!(kTasks & bit(kQb))) break;
            const Opnd A{Mq, C, 1, nullptr}, Bo{Dl, 1, nout, nullptr};
            if (l < L) {
                tile_pre<kMfma, 4>(i0, j0, n, nout, n, A, Bo, lds,
                                   [&](int i, int jj) { return U[i * nout + jj]; },
                                   [&](int i, int jj, float x, float u0) {
                                       const float u = u0 - x;
                                       U[i * nout + jj] = u * sigm<kMfma>(u);
                                   });
            } else {
                tile_pre<kMfma, 4>(i0, j0, n, nout, n, A, Bo, lds,
                                   [&](int i, int jj) { return U[i * nout + jj]; },
                                   [&](int i, int jj, float x, float u0) {
                                       store_io(a.y, ybase + (c0 + i) * a.ys[1] + jj, a.io, u0 - x);
                                   });
            }
            break;
        }
        case kCarry: {  // W_l, S_l to the chunk end (W first: it needs the chunk-start S)
            if constexpr (!(kTasks & bit(kCarry))) break;
            const float an = coef_a[n], bn = coef_b[n], pn = coef_p[0];
            const float* crow = Cm + (int64_t)n * C;
            const Opnd Bo = hk_cols;
            if constexpr (kMfma) {  // both products from one staging of Delta_l and Hk
                tile_carry(i0, j0, nout, nin, n, Opnd{Dl, 1, nout, crow}, Opnd{Dl, 1, nout, coef_w},
                           Bo, W, S, nin, an, bn, pn, static_cast<__bf16*>(lds));
                break;
            }
            tile<kMfma>(i0, j0, nout, nin, n, Opnd{Dl, 1, nout, crow}, Bo, lds,
                        [&](int i, int jj, float x) {
                            const int64_t o = (int64_t)i * nin + jj;
                            W[o] = an * W[o] - bn * S[o] - x;
                        });
            tile<kMfma>(i0, j0, nout, nin, n, Opnd{Dl, 1, nout, coef_w}, Bo, lds,
                        [&](int i, int jj, float x) {
                            const int64_t o = (int64_t)i * nin + jj;
                            S[o] = pn * S[o] + x;
                        });
            break;
        }
        default: break;
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

int tiles(int x) { return (x + kTile - 1) / kTile; }

// Host-side builder of one launch.
struct Launch {
    Phase ph{};
    int blocks = 0;
    int lds = 0;   // bf16 staging bytes its largest product needs
    unsigned tasks = 0;
    void add(int task, int l, int M, int N, int K) {
        Seg& s = ph.seg[ph.nseg++];
        s.task = task;
        s.l = l;
        const bool single = task == kPrep || task == kNorm;  // one block per memory
        s.tj = single ? 1 : tiles(N);
        tasks |= bit(task);
        s.count = single ? 1 : tiles(M) * s.tj;
        blocks += s.count;
        const int need = (task == kPrep || task == kNorm) ? 0
                         : (task == kCarry || task == kU) ? mfma_lds_bytes(K < kWin3 ? K : kWin3, 3)
                                                          : mfma_lds_bytes(K, 2);
        if (need > lds) lds = need;
    }
};

template <bool kMfma>
hipError_t run(const ScanArgs& a, hipStream_t stream) {
    const int64_t nseq = a.B * a.H;
    const int L = a.L, C = a.C;
    const int64_t nchunks = (a.T + C - 1) / C;
    const PhLayout wl = ph_layout(C, L, a.n);
    auto chunk_len = [&](int64_t c) { return (int)((a.T - c * C) < C ? (a.T - c * C) : C); };

    if (kMfma) {
        const void* fns[] = {reinterpret_cast<const void*>(&phase_kernel<true, kSetFirst>),
                             reinterpret_cast<const void*>(&phase_kernel<true, kSetFwd>),
                             reinterpret_cast<const void*>(&phase_kernel<true, kSetBwd>),
                             reinterpret_cast<const void*>(&phase_kernel<true, kSetRead>),
                             reinterpret_cast<const void*>(&phase_kernel<true, kSetLast>)};
        for (const void* f : fns) {
            const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     mfma_lds_bytes(512));
            if (e != hipSuccess) return e;
        }
    }
    auto go = [&](Launch& x) -> hipError_t {
        const size_t lds = kMfma ? (size_t)(x.lds > 0 ? x.lds : mfma_lds_bytes(32)) : (size_t)kF32Lds;
        x.ph.gx = x.blocks;
        const dim3 grid((unsigned)(x.blocks * nseq));
        auto within = [&](unsigned set) { return (x.tasks & ~set) == 0; };
        if (within(kSetFwd))
            phase_kernel<kMfma, kSetFwd><<<grid, kThreads, lds, stream>>>(a, x.ph);
        else if (within(kSetBwd))
            phase_kernel<kMfma, kSetBwd><<<grid, kThreads, lds, stream>>>(a, x.ph);
        else if (within(kSetRead))
            phase_kernel<kMfma, kSetRead><<<grid, kThreads, lds, stream>>>(a, x.ph);
        else if (within(kSetLast))
            phase_kernel<kMfma, kSetLast><<<grid, kThreads, lds, stream>>>(a, x.ph);
        else if (within(kSetNorm))
            phase_kernel<kMfma, kSetNorm><<<grid, kThreads, lds, stream>>>(a, x.ph);
        else
            phase_kernel<kMfma, kSetFirst><<<grid, kThreads, lds, stream>>>(a, x.ph);
        return hipGetLastError();
    };

    {
        const dim3 grid((unsigned)((a.P + 255) / 256 < 64 ? (a.P + 255) / 256 : 64), (unsigned)nseq);
        copy_state_kernel<<<grid, 256, 0, stream>>>(a);
        Launch p0;
        p0.ph.wl = wl;
        p0.ph.c0p = 0;
        p0.ph.np = chunk_len(0);
        p0.ph.ppar = 0;
        p0.add(kPrep, 1, 0, 0, 0);
        hipError_t e = go(p0);
        if (e != hipSuccess) return e;
    }
    for (int64_t c = 0; c < nchunks; ++c) {
        const int n = chunk_len(c), par = (int)(c & 1);
        auto base = [&]() {
            Launch x;
            x.ph.wl = wl;
            x.ph.c0 = c * C;
            x.ph.n = n;
            x.ph.par = par;
            return x;
        };
        hipError_t e;
        {  // key forward of layer 1, layer-1 read products, next chunk's coefficients
            Launch x = base();
            x.add(kFwd, 1, n, a.n[1], a.n[0]);
            x.add(kMq, 1, n, n, a.n[0]);
            x.add(kU, 1, n, a.n[1], a.n[0]);
            if (c + 1 < nchunks) {
                x.ph.c0p = (c + 1) * C;
                x.ph.np = chunk_len(c + 1);
                x.ph.ppar = par ^ 1;
                x.add(kPrep, 1, 0, 0, 0);
            }
            if ((e = go(x)) != hipSuccess) return e;
        }
        for (int l = 2; l <= L; ++l) {
            Launch x = base();
            x.add(kFwd, l, n, a.n[l], a.n[l - 1]);
            if ((e = go(x)) != hipSuccess) return e;
        }
        for (int l = L; l >= 2; --l) {
            Launch x = base();
            x.add(kBwd, l, n, a.n[l - 1], a.n[l]);
            if ((e = go(x)) != hipSuccess) return e;
        }
        for (int l = 1; l <= L; ++l) {
            if (l > 1) {
                Launch x = base();
                x.add(kMq, l, n, n, a.n[l - 1]);
                x.add(kU, l, n, a.n[l], a.n[l - 1]);
                if ((e = go(x)) != hipSuccess) return e;
            }
            if (l == 1 && a.surprise) {  // every Delta is written: the token gradient norms
                Launch x = base();
                x.add(kNorm, 1, 0, 0, 0);
                if ((e = go(x)) != hipSuccess) return e;
            }
            Launch x = base();
            x.add(kQb, l, n, a.n[l], n);
            if (l == L)
                for (int m = 1; m <= L; ++m) x.add(kCarry, m, a.n[m], a.n[m - 1], n);
            if ((e = go(x)) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace

size_t scan_phased_workspace_bytes(const ScanArgs& a) {
    const PhLayout w = ph_layout(a.C, a.L, a.n);
    return (size_t)(a.B * a.H) * (size_t)w.per_seq * sizeof(float);
}

hipError_t launch_scan_phased(const ScanArgs& a, hipStream_t stream) {
    if (a.B * a.H == 0) return hipSuccess;
    return a.io == TITANS_BF16 ? run<true>(a, stream) : run<false>(a, stream);
}

}  // namespace titans
