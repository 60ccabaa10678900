// Titans MAG block (memory as gate) and MAC block (memory as context) on gfx950:
// everything of the blocks except the memory scan and read, which run through the scan
// and retrieve launchers.
//
// The block (Titans explainer, the three architecture variants, memory as gate; the
// lowest.today summary, "Varianti dell'Architettura Titans"): the memory branch reads the
// long-term memory, sliding-window attention is the short-term branch, and the memory's
// output gates the attention output through a sigmoid, o = sigmoid(y_mem) * y_attn.  The
// projection front end and the output projection take the plainest reading:
//
//   [q | k | v | g] = x W_in^T         W_in [3D + 3H, D] (out features x in features)
//   q, k <- unit L2 norm per (token, head); v as is
//   alpha = sigmoid(g_a + b_a), eta = eta_scale sigmoid(g_e + b_e), beta = sigmoid(g_b + b_b)
//   y_attn = causal softmax attention over the last `window` tokens (itself included),
//            scores q.k / sqrt(d)
//   out = (sigmoid(y_mem) * y_attn) W_out^T                W_out [D, D]
//
// Kernels:
//   gemm_nt_kernel   C = A W^T on v_mfma_f32_16x16x32_bf16, 256 x 128 tiles, 8 waves of
//                    64 x 64, k staged 32 deep through double-buffered LDS; the front-end
//                    projection normalizes and gates in its epilogue, the output
//                    projection writes bf16.
//                    When D is a multiple of 64 the projection's epilogue also normalizes
//                    q and k per head and applies the gates (ProjFront); otherwise:
//   prep_kernel      one workgroup per token: per-head norms of q and k (shuffle sums over
//                    the lanes that hold one head), bf16 q, k, v, and the three gates.
//   attn_kernel      flash-style attention: 128 queries (32 per wave) against 64-key
//                    blocks double-buffered in LDS, scores computed transposed (keys x
//                    queries) so each lane owns one query's running max and sum,
//                    probabilities fed back to the value product straight from the score
//                    accumulators.  MAG: causal sliding window, the epilogue gates with
//                    sigmoid(y_mem).  MAC: one segment whose memory reads form a prefix of
//                    keys and values visible to every query, own keys causal, no gate.
#include <hip/hip_runtime.h>

#include <math.h>

#include "mfma_util.h"
#include "titans_internal.h"

namespace titans {
namespace mag {

using fused::bf16x4;
using fused::bf16x8;
using fused::f32x4;

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 zero8() {
    const __bf16 z = static_cast<__bf16>(0.0f);
    return bf16x8{z, z, z, z, z, z, z, z};
}

// Max over the lane pairs l, l ^ 16 and l, l ^ 32 by the permlane swaps (register moves,
// no LDS round trip): each swap returns the pair's two values, in some order, to both lanes.
__device__ __forceinline__ float max_pair16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_pair32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Workgroups are dealt to the 8 XCDs round-robin; when the grid divides evenly, give each
// XCD one contiguous range of logical tiles so that tiles sharing operands share an L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nb) {
    if (nb % 8) return bid;
    return (bid % 8) * (nb / 8) + bid / 8;
}

// ------------------------------------------------------------------------------ GEMM

constexpr int kGT = 128;       // tile extent in N
constexpr int kGM = 256;       // tile extent in M (8 waves: 4 x 2 of 64 x 64)
constexpr int kGK = 32;        // k per stage
constexpr int kGP = kGK + 8;   // LDS row pitch in bf16
constexpr int kGPR = kGK / 8;                // 16-byte pieces per tile row and stage
constexpr int kGRows = 512 / kGPR;           // tile rows one pass of 512 threads stages
constexpr int kGItA = kGM / kGRows;          // passes per stage: A (256 rows), W (128 rows)
constexpr int kGItW = kGT / kGRows;

// Epilogues see a wave's whole 64 x 64 result: acc[in][im] holds C[r0 + 16 im + j]
// [c0 + 16 in + 4 g + r]; red is 2 KiB of LDS free for the epilogue, and every wave of the
// workgroup calls tile() (so it may synchronize).
template <class Store>
struct PerElement {
    Store st;
    __device__ void tile(const f32x4 (&acc)[4][4], int64_t r0, int c0, int wn, int g, int j,
                         int64_t M, float* red) const {
#pragma unroll
        for (int im = 0; im < 4; ++im) {
            const int64_t m = r0 + 16 * im + j;
            if (m >= M) continue;
#pragma unroll
            for (int in = 0; in < 4; ++in) st(m, c0 + 16 * in + 4 * g, acc[in][im]);
        }
    }
};
struct StoreF32 {
    float* p;
    int64_t ld;
    int n_lim;  // a multiple of 4: column groups at or beyond it are not stored
    __device__ void operator()(int64_t m, int n, f32x4 v) const {
        if (n < n_lim) *reinterpret_cast<f32x4*>(p + m * ld + n) = v;
    }
};
struct StoreBf16 {
    __bf16* p;
    int64_t ld;
    int n_lim;
    __device__ void operator()(int64_t m, int n, f32x4 v) const {
        if (n < n_lim) *reinterpret_cast<bf16x4*>(p + m * ld + n) = fused::bf4(v);
    }
};

__device__ __forceinline__ float sigm(float z) { return 1.0f / (1.0f + expf(-z)); }

// The front end in the projection's epilogue (D a multiple of 64, d = 32, 64 or 128): a
// wave's 64-column strip lies in one of the q, k, v, gate sections; in q and k it holds two
// heads (d = 32), one (64) or half of one (128, the other half in the partner wave
// wn ^ 1, combined through LDS).  Sums of squares per row: the lane's 16 (or 8) values,
// then xor shuffles over the four lanes g that share a row.
struct ProjFront {
    int D, H, d;
    float eta_scale;
    const float* bg;
    __bf16 *q, *k, *v;
    float *alpha, *eta, *beta;
    __device__ void tile(const f32x4 (&acc)[4][4], int64_t r0, int c0, int wn, int g, int j,
                         int64_t M, float* red) const {
        const int sec = c0 < 3 * D ? c0 / D : 3;
#pragma unroll
        for (int im = 0; im < 4; ++im) {
            const int64_t m = r0 + 16 * im + j;
            float s0 = 0.f, s1 = 0.f;  // columns 0..31 and 32..63 of the strip
#pragma unroll
            for (int in = 0; in < 4; ++in) {
                const float e = acc[in][im][0] * acc[in][im][0] + acc[in][im][1] * acc[in][im][1] +
                                acc[in][im][2] * acc[in][im][2] + acc[in][im][3] * acc[in][im][3];
                if (in < 2) s0 += e; else s1 += e;
            }
            s0 += __shfl_xor(s0, 16);
            s0 += __shfl_xor(s0, 32);
            s1 += __shfl_xor(s1, 16);
            s1 += __shfl_xor(s1, 32);
            float n0 = s0 + s1, n1 = s0 + s1;  // d = 64: one head
            if (d == 32) {
                n0 = s0;
                n1 = s1;
            } else if (d == 128) {
                // both halves' sums meet in LDS: red[wm-local row][wn]
                __syncthreads();
                if (g == 0) red[(static_cast<int>(r0 % kGM) + 16 * im + j) * 2 + wn] = s0 + s1;
                __syncthreads();
                n0 = n1 = red[(static_cast<int>(r0 % kGM) + 16 * im + j) * 2] +
                          red[(static_cast<int>(r0 % kGM) + 16 * im + j) * 2 + 1];
            }
            if (m >= M || (sec == 3 && c0 >= 3 * D + 3 * H)) continue;
            if (sec < 3) {
                __bf16* dst = sec == 0 ? q : sec == 1 ? k : v;
                const float i0 = sec == 2 ? 1.0f : 1.0f / sqrtf(n0);
                const float i1 = sec == 2 ? 1.0f : 1.0f / sqrtf(n1);
                const int cs = c0 - sec * D;
#pragma unroll
                for (int in = 0; in < 4; ++in)
                    *reinterpret_cast<bf16x4*>(dst + m * D + cs + 16 * in + 4 * g) =
                        fused::bf4(acc[in][im] * (in < 2 ? i0 : i1));
            } else {
#pragma unroll
                for (int in = 0; in < 4; ++in)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int gc = c0 - 3 * D + 16 * in + 4 * g + r;
                        if (gc >= 3 * H) continue;
                        const float sgm = sigm(acc[in][im][r] + bg[gc]);
                        const int which = gc / H, h = gc - which * H;
                        float* dst = which == 0 ? alpha : which == 1 ? eta : beta;
                        dst[m * H + h] = which == 1 ? eta_scale * sgm : sgm;
                    }
            }
        }
    }
};

// C[m][n] = sum_k A[m][k] W[n][k] for A [M, K] (row pitch lda) and W [N, K] (row pitch K),
// K a multiple of 8, A and W 16-byte aligned.  Workgroup tile (tm, tn) covers rows
// 256 tm .. +255 and columns 128 tn .. +127; wave w the 64 x 64 block (w / 2, w % 2).
// The product is formed transposed (W rows as the MFMA's A operand) so that a lane's
// accumulator holds four consecutive columns of one row: lane (g, j) of block (in, im)
// holds C[16 im + j][16 in + 4 g + r], r = 0..3.
template <class Epi>
__global__ __launch_bounds__(512) void gemm_nt_kernel(const __bf16* __restrict__ A, int64_t lda,
                                                      const __bf16* __restrict__ W, int64_t M,
                                                      int N, int K, int tiles_n, Epi epi) {
    __shared__ __align__(16) __bf16 sa[2][kGM * kGP];
    __shared__ __align__(16) __bf16 sw[2][kGT * kGP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t m0 = (bid / tiles_n) * kGM;
    const int n0 = static_cast<int>(bid % tiles_n) * kGT;
    // staging: thread t stages the 16-byte piece (t % kGPR) of rows t / kGPR + kGRows i
    const int r0 = tid / kGPR, kc = (tid % kGPR) * 8;
    bf16x8 ra[kGItA], rw[kGItW];
    auto load = [&](int k0) {
        const bool kok = k0 + kc < K;
#pragma unroll
        for (int i = 0; i < kGItA; ++i) {
            const int64_t m = m0 + r0 + kGRows * i;
            ra[i] = (kok && m < M) ? *reinterpret_cast<const bf16x8*>(A + m * lda + k0 + kc) : zero8();
        }
#pragma unroll
        for (int i = 0; i < kGItW; ++i) {
            const int n = n0 + r0 + kGRows * i;
            rw[i] = (kok && n < N) ? *reinterpret_cast<const bf16x8*>(W + (int64_t)n * K + k0 + kc)
                                   : zero8();
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kGItA; ++i)
            *reinterpret_cast<bf16x8*>(&sa[buf][(r0 + kGRows * i) * kGP + kc]) = ra[i];
#pragma unroll
        for (int i = 0; i < kGItW; ++i)
            *reinterpret_cast<bf16x8*>(&sw[buf][(r0 + kGRows * i) * kGP + kc]) = rw[i];
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fused::zero4();
    const int wm = wave >> 1, wn = wave & 1;  // wm 0..3
    const int nk = (K + kGK - 1) / kGK;
    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
        const int cur = s & 1;
        if (s + 1 < nk) load((s + 1) * kGK);
#pragma unroll
        for (int ks = 0; ks < kGK / 32; ++ks) {
            bf16x8 fa[4], fw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[i] = *reinterpret_cast<const bf16x8*>(&sa[cur][(wm * 64 + 16 * i + j) * kGP + 32 * ks + 8 * g]);
                fw[i] = *reinterpret_cast<const bf16x8*>(&sw[cur][(wn * 64 + 16 * i + j) * kGP + 32 * ks + 8 * g]);
            }
#pragma unroll
            for (int in = 0; in < 4; ++in)
#pragma unroll
                for (int im = 0; im < 4; ++im) acc[in][im] = mma(fw[in], fa[im], acc[in][im]);
        }
        if (s + 1 < nk) store(cur ^ 1);
        __syncthreads();
    }
    // the main loop ended on a barrier: the staging buffers are free
    epi.tile(acc, m0 + wm * 64, n0 + wn * 64, wn, g, j, M, reinterpret_cast<float*>(&sa[0][0]));
}

template <class Epi>
static hipError_t gemm_nt(const __bf16* A, int64_t lda, const __bf16* W, int64_t M, int N, int K,
                          Epi epi, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const int tiles_n = (N + kGT - 1) / kGT;
    const int64_t tiles = (M + kGM - 1) / kGM * tiles_n;
    hipLaunchKernelGGL(gemm_nt_kernel<Epi>, dim3(static_cast<unsigned>(tiles)), dim3(512), 0,
                       stream, A, lda, W, M, N, K, tiles_n, epi);
    return hipGetLastError();
}

// ------------------------------------------------------------------------- front end

// Token row m of the projection (fp32, pitch ldp): columns [0, D) q, [D, 2D) k,
// [2D, 3D) v, [3D, 3D + 3H) the gate logits.  Thread t handles the four columns 4t .. 4t+3
// of each 1024-column group; with d a multiple of 32 dividing 256, the d / 4 lanes
// holding one head are consecutive lanes of one wave, and a butterfly over them leaves
// every lane with its head's sum of squares.
__global__ __launch_bounds__(256) void prep_kernel(const float* __restrict__ proj, int64_t ldp,
                                                   int H, int d, float eta_scale,
                                                   const float* __restrict__ bg,
                                                   __bf16* __restrict__ q, __bf16* __restrict__ k,
                                                   __bf16* __restrict__ v, float* __restrict__ alpha,
                                                   float* __restrict__ eta, float* __restrict__ beta) {
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const int D = H * d;
    const float* row = proj + m * ldp;
    for (int c0 = 0; c0 < D; c0 += 1024) {
        const int c = c0 + 4 * tid;
        const bool ok = c < D;
        f32x4 qv = fused::zero4(), kv = fused::zero4(), vv = fused::zero4();
        if (ok) {
            qv = *reinterpret_cast<const f32x4*>(row + c);
            kv = *reinterpret_cast<const f32x4*>(row + D + c);
            vv = *reinterpret_cast<const f32x4*>(row + 2 * D + c);
        }
        float sq = qv[0] * qv[0] + qv[1] * qv[1] + qv[2] * qv[2] + qv[3] * qv[3];
        float sk = kv[0] * kv[0] + kv[1] * kv[1] + kv[2] * kv[2] + kv[3] * kv[3];
        for (int o = 1; o < d / 4; o <<= 1) {
            sq += __shfl_xor(sq, o);
            sk += __shfl_xor(sk, o);
        }
        if (ok) {
            const float iq = 1.0f / sqrtf(sq), ik = 1.0f / sqrtf(sk);
            *reinterpret_cast<bf16x4*>(q + m * D + c) = fused::bf4(qv * iq);
            *reinterpret_cast<bf16x4*>(k + m * D + c) = fused::bf4(kv * ik);
            *reinterpret_cast<bf16x4*>(v + m * D + c) = fused::bf4(vv);
        }
    }
    for (int t = tid; t < 3 * H; t += 256) {
        const float s = sigm(row[3 * D + t] + bg[t]);
        const int which = t / H, h = t - which * H;
        float* dst = which == 0 ? alpha : which == 1 ? eta : beta;
        dst[m * H + h] = which == 1 ? eta_scale * s : s;
    }
}

// ------------------------------------------------------------------------- attention

constexpr int kQW = 32;         // queries per wave: two 16-query tiles
constexpr int kQB = 4 * kQW;    // queries per workgroup
constexpr int kKB = 64;         // keys per LDS block
constexpr int kVP = kKB + 4;    // transposed value rows in LDS (bf16 pitch)

// Attention over "virtual" key positions 0 .. P + Tq - 1 of one (b, h): positions below P
// are prefix entries (MAC: the segment's memory reads, each used as key and value), the
// rest are the tokens row0 .. row0 + Tq - 1 themselves; query i (token row0 + i) sits at
// position P + i and sees the positions j <= P + i with j > P + i - window.  The MAG
// block's attention is P = 0, row0 = 0, Tq = T with its sliding window; the MAC block's is
// one segment (row0 its first token, Tq = P its length) with an unbounded window.
struct AttnArgs {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    const __bf16* ymem;  // MAG: the memory read that gates the output
    const __bf16* hpre;  // MAC: the memory reads (rows of the [B, T, H, d] buffer)
    __bf16* o;
    int64_t T;           // tokens per sequence of the [B, T, H, d] buffers
    int64_t row0, Tq, P;
    int H, window, nqb;
    float scale_log2;
};

// One workgroup per (b, h, 128-query block); all buffers are [B, T, H, kD] bf16 rows of
// pitch D = H kD.  Wave w owns queries q0 + 32 w + 16 u + j (u = 0, 1) at lane (g, j).
// Per 64-key block: S^T tile (u, t) = K_t Q_u^T, so lane (g, j) holds the scores of keys
// 16 t + 4 g + r for its query of tile u; the max is shared by the four lanes of a query
// (two permlane swaps); O^T += V^T P^T and the row sums (ones x P^T) take P^T straight from
// the score registers (the accumulator's row index, the key, is the reduction index of the
// value product) and V^T from a transposed LDS copy.  Key and value blocks are
// double-buffered: the next block's global loads are in flight while the current one is
// used.  Blocks that lie wholly outside a wave's windows are skipped by that wave; masks
// are applied only on blocks at the diagonal or the window's edge.  Exponentials are the
// hardware's base-2 exponential (v_exp_f32): arguments are <= 0 and results below fp32's
// normal range flush to 0, which a probability that small does not notice.  The softmax
// reference moves only when a block's max exceeds it by more than 8 (a factor of 2^8), so
// most blocks rescale nothing.
template <int kD, bool kMac>
__global__ __launch_bounds__(256, kD <= 64 ? 3 : 1) void attn_kernel(AttnArgs a) {
    constexpr int kKP = kD + 8;                   // key rows in LDS (bf16 pitch)
    constexpr int kKPieces = kKB * kD / 8;        // 16-byte pieces of a key block
    constexpr int kVTasks = (kKB / 4) * (kD / 4); // 4 keys x 4 columns of a value block
    constexpr int kNK = (kKPieces + 255) / 256, kNV = (kVTasks + 255) / 256;
    __shared__ __align__(16) __bf16 ks[2][kKB * kKP];
    __shared__ __align__(16) __bf16 vt[2][kD * kVP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = static_cast<int>(bid % a.nqb);
    const int64_t bh = bid / a.nqb;
    const int64_t b = bh / a.H;
    const int h = static_cast<int>(bh % a.H);
    const int64_t D = static_cast<int64_t>(a.H) * kD;
    const int64_t base = b * a.T * D + static_cast<int64_t>(h) * kD;  // (b, 0, h, 0)
    const int64_t Tq = a.Tq, P = kMac ? a.P : 0, Tk = P + Tq, row0 = kMac ? a.row0 : 0;
    const int window = a.window;
    const int64_t q0 = static_cast<int64_t>(qb) * kQB;          // first query of the block
    const int64_t wq0 = q0 + kQW * wave;                         // first query of the wave
    const int64_t wq0v = P + wq0, wlastv = wq0v + kQW - 1;       // their key positions

    bf16x8 qf[2][kD / 32];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t qi = wq0 + 16 * u + j;
#pragma unroll
        for (int kb = 0; kb < kD / 32; ++kb)
            qf[u][kb] = qi < Tq ? *reinterpret_cast<const bf16x8*>(a.q + base + (row0 + qi) * D +
                                                                   32 * kb + 8 * g)
                                : zero8();
    }
    f32x4 acc[2][kD / 16], lsum[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        lsum[u] = fused::zero4();
#pragma unroll
        for (int dt = 0; dt < kD / 16; ++dt) acc[u][dt] = fused::zero4();
    }
    float m_ref[2] = {-INFINITY, -INFINITY};
    const __bf16 one = static_cast<__bf16>(1.0f);
    const bf16x8 ones = {one, one, one, one, one, one, one, one};

    const int64_t qlastv = P + ((q0 + kQB - 1 < Tq - 1) ? q0 + kQB - 1 : Tq - 1);
    const int64_t kfirst = P + q0 - window + 1 > 0 ? P + q0 - window + 1 : 0;
    const int64_t kbeg = kfirst / kKB * kKB;
    const int nblk = static_cast<int>((qlastv - kbeg) / kKB) + 1;

    // row of key position kv: a prefix entry (MAC) or a token; positions past Tk are zero
    auto key_row = [&](const __bf16* own, int64_t kv) -> const __bf16* {
        if (kMac && kv < P) return a.hpre + base + (row0 + kv) * D;
        return own + base + (row0 + kv - P) * D;
    };
    bf16x8 rk[kNK];
    bf16x4 rv[kNV][4];
    auto fetch = [&](int64_t kb0) {
        // the common case: a whole block of one source, no bound checks
        if (kb0 + kKB <= Tk && (!kMac || kb0 + kKB <= P || kb0 >= P)) {
            const __bf16* ksrc = key_row(a.k, kb0);
            const __bf16* vsrc = key_row(a.v, kb0);
#pragma unroll
            for (int i = 0; i < kNK; ++i) {
                const int c = tid + 256 * i;
                if (kKPieces % 256 == 0 || c < kKPieces)
                    rk[i] = *reinterpret_cast<const bf16x8*>(ksrc + (c / (kD / 8)) * D + (c % (kD / 8)) * 8);
            }
#pragma unroll
            for (int i = 0; i < kNV; ++i) {
                const int t = tid + 256 * i;
                if (kVTasks % 256 == 0 || t < kVTasks) {
                    const __bf16* vp = vsrc + (4 * (t / (kD / 4))) * D + 4 * (t % (kD / 4));
#pragma unroll
                    for (int e = 0; e < 4; ++e) rv[i][e] = *reinterpret_cast<const bf16x4*>(vp + e * D);
                }
            }
            return;
        }
        const bool full = false;
#pragma unroll
        for (int i = 0; i < kNK; ++i) {
            const int c = tid + 256 * i;
            if (c < kKPieces) {
                const int64_t kv = kb0 + c / (kD / 8);
                rk[i] = (full || kv < Tk)
                            ? *reinterpret_cast<const bf16x8*>(key_row(a.k, kv) + (c % (kD / 8)) * 8)
                            : zero8();
            }
        }
#pragma unroll
        for (int i = 0; i < kNV; ++i) {
            const int t = tid + 256 * i;
            if (t < kVTasks) {
                const int cg = t % (kD / 4), kg = t / (kD / 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t kv = kb0 + 4 * kg + e;
                    const __bf16 z = static_cast<__bf16>(0.0f);
                    rv[i][e] = (full || kv < Tk)
                                   ? *reinterpret_cast<const bf16x4*>(key_row(a.v, kv) + 4 * cg)
                                   : bf16x4{z, z, z, z};
                }
            }
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kNK; ++i) {
            const int c = tid + 256 * i;
            if (c < kKPieces)
                *reinterpret_cast<bf16x8*>(&ks[buf][(c / (kD / 8)) * kKP + (c % (kD / 8)) * 8]) = rk[i];
        }
#pragma unroll
        for (int i = 0; i < kNV; ++i) {
            const int t = tid + 256 * i;
            if (t < kVTasks) {
                const int cg = t % (kD / 4), kg = t / (kD / 4);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<bf16x4*>(&vt[buf][(4 * cg + c) * kVP + 4 * kg]) =
                        bf16x4{rv[i][0][c], rv[i][1][c], rv[i][2][c], rv[i][3][c]};
            }
        }
    };

    fetch(kbeg);
    stash(0);
    __syncthreads();
    for (int ib = 0; ib < nblk; ++ib) {
        const int buf = ib & 1;
        const int64_t kb0 = kbeg + static_cast<int64_t>(ib) * kKB;
        const bool more = ib + 1 < nblk;
        if (more) fetch(kb0 + kKB);
        // some (query, key) of this wave and block with key <= query < key + window
        const bool live = wq0 < Tq && kb0 <= wlastv && kb0 + kKB - 1 > wq0v - window;
        if (live) {
            const bool edge = kb0 + kKB - 1 > wq0v || kb0 <= wlastv - window;
            f32x4 st[2][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                bf16x8 kf[kD / 32];
#pragma unroll
                for (int kb = 0; kb < kD / 32; ++kb)
                    kf[kb] = *reinterpret_cast<const bf16x8*>(&ks[buf][(16 * t + j) * kKP + 32 * kb + 8 * g]);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    st[u][t] = fused::zero4();
#pragma unroll
                    for (int kb = 0; kb < kD / 32; ++kb) st[u][t] = mma(kf[kb], qf[u][kb], st[u][t]);
                }
            }
            bf16x8 pf[2][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (edge) {
                    // key - query position for key kb0 + 4 g (|.| < P + Tq + 2 kQB: int32 by
                    // the host's limit on T)
                    const int rel0 = static_cast<int>(kb0 - (wq0v + 16 * u + j)) + 4 * g;
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int rel = rel0 + 16 * t + r;
                            if (!(rel <= 0 && rel > -window)) st[u][t][r] = -INFINITY;
                        }
                }
                float mx = -INFINITY;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    mx = fmaxf(fmaxf(fmaxf(mx, st[u][t][0]), fmaxf(st[u][t][1], st[u][t][2])), st[u][t][3]);
                mx = max_pair32(max_pair16(mx));
                const float ms = mx * a.scale_log2;
                const bool grow = ms > m_ref[u] + 8.0f;
                if (__ballot(grow)) {
                    // lanes that keep their reference (possibly still -inf) scale by 1
                    const float corr = grow ? __builtin_amdgcn_exp2f(m_ref[u] - ms) : 1.0f;
                    if (grow) m_ref[u] = ms;
                    lsum[u] *= corr;
#pragma unroll
                    for (int dt = 0; dt < kD / 16; ++dt) acc[u][dt] *= corr;
                }
                const float m_use = m_ref[u] == -INFINITY ? 0.0f : m_ref[u];
                bf16x4 pb[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    f32x4 p;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        p[r] = __builtin_amdgcn_exp2f(fmaf(st[u][t][r], a.scale_log2, -m_use));
                    pb[t] = fused::bf4(p);
                }
                pf[u][0] = fused::cat(pb[0], pb[1]);
                pf[u][1] = fused::cat(pb[2], pb[3]);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int dt = 0; dt < kD / 16; ++dt) {
                    const __bf16* p = &vt[buf][(16 * dt + j) * kVP + 32 * kb + 4 * g];
                    const bf16x8 vf = fused::cat(*reinterpret_cast<const bf16x4*>(p),
                                                 *reinterpret_cast<const bf16x4*>(p + 16));
#pragma unroll
                    for (int u = 0; u < 2; ++u) acc[u][dt] = mma(vf, pf[u][kb], acc[u][dt]);
                }
            // row sums of the rounded probabilities on the matrix cores: every row of
            // ones * P^T is the sum, so each lane's four results are its query's
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int u = 0; u < 2; ++u) lsum[u] = mma(ones, pf[u][kb], lsum[u]);
        }
        if (more) stash(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float l = lsum[u][0];
        const int64_t qi = wq0 + 16 * u + j;
        if (qi >= Tq) continue;
        const float inv = 1.0f / l;
#pragma unroll
        for (int dt = 0; dt < kD / 16; ++dt) {
            const int64_t at = base + (row0 + qi) * D + 16 * dt + 4 * g;
            f32x4 out;
            if (kMac) {
                out = acc[u][dt] * inv;
            } else {
                const f32x4 ym = fused::f4(*reinterpret_cast<const bf16x4*>(a.ymem + at));
#pragma unroll
                for (int r = 0; r < 4; ++r) out[r] = sigm(ym[r]) * (acc[u][dt][r] * inv);
            }
            *reinterpret_cast<bf16x4*>(a.o + at) = fused::bf4(out);
        }
    }
}

}  // namespace mag

bool mag_head_dim_supported(int d) { return d == 32 || d == 64 || d == 128; }

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Workspace: proj fp32 [M, ldp], q / k / v / y_mem / o bf16 [M, D], alpha / eta / beta
// fp32 [M, H], each piece 256-byte aligned; the memory scan's own workspace follows.
size_t mag_workspace_bytes(const MagArgs& g) {
    const int64_t M = g.B * g.T, D = g.H * g.d;
    const int64_t ldp = (3 * D + 3 * g.H + 3) / 4 * 4;
    return static_cast<size_t>(align256(M * ldp * 4) + 5 * align256(M * D * 2) +
                               3 * align256(M * g.H * 4));
}

void mag_place(MagArgs& g, void* ws) {
    const int64_t M = g.B * g.T, D = g.H * g.d;
    g.ldp = (3 * D + 3 * g.H + 3) / 4 * 4;
    char* p = static_cast<char*>(ws);
    g.proj = reinterpret_cast<float*>(p);
    p += align256(M * g.ldp * 4);
    __bf16** bufs[5] = {&g.q, &g.k, &g.v, &g.ymem, &g.o};
    for (__bf16** b : bufs) {
        *b = reinterpret_cast<__bf16*>(p);
        p += align256(M * D * 2);
    }
    float** gates[3] = {&g.alpha, &g.eta, &g.beta};
    for (float** a : gates) {
        *a = reinterpret_cast<float*>(p);
        p += align256(M * g.H * 4);
    }
}

hipError_t launch_mag_front(const MagArgs& g, hipStream_t stream) {
    const int64_t M = g.B * g.T;
    const int D = static_cast<int>(g.H * g.d);
    const int N = 3 * D + 3 * static_cast<int>(g.H);
    if (D % 64 == 0)  // normalization and gates in the GEMM's epilogue
        return mag::gemm_nt(g.x, D, g.w_in, M, N, D,
                            mag::ProjFront{D, static_cast<int>(g.H), g.d, g.eta_scale, g.b_gate,
                                           g.q, g.k, g.v, g.alpha, g.eta, g.beta},
                            stream);
    hipError_t e = mag::gemm_nt(g.x, D, g.w_in, M, N, D,
                                mag::PerElement<mag::StoreF32>{{g.proj, g.ldp, static_cast<int>(g.ldp)}},
                                stream);
    if (e != hipSuccess || M == 0) return e;
    hipLaunchKernelGGL(mag::prep_kernel, dim3(static_cast<unsigned>(M)), dim3(256), 0, stream,
                       g.proj, g.ldp, static_cast<int>(g.H), g.d, g.eta_scale, g.b_gate, g.q, g.k,
                       g.v, g.alpha, g.eta, g.beta);
    return hipGetLastError();
}

template <bool kMac>
static hipError_t launch_attn(mag::AttnArgs a, int d, int64_t B, hipStream_t stream) {
    if (B * a.H * a.Tq == 0) return hipSuccess;
    a.nqb = static_cast<int>((a.Tq + mag::kQB - 1) / mag::kQB);
    const dim3 grid(static_cast<unsigned>(B * a.H * a.nqb));
    a.scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(d));
    switch (d) {
        case 32: hipLaunchKernelGGL((mag::attn_kernel<32, kMac>), grid, dim3(256), 0, stream, a); break;
        case 64: hipLaunchKernelGGL((mag::attn_kernel<64, kMac>), grid, dim3(256), 0, stream, a); break;
        case 128: hipLaunchKernelGGL((mag::attn_kernel<128, kMac>), grid, dim3(256), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mag_attention(const MagArgs& g, hipStream_t stream) {
    mag::AttnArgs a{};
    a.q = g.q; a.k = g.k; a.v = g.v; a.ymem = g.ymem; a.hpre = nullptr; a.o = g.o;
    a.T = g.T; a.row0 = 0; a.Tq = g.T; a.P = 0;
    a.H = static_cast<int>(g.H);
    a.window = g.window;
    return launch_attn<false>(a, g.d, g.B, stream);
}

hipError_t launch_mac_attention(const MagArgs& g, const __bf16* h, int64_t row0, int64_t len,
                                hipStream_t stream) {
    mag::AttnArgs a{};
    a.q = g.q; a.k = g.k; a.v = g.v; a.ymem = nullptr; a.hpre = h; a.o = g.o;
    a.T = g.T; a.row0 = row0; a.Tq = len; a.P = len;
    a.H = static_cast<int>(g.H);
    a.window = 0x7fffffff;
    return launch_attn<true>(a, g.d, g.B, stream);
}

hipError_t launch_mag_out(const MagArgs& g, hipStream_t stream) {
    const int64_t M = g.B * g.T;
    const int D = static_cast<int>(g.H * g.d);
    return mag::gemm_nt(g.o, D, g.w_out, M, D, D, mag::PerElement<mag::StoreBf16>{{g.out, D, D}},
                        stream);
}

}  // namespace titans
