// Device helpers shared by the fused MFMA scan kernels (gfx950, wave64).
//
// MFMA operand layouts.  For v_mfma_f32_16x16x32_bf16, lane l (g = l / 16, j = l % 16)
// holds A[j][k] and B[k][j] for eight k of a 32-wide block and D[4g + r][j], r = 0..3.
// An accumulator block is reused as an operand without leaving registers when its row
// index is the next product's reduction index: the eight k-slots of lane (g, j) are then
// rows {4g .. 4g+3} of the block's first 16-row tile and {16+4g .. 16+4g+3} of its
// second.  Every product uses that k order, so LDS fragments are read as two 8-byte
// pieces at columns 4g and 16 + 4g of a k-contiguous row.  LDS matrices are 64 x 64 with
// rows padded to 68 elements: the 16 rows a fragment read touches then start in
// distinct banks, and every LDS address is one per-lane base register plus an
// immediate offset.
#pragma once

#include <hip/hip_runtime.h>

#include "bias_util.h"

namespace titans {
namespace fused {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 bf4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ f32x4 f4(bf16x4 x) { return __builtin_convertvector(x, f32x4); }
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 acc_frag(f32x4 x0, f32x4 x1) { return cat(bf4(x0), bf4(x1)); }
__device__ __forceinline__ bf16x4 half4(bf16x8 x, int hi) {
    return hi ? __builtin_shufflevector(x, x, 4, 5, 6, 7) : __builtin_shufflevector(x, x, 0, 1, 2, 3);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

constexpr int kLd = 68;  // padded row length of every 64 x 64 LDS matrix

// Element (r, c) of a padded 64 x 64 matrix.
__device__ __forceinline__ int sw(int r, int c) { return r * kLd + c; }

// Operand fragment from a k-contiguous LDS row.  p = matrix + (j * kLd + 4 g) (lane
// base), off = 16 t * kLd + 32 kb for row tile t and k-block kb.
__device__ __forceinline__ bf16x8 frag(const __bf16* p, int off) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + off);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + off + 16);
    return cat(lo, hi);
}
__device__ __forceinline__ constexpr int fo(int t, int kb) { return 16 * t * kLd + 32 * kb; }

__device__ __forceinline__ float sigmoid(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * z));
}

// Register-pressure controls.  The compiler would otherwise keep every loop-invariant
// operand fragment of a fully unrolled loop live at once, and share one bf16
// conversion of a state tile between phases far apart.
//   opaque(x): a copy the compiler cannot prove equal to x, so conversions made from
//              it are not shared with other uses of x.
//   reload():  LDS reads after this point are not merged with reads before it.
// An int the compiler cannot see through: LDS lane bases built from it are recomputed in
// each phase instead of being hoisted out of the chunk loop and kept live throughout.
__device__ __forceinline__ int opq(int x) {
    asm volatile("" : "+v"(x));
    return x;
}
template <class T>
__device__ __forceinline__ T opaque(T x) {
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ void reload() { asm volatile("" ::: "memory"); }
// Keeps the scheduler from hoisting the next tile's state reads into this one.
__device__ __forceinline__ void tile_fence() { __builtin_amdgcn_sched_barrier(0); }
__device__ __forceinline__ bf16x8 state_frag(f32x4 x0, f32x4 x1) {
    return acc_frag(opaque(x0), opaque(x1));
}

// Wave-wide inclusive scans with DPP (row shifts within 16 lanes, then row broadcasts).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp(float identity, float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(x),
                                                      kCtrl, kRowMask, 0xf, false));
}
__device__ __forceinline__ float wave_scan_mul(float x) {
    x *= dpp<0x111, 0xf>(1.f, x);
    x *= dpp<0x112, 0xf>(1.f, x);
    x *= dpp<0x114, 0xf>(1.f, x);
    x *= dpp<0x118, 0xf>(1.f, x);
    x *= dpp<0x142, 0xa>(1.f, x);
    x *= dpp<0x143, 0xc>(1.f, x);
    return x;
}
__device__ __forceinline__ float wave_scan_add(float x) {
    x += dpp<0x111, 0xf>(0.f, x);
    x += dpp<0x112, 0xf>(0.f, x);
    x += dpp<0x114, 0xf>(0.f, x);
    x += dpp<0x118, 0xf>(0.f, x);
    x += dpp<0x142, 0xa>(0.f, x);
    x += dpp<0x143, 0xc>(0.f, x);
    return x;
}
// Inclusive scan of affine maps x -> k x + c in lane order (earlier lanes applied first).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ void affine_step(float& k, float& c) {
    const float ek = dpp<kCtrl, kRowMask>(1.f, k), ec = dpp<kCtrl, kRowMask>(0.f, c);
    c = k * ec + c;
    k *= ek;
}
__device__ __forceinline__ void wave_scan_affine(float& k, float& c) {
    affine_step<0x111, 0xf>(k, c);
    affine_step<0x112, 0xf>(k, c);
    affine_step<0x114, 0xf>(k, c);
    affine_step<0x118, 0xf>(k, c);
    affine_step<0x142, 0xa>(k, c);
    affine_step<0x143, 0xc>(k, c);
}
// Value of lane l - 1 (lane 0 gets `first`).
__device__ __forceinline__ float lane_prev(float x, float first) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(first), __float_as_int(x), 0x138,
                                                      0xf, 0xf, false));
}

// Make this wave's LDS writes visible to its own later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The output-layer error E2 = loss'(O - V) of four components; the squared error (the
// default) stays one multiply.
__device__ __forceinline__ f32x4 bias_grad4(f32x4 r, int kind, float prm) {
    if (kind == TITANS_BIAS_L2) return 2.f * r;
    f32x4 e;
#pragma unroll
    for (int u = 0; u < 4; ++u) e[u] = bias_grad(r[u], kind, prm);
    return e;
}

}  // namespace fused
}  // namespace titans
