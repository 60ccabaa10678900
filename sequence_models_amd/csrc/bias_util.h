// The attentional bias of the memory's writes (titans_bias): the derivative of its
// per-component loss at a residual r = M(k) - v, which takes the place of 2 r in the
// output-layer error of every scan kernel.
#pragma once

#include <hip/hip_runtime.h>

#include "titans_mem.h"

namespace titans {

// 2 r (squared error); 2 clamp(r, -delta, delta) (Huber, threshold delta);
// p sign(r) |r|^(p-1), 0 at r = 0 (l_p, p >= 1).  |r|^(p-1) = 2^((p-1) log2 |r|) on the
// hardware exp2 / log2 (about one ulp each; a handful of registers, so the fused kernels
// keep their allocation).
__device__ __forceinline__ float bias_grad(float r, int kind, float prm) {
    if (kind == TITANS_BIAS_HUBER) return 2.0f * fminf(fmaxf(r, -prm), prm);
    if (kind == TITANS_BIAS_LP) {
        const float m = prm == 1.0f ? 1.0f
                                    : __builtin_amdgcn_exp2f((prm - 1.0f) *
                                                             __builtin_amdgcn_logf(fabsf(r)));
        return r == 0.0f ? 0.0f : copysignf(prm * m, r);
    }
    return 2.0f * r;
}

// The second derivative of the per-component loss (the reverse pass differentiates the
// output-layer error once more): 2; 2 inside [-delta, delta] and 0 outside (Huber);
// p (p - 1) |r|^(p-2) (l_p, p >= 2; 0 at r = 0 for p > 2).
__device__ __forceinline__ float bias_grad_prime(float r, int kind, float prm) {
    if (kind == TITANS_BIAS_HUBER) return fabsf(r) <= prm ? 2.0f : 0.0f;
    if (kind == TITANS_BIAS_LP) {
        if (prm == 2.0f) return 2.0f;
        if (r == 0.0f) return 0.0f;
        return prm * (prm - 1.0f) *
               __builtin_amdgcn_exp2f((prm - 2.0f) * __builtin_amdgcn_logf(fabsf(r)));
    }
    return 2.0f;
}

}  // namespace titans
