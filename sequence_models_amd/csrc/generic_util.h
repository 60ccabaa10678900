// Element I/O and activation helpers shared by the generic (any-shape) scan kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bias_util.h"
#include "titans_mem.h"

namespace titans {
namespace generic {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float load_io(const void* p, int64_t idx, int io) {
    return io == TITANS_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[idx])
                             : static_cast<const float*>(p)[idx];
}

__device__ __forceinline__ void store_io(void* p, int64_t idx, int io, float x) {
    if (io == TITANS_BF16)
        static_cast<uint16_t*>(p)[idx] = f32_to_bf16(x);
    else
        static_cast<float*>(p)[idx] = x;
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

}  // namespace generic
}  // namespace titans
