// bkv_device.hpp -- device helpers shared by the gfx950 kernels.
//
// Built with -ffp-contract=off: every fp32 product and sum written here is
// rounded on its own unless a fused multiply-add is written explicitly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bkv.h"

namespace bkv {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN of that sign.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Monotone map of fp32 to uint32 (larger float -> larger code), for
// integer max / radix ordering.  -0 and +0 map to neighbouring codes.
__device__ __forceinline__ uint32_t f32_order(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_unorder(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

template <typename T>
__device__ __forceinline__ T clampi(T v, T lo, T hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

// Wave-wide argmin of (v, i): smallest v, then smallest i.  Every lane gets
// the result.
__device__ __forceinline__ void wave_argmin(float& v, int& i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        float v2 = __shfl_xor(v, off, kWave);
        int i2 = __shfl_xor(i, off, kWave);
        if (v2 < v || (v2 == v && i2 < i)) {
            v = v2;
            i = i2;
        }
    }
}

}  // namespace bkv
