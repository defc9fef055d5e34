// wgn_numerics.h -- element-wise numerics shared by the kernels: BF16
// conversions, the epilogue activations (and the GELU slope of the backward
// pass) and the order-preserving key of the argmax.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wgn {

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }
// FP32 -> BF16, round to nearest even (gfx950's v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// FP64 -> BF16, round to nearest even, in two steps that round once: to FP32
// with round-to-odd (an inexact result keeps an odd last bit, so it can never
// sit on a BF16 tie), then FP32 -> BF16 to nearest even (v_cvt_pk_bf16_f32).
// FP32 carries 16 more bits than BF16, so the result equals rounding the FP64
// value directly (round-to-odd, Boldo and Melquiond).
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
    const float f = (float)d;
    uint32_t b = __float_as_uint(f);
    if ((double)f != d && (b & 1u) == 0u) b += fabs((double)f) < fabs(d) ? 1u : 0xFFFFFFFFu;
    return f2bf(__uint_as_float(b));
}

// FP32 value -> 32-bit key whose unsigned order is the value order (negative
// values bit-inverted, positive ones with the sign bit set), and back.
__device__ __forceinline__ uint32_t orderable(float f) {
    uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unorderable(uint32_t o) {
    uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(b);
}

// GELU, tanh form, and SiLU (x * sigmoid(x)) in FP32.
__device__ __forceinline__ float gelu_tanh(float z) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
}
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// d/dz of gelu_tanh: with t = tanh(c (z + 0.044715 z^3)),
// 0.5 (1 + t) + 0.5 z (1 - t^2) c (1 + 3 * 0.044715 z^2).
__device__ __forceinline__ float gelu_tanh_grad(float z) {
    const float c = 0.7978845608028654f;
    const float z2 = z * z;
    const float t = tanhf(c * (z + 0.044715f * z2 * z));
    return 0.5f * (1.0f + t) + 0.5f * z * (1.0f - t * t) * c * (1.0f + 0.134145f * z2);
}

}  // namespace wgn
