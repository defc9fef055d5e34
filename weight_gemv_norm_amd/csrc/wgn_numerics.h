// wgn_numerics.h -- element-wise numerics shared by the kernels: BF16
// conversions, the epilogue activations and the order-preserving key of the
// argmax.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wgn {

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }
// FP32 -> BF16, round to nearest even (gfx950's v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

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

}  // namespace wgn
