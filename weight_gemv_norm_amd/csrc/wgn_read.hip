// wgn_read.hip -- a plain streaming read of device memory: the measured HBM
// read ceiling of the GPU the weight stream runs on.  The pages quote every
// bandwidth figure against a ceiling measured on the same card beside the
// rated one ("One Token, Kernel by Kernel: A Decode Step on a Laptop GPU",
// section "Step 2: every kernel class on the roofline"); this kernel is that
// measurement here.
//
// Every 16-byte chunk of the buffer is read exactly once with a non-temporal
// 128-bit load; a wave's load covers 1 KB of consecutive bytes and each lane
// keeps DEPTH independent loads in flight.  The loaded values are folded into
// one word per lane, which is stored only if it equals a fixed pattern, so the
// loads cannot be removed and the kernel (practically) writes nothing.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace wgn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t SINK_PATTERN = 0x9E3779B9u;

template <int DEPTH>
__global__ void stream_read_kernel(const u32x4 *__restrict__ p, uint64_t n16, uint32_t *sink) {
    const uint64_t nt = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (uint64_t)(DEPTH - 1) * nt < n16; i += (uint64_t)DEPTH * nt) {
        u32x4 v[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) v[d] = __builtin_nontemporal_load(p + i + (uint64_t)d * nt);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    for (; i < n16; i += nt) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == SINK_PATTERN) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *src, uint64_t n16, int32_t grid, int32_t threads, int32_t depth,
                              uint32_t *sink, hipStream_t s) {
    const u32x4 *p = (const u32x4 *)src;
    switch (depth) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(grid), dim3(threads), 0, s, p, n16, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(grid), dim3(threads), 0, s, p, n16, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(threads), 0, s, p, n16, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(threads), 0, s, p, n16, sink); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(grid), dim3(threads), 0, s, p, n16, sink); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace wgn
