// Product with 4-bit weights in groups of 128 along K ("One Token, Kernel by
// Kernel", section "4-bit weights"): y[b][n] = R(sum_k (s q + z) x[b][k]),
// with q the 4-bit code (low nibble = even k), s and z the BF16 scale and zero
// of (row n, group k/128).
//
// Each lane owns 16 bytes (32 codes, a quarter of a group) of a row per 1 KB
// slice; a wave takes 4 rows at a time, the loads of several such items
// issued together before use.
// Codes become BF16 pairs without conversion instructions: the byte permute
// v_perm_b32 places one code in the mantissa of each half and an OR with
// 0x4300 gives the BF16 values 128 + q, exact; v_dot2_f32_bf16 then forms
// sum (128 + q) x in FP32.  With S = sum x over the lane's 32 inputs
// (computed once per workgroup), the lane's share of the row is
//   s * dot + (z - 128 s) * S  =  sum (s q + z) x.
// x (all batch rows) and the 32-input sums are staged in LDS once per
// workgroup; workgroups stride over row groups.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace wgn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#ifndef WGN_I4_ROWS
#define WGN_I4_ROWS 4
#endif
constexpr int I4_ROWS = WGN_I4_ROWS;         // rows per wave at a time
#ifndef WGN_I4_WAVES
#define WGN_I4_WAVES 4
#endif
#ifndef WGN_I4_BLOCKS_PER_CU
#define WGN_I4_BLOCKS_PER_CU 8
#endif
constexpr int I4_WAVES = WGN_I4_WAVES;
constexpr int I4_BLOCKS_PER_CU = WGN_I4_BLOCKS_PER_CU;  // cap of the grid (workgroups stride over row groups)
#ifndef WGN_I4_BATCH
#define WGN_I4_BATCH 2
#endif
// items whose loads are issued together, at batch 1 and 2 (one at larger
// batches, whose registers go to x; measured: 2 is 5 % faster than 1 at batch
// 1, 4 slower than 2, and 2 slower than 1 at batch 8)
constexpr int I4_BATCH = WGN_I4_BATCH;
constexpr uint32_t I4_MAGIC = 0x43004300u;   // BF16 128.0 in both halves
constexpr int I4_MAX_LDS = 160 * 1024;       // dynamic LDS of one workgroup on gfx950

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over the 64 lanes, complete in lane 63 only: rows of 16 lanes by DPP,
// then DPP row broadcasts (lane 15 into rows 1 and 3, lane 31 into rows 2
// and 3), so no LDS permute is on the path.
__device__ __forceinline__ float wave_sum_last(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31
    return v;
}

template <int B>
__global__ __launch_bounds__(64 * I4_WAVES) void gemv_int4_kernel(const uint16_t *x, int64_t xs, int32_t K,
                                                                 const uint8_t *W4, const uint16_t *sc,
                                                                 const uint16_t *zr, int32_t N, uint16_t *y,
                                                                 int64_t ys) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    uint16_t *sx = (uint16_t *)lds;                        // [B][K] BF16
    float *ssum = (float *)(lds + (size_t)B * K * 2);      // [B][K/32]
    const int32_t tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int32_t K8 = K / 8, K32 = K / 32, half = K / 2, ng = K / 128;
    for (int32_t i = tid; i < B * K8; i += 64 * I4_WAVES) {
        const int32_t b = i / K8, j = i - b * K8;
        *(u32x4 *)(sx + (size_t)b * K + j * 8) = *(const u32x4 *)(x + (size_t)b * xs + j * 8);
    }
    __syncthreads();
    for (int32_t i = tid; i < B * K32; i += 64 * I4_WAVES) {
        const int32_t b = i / K32, j = i - b * K32;
        const uint32_t *p = (const uint32_t *)(sx + (size_t)b * K + j * 32);
        float s = 0.0f;
#pragma unroll
        for (int m = 0; m < 16; ++m) s += bf2f(p[m] & 0xFFFFu) + bf2f(p[m] >> 16);
        ssum[i] = s;
    }
    __syncthreads();

    const int32_t slices = (half + 1023) / 1024;
    const int32_t groups = (N + I4_ROWS * I4_WAVES - 1) / (I4_ROWS * I4_WAVES);
    // One item is a slice c of the wave's 4 rows of row group rg; a
    // workgroup's items are (rg, c) for rg = blockIdx.x, + gridDim.x, ... in
    // order.  Items are taken IB at a time: all their codes, scales and
    // zeros are requested before the first is used, so one memory round trip
    // serves IB items.  Loads past the last item re-read the last
    // row group (in range, never used), so every pass issues the same loads.
    struct Item {
        u32x4 code[I4_ROWS];
        float s[I4_ROWS], z[I4_ROWS];
    };
    // Buffer loads with 32-bit offsets (the host keeps the codes below 2 GB):
    // one offset register per load, so that computing the next item's
    // addresses needs no registers a load in flight still owns.
    const __amdgpu_buffer_rsrc_t rcode = __builtin_amdgcn_make_buffer_rsrc((void *)W4, (short)0,
                                                                           (int)((int64_t)N * half), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc((void *)sc, (short)0,
                                                                         (int)((int64_t)N * ng * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rzr = __builtin_amdgcn_make_buffer_rsrc((void *)zr, (short)0,
                                                                         (int)((int64_t)N * ng * 2), 0x00020000);
    auto load = [&](int32_t rg, int32_t c, Item &it) {
        rg = min(rg, groups - 1);
        const int32_t n0 = (rg * I4_WAVES + w) * I4_ROWS;
        const int32_t byte0 = (c * 64 + lane) * 16;  // this lane's bytes within a row
        const bool act = byte0 < half;
        const uint32_t g = (uint32_t)(act ? byte0 * 2 : 0) / 128u;
#pragma unroll
        for (int r = 0; r < I4_ROWS; ++r) {
            const uint32_t n = (uint32_t)min(n0 + r, N - 1);  // in range; rows past N are not stored
            it.code[r] = __builtin_amdgcn_raw_buffer_load_b128(rcode, n * (uint32_t)half + (act ? byte0 : 0), 0, 0);
            it.s[r] = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rsc, (n * (uint32_t)ng + g) * 2u, 0, 0));
            it.z[r] = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rzr, (n * (uint32_t)ng + g) * 2u, 0, 0));
        }
    };
    float acc[I4_ROWS][B];
#pragma unroll
    for (int r = 0; r < I4_ROWS; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
    auto use = [&](int32_t rg, int32_t c, const Item &it) {
        const int32_t byte0 = (c * 64 + lane) * 16;
        if (byte0 < half) {
            const int32_t kb = byte0 * 2;  // first k of this lane's bytes
            // x of every batch row for this lane's 32 inputs, and their sums
            uint32_t xw[B][16];
            float S[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const u32x4 *xp = (const u32x4 *)(sx + (size_t)b * K + kb);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const u32x4 v = xp[u];
                    xw[b][4 * u] = v.x; xw[b][4 * u + 1] = v.y; xw[b][4 * u + 2] = v.z; xw[b][4 * u + 3] = v.w;
                }
                S[b] = ssum[b * K32 + kb / 32];
            }
#pragma unroll
            for (int r = 0; r < I4_ROWS; ++r) {
                // the row's 16 code pairs as BF16 (128 + q) pairs, decoded once for all batch rows
                const uint32_t cw[4] = {it.code[r].x, it.code[r].y, it.code[r].z, it.code[r].w};
                uint32_t pr[16];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t lo = cw[u] & 0x0F0F0F0Fu, hi = (cw[u] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        // bytes [lo_q, 0, hi_q, 0]: codes of k = 2q (low half) and 2q+1 (high half)
                        const uint32_t sel = (uint32_t)q | (0x0Cu << 8) | ((uint32_t)(4 + q) << 16) | (0x0Cu << 24);
                        pr[4 * u + q] = __builtin_amdgcn_perm(hi, lo, sel) | I4_MAGIC;
                    }
                }
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    float dot = 0.0f;
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr[m]),
                                                              __builtin_bit_cast(bf16x2, xw[b][m]), dot, false);
                    acc[r][b] += it.s[r] * dot + (it.z[r] - 128.0f * it.s[r]) * S[b];
                }
            }
        }
        if (c == slices - 1) {
            const int32_t n0 = (rg * I4_WAVES + w) * I4_ROWS;
#pragma unroll
            for (int r = 0; r < I4_ROWS; ++r) {
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const float t = wave_sum_last(acc[r][b]);
                    if (lane == 63 && n0 + r < N)
                        y[(size_t)b * ys + n0 + r] = __builtin_bit_cast(uint16_t, (__bf16)t);
                    acc[r][b] = 0.0f;
                }
            }
        }
    };
    constexpr int IB = B <= 2 ? I4_BATCH : 1;
    int32_t rg = blockIdx.x, c = 0;
    while (rg < groups) {
        Item it[IB];
        int32_t rgs[IB], cs[IB];
#pragma unroll
        for (int u = 0; u < IB; ++u) {
            rgs[u] = rg;
            cs[u] = c;
            load(rg, c, it[u]);
            if (++c == slices) {
                c = 0;
                rg += gridDim.x;
            }
        }
#pragma unroll
        for (int u = 0; u < IB; ++u)
            if (rgs[u] < groups) use(rgs[u], cs[u], it[u]);
    }
}

}  // namespace

size_t gemv_int4_lds_bytes(int32_t batch, int32_t K) { return (size_t)batch * K * 2 + (size_t)batch * (K / 32) * 4; }

// x and its sums may take the whole 160 KB of a gfx950 workgroup's LDS (the
// down projection's 8960 inputs at batch 8 need 152 KB); the attribute is set
// once per batch size before its first launch.
template <int B>
static hipError_t allow_full_lds() {
    static bool done = false;
    if (done) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute((const void *)gemv_int4_kernel<B>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, I4_MAX_LDS);
    if (e == hipSuccess) done = true;
    return e;
}

hipError_t launch_gemv_int4(const uint16_t *x, int64_t xs, int32_t batch, int32_t K, const uint8_t *W4,
                            const uint16_t *sc, const uint16_t *zr, int32_t N, uint16_t *y, int64_t ys,
                            int32_t cus, hipStream_t s) {
    const int32_t groups = (N + I4_ROWS * I4_WAVES - 1) / (I4_ROWS * I4_WAVES);
    const int32_t blocks = groups < I4_BLOCKS_PER_CU * cus ? groups : I4_BLOCKS_PER_CU * cus;
    const size_t lds = gemv_int4_lds_bytes(batch, K);
    dim3 grid(blocks), block(64 * I4_WAVES);
    switch (batch) {
#define WGN_I4_CASE(BB)                                                                                   \
    case BB: {                                                                                            \
        const hipError_t ea = allow_full_lds<BB>();                                                       \
        if (ea != hipSuccess) return ea;                                                                  \
        hipLaunchKernelGGL(gemv_int4_kernel<BB>, grid, block, lds, s, x, xs, K, W4, sc, zr, N, y, ys);    \
        break;                                                                                            \
    }
    WGN_I4_CASE(1) WGN_I4_CASE(2) WGN_I4_CASE(3) WGN_I4_CASE(4)
    WGN_I4_CASE(5) WGN_I4_CASE(6) WGN_I4_CASE(7) WGN_I4_CASE(8)
#undef WGN_I4_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace wgn
