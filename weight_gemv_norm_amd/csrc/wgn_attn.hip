// Attention of one new token over a static key/value cache, in one launch
// ("Making small PyTorch ops faster on a laptop GPU", section "A full decode
// step is a different story": append the new key and value, FP32 softmax,
// the cache split across blocks, the last block to finish merges; "One
// Token, Kernel by Kernel", section "The fix: Part 10's split-KV kernel":
// (batch, head, slot, dimension) layout, the valid length read on the device,
// each key/value head read once for its whole group of query heads).
//
// Grid: (chunks of 128 slots, key/value heads, batch rows); 256 threads = 4
// waves, each wave 32 slots.  A lane holds 16 bytes (8 dimensions) of 8 key
// rows and 8 value rows, all loaded before the first use; 16 lanes cover one
// 256-byte row.  Scores are FP32 dot products (v_dot2_f32_bf16) reduced over
// the 16 lanes of a row by DPP; weights are 2^(s - m) with the score scale
// pre-multiplied by log2(e).  Each row of lanes keeps its own maximum and
// weight sum (no cross-lane step); the workgroup combines its 16 rows in LDS.
//
// Merge: a chunk that holds valid slots writes its partial (per query head:
// maximum m, weight sum l, weighted value sums) and takes a ticket; the last
// of up to 8 siblings to arrive merges their partials into one for the next
// level, and the last arrival at the top level writes the output.  On this
// chip one workgroup merging many 3 KB partials takes several microseconds of
// coherent loads, so the merge is a tree of fan-in 8 rather than one level.
// Partials and tickets use the system-coherent cache policy (sc0|sc1), so no
// L2 write-back or invalidate is needed between workgroups on different XCDs.
// The ticket's last arrival resets it to zero, so the next call (or a graph
// replay) starts from zero.  Nothing waits on another workgroup.
#include "wgn_attn.h"

namespace wgn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int ATT_COH = 17;                 // sc0|sc1: the system-coherent level
constexpr uint32_t ATT_RSRC_W3 = 0x00020000u;
constexpr int ATT_LOADS = ATT_SLOTS_PER_WAVE / 4;  // 4 rows per wave-wide load

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// 8 BF16 products summed in FP32.  The vector elements are copied to scalars
// first: bit-casting an ext-vector element expression directly miscompiles to
// element 0 with this toolchain.
__device__ __forceinline__ float dot8(const u32x4 &a, const u32x4 &b) {
    const uint32_t aa[4] = {a.x, a.y, a.z, a.w}, bb[4] = {b.x, b.y, b.z, b.w};
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aa[i]), __builtin_bit_cast(bf16x2, bb[i]),
                                              acc, false);
    return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over each row of 16 lanes; every lane of the row gets the same bits.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);  // row_half_mirror
    v += dpp_f<0x140>(v);  // row_mirror
    return v;
}

// Buffer resource over 2 GB from base; a null base gets an empty range, so a
// store through it is dropped without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, base ? 0x7FFFFFFF : 0, (int)ATT_RSRC_W3);
}
__device__ __forceinline__ void coh_store(__amdgpu_buffer_rsrc_t r, int32_t idx, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, idx * 4, 0, ATT_COH);
}
__device__ __forceinline__ float coh_load(__amdgpu_buffer_rsrc_t r, int32_t idx) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, idx * 4, 0, ATT_COH));
}
// 16-byte forms; idx is a multiple of 4 floats.
__device__ __forceinline__ void coh_store4(__amdgpu_buffer_rsrc_t r, int32_t idx, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, idx * 4, 0, ATT_COH);
}
__device__ __forceinline__ f32x4 coh_load4(__amdgpu_buffer_rsrc_t r, int32_t idx) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, idx * 4, 0, ATT_COH));
}
// Four outputs rounded to BF16 (8 bytes; the destination is 8-byte aligned).
__device__ __forceinline__ void store_out4(uint16_t *p, f32x4 v) {
    const uint32_t lo = (uint32_t)to_bf16(v.x) | ((uint32_t)to_bf16(v.y) << 16);
    const uint32_t hi = (uint32_t)to_bf16(v.z) | ((uint32_t)to_bf16(v.w) << 16);
    *(uint2 *)p = make_uint2(lo, hi);
}

// At least 3 waves per SIMD (at most 168 VGPRs): 3 workgroups per CU, so one
// workgroup's arithmetic overlaps the others' loads.  Measured: +20 % at long
// caches and batch 4; 4 waves per SIMD does not fit without spilling.
#ifndef WGN_ATT_MIN_WAVES
#define WGN_ATT_MIN_WAVES 3
#endif
template <int G>
__global__ __launch_bounds__(ATT_THREADS, WGN_ATT_MIN_WAVES) void decode_attention_kernel(AttnArgs a) {
    constexpr int E = att_entry_floats(G);
    constexpr int NO = G * ATT_D;                 // outputs per (batch row, key/value head)
    constexpr int NQ4 = NO / 4;                   // float4 groups of outputs (at most 256)
    constexpr int ROWS = 4 * ATT_WAVES;           // rows of 16 lanes in the workgroup
    static_assert(NQ4 <= ATT_THREADS, "one float4 of outputs per thread");
    __shared__ __attribute__((aligned(16))) float s_acc[ROWS * G * ATT_D];  // [wave][row][head][dim]
    __shared__ float s_m[ROWS * G], s_l[ROWS * G];                         // [wave][row][head]
    __shared__ float s_mm[ATT_FAN * G], s_ll[ATT_FAN * G];
    __shared__ uint32_t s_tick;

    const int32_t c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int32_t tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane >> 4, col = lane & 15;
    const int32_t bg = b * a.hkv + g;
    const int32_t p0 = a.pos[b];
    // last valid slot; -1 for a row whose position is out of range (nothing valid)
    const int32_t last = (p0 >= 0 && p0 < a.slots) ? p0 : -1;
    const int32_t t0 = c * ATT_CHUNK;
    uint16_t *out_bg = a.out + ((size_t)b * a.hq + (size_t)g * G) * ATT_D;

    if (t0 <= last) {
        const size_t row0 = (size_t)bg * a.slots;
        const uint16_t *kn = a.k_new + (size_t)bg * ATT_D + col * 8;
        const uint16_t *vn = a.v_new + (size_t)bg * ATT_D + col * 8;
        u32x4 qv[G], kd[ATT_LOADS], vd[ATT_LOADS];
#pragma unroll
        for (int h = 0; h < G; ++h)
            qv[h] = *(const u32x4 *)(a.q + ((size_t)b * a.hq + (size_t)g * G + h) * ATT_D + col * 8);
        // Slots after the last valid one read the last one again (never beyond
        // it, so an unwritten tail of the cache is never touched); their
        // weight is zero.  The last slot comes from the new key/value.
#pragma unroll
        for (int i = 0; i < ATT_LOADS; ++i) {
            const int32_t t = min(t0 + w * ATT_SLOTS_PER_WAVE + i * 4 + r, last);
            const bool fresh = t == last;
            kd[i] = *(const u32x4 *)(fresh ? kn : a.k_cache + (row0 + t) * ATT_D + col * 8);
            vd[i] = *(const u32x4 *)(fresh ? vn : a.v_cache + (row0 + t) * ATT_D + col * 8);
        }
        // One query head at a time: its 8 scores, the wave's maximum, the
        // weights and this lane's 8 weighted value sums, posted to LDS.
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float sc[ATT_LOADS], mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < ATT_LOADS; ++i) {
                const bool ok = t0 + w * ATT_SLOTS_PER_WAVE + i * 4 + r <= last;
                const float sv = row16_sum(dot8(kd[i], qv[h])) * a.scale_log2;
                sc[i] = ok ? sv : -INFINITY;
                mx = fmaxf(mx, sc[i]);
            }
            // the 16 lanes of a row hold the same scores: mx is this row's maximum
            const float mu = mx == -INFINITY ? 0.0f : mx;  // a row with no valid slot
            float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f}, lw = 0.0f;
#pragma unroll
            for (int i = 0; i < ATT_LOADS; ++i) {
                const float p = __builtin_amdgcn_exp2f(sc[i] - mu);
                const uint32_t vv[4] = {vd[i].x, vd[i].y, vd[i].z, vd[i].w};
                lw += p;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[2 * j] += p * bf_lo(vv[j]);
                    acc[2 * j + 1] += p * bf_hi(vv[j]);
                }
            }
            float *dst = s_acc + ((w * 4 + r) * G + h) * ATT_D + col * 8;
            *(f32x4 *)dst = (f32x4){acc[0], acc[1], acc[2], acc[3]};
            *(f32x4 *)(dst + 4) = (f32x4){acc[4], acc[5], acc[6], acc[7]};
            if (col == 0) {
                s_m[(w * 4 + r) * G + h] = mx;
                s_l[(w * 4 + r) * G + h] = lw;
            }
        }
        // the append: the lanes that hold the new token's row store it
#pragma unroll
        for (int i = 0; i < ATT_LOADS; ++i) {
            if (t0 + w * ATT_SLOTS_PER_WAVE + i * 4 + r == last) {
                *(u32x4 *)(a.k_cache + (row0 + last) * ATT_D + col * 8) = kd[i];
                *(u32x4 *)(a.v_cache + (row0 + last) * ATT_D + col * 8) = vd[i];
            }
        }
    }
    __syncthreads();
    // One float4 of outputs (4 dimensions of one query head) per thread.
    const bool mine = tid < NQ4;
    const int32_t h = tid / (ATT_D / 4), d0 = (tid % (ATT_D / 4)) * 4;
    if (t0 <= last) {
        if (mine) {
            // over the rows (4 per wave); finite: row 0 of wave 0 holds slot t0
            float M = -INFINITY;
#pragma unroll
            for (int wr = 0; wr < ROWS; ++wr) M = fmaxf(M, s_m[wr * G + h]);
            f32x4 A = {0.0f, 0.0f, 0.0f, 0.0f};
            float L = 0.0f;
#pragma unroll
            for (int wr = 0; wr < ROWS; ++wr) {
                const float f = __builtin_amdgcn_exp2f(s_m[wr * G + h] - M);
                A += f * *(const f32x4 *)(s_acc + (wr * G + h) * ATT_D + d0);
                L += f * s_l[wr * G + h];
            }
            if (a.top == 0) {
                store_out4(out_bg + h * ATT_D + d0, A / L);
            } else {
                const __amdgpu_buffer_rsrc_t rp = rsrc(a.part[0] + (size_t)bg * a.count[0] * E);
                coh_store4(rp, c * E + h * ATT_D + d0, A);
                if (d0 == 0) {
                    coh_store(rp, c * E + NO + h, M);
                    coh_store(rp, c * E + NO + G + h, L);
                }
            }
        }
    } else if (a.top == 0 && mine) {
        store_out4(out_bg + h * ATT_D + d0, (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
    }

    // ------------------------------------------------------------- merge tree
    int32_t idx = c;
    for (int32_t level = 0; level < a.top; ++level) {
        __builtin_amdgcn_s_waitcnt(0);  // this workgroup's partial is written through
        __syncthreads();
        const int32_t J = idx / ATT_FAN;
        const int32_t nm = min(ATT_FAN, a.count[level] - J * ATT_FAN);
        uint32_t *tk = a.tick[level + 1] + (size_t)bg * a.count[level + 1] + J;
        if (tid == 0) s_tick = __hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (s_tick != (uint32_t)(nm - 1)) return;  // a sibling is still running: it merges
        if (tid == 0) __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        idx = J;
        // siblings [J*FAN, J*FAN + nm) of this level; item i covers slots from i * span
        const int64_t span = (int64_t)ATT_CHUNK << (ATT_FAN_LOG2 * level);
        const int32_t first = J * ATT_FAN;
        const __amdgpu_buffer_rsrc_t rin = rsrc(a.part[level] + (size_t)bg * a.count[level] * E);
        if (tid < nm * G) {
            const int32_t i = tid / G, hh = tid % G;
            const bool ok = (int64_t)(first + i) * span <= last;
            const float m = coh_load(rin, (first + i) * E + NO + hh);
            const float l = coh_load(rin, (first + i) * E + NO + G + hh);
            s_mm[i * G + hh] = ok ? m : -INFINITY;
            s_ll[i * G + hh] = ok ? l : 0.0f;
        }
        f32x4 av[ATT_FAN];
        if (mine) {
#pragma unroll
            for (int i = 0; i < ATT_FAN; ++i) {
                const int32_t it = i < nm ? first + i : first;  // in range; unused values are masked
                av[i] = coh_load4(rin, it * E + h * ATT_D + d0);
            }
        }
        __syncthreads();
        const bool top = level + 1 == a.top;
        if (mine) {
            float M = -INFINITY;
#pragma unroll
            for (int i = 0; i < ATT_FAN; ++i)
                if (i < nm) M = fmaxf(M, s_mm[i * G + h]);
            f32x4 A = {0.0f, 0.0f, 0.0f, 0.0f};
            float L = 0.0f;
            if (M != -INFINITY) {
#pragma unroll
                for (int i = 0; i < ATT_FAN; ++i) {
                    if (i < nm) {
                        const bool ok = (int64_t)(first + i) * span <= last;
                        const float f = __builtin_amdgcn_exp2f(s_mm[i * G + h] - M);
                        A += f * (ok ? av[i] : (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
                        L += f * s_ll[i * G + h];
                    }
                }
            }
            if (top) {
                store_out4(out_bg + h * ATT_D + d0, L > 0.0f ? A / L : (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
            } else if (M != -INFINITY) {
                const __amdgpu_buffer_rsrc_t rout = rsrc(a.part[level + 1] + (size_t)bg * a.count[level + 1] * E);
                coh_store4(rout, J * E + h * ATT_D + d0, A);
                if (d0 == 0) {
                    coh_store(rout, J * E + NO + h, M);
                    coh_store(rout, J * E + NO + G + h, L);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_decode_attention(const AttnArgs &a, int32_t group, int32_t batch, hipStream_t s) {
    dim3 grid(a.count[0], a.hkv, batch), block(ATT_THREADS);
    switch (group) {
    case 1: hipLaunchKernelGGL(decode_attention_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(decode_attention_kernel<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(decode_attention_kernel<3>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(decode_attention_kernel<4>, grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL(decode_attention_kernel<5>, grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL(decode_attention_kernel<6>, grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL(decode_attention_kernel<7>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(decode_attention_kernel<8>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace wgn
