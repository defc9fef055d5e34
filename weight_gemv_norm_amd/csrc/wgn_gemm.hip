// wgn_gemm.hip -- norm-fused weight products for larger batches (up to 128
// rows) on the matrix cores.
//
// "One Token, Kernel by Kernel: A Decode Step on a Laptop GPU", section
// "Batching: when does decode stop being memory-bound?", runs the same weight
// products at growing batch: each weight read then serves every batch row, so
// the arithmetic per byte grows with the batch until the products turn
// compute-bound.  At 17 to 128 rows the persistent kernel's layout (every
// workgroup holds the whole normalised input of a phase in LDS) no longer
// fits: 128 rows of the down projection's 8960 inputs are 2.3 MB.  Here each
// call is one launch of a tiled product instead:
//   * an item is a tile of 64 output rows (16 per wave) over one K slice, for
//     all batch rows at once (padded to a multiple of 16);
//   * the input slice goes through LDS in windows of 128 elements (each batch
//     row padded by 16 bytes so the 16 rows read by one instruction fall in
//     different banks), double-buffered: the next window's copy and weight
//     loads are in flight while the current one is multiplied.  Each wave
//     streams its 16 weight rows straight into registers as the A operand of
//     v_mfma_f32_16x16x32_bf16 (FP32 accumulation), one 16 x 16 accumulator
//     tile per 16 batch rows;
//   * a stage with few row tiles is split over K so that the launch fills the
//     GPU: each item then stores its accumulators (system-scope stores), and
//     the last item of a tile to take the tile's ticket adds the slices in
//     slice order -- a fixed FP32 order, so results do not depend on timing --
//     and applies the epilogue;
//   * the epilogue is the one of the vector path: bias, GELU (tanh form) or
//     SwiGLU on the FP32 sum, residual add, one rounding to BF16; or, for the
//     LM head, packed (value, index) keys merged by an atomic maximum and
//     turned into indices by the last tile.
// The normalisation runs before, as its own pass over the batch rows (x-hat
// written once in BF16, from binary64 statistics and products), which is what
// the unfused pipeline of the same page does between its RMSNorm kernel and
// its matrix-vector kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wgn_gemm.h"
#include "wgn_numerics.h"
#include "wgn_prog.h"

namespace wgn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int GEMM_COH = 17;                   // sc0|sc1: data exchanged between workgroups
constexpr int GEMM_WEIGHT_AUX = 2;             // nt: weights are read once
constexpr uint32_t GEMM_RSRC_W3 = 0x00020000u; // raw buffer descriptor, range-checked
constexpr uint32_t GEMM_OUT_OF_RANGE = 0xFFFFFFF0u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t grsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, (int)GEMM_RSRC_W3);
}
__device__ __forceinline__ f32x4 mfma(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

#define GEMM_LAS __attribute__((address_space(3)))

// Wait until at most N loads of this wave are in flight and its LDS accesses
// are done (s_waitcnt: vmcnt in bits 3:0 and 15:14, lgkmcnt 0, expcnt left).
template <int N>
__device__ __forceinline__ void wait_vm_lds0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
}
// A buffer offset, or one past every buffer's range (reads as zero) when ok
// is false: an OR with a mask rather than a choice between two offsets,
// which the compiler would turn into two loads under complementary masks.
__device__ __forceinline__ uint32_t oor_unless(bool ok, uint32_t off) {
    return off | (((uint32_t)ok - 1u) & GEMM_OUT_OF_RANGE);
}
// Workgroup barrier without the memory fences of __syncthreads, whose
// release would wait for every load in flight, LDS copies included; the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Slices whose partial tiles are loaded together when a tile's slices are
// added (one memory round trip per group).
template <int NT, bool SWI>
constexpr int sum_group() { return (SWI ? 2 : 1) * NT <= 4 ? 4 : (SWI ? 2 : 1) * NT <= 8 ? 2 : 1; }

template <int NT, bool SWI>
__global__ __launch_bounds__(GEMM_THREADS, WGN_GEMM_OCC) void gemm_kernel(GemmLaunch G) {
    extern __shared__ __align__(16) char lds[];
    // this workgroup's stage and place among the stage's workgroups
    int32_t si = 0;
#pragma unroll
    for (int k = 1; k < GEMM_MAX_GROUP; ++k) si += (k < G.n && (int32_t)blockIdx.x >= G.start[k]) ? 1 : 0;
    const GemmArgs &a = G.s[si];
    const int32_t g = (int32_t)blockIdx.x - G.start[si];
    constexpr int P = SWI ? 2 : 1;                           // accumulator sets (gate and up)
    constexpr int MS = GEMM_KWIN / 32;                       // K steps per window
    constexpr int D = GEMM_RING;                             // windows in flight
    constexpr int XI = gemm_copies_per_wave(NT);             // 1 KB input copies per wave and window
    constexpr uint32_t XB = gemm_slot_bytes(NT);             // one ring slot
    constexpr int LPW = P * MS + XI;                         // loads per wave and window
    constexpr uint32_t TSTRIDE = GEMM_TILE_ROWS * 4 + 16;    // epilogue staging: bytes per batch row
    static_assert(NT * 16 * TSTRIDE <= D * XB, "the epilogue's staging fits the ring");
    constexpr int RI = (NT * 16 * 8 + GEMM_THREADS - 1) / GEMM_THREADS;  // output chunks per thread
    const int32_t w = (int32_t)(threadIdx.x >> 6);
    const size_t merge_off = (size_t)D * XB;          // argmax merge area, then the last-contributor flag
    int32_t *s_last = (int32_t *)(lds + merge_off + 4 * GEMM_MAX_BATCH * 8);
    const uint32_t wbytes = (uint32_t)((int64_t)a.N * a.K * 2);
    const __amdgpu_buffer_rsrc_t rw = grsrc(a.W, wbytes);
    const __amdgpu_buffer_rsrc_t ru = grsrc(SWI ? a.W_up : a.W, wbytes);
    const __amdgpu_buffer_rsrc_t rx = grsrc(a.x, (uint32_t)(((int64_t)(a.B - 1) * a.x_stride + a.K) * 2));
    const __amdgpu_buffer_rsrc_t rp = grsrc(a.part, 0x7FFFFFF0u);
    uint16_t *y = (uint16_t *)a.y;
    // 16-byte output accesses need 16-byte aligned rows of y (and of the residual)
    const bool vy = ((uintptr_t)y & 15u) == 0 && (a.y_stride & 7) == 0 &&
                    (!a.residual || (((uintptr_t)a.residual & 15u) == 0 && (a.res_stride & 7) == 0));

    // The stage's units are the windows of its row tiles, tile by tile
    // (nwin per tile); workgroup g takes units [g U / wgs, (g + 1) U / wgs),
    // so every workgroup streams the same number of windows.  A tile whose
    // units fall to several workgroups (its contributors, consecutive) is
    // added up by the last of them to finish, in contributor order.
    const int64_t U = (int64_t)a.ntiles * a.nwin;
    const int32_t u0 = (int32_t)((int64_t)g * U / a.wgs), u1 = (int32_t)((int64_t)(g + 1) * U / a.wgs);
    auto owner = [&](int64_t u) -> int32_t { return (int32_t)(((u + 1) * a.wgs - 1) / U); };

    for (int32_t u = u0; u < u1;) {
        // one segment: windows [wb0, we0) of row tile `tile`
        const int32_t tile = u / a.nwin;
        const int32_t wb0 = u - tile * a.nwin;
        const int32_t we0 = min(a.nwin, wb0 + (u1 - u));
        u += we0 - wb0;
        const int32_t n0 = tile * GEMM_TILE_ROWS;
        const int32_t k0 = wb0 * GEMM_KWIN, k1 = min(a.K, we0 * GEMM_KWIN);
        const int32_t nwin = we0 - wb0;
        // The thread's index is taken afresh in every segment (an empty asm
        // statement hides its value), so that the compiler derives the
        // thread's addresses here rather than keeping all of them live
        // across the whole loop, epilogue included.
        uint32_t tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const uint32_t lane = tid & 63u;
        const uint32_t q = lane >> 4, j = lane & 15u;
        const int32_t arow = n0 + 16 * w + (int32_t)j;  // weight row of this lane's A fragments

        f32x4 acc[P][NT];
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) acc[p][ct] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

        // weight fragments of the window at kw: row arow, K offset kw + 32 t + 8 q
        // (past the segment, or for a window after the last, the loads read zero)
        auto load_w = [&](int32_t kw, u32x4 (&wa)[P][MS]) {
#pragma unroll
            for (int t = 0; t < MS; ++t) {
                const int32_t k = kw + 32 * t + 8 * (int32_t)q;
                const uint32_t off = oor_unless(arow < a.N && k < k1, (uint32_t)(((int64_t)arow * a.K + k) * 2));
                wa[0][t] = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, GEMM_WEIGHT_AUX);
                if constexpr (SWI) wa[P - 1][t] = __builtin_amdgcn_raw_buffer_load_b128(ru, off, 0, GEMM_WEIGHT_AUX);
            }
        };
        // The input window at kw, copied into a ring slot by LDS-DMA loads:
        // 1 KB copies m = w, w + 4, ... of 8 batch rows each.  Batch row r
        // sits at r * 128 bytes with its 16-byte chunk c in place
        // c ^ ((r >> 1) & 7), so that the 16 rows one read instruction
        // touches fall in different banks.  A chunk past the segment takes
        // the segment's first chunk instead (finite input against a zero
        // weight); rows past the batch are left out of range (no memory
        // traffic; those columns are never used).
        auto issue_x = [&](int32_t kw, char *slot) {
#pragma unroll
            for (int e = 0; e < XI; ++e) {
                const int32_t m = w + 4 * e;
                const int32_t row = 8 * m + (int32_t)(lane >> 3);
                const int32_t k = kw + 8 * ((int32_t)(lane & 7u) ^ ((4 * m + (int32_t)(lane >> 4)) & 7));
                const uint32_t off =
                    oor_unless(row < a.B, (uint32_t)(((int64_t)row * a.x_stride + (k < k1 ? k : k0)) * 2));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (GEMM_LAS void *)(slot + m * 1024), 16, off, 0, 0, 0);
            }
        };
        // the window's products: B operand = batch row 16 ct + j, chunk 4 t + q
        auto compute = [&](const char *slot, const u32x4 (&wa)[P][MS]) {
#pragma unroll
            for (int t = 0; t < MS; ++t)
#pragma unroll
                for (int ct = 0; ct < NT; ++ct) {
                    const u32x4 xv = *(const u32x4 *)(slot + (uint32_t)ct * 2048u + j * 128u +
                                                      ((((uint32_t)(4 * t) + q) ^ (j >> 1)) << 4));
#pragma unroll
                    for (int p = 0; p < P; ++p) acc[p][ct] = mfma(wa[p][t], xv, acc[p][ct]);
                }
        };

        // Ring of GEMM_RING windows: window i is multiplied from slot i % RING
        // and register set i % RING while windows i + 1 .. i + RING - 1 are in
        // flight.  Every step issues the same loads (zero weights past the
        // segment), so a fixed count of outstanding loads marks window i as
        // landed; each wave waits for its own copies, then the barrier makes
        // every wave's copies visible and frees the slot of window i - 1 for
        // window i + RING - 1.  Unrolled by RING, so that no register array
        // is indexed at run time; the windows that pad the segment to a
        // multiple of RING add zero products.
        __syncthreads();  // the previous segment's epilogue is done with the ring
        u32x4 wa[D][P][MS];
#pragma unroll
        for (int d = 0; d < D - 1; ++d) {
            load_w(k0 + d * GEMM_KWIN, wa[d]);
            issue_x(k0 + d * GEMM_KWIN, lds + d * XB);
            asm volatile("" ::: "memory");  // windows issued in order: the count below relies on it
        }
        for (int32_t i = 0; i < nwin; i += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                wait_vm_lds0<(D - 2) * LPW>();
                ring_barrier();
                const int32_t kn = k0 + (i + d + D - 1) * GEMM_KWIN;
                load_w(kn, wa[(d + D - 1) % D]);
                issue_x(kn, lds + ((d + D - 1) % D) * XB);
                compute(lds + d * XB, wa[d]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // the ring's copies past the last window have landed

        // The epilogue's own inputs, requested as soon as this workgroup
        // knows it applies the epilogue (before the contributions are added,
        // whose loads then overlap them): the bias of this lane's 4 rows and,
        // where 16-byte accesses are allowed, the residual chunks of this
        // thread's outputs (8 rows of one batch row, as the output loop takes
        // them).
        float bz[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        u32x4 rv[RI];
        auto fetch_epilogue_inputs = [&]() {
            if (a.epi == EPI_ARGMAX) return;
            if (a.bias) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int32_t n = n0 + 16 * w + 4 * (int32_t)q + r;
                    if (n < a.N) bz[r] = bf2f(a.bias[n]);
                }
            }
            if (a.residual && vy) {
#pragma unroll
                for (int it = 0; it < RI; ++it) {
                    const int32_t idx = (int32_t)tid + it * GEMM_THREADS;
                    const int32_t b = idx >> 3, n = n0 + 8 * (idx & 7);
                    if (idx < NT * 16 * 8 && b < a.B && n + 8 <= a.N)
                        rv[it] = *(const u32x4 *)(a.residual + (int64_t)b * a.res_stride + n);
                }
            }
        };

        bool epi = true;
        if (wb0 > 0 || we0 < a.nwin) {
            // a shared tile: this workgroup's accumulators go to its
            // contributor slot, then the tile's ticket
            const int32_t first = owner((int64_t)tile * a.nwin);
            const int32_t nc = owner((int64_t)tile * a.nwin + a.nwin - 1) - first + 1;  // contributors
            const int32_t kc = g - first;                                               // this one
            const int32_t base = first + tile;  // slot of contributor 0: slots of successive tiles never overlap
            auto frag = [&](int32_t c, int p, int ct) -> uint32_t {  // byte offset of this lane's part of a fragment
                return (uint32_t)(((((size_t)(base + c)) * 4 + w) * P * NT + (size_t)p * NT + ct) * GEMM_FRAG_BYTES +
                                  lane * 16u);
            };
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int ct = 0; ct < NT; ++ct)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[p][ct]), rp, frag(kc, p, ct), 0,
                                                           GEMM_COH);
            __builtin_amdgcn_s_waitcnt(0);  // the stores have completed: visible at the coherent level
            __syncthreads();
            if (tid == 0u) {
                const uint32_t old =
                    __hip_atomic_fetch_add(&a.tickets[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int32_t last = old == (uint32_t)(nc - 1) ? 1 : 0;
                if (last) __hip_atomic_store(&a.tickets[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                *s_last = last;
            }
            __syncthreads();
            epi = *s_last != 0;
            if (epi) {
                fetch_epilogue_inputs();
                // the last contributor adds the contributions in contributor
                // order, its own too (stored like the others), into acc
                constexpr int GS = sum_group<NT, SWI>();
                for (int32_t c0 = 0; c0 < nc; c0 += GS) {
                    f32x4 v[GS][P][NT];
#pragma unroll
                    for (int gg = 0; gg < GS; ++gg) {
                        if (c0 + gg < nc) {
#pragma unroll
                            for (int p = 0; p < P; ++p)
#pragma unroll
                                for (int ct = 0; ct < NT; ++ct)
                                    v[gg][p][ct] = __builtin_bit_cast(
                                        f32x4,
                                        __builtin_amdgcn_raw_buffer_load_b128(rp, frag(c0 + gg, p, ct), 0, GEMM_COH));
                        }
                    }
#pragma unroll
                    for (int gg = 0; gg < GS; ++gg) {
                        if (c0 + gg < nc) {
#pragma unroll
                            for (int p = 0; p < P; ++p)
#pragma unroll
                                for (int ct = 0; ct < NT; ++ct)
                                    acc[p][ct] = c0 + gg == 0 ? v[gg][p][ct] : acc[p][ct] + v[gg][p][ct];
                        }
                    }
                }
            }
        } else {
            fetch_epilogue_inputs();
        }
        if (!epi) continue;

        // ------------------------------------------------------------ epilogue
        // lane: rows n0 + 16 w + 4 q + r (r = 0..3) of batch rows 16 ct + j.
        if (a.epi != EPI_ARGMAX) {
            // The activated tile goes through LDS (the ring, free now) so
            // that the residual is read and the output written in 16-byte
            // chunks of 8 consecutive rows of one batch row: the fragment
            // layout would make every store instruction touch 16 batch rows
            // with 2-byte writes.
            __syncthreads();  // every wave is done with the ring
            float *tb = (float *)lds;  // [16 NT batch rows][64 rows], row stride TSTRIDE bytes
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                f32x4 e4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int32_t n = n0 + 16 * w + 4 * (int32_t)q + r;
                    const float z = acc[0][ct][r] + bz[r];
                    float e;
                    if (a.epi == EPI_GELU_TANH) {
                        e = gelu_tanh(z);
                        const int32_t b = ct * 16 + (int32_t)j;
                        if (a.logits && n < a.N && b < a.B)
                            a.logits[(int64_t)b * a.N + n] = z;  // pre-activation for the backward pass
                    } else if (a.epi == EPI_SWIGLU) e = silu(z) * acc[P - 1][ct][r];
                    else e = z;
                    e4[r] = e;
                }
                *(f32x4 *)((char *)tb + (uint32_t)(ct * 16 + (int32_t)j) * TSTRIDE +
                           (uint32_t)(16 * w + 4 * (int32_t)q) * 4u) = e4;
            }
            __syncthreads();
#pragma unroll
            for (int it = 0; it < RI; ++it) {
                const int32_t idx = (int32_t)tid + it * GEMM_THREADS;
                const int32_t b = idx >> 3, c8 = idx & 7, n = n0 + 8 * c8;
                if (idx >= NT * 16 * 8 || b >= a.B || n >= a.N) continue;
                const float *src = (const float *)((const char *)tb + (uint32_t)b * TSTRIDE + (uint32_t)c8 * 32u);
                const f32x4 lo = *(const f32x4 *)src, hi = *(const f32x4 *)(src + 4);
                float e[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                if (vy && n + 8 <= a.N) {
                    if (a.residual) {
                        const uint32_t rr[4] = {rv[it].x, rv[it].y, rv[it].z, rv[it].w};
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            e[2 * k] += bf2f(rr[k] & 0xFFFFu);
                            e[2 * k + 1] += bf2f(rr[k] >> 16);
                        }
                    }
                    u32x4 o;
                    o.x = (uint32_t)f2bf(e[0]) | ((uint32_t)f2bf(e[1]) << 16);
                    o.y = (uint32_t)f2bf(e[2]) | ((uint32_t)f2bf(e[3]) << 16);
                    o.z = (uint32_t)f2bf(e[4]) | ((uint32_t)f2bf(e[5]) << 16);
                    o.w = (uint32_t)f2bf(e[6]) | ((uint32_t)f2bf(e[7]) << 16);
                    *(u32x4 *)(y + (int64_t)b * a.y_stride + n) = o;
                } else {
                    for (int k = 0; k < 8 && n + k < a.N; ++k) {
                        float v = e[k];
                        if (a.residual) v += bf2f(a.residual[(int64_t)b * a.res_stride + n + k]);
                        y[(int64_t)b * a.y_stride + n + k] = f2bf(v);
                    }
                }
            }
            continue;
        }
        // argmax: the tile's best key per batch row, merged over the tiles by
        // an atomic maximum; the last tile writes the indices and clears the
        // keys
        uint64_t *mk = (uint64_t *)(lds + merge_off);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const int32_t b = ct * 16 + (int32_t)j;
            uint64_t best = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int32_t n = n0 + 16 * w + 4 * (int32_t)q + r;
                if (n < a.N && b < a.B) {
                    const float z = acc[0][ct][r];
                    if (a.logits) a.logits[(int64_t)b * a.N + n] = z;
                    const uint64_t key = ((uint64_t)orderable(z) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)n);
                    best = key > best ? key : best;
                }
            }
            uint64_t o = __shfl_xor(best, 16);
            best = o > best ? o : best;
            o = __shfl_xor(best, 32);
            best = o > best ? o : best;
            if (q == 0) mk[w * GEMM_MAX_BATCH + b] = best;
        }
        __syncthreads();
        if ((int32_t)tid < a.B) {
            const int32_t b = (int32_t)tid;
            uint64_t best = mk[b];
#pragma unroll
            for (int ww = 1; ww < 4; ++ww)
                best = mk[ww * GEMM_MAX_BATCH + b] > best ? mk[ww * GEMM_MAX_BATCH + b] : best;
            __hip_atomic_fetch_max(&a.keys[b], best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this tile's maxima and logits are done
        __syncthreads();
        if (tid == 0u) {
            const uint32_t old =
                __hip_atomic_fetch_add(&a.tickets[a.ntiles], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int32_t last = old == (uint32_t)(a.ntiles - 1) ? 1 : 0;
            if (last) __hip_atomic_store(&a.tickets[a.ntiles], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *s_last = last;
        }
        __syncthreads();
        if (*s_last != 0 && (int32_t)tid < a.B) {
            const int32_t b = (int32_t)tid;
            const uint64_t key = __hip_atomic_load(&a.keys[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.keys[b], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ((int32_t *)a.y)[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
            if (a.maxval) a.maxval[b] = unorderable((uint32_t)(key >> 32));
        }
    }
}

// Sum of one value per thread over the workgroup (FP64): waves, then LDS.
__device__ __forceinline__ double block_sum(double v, double *red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    const int32_t w = (int32_t)(threadIdx.x >> 6);
    if ((threadIdx.x & 63u) == 0u) red[w] = v;
    __syncthreads();
    const double t = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();  // red is reused by the next sum
    return t;
}

// x-hat of one batch row per workgroup, in binary64 as the norms are defined
// ("GPU Kernel Optimization" README, section "Architecture": mean square,
// rsqrt, gain multiply; LayerNorm with its mean and biased variance about the
// mean), rounded once to BF16: RMSNorm x r g with r = (sum x^2 / K + eps)^-1/2;
// LayerNorm (x - mu) r g + beta with r = (sum (x - mu)^2 / K + eps)^-1/2.
// The products and sums are kept separate (no fused multiply-add), so each
// rounds as written.
template <bool LAYER>
__global__ __launch_bounds__(256) void norm_rows64_kernel(const uint16_t *x, int64_t x_stride, const uint16_t *gamma,
                                                          const uint16_t *beta, double eps, uint16_t *y, int32_t K) {
#pragma clang fp contract(off)
    __shared__ double red[4];
    const uint16_t *xr = x + (int64_t)blockIdx.x * x_stride;
    uint16_t *yr = y + (int64_t)blockIdx.x * K;
    const int32_t n8 = K >> 3;
    double mu = 0.0;
    if constexpr (LAYER) {
        double s = 0.0;
        for (int32_t i = (int32_t)threadIdx.x; i < n8; i += 256) {
            const u32x4 v = *(const u32x4 *)(xr + (int64_t)i * 8);
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) s += (double)bf2f(vv[e] & 0xFFFFu) + (double)bf2f(vv[e] >> 16);
        }
        mu = block_sum(s, red) / (double)K;
    }
    double ss = 0.0;
    for (int32_t i = (int32_t)threadIdx.x; i < n8; i += 256) {
        const u32x4 v = *(const u32x4 *)(xr + (int64_t)i * 8);
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double lo = (double)bf2f(vv[e] & 0xFFFFu) - mu, hi = (double)bf2f(vv[e] >> 16) - mu;
            ss += lo * lo;
            ss += hi * hi;
        }
    }
    const double r = 1.0 / sqrt(block_sum(ss, red) / (double)K + eps);
    for (int32_t i = (int32_t)threadIdx.x; i < n8; i += 256) {
        const u32x4 v = *(const u32x4 *)(xr + (int64_t)i * 8);
        const u32x4 gv = gamma ? *(const u32x4 *)(gamma + (int64_t)i * 8) : (u32x4){0x3F803F80u, 0x3F803F80u,
                                                                                     0x3F803F80u, 0x3F803F80u};
        const u32x4 bv = beta ? *(const u32x4 *)(beta + (int64_t)i * 8) : (u32x4){0u, 0u, 0u, 0u};
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w}, gg[4] = {gv.x, gv.y, gv.z, gv.w}, bb[4] = {bv.x, bv.y, bv.z, bv.w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            double t[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const double xv = (double)bf2f((vv[e] >> (16 * h)) & 0xFFFFu);
                const double g = (double)bf2f((gg[e] >> (16 * h)) & 0xFFFFu);
                t[h] = LAYER ? (xv - mu) * r * g + (double)bf2f((bb[e] >> (16 * h)) & 0xFFFFu) : xv * r * g;
            }
            o[e] = (uint32_t)f64_to_bf16(t[0]) | ((uint32_t)f64_to_bf16(t[1]) << 16);
        }
        *(u32x4 *)(yr + (int64_t)i * 8) = (u32x4){o[0], o[1], o[2], o[3]};
    }
}
// The same norm with the row held in registers (at most C 16-byte chunks per
// thread, K <= 2048 C): the row, its gain and its shift are loaded once, at
// the start, instead of once per pass.  Each thread takes the same chunks in
// the same order and the sums are the same, so x-hat has the same bits.
template <bool LAYER, int C>
__global__ __launch_bounds__(256) void norm_rows64_reg_kernel(const uint16_t *x, int64_t x_stride,
                                                              const uint16_t *gamma, const uint16_t *beta, double eps,
                                                              uint16_t *y, int32_t K) {
#pragma clang fp contract(off)
    __shared__ double red[4];
    const uint16_t *xr = x + (int64_t)blockIdx.x * x_stride;
    uint16_t *yr = y + (int64_t)blockIdx.x * K;
    const int32_t n8 = K >> 3;
    u32x4 v[C], gv[C], bv[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int32_t i = (int32_t)threadIdx.x + 256 * c;
        const bool in = i < n8;
        v[c] = in ? *(const u32x4 *)(xr + (int64_t)i * 8) : (u32x4){0u, 0u, 0u, 0u};
        gv[c] = (in && gamma) ? *(const u32x4 *)(gamma + (int64_t)i * 8)
                              : (u32x4){0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
        bv[c] = (in && beta) ? *(const u32x4 *)(beta + (int64_t)i * 8) : (u32x4){0u, 0u, 0u, 0u};
    }
    double mu = 0.0;
    if constexpr (LAYER) {
        double s = 0.0;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if ((int32_t)threadIdx.x + 256 * c >= n8) break;
            const uint32_t vv[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) s += (double)bf2f(vv[e] & 0xFFFFu) + (double)bf2f(vv[e] >> 16);
        }
        mu = block_sum(s, red) / (double)K;
    }
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if ((int32_t)threadIdx.x + 256 * c >= n8) break;
        const uint32_t vv[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double lo = (double)bf2f(vv[e] & 0xFFFFu) - mu, hi = (double)bf2f(vv[e] >> 16) - mu;
            ss += lo * lo;
            ss += hi * hi;
        }
    }
    const double r = 1.0 / sqrt(block_sum(ss, red) / (double)K + eps);
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int32_t i = (int32_t)threadIdx.x + 256 * c;
        if (i >= n8) break;
        const uint32_t vv[4] = {v[c].x, v[c].y, v[c].z, v[c].w}, gg[4] = {gv[c].x, gv[c].y, gv[c].z, gv[c].w},
                       bb[4] = {bv[c].x, bv[c].y, bv[c].z, bv[c].w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            double t[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const double xv = (double)bf2f((vv[e] >> (16 * h)) & 0xFFFFu);
                const double g = (double)bf2f((gg[e] >> (16 * h)) & 0xFFFFu);
                t[h] = LAYER ? (xv - mu) * r * g + (double)bf2f((bb[e] >> (16 * h)) & 0xFFFFu) : xv * r * g;
            }
            o[e] = (uint32_t)f64_to_bf16(t[0]) | ((uint32_t)f64_to_bf16(t[1]) << 16);
        }
        *(u32x4 *)(yr + (int64_t)i * 8) = (u32x4){o[0], o[1], o[2], o[3]};
    }
}

__global__ void zero_words_kernel(uint32_t *p, int32_t n) {
    const int32_t i = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0u;
}

// The window may take more than the default 64 KB of dynamic LDS; the
// attribute is set once per kernel before its first launch.
template <int NT, bool SWI>
hipError_t launch_nt(const GemmLaunch &G, size_t lds, hipStream_t s) {
    static bool done = false;
    if (!done) {
        const hipError_t e = hipFuncSetAttribute((const void *)gemm_kernel<NT, SWI>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_cap());
        if (e != hipSuccess) return e;
        done = true;
    }
    hipLaunchKernelGGL((gemm_kernel<NT, SWI>), dim3(G.start[G.n]), dim3(GEMM_THREADS), lds, s, G);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmLaunch &G, bool swiglu, size_t lds, hipStream_t s) {
    if (G.n < 1 || G.n > GEMM_MAX_GROUP || G.start[0] != 0 || lds > lds_cap()) return hipErrorInvalidValue;
    const int32_t nt = (G.s[0].B + 15) / 16;
    for (int i = 0; i < G.n; ++i) {
        const GemmArgs &a = G.s[i];
        // the kernel's window and slice arithmetic assumes these
        // (every workgroup of a stage has at least one unit: contributor
        // counts rely on it)
        if (a.ntiles < 1 || a.B < 1 || a.B > GEMM_MAX_BATCH || (a.B + 15) / 16 != nt || a.K < 1 ||
            a.nwin != (a.K + GEMM_KWIN - 1) / GEMM_KWIN || a.wgs < 1 || (int64_t)a.wgs > (int64_t)a.ntiles * a.nwin ||
            G.start[i + 1] - G.start[i] != a.wgs || (gemm_tiles_shared(a.ntiles, a.nwin, a.wgs) && !a.part))
            return hipErrorInvalidValue;
    }
    switch (nt * 2 + (swiglu ? 1 : 0)) {
#define WGN_GEMM_CASE(NT)                                  \
    case 2 * NT: return launch_nt<NT, false>(G, lds, s);   \
    case 2 * NT + 1: return launch_nt<NT, true>(G, lds, s);
        WGN_GEMM_CASE(1) WGN_GEMM_CASE(2) WGN_GEMM_CASE(3) WGN_GEMM_CASE(4)
        WGN_GEMM_CASE(5) WGN_GEMM_CASE(6) WGN_GEMM_CASE(7) WGN_GEMM_CASE(8)
#undef WGN_GEMM_CASE
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_zero_words(uint32_t *p, int32_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_norm_rows64(const uint16_t *x, int64_t x_stride, const uint16_t *gamma, const uint16_t *beta,
                              float eps, bool layer, uint16_t *y, int32_t rows, int32_t K, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int32_t c = ((K >> 3) + 255) / 256;  // 16-byte chunks per thread
    const double e = (double)eps;
#define WGN_NORM_REG(L, C) hipLaunchKernelGGL((norm_rows64_reg_kernel<L, C>), dim3(rows), dim3(256), 0, s, x, \
                                              x_stride, gamma, beta, e, y, K)
    if (c <= 1) {
        if (layer) WGN_NORM_REG(true, 1);
        else WGN_NORM_REG(false, 1);
    } else if (c == 2) {
        if (layer) WGN_NORM_REG(true, 2);
        else WGN_NORM_REG(false, 2);
    } else if (c <= 4) {
        if (layer) WGN_NORM_REG(true, 4);
        else WGN_NORM_REG(false, 4);
    } else if (layer)
        hipLaunchKernelGGL(norm_rows64_kernel<true>, dim3(rows), dim3(256), 0, s, x, x_stride, gamma, beta, e, y, K);
    else
        hipLaunchKernelGGL(norm_rows64_kernel<false>, dim3(rows), dim3(256), 0, s, x, x_stride, gamma, beta, e, y, K);
#undef WGN_NORM_REG
    return hipGetLastError();
}

}  // namespace wgn
