// wgn_kernels.hip -- gfx950 kernels of the decode-step weight stream.
//
// One kernel runs a whole chain of norm-fused weight products (or a single
// stage).  Each workgroup (one per compute unit when persistent) has
//   * 7 streaming waves: they only stream weight units (128-bit buffer loads,
//     1 KB per wave-load, fully coalesced) into registers, dot them with the
//     BF16 normalised input held in LDS (v_dot2c_f32_bf16, FP32 accumulation),
//     reduce each row-part across lanes (DPP + bpermute) and write partial sums
//     to LDS.  They never touch global memory otherwise, so they never wait on
//     anything but their own weight loads, and the loads of the next block of
//     units -- possibly of the next phase -- are issued before the current
//     block is consumed;
//   * 1 control wave: it waits for the previous phase to finish device-wide,
//     loads the phase's input vectors, computes the norm statistics (FP32) and
//     writes x-hat as BF16 into LDS, then sums the partials in a fixed order,
//     applies the epilogue (bias, GELU-tanh, SwiGLU, residual or argmax) and
//     stores the outputs, then releases its completion counter.
// Shapes of the pages' workload: "One Token, Kernel by Kernel: A Decode Step on
// a Laptop GPU", sections "The setup" and "What one block launches" (BF16
// weights, FP32 accumulation, RMSNorm + SwiGLU, residual folded into a
// neighbouring kernel) and "The whole step" (LM head + argmax).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wgn_loader.h"

namespace wgn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int DEPTH = 16;                 // units per block (loads in flight per block)
constexpr uint32_t RSRC_W3 = 0x00020000u; // buffer descriptor word 3 for raw dword loads

// ------------------------------------------------------------------ numerics
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

// FP32 -> BF16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Dot product of 8 BF16 pairs, FP32 accumulation (v_dot2c_f32_bf16).  The
// vector elements are copied to scalars first: bit-casting an ext-vector
// element expression directly miscompiles to element 0 with this toolchain.
__device__ __forceinline__ float dot8(const u32x4 &w, const u32x4 &x, float acc) {
    const uint32_t wa[4] = {w.x, w.y, w.z, w.w}, xa[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wa[i]), __builtin_bit_cast(bf16x2, xa[i]),
                                              acc, false);
    return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes; every lane gets the same bits (each step adds a
// symmetric pair, so all lanes hold identical values after every step).
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    v += dpp<0x140>(v);   // row_mirror
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    for (int o = 32; o >= 1; o >>= 1) {
        uint64_t t = __shfl_xor(v, o);
        v = t > v ? t : v;
    }
    return v;
}

__device__ __forceinline__ uint32_t orderable(float f) {
    uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unorderable(uint32_t o) {
    uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(b);
}

__device__ __forceinline__ float gelu_tanh(float z) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
}
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ------------------------------------------------------------- sync helpers
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ void release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Set by the control wave when an in-kernel wait times out; read by the
// streaming waves after a workgroup barrier.  A typed LDS variable (not a
// generic pointer) so that reading it never waits on vector memory.
__shared__ int32_t g_abort;
__device__ __forceinline__ int32_t abort_flag_get() {
    return __hip_atomic_load(&g_abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void abort_flag_set(int32_t v) {
    __hip_atomic_store(&g_abort, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ uint32_t lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// ------------------------------------------------------------ streaming waves
struct BlockMeta {
    uint32_t meta_v;       // lane j holds the meta word of the block's unit j
    int32_t xb_bytes;      // LDS bytes per batch row of x-hat in this block's phase
    bool last;             // last block of this wave in its phase
};

struct StreamState {
    PhaseGeo G;
    int32_t u, u_beg, u_end;
    int32_t g, w, p1;
    bool done_all;
};

template <bool CHAIN>
__device__ __forceinline__ void stream_begin_phase(const KArgs &a, StreamState &S, int32_t p) {
    S.G = phase_geo<CHAIN>(a, p, S.g);
    S.u_beg = S.G.U > 0 ? wave_begin(S.w, S.G.U, STREAM_WAVES) : 0;
    S.u_end = S.G.U > 0 ? wave_begin(S.w + 1, S.G.U, STREAM_WAVES) : 0;
    S.u = S.u_beg;
}

// Issue DEPTH unit loads (a block never spans a phase boundary).  Lane j first
// computes the descriptor of unit j; each load then takes its base address and
// length from lane j through v_readlane.  Invalid slots load from an empty
// range (no memory traffic, value 0), so every block issues the same number of
// loads and the compiler's vmcnt accounting stays exact.
template <int B, bool CHAIN>
__device__ __forceinline__ void load_block(const KArgs &a, StreamState &S, u32x4 (&d)[DEPTH], BlockMeta &bm,
                                           uint32_t lane) {
    UnitDesc ud;
    ud.ptr = 0;
    ud.nbytes = 0;
    ud.meta = 0;
    if (!S.done_all && lane < (uint32_t)DEPTH)
        ud = unit_desc<CHAIN>(a, S.G, S.u + (int32_t)lane, S.u_beg, S.u_end, S.w, B);
    if (ud.nbytes == 0) ud.ptr = (uint64_t)(uintptr_t)a.ist.W;
    const uint32_t plo = (uint32_t)ud.ptr, phi = (uint32_t)(ud.ptr >> 32);
    bm.meta_v = ud.meta;
    bm.xb_bytes = S.done_all ? 0 : S.G.xb_bytes;
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
        const uint32_t lo = __builtin_amdgcn_readlane(plo, j);
        const uint32_t hi = __builtin_amdgcn_readlane(phi, j);
        const uint32_t nb = __builtin_amdgcn_readlane(ud.nbytes, j);
        const void *base = (const void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
        __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)nb, (int)RSRC_W3);
        d[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(lane * 16u), 0, 0);
    }
    if (S.done_all) {
        bm.last = false;  // past the final phase: nothing to synchronise
        return;
    }
    S.u = S.u + DEPTH < S.u_end ? S.u + DEPTH : S.u_end;
    bm.last = S.u >= S.u_end;
    if (bm.last) {
        if (S.G.p + 1 < S.p1) stream_begin_phase<CHAIN>(a, S, S.G.p + 1);
        else S.done_all = true;
    }
}

// Every slot of a block is consumed unconditionally (an invalid slot holds
// zeros and points at x-hat offset 0, which is initialised in every phase), so
// every load is waited for in issue order on every path and the compiler's
// vmcnt bookkeeping stays exact.
template <int B>
__device__ __forceinline__ void consume_block(const u32x4 (&d)[DEPTH], const BlockMeta &bm, float (&acc)[B],
                                              const char *xh, float *part, uint32_t lane) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
        const uint32_t m = __builtin_amdgcn_readlane(bm.meta_v, j);
        const char *xp = xh + ((m & 0x3FFFu) << 4) + lane * 16u;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            u32x4 xv = *(const u32x4 *)(xp + b * bm.xb_bytes);
            acc[b] = dot8(d[j], xv, acc[b]);
        }
        if (m & 0x4000u) {
            const uint32_t slot = m >> 16;
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float s = wave_sum(acc[b]);
                if (lane == 0) part[slot + b] = s;
                acc[b] = 0.0f;
            }
        }
    }
}

template <int B, bool CHAIN>
__device__ void stream_wave(const KArgs &a, int32_t g, int32_t w, char *lds) {
    const uint32_t lane = lane_id();
    const char *xh = lds;
    float *part = (float *)(lds + a.lds_x_bytes);
    StreamState S;
    S.g = g;
    S.w = w;
    S.p1 = a.p1;
    S.done_all = false;
    stream_begin_phase<CHAIN>(a, S, a.p0);
    u32x4 dA[DEPTH], dB[DEPTH];
    BlockMeta mA, mB;
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;

    load_block<B, CHAIN>(a, S, dA, mA, lane);
    wg_barrier();  // x-hat of the first phase is ready
    bool ok = abort_flag_get() == 0;
    int32_t p = a.p0;
    // Two blocks per iteration (register double buffering) and a single exit
    // at the bottom, so the compiler sees one straight-line pipeline.
    while (ok && p < a.p1) {
        load_block<B, CHAIN>(a, S, dB, mB, lane);
        consume_block<B>(dA, mA, acc, xh, part, lane);
        if (mA.last) {
            wg_barrier();  // partials of phase p are complete
            if (++p < a.p1) {
                wg_barrier();  // x-hat of phase p+1 is ready
                ok = abort_flag_get() == 0;
            }
        }
        load_block<B, CHAIN>(a, S, dA, mA, lane);
        consume_block<B>(dB, mB, acc, xh, part, lane);
        if (ok && mB.last) {
            wg_barrier();
            if (++p < a.p1) {
                wg_barrier();
                ok = abort_flag_get() == 0;
            }
        }
    }
}

// --------------------------------------------------------------- control wave
__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *(const u32x4 *)p; }

// Stage every source of phase ph into LDS as BF16 x-hat (FP32 statistics).
template <int B, bool CHAIN>
__device__ void prepare_sources(const KArgs &a, const DevPhase &ph, char *xh, uint32_t lane) {
    for (int32_t si = 0; si < ph.nsrc; ++si) {
        const DevSource src = source_of<CHAIN>(a, ph.src0 + si);
        const int32_t K = src.K;
        const int32_t n8 = K >> 3;
        const int32_t padded8 = nchunks_of(K) * (UNIT / 8);
        const float invK = 1.0f / (float)K;
        for (int b = 0; b < B; ++b) {
            uint16_t *dst = (uint16_t *)(xh + ((size_t)b * ph.xb + src.lds_off) * 2);
            const uint16_t *xr = src.x + (int64_t)b * src.x_stride;
            float s1 = 0.0f, s2 = 0.0f;
            for (int32_t i = lane; i < n8; i += 64) {
                u32x4 v = ld16(xr + i * 8);
                *(u32x4 *)(dst + i * 8) = v;
                uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float lo = bf2f(vv[e] & 0xFFFFu), hi = bf2f(vv[e] >> 16);
                    s1 += lo + hi;
                    s2 += lo * lo + hi * hi;
                }
            }
            for (int32_t i = n8 + lane; i < padded8; i += 64) *(u32x4 *)(dst + i * 8) = (u32x4){0u, 0u, 0u, 0u};
            if (src.norm == NORM_NONE) continue;
            float mean = 0.0f, rstd;
            if (src.norm == NORM_RMS) {
                s2 = wave_sum(s2);
                rstd = 1.0f / sqrtf(s2 * invK + src.eps);
            } else {
                s1 = wave_sum(s1);
                mean = s1 * invK;
                float sv = 0.0f;
                for (int32_t i = lane; i < n8; i += 64) {
                    u32x4 v = *(const u32x4 *)(dst + i * 8);
                    uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float lo = bf2f(vv[e] & 0xFFFFu) - mean, hi = bf2f(vv[e] >> 16) - mean;
                        sv += lo * lo + hi * hi;
                    }
                }
                sv = wave_sum(sv);
                rstd = 1.0f / sqrtf(sv * invK + src.eps);
            }
            for (int32_t i = lane; i < n8; i += 64) {
                u32x4 v = *(const u32x4 *)(dst + i * 8);
                u32x4 gv = src.gamma ? ld16(src.gamma + i * 8)
                                     : (u32x4){0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
                u32x4 bv = (src.norm == NORM_LAYER && src.beta) ? ld16(src.beta + i * 8) : (u32x4){0u, 0u, 0u, 0u};
                uint32_t vv[4] = {v.x, v.y, v.z, v.w}, gg[4] = {gv.x, gv.y, gv.z, gv.w},
                         bb[4] = {bv.x, bv.y, bv.z, bv.w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float lo = (bf2f(vv[e] & 0xFFFFu) - mean) * rstd * bf2f(gg[e] & 0xFFFFu) + bf2f(bb[e] & 0xFFFFu);
                    float hi = (bf2f(vv[e] >> 16) - mean) * rstd * bf2f(gg[e] >> 16) + bf2f(bb[e] >> 16);
                    o[e] = (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
                }
                *(u32x4 *)(dst + i * 8) = (u32x4){o[0], o[1], o[2], o[3]};
            }
        }
    }
}

// Merge the per-workgroup argmax keys of one ARGMAX stage (called by the last
// workgroup to arrive) and write the index / maximum outputs.
template <int B>
__device__ void argmax_merge(const KArgs &a, const DevStage &st, uint32_t lane) {
    for (int b = 0; b < B; ++b) {
        uint64_t best = 0;
        for (int32_t gg = lane; gg < a.G; gg += 64) {
            uint64_t k = __hip_atomic_load(&a.am_part[((size_t)st.am_slot * a.G + gg) * B + b], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            best = k > best ? k : best;
        }
        best = wave_max_u64(best);
        if (lane == 0) {
            ((int32_t *)st.y)[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)best);
            if (st.maxval) st.maxval[b] = unorderable((uint32_t)(best >> 32));
        }
    }
}

template <int B, bool CHAIN>
__device__ void epilogue(const KArgs &a, const PhaseGeo &G, int32_t g, const float *part, uint32_t lane) {
    int32_t rp_base = 0, u_base = 0;
    for (int32_t si = 0; si < G.nstages; ++si) {
        const DevStage st = stage_of<CHAIN>(a, G.stage0 + si);
        const StageSpan sp = stage_span(st, G.r0, G.r1, 0, 0);
        const int32_t parts = st.parts, nch = st.nchunks;
        uint64_t best[B];
#pragma unroll
        for (int b = 0; b < B; ++b) best[b] = 0;
        for (int32_t i = lane; i < sp.nrows; i += 64) {
            const int32_t n = sp.row0 + i;
            float acc0[B], acc1[B];
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                if (pt >= parts) break;
                const int32_t rp = rp_base + i * parts + pt;
                const int32_t a0 = u_base + (i * parts + pt) * nch;
                const int32_t span =
                    first_wave(a0 + nch - 1, G.U, STREAM_WAVES) - first_wave(a0, G.U, STREAM_WAVES) + 1;
                const float *pp = part + (size_t)rp * G.jmax * B;
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    float s = pp[b];
                    for (int32_t j = 1; j < span; ++j) s += pp[j * B + b];
                    if (pt == 0) acc0[b] = s;
                    else acc1[b] = s;
                }
            }
            const float bias = st.bias ? bf2f(st.bias[n]) : 0.0f;
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float z = acc0[b] + bias;
                if (st.epi == EPI_ARGMAX) {
                    if (st.logits) st.logits[(size_t)b * st.N + n] = z;
                    const uint64_t key = ((uint64_t)orderable(z) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)n);
                    best[b] = key > best[b] ? key : best[b];
                    continue;
                }
                float e;
                if (st.epi == EPI_GELU_TANH) e = gelu_tanh(z);
                else if (st.epi == EPI_SWIGLU) e = silu(z) * acc1[b];
                else e = z;
                if (st.residual) e += bf2f(st.residual[(int64_t)b * st.res_stride + n]);
                ((uint16_t *)st.y)[(int64_t)b * st.y_stride + n] = f2bf(e);
            }
        }
        if (st.epi == EPI_ARGMAX) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const uint64_t k = wave_max_u64(best[b]);
                if (lane == 0)
                    __hip_atomic_store(&a.am_part[((size_t)st.am_slot * a.G + g) * B + b], k, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            release_agent();
            uint32_t old = 0;
            if (lane == 0)
                old = __hip_atomic_fetch_add(&a.tickets[st.am_slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            old = __shfl(old, 0);
            if (old == (uint32_t)(a.G - 1)) {
                acquire_agent();
                argmax_merge<B>(a, st, lane);
                if (lane == 0)
                    __hip_atomic_store(&a.tickets[st.am_slot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        rp_base += sp.nrows * parts;
        u_base += sp.nrows * parts * nch;
    }
}

template <int B, bool CHAIN>
__device__ void control_wave(const KArgs &a, int32_t g, char *lds) {
    const uint32_t lane = lane_id();
    const float *part = (const float *)(lds + a.lds_x_bytes);
    if (lane == 0) abort_flag_set(0);
    for (int32_t p = a.p0; p < a.p1; ++p) {
        const DevPhase ph = phase_of<CHAIN>(a, p);
        if (a.persistent && p > a.p0 && ph.wait) {
            const uint64_t t0 = wall_clock64();
            bool timed_out = false;
            while (__hip_atomic_load(&a.ctr[p - 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)a.G) {
                __builtin_amdgcn_s_sleep(1);
                if (wall_clock64() - t0 > WAIT_TICKS) {
                    timed_out = true;
                    break;
                }
            }
            if (timed_out) {
                if (lane == 0) {
                    abort_flag_set(1);
                    __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                wg_barrier();  // releases the streaming waves, which then exit
                return;
            }
            acquire_agent();
        }
        prepare_sources<B, CHAIN>(a, ph, lds, lane);
        wg_barrier();  // x-hat ready
        wg_barrier();  // partials complete
        const PhaseGeo G = phase_geo<CHAIN>(a, p, g);
        epilogue<B, CHAIN>(a, G, g, part, lane);
        if (a.persistent) {
            release_agent();
            if (lane == 0) __hip_atomic_fetch_add(&a.ctr[p], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (a.persistent) {
        // The last workgroup to finish resets the counters so the next run (or
        // graph replay) starts from zero; every other workgroup is past all of
        // its waits by then.
        release_agent();
        uint32_t old = 0;
        if (lane == 0)
            old = __hip_atomic_fetch_add(&a.tickets[a.n_argmax], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0);
        if (old == (uint32_t)(a.G - 1)) {
            acquire_agent();
            for (int32_t p = a.p0 + (int32_t)lane; p < a.p1; p += 64)
                __hip_atomic_store(&a.ctr[p], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (lane == 0) __hip_atomic_store(&a.tickets[a.n_argmax], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int B, bool CHAIN>
__global__ __launch_bounds__(THREADS, 1) void chain_kernel(KArgs a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int32_t g = blockIdx.x;
    const int32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w < STREAM_WAVES) stream_wave<B, CHAIN>(a, g, w, lds);
    else control_wave<B, CHAIN>(a, g, lds);
}

// ------------------------------------------------------- standalone norm rows
// One wave per row: 128-bit loads, FP32 mean square, one rounding on store
// ("GPU Kernel Optimization" README, section "Architecture": one program per
// row instead of separate reduction and elementwise kernels).
template <bool F16>
__device__ __forceinline__ float h2f(uint32_t h) {
    if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    else return bf2f(h);
}
template <bool F16>
__device__ __forceinline__ uint32_t f2h(float f) {
    if constexpr (F16) return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
    else return (uint32_t)f2bf(f);
}

constexpr int NR_REG = 8;  // 128-bit chunks per lane kept in registers (K <= 4096)

template <bool F16>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const uint16_t *x, int64_t x_stride, const uint16_t *gamma,
                                                           float eps, uint16_t *y, int64_t y_stride, int32_t rows,
                                                           int32_t K) {
    const uint32_t lane = lane_id();
    const int32_t row = blockIdx.x * 4 + (int32_t)(threadIdx.x >> 6);
    if (row >= rows) return;
    const uint16_t *xr = x + (int64_t)row * x_stride;
    uint16_t *yr = y + (int64_t)row * y_stride;
    const int32_t n8 = K >> 3;
    float ss = 0.0f;
    if (n8 <= 64 * NR_REG) {
        u32x4 v[NR_REG];
#pragma unroll
        for (int c = 0; c < NR_REG; ++c) {
            int32_t i = c * 64 + (int32_t)lane;
            v[c] = i < n8 ? ld16(xr + i * 8) : (u32x4){0u, 0u, 0u, 0u};
            uint32_t vv[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float lo = h2f<F16>(vv[e] & 0xFFFFu), hi = h2f<F16>(vv[e] >> 16);
                ss += lo * lo + hi * hi;
            }
        }
        ss = wave_sum(ss);
        const float r = 1.0f / sqrtf(ss / (float)K + eps);
#pragma unroll
        for (int c = 0; c < NR_REG; ++c) {
            int32_t i = c * 64 + (int32_t)lane;
            if (i >= n8) break;
            u32x4 gv = ld16(gamma + i * 8);
            uint32_t vv[4] = {v[c].x, v[c].y, v[c].z, v[c].w}, gg[4] = {gv.x, gv.y, gv.z, gv.w}, o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float lo = h2f<F16>(vv[e] & 0xFFFFu) * r * h2f<F16>(gg[e] & 0xFFFFu);
                float hi = h2f<F16>(vv[e] >> 16) * r * h2f<F16>(gg[e] >> 16);
                o[e] = f2h<F16>(lo) | (f2h<F16>(hi) << 16);
            }
            *(u32x4 *)(yr + i * 8) = (u32x4){o[0], o[1], o[2], o[3]};
        }
        return;
    }
    for (int32_t i = lane; i < n8; i += 64) {
        u32x4 v = ld16(xr + i * 8);
        uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float lo = h2f<F16>(vv[e] & 0xFFFFu), hi = h2f<F16>(vv[e] >> 16);
            ss += lo * lo + hi * hi;
        }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)K + eps);
    for (int32_t i = lane; i < n8; i += 64) {
        u32x4 v = ld16(xr + i * 8), gv = ld16(gamma + i * 8);
        uint32_t vv[4] = {v.x, v.y, v.z, v.w}, gg[4] = {gv.x, gv.y, gv.z, gv.w}, o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float lo = h2f<F16>(vv[e] & 0xFFFFu) * r * h2f<F16>(gg[e] & 0xFFFFu);
            float hi = h2f<F16>(vv[e] >> 16) * r * h2f<F16>(gg[e] >> 16);
            o[e] = f2h<F16>(lo) | (f2h<F16>(hi) << 16);
        }
        *(u32x4 *)(yr + i * 8) = (u32x4){o[0], o[1], o[2], o[3]};
    }
}

}  // namespace wgn

// ------------------------------------------------------------ host launchers
namespace wgn {

template <int B, bool CHAIN>
static hipError_t launch_chain_b(const KArgs &a, int32_t grid, size_t lds, hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
        // 160 KB of LDS per workgroup on gfx950, minus the kernel's static LDS
        hipError_t e = hipFuncSetAttribute((const void *)chain_kernel<B, CHAIN>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((chain_kernel<B, CHAIN>), dim3(grid), dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

template <bool CHAIN>
static hipError_t launch_chain_c(int32_t batch, const KArgs &a, int32_t grid, size_t lds, hipStream_t s) {
    switch (batch) {
    case 1: return launch_chain_b<1, CHAIN>(a, grid, lds, s);
    case 2: return launch_chain_b<2, CHAIN>(a, grid, lds, s);
    case 3: return launch_chain_b<3, CHAIN>(a, grid, lds, s);
    case 4: return launch_chain_b<4, CHAIN>(a, grid, lds, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chain(int32_t batch, const KArgs &a, int32_t grid, size_t lds, hipStream_t s) {
    return a.phases ? launch_chain_c<true>(batch, a, grid, lds, s) : launch_chain_c<false>(batch, a, grid, lds, s);
}

hipError_t launch_rmsnorm_rows(const uint16_t *x, int64_t xs, const uint16_t *g, float eps, uint16_t *y, int64_t ys,
                               int32_t rows, int32_t K, bool f16, hipStream_t s) {
    dim3 grid((rows + 3) / 4), block(256);
    if (f16) hipLaunchKernelGGL(rmsnorm_rows_kernel<true>, grid, block, 0, s, x, xs, g, eps, y, ys, rows, K);
    else hipLaunchKernelGGL(rmsnorm_rows_kernel<false>, grid, block, 0, s, x, xs, g, eps, y, ys, rows, K);
    return hipGetLastError();
}

}  // namespace wgn
