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

#include <mutex>

#include "wgn_loader.h"
#include "wgn_numerics.h"

namespace wgn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef WGN_WEIGHT_AUX
#define WGN_WEIGHT_AUX 2  // nt: weights are streamed once
#endif
constexpr int TILE_LOADS = UNIT / 32;     // matrix-core path: loads per unit (= per block)
constexpr int WEIGHT_AUX = WGN_WEIGHT_AUX;  // cache policy of the weight loads (streamed once)
// Cache policy of every access to data that another workgroup produces or
// consumes inside the same launch (stage outputs, completion flags, argmax
// partials): sc0|sc1, the system-coherent level.  Stores are written through
// and loads are served from the coherent level, so data written on one XCD
// is visible to another without L2 write-back/invalidate fences (which cost
// several microseconds per phase boundary on this chip).
constexpr int COH = 17;
#ifndef WGN_POLL_GAP
#define WGN_POLL_GAP 0
#endif
#ifndef WGN_POLL_DELAY
#define WGN_POLL_DELAY 0
#endif
// s_sleep units (64 clocks): between flag-row reads, and before the first
constexpr int POLL_GAP = WGN_POLL_GAP, POLL_DELAY = WGN_POLL_DELAY;
constexpr uint32_t RSRC_W3 = 0x00020000u; // buffer descriptor word 3 for raw dword loads

// ------------------------------------------------------------------ numerics

// FP64 reciprocal and FP32-rounded reciprocal square root: the hardware's
// FP64 estimates, each refined by two Newton-Raphson steps (every step
// squares the relative error), leave only FP64 rounding before the final
// FP32 rounding -- at a fraction of the latency of IEEE divide and sqrt.
__device__ __forceinline__ double recip_f64(double k) {
    double r = __builtin_amdgcn_rcp(k);
    r = __builtin_fma(__builtin_fma(-k, r, 1.0), r, r);
    r = __builtin_fma(__builtin_fma(-k, r, 1.0), r, r);
    return r;
}
__device__ __forceinline__ float rsqrt_f64_to_f32(double v) {
    double y = __builtin_amdgcn_rsq(v);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const double e = __builtin_fma(-v * y, y, 1.0);  // 1 - v y^2
        y = __builtin_fma(0.5 * y, e, y);
    }
    return (float)y;
}
// (s / K + eps)^(-1/2) for an FP64 sum s over K values.
__device__ __forceinline__ float inv_sqrt_mean(double s, int32_t K, float eps) {
    return rsqrt_f64_to_f32(__builtin_fma(s, recip_f64((double)K), (double)eps));
}

// Two values packed as BF16 (lo in the low half), one instruction.
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
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

// Statistic of one 16-byte chunk of 8 BF16 values: the sum of squares
// (RMSNorm) or the sum (LayerNorm), formed in FP32 by v_dot2_f32_bf16 (the
// products of BF16 values are exact in FP32) in two interleaved chains, and
// widened to FP64 for the accumulation over chunks.
__device__ __forceinline__ double chunk_stat(const u32x4 &v, bool layer) {
    const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
    const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3F803F80u);
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16x2 x = __builtin_bit_cast(bf16x2, vv[e]);
        const bf16x2 y = layer ? one : x;
        if (e & 1) b = __builtin_amdgcn_fdot2_f32_bf16(x, y, b, false);
        else a = __builtin_amdgcn_fdot2_f32_bf16(x, y, a, false);
    }
    return (double)a + (double)b;
}

// x-hat of one chunk, rounded to BF16: ((x - mean) * rstd) * g + beta for
// LayerNorm, (x * rstd) * g for RMSNorm (g = 1 and beta = 0 when absent).
__device__ __forceinline__ u32x4 chunk_apply(const u32x4 &v, const u32x4 &gv, const u32x4 &bv, float mean,
                                             float rstd, bool layer) {
    const uint32_t vv[4] = {v.x, v.y, v.z, v.w}, gg[4] = {gv.x, gv.y, gv.z, gv.w}, bb[4] = {bv.x, bv.y, bv.z, bv.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float lo = bf2f(vv[e] & 0xFFFFu), hi = bf2f(vv[e] >> 16);
        if (layer) {
            lo = (lo - mean) * rstd * bf2f(gg[e] & 0xFFFFu) + bf2f(bb[e] & 0xFFFFu);
            hi = (hi - mean) * rstd * bf2f(gg[e] >> 16) + bf2f(bb[e] >> 16);
        } else {
            lo = lo * rstd * bf2f(gg[e] & 0xFFFFu);
            hi = hi * rstd * bf2f(gg[e] >> 16);
        }
        o[e] = f2bf2(lo, hi);
    }
    return (u32x4){o[0], o[1], o[2], o[3]};
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

// Sum over the 64 lanes, complete in lane 63 only (the other lanes hold
// partial sums).  The row sums of 16 lanes are formed as in wave_sum; the
// rows are then combined with DPP row broadcasts -- lane 15 of rows 0 and 2
// into rows 1 and 3, then lane 31 into rows 2 and 3 -- so no LDS permute (and
// no wait on the LDS queue) is needed.  The order is fixed: reproducible.
__device__ __forceinline__ float wave_sum_last(float v) {
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    v += dpp<0x140>(v);   // row_mirror
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31
    return v;
}

// Sum over aligned groups of lpr lanes (lpr = 4, 8, 16, 32 or 64, wave-uniform);
// every lane of a group gets the same bits.  lpr = 64 is exactly wave_sum.
__device__ __forceinline__ float group_sum(float v, int32_t lpr) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    if (lpr >= 8) v += dpp<0x141>(v);
    if (lpr >= 16) v += dpp<0x140>(v);
    if (lpr >= 32) v += __shfl_xor(v, 16);
    if (lpr >= 64) v += __shfl_xor(v, 32);
    return v;
}

template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// A DPP row broadcast of an FP64 value into the rows of ROW_MASK (0 elsewhere).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp64_rows(double v) {
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Sum of an FP64 value over the 64 lanes, returned to every lane from scalar
// registers: row sums by DPP, rows combined by the row broadcasts (as in
// wave_sum_last), then lane 63 read out -- no LDS permute.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp64<0xB1>(v);
    v += dpp64<0x4E>(v);
    v += dpp64<0x141>(v);
    v += dpp64<0x140>(v);
    v += dpp64_rows<0x142, 0xA>(v);  // row_bcast:15
    v += dpp64_rows<0x143, 0xC>(v);  // row_bcast:31
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, 63), hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), 63);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// The same steps as group_sum for FP64 values.
__device__ __forceinline__ double group_sum_f64(double v, int32_t lpr) {
    v += dpp64<0xB1>(v);
    v += dpp64<0x4E>(v);
    if (lpr >= 8) v += dpp64<0x141>(v);
    if (lpr >= 16) v += dpp64<0x140>(v);
    if (lpr >= 32) v += __shfl_xor(v, 16);
    if (lpr >= 64) v += __shfl_xor(v, 32);
    return v;
}

// Lane -> (batch row, slot) split used by the control wave: batch rows are
// padded to a power of two P <= 16; lane l serves batch row l % P and the
// (l / P)-th of every 64 / P consecutive items (norm chunks, output rows).
struct LaneSplit {
    int32_t P, shift;      // P = 1 << shift >= batch
    int32_t b;             // batch row of this lane
    int32_t i0, step;      // first item and item stride of this lane
    bool active;           // b < batch
};
__device__ __forceinline__ LaneSplit lane_split(int32_t nb, uint32_t lane) {
    LaneSplit L;
    L.shift = nb <= 1 ? 0 : 32 - __builtin_clz((uint32_t)(nb - 1));
    L.P = 1 << L.shift;
    L.b = (int32_t)(lane & (uint32_t)(L.P - 1));
    L.i0 = (int32_t)(lane >> L.shift);
    L.step = 64 >> L.shift;
    L.active = L.b < nb;
    return L;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    for (int o = 32; o >= 1; o >>= 1) {
        uint64_t t = __shfl_xor(v, o);
        v = t > v ? t : v;
    }
    return v;
}


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

__device__ __forceinline__ void trace_point(const KArgs &a, int32_t p, int32_t g, int i, uint32_t lane) {
    if (a.trace && lane == 0) a.trace[((size_t)p * a.G + g) * TRACE_POINTS + i] = wall_clock64();
}

// ------------------------------------------------------ normalisation (all waves)
// The inputs of a phase are normalised by the waves of the workgroup
// together.  The work items are the (job, batch row) pairs -- item
// q = j * Pb + b, Pb = batch rounded up to a power of two, the number of items
// P padded to a power of two -- and they are spread over the waves like rows
// by norm_split.  Each lane serves one item and walks a strided share of its
// 16-byte chunks.  Sums are formed per chunk in FP32 (chunk_stat),
// accumulated in FP64 and reduced inside the wave, so the statistics are as
// good as exact and their order is fixed.  Two splits:
//   * batch 3 and above (at least 4 items): never more than one wave per
//     item (the extra waves idle, or a wave holds several items); every lane
//     of an item then holds its statistics after the wave's reduction, and
//     no barrier or LDS round trip lies between the statistics and the
//     normalisation;
//   * batch 1 and 2 (a few items): an item spreads over several whole waves,
//     whose partial statistics are posted in LDS and combined in wave order
//     after a barrier -- shorter per-lane loops, which beat the saved barrier
//     there (measured: batch-1 decode step 740 against 742 us; LayerNorm
//     chain at batch 4 and 16 530 and 685 against 544 and 725 us).
// The split is fixed per kernel instance (one code path each: the batch-1
// kernel spills to scratch with both).
template <int B>
constexpr bool norm_one_wave() { return B >= 3; }

// log2 of the padded item count of the phase's jobs
__device__ __forceinline__ int32_t norm_items_log2(const NormHdr &J) {
    const int32_t lb = J.nb <= 1 ? 0 : 32 - wgn_clz((uint32_t)(J.nb - 1));
    const int32_t lj = J.njobs <= 1 ? 0 : 32 - wgn_clz((uint32_t)(J.njobs - 1));
    return lb + lj;
}

struct NormItem {
    NormSplit S;
    int32_t j, b;        // job and batch row of this lane's item
    bool active;         // this lane serves a real item
    bool wave_active;    // this wave serves items at all
};
__device__ __forceinline__ NormItem norm_item(const NormHdr &J, int32_t w, uint32_t lane, int32_t nw) {
    NormItem it;
    const int32_t lb = J.nb <= 1 ? 0 : 32 - wgn_clz((uint32_t)(J.nb - 1));
    const int32_t P = 1 << norm_items_log2(J);
    const int32_t nwe = P < nw ? P : nw;  // waves that serve items: one wave per item at most
    it.wave_active = w < nwe;
    it.S = norm_split(P, it.wave_active ? w : 0, lane, nwe);
    it.j = it.S.row >> lb;
    it.b = it.S.row & ((1 << lb) - 1);
    it.active = it.wave_active && it.S.active && it.j < J.njobs && it.b < J.nb;
    return it;
}

// One-wave split: statistics of this lane's item, then its share of the item
// normalised and rounded to BF16 in place.
__device__ void norm_item_apply(char *lds, int32_t w, uint32_t lane, int32_t nw) {
    const NormHdr &J = *(const NormHdr *)(lds + LDS_NORM_OFF);
    const NormItem it = norm_item(J, w, lane, nw);
    if (!it.wave_active) return;
    const NormSplit &S = it.S;
    const NormJob &jb = J.job[it.active ? it.j : 0];
    const bool layer = jb.norm == NORM_LAYER;
    const int32_t K = jb.K, n8 = it.active ? K >> 3 : 0;
    uint16_t *dst = (uint16_t *)(lds + J.x_off + ((size_t)(it.active ? it.b : 0) * J.xb + jb.xoff) * 2);
    double s1 = 0.0, s2 = 0.0;
    for (int32_t i = S.sub; i < n8; i += S.lanes) {
        const u32x4 v = *(const u32x4 *)(dst + i * 8);
        s2 += chunk_stat(v, false);
        if (layer) s1 += chunk_stat(v, true);
    }
    if (S.lpr == 64) {
        s1 = wave_sum_f64(s1);
        s2 = wave_sum_f64(s2);
    } else {
        s1 = group_sum_f64(s1, S.lpr);
        s2 = group_sum_f64(s2, S.lpr);
    }
    if (!it.active) return;
    float mean = 0.0f, rstd;
    if (!layer) {
        rstd = inv_sqrt_mean(s2, K, jb.eps);
    } else {
        const double rk = recip_f64((double)K);
        const double m = s1 * rk;
        const double var = __builtin_fma(s2, rk, -m * m);  // biased; FP64 sums, see above
        mean = (float)m;
        rstd = rsqrt_f64_to_f32((var > 0.0 ? var : 0.0) + (double)jb.eps);
    }
    const char *gp = lds + jb.prm;
    const char *bp = lds + jb.prm + jb.prm_half;
    for (int32_t i = S.sub; i < n8; i += S.lanes) {
        const u32x4 v = *(const u32x4 *)(dst + i * 8);
        const u32x4 gv = jb.has_gamma ? *(const u32x4 *)(gp + i * 16)
                                      : (u32x4){0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
        const u32x4 bv = jb.has_beta ? *(const u32x4 *)(bp + i * 16) : (u32x4){0u, 0u, 0u, 0u};
        *(u32x4 *)(dst + i * 8) = chunk_apply(v, gv, bv, mean, rstd, layer);
    }
}

// Spread split: statistics over several waves, posted per wave in LDS.
__device__ __forceinline__ double2 *norm_stats(char *lds, int32_t w, int32_t slot) {
    return (double2 *)(lds + LDS_STATS_OFF) + (w * STATS_ROWS + slot);
}

struct NormItemW {
    NormSplit S;
    int32_t j, b;  // job and batch row of this lane's item
    bool active;
};
__device__ __forceinline__ NormItemW norm_item_w(const NormHdr &J, int32_t w, uint32_t lane, int32_t nw) {
    NormItemW it;
    const int32_t lb = J.nb <= 1 ? 0 : 32 - wgn_clz((uint32_t)(J.nb - 1));
    const int32_t lj = J.njobs <= 1 ? 0 : 32 - wgn_clz((uint32_t)(J.njobs - 1));
    it.S = norm_split(1 << (lj + lb), w, lane, nw);
    it.j = it.S.row >> lb;
    it.b = it.S.row & ((1 << lb) - 1);
    it.active = it.S.active && it.j < J.njobs && it.b < J.nb;
    return it;
}

// Step 1 (after the inputs have landed in LDS): partial statistics.
__device__ void norm_all_stats(char *lds, int32_t w, uint32_t lane, int32_t nw) {
    const NormHdr &J = *(const NormHdr *)(lds + LDS_NORM_OFF);
    const NormItemW it = norm_item_w(J, w, lane, nw);
    const NormSplit &S = it.S;
    const NormJob &jb = J.job[it.active ? it.j : 0];
    const bool layer = jb.norm == NORM_LAYER;
    const int32_t n8 = it.active ? jb.K >> 3 : 0;
    const uint16_t *src = (const uint16_t *)(lds + J.x_off + ((size_t)(it.active ? it.b : 0) * J.xb + jb.xoff) * 2);
    double s1 = 0.0, s2 = 0.0;
    for (int32_t i = S.sub; i < n8; i += S.lanes) {
        const u32x4 v = *(const u32x4 *)(src + i * 8);
        s2 += chunk_stat(v, false);
        if (layer) s1 += chunk_stat(v, true);
    }
    if (S.lpr == 64) {
        s1 = wave_sum_f64(s1);
        s2 = wave_sum_f64(s2);
    } else {
        s1 = group_sum_f64(s1, S.lpr);
        s2 = group_sum_f64(s2, S.lpr);
    }
    if ((S.sub % S.lpr) == 0) {
        double2 st;
        st.x = s1;
        st.y = s2;
        *norm_stats(lds, w, S.slot) = st;
    }
}

// Step 2 (after every wave has posted its statistics): normalise this lane's
// share and round to BF16 in place.
__device__ void norm_all_apply(char *lds, int32_t w, uint32_t lane, int32_t nw) {
    const NormHdr &J = *(const NormHdr *)(lds + LDS_NORM_OFF);
    const NormItemW it = norm_item_w(J, w, lane, nw);
    if (!it.active) return;
    const NormSplit &S = it.S;
    const NormJob &jb = J.job[it.j];
    const int32_t K = jb.K, n8 = K >> 3;
    double s1 = 0.0, s2 = 0.0;
    for (int32_t ww = S.w0; ww < S.w1; ++ww) {
        const double2 st = *norm_stats(lds, ww, S.rslot);
        s1 += st.x;
        s2 += st.y;
    }
    const bool layer = jb.norm == NORM_LAYER;
    float mean = 0.0f, rstd;
    if (!layer) {
        rstd = inv_sqrt_mean(s2, K, jb.eps);
    } else {
        const double rk = recip_f64((double)K);
        const double m = s1 * rk;
        const double var = __builtin_fma(s2, rk, -m * m);  // biased; FP64 sums, see above
        mean = (float)m;
        rstd = rsqrt_f64_to_f32((var > 0.0 ? var : 0.0) + (double)jb.eps);
    }
    uint16_t *dst = (uint16_t *)(lds + J.x_off + ((size_t)it.b * J.xb + jb.xoff) * 2);
    const char *gp = lds + jb.prm;
    const char *bp = lds + jb.prm + jb.prm_half;
    for (int32_t i = S.sub; i < n8; i += S.lanes) {
        const u32x4 v = *(const u32x4 *)(dst + i * 8);
        const u32x4 gv = jb.has_gamma ? *(const u32x4 *)(gp + i * 16)
                                      : (u32x4){0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
        const u32x4 bv = jb.has_beta ? *(const u32x4 *)(bp + i * 16) : (u32x4){0u, 0u, 0u, 0u};
        *(u32x4 *)(dst + i * 8) = chunk_apply(v, gv, bv, mean, rstd, layer);
    }
}

// Every wave calls this for a phase whose run header says it has a
// normalised input, right before the x-hat barrier.  Barriers: one (inputs
// in LDS, jobs posted), and with the spread split one more (statistics of
// every wave posted).
template <int B>
__device__ __forceinline__ void norm_all(char *lds, int32_t w, uint32_t lane) {
    wg_barrier();  // inputs in LDS, jobs posted
    if constexpr (norm_one_wave<B>()) {
        norm_item_apply(lds, w, lane, WAVES);
    } else {
        norm_all_stats(lds, w, lane, WAVES);
        wg_barrier();  // statistics of every wave posted
        norm_all_apply(lds, w, lane, WAVES);
    }
}


// ------------------------------------------------------------ streaming waves
struct BlockMeta {
    uint32_t meta_v;       // vector path: lane j holds the meta word of the block's unit j
    int32_t xb_bytes;      // LDS bytes per batch row of x-hat in this block's phase
    int32_t x_off;         // LDS offset of the phase's x-hat
    int32_t part_off;      // LDS offset of the phase's partial slots
    // matrix-core path (one unit per block; wave-uniform)
    uint32_t xoff;         // chunk offset inside a batch row of x-hat
    int32_t rows, slot0, slot_stride;
    bool seg_end;
    bool last;             // last block of this wave in its phase
};

struct StreamState {
    const char *desc;      // LDS run-list buffers
    RunHdr h;              // header of the current phase's run list
    const Run *runs;       // run list of the current phase (LDS)
    int32_t p;
    int32_t u, u_beg, u_end;
    int32_t g, w, p1;
    int32_t dmask;         // run-list ring size - 1
    bool done_all;
};

__device__ __forceinline__ const char *run_buf(const char *desc, int32_t p, int32_t dmask) {
    return desc + (p & dmask) * RUN_BUF_STRIDE;
}
__device__ __forceinline__ const char *run_buf_s(const StreamState &S, int32_t p) {
    return run_buf(S.desc, p, S.dmask);
}

__device__ __forceinline__ void stream_begin_phase(StreamState &S, int32_t p) {
    const char *buf = run_buf_s(S, p);
    S.h = *(const RunHdr *)buf;
    S.runs = (const Run *)(buf + sizeof(RunHdr));
    S.p = p;
    S.u_beg = ((const RunHdr *)buf)->wb[S.w];  // indexed in LDS, not in registers
    S.u_end = ((const RunHdr *)buf)->wb[S.w + 1];
    S.u = S.u_beg;
}

__device__ __forceinline__ void stream_advance(StreamState &S, BlockMeta &bm, int32_t step) {
    if (S.done_all) {
        bm.last = false;  // past the final phase: nothing to synchronise
        return;
    }
    S.u = S.u + step < S.u_end ? S.u + step : S.u_end;
    bm.last = S.u >= S.u_end;
    if (bm.last) {
        if (S.p + 1 < S.p1) stream_begin_phase(S, S.p + 1);
        else S.done_all = true;
    }
}

// Vector path: issue DEPTH unit loads (a block never spans a phase boundary).
// Lane j first computes the descriptor of unit j from the phase's run list in
// LDS; each load then takes its base address and length from lane j through
// v_readlane.  Invalid slots load from an empty range (no memory traffic,
// value 0), so every block issues the same number of loads and the
// compiler's vmcnt bookkeeping stays exact.
// Per-lane unit addresses of a block whose loads have not been issued yet
// (lane j: unit j), so that they can be issued one by one later.
struct PendLoads {
    uint32_t plo, phi, nb;
};

template <int B, int D>
__device__ __forceinline__ PendLoads prepare_block(const KArgs &a, StreamState &S, BlockMeta &bm, uint32_t lane) {
    UnitDesc ud;
    ud.ptr = 0;
    ud.nbytes = 0;
    ud.meta = 0;
    if (!S.done_all && lane < (uint32_t)D)
        ud = unit_desc_runs(S.h, S.runs, S.u + (int32_t)lane, S.u_beg, S.u_end, S.w, B);
    if (ud.nbytes == 0) ud.ptr = (uint64_t)(uintptr_t)a.ist.W;
    PendLoads q;
    q.plo = (uint32_t)ud.ptr;
    q.phi = (uint32_t)(ud.ptr >> 32);
    q.nb = ud.nbytes;
    bm.meta_v = ud.meta;
    bm.xb_bytes = S.done_all ? 0 : S.h.xb_bytes;
    bm.x_off = S.h.x_off;
    bm.part_off = S.h.part_off;
    stream_advance(S, bm, D);
    return q;
}

// Load unit j of a prepared block: 16 bytes per lane, 1 KB per wave.
__device__ __forceinline__ u32x4 issue_unit(const PendLoads &q, int j, uint32_t lane) {
    const uint32_t lo = __builtin_amdgcn_readlane(q.plo, j);
    const uint32_t hi = __builtin_amdgcn_readlane(q.phi, j);
    const uint32_t nb = __builtin_amdgcn_readlane(q.nb, j);
    const void *base = (const void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)nb, (int)RSRC_W3);
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)(lane * 16u), 0, WEIGHT_AUX);
}

template <int B, int D>
__device__ __forceinline__ void load_block(const KArgs &a, StreamState &S, u32x4 (&d)[D], BlockMeta &bm,
                                           uint32_t lane) {
    const PendLoads q = prepare_block<B, D>(a, S, bm, lane);
#pragma unroll
    for (int j = 0; j < D; ++j) d[j] = issue_unit(q, j, lane);
}

// Every slot of a block is consumed unconditionally (an invalid slot holds
// zeros and points at the start of x-hat, which is initialised in every
// phase), so every load is waited for in issue order on every path and the
// compiler's vmcnt bookkeeping stays exact.
//
// Units are consumed in groups of G: the group's x-hat reads are issued
// together, so one LDS latency covers G units, and a row-part that ends in
// the block is reduced by wave_sum_last (DPP only) and its partial written by
// lane 63.  G is the largest group whose x-hat values fit in the registers
// left beside the two in-flight blocks.
template <int B, int D>
constexpr int xhat_group() {
    return (B == 1 && D % 16 == 0 && D <= 16) ? 16 : (B == 1 && D % 8 == 0) ? 8
         : ((B == 1 || B == 2) && D % 4 == 0) ? 4 : 2;
}

// IL: while consuming, also issue the loads of a prepared block q into dn,
// one per consumed unit (after each group's x-hat reads), so that the compute
// unit's memory pipeline receives a steady trickle instead of a burst.
template <int B, int D, bool IL = false>
__device__ __forceinline__ void consume_block(const u32x4 (&d)[D], const BlockMeta &bm, float (&acc)[B],
                                              const char *lds, uint32_t lane, const PendLoads *q = nullptr,
                                              u32x4 *dn = nullptr) {
    constexpr int G = xhat_group<B, D>();
    static_assert(D % G == 0, "block depth must be a multiple of the x-hat group");
    const char *xh = lds + bm.x_off + lane * 16u;
    float *part = (float *)(lds + bm.part_off);
#pragma unroll
    for (int g0 = 0; g0 < D; g0 += G) {
        u32x4 xv[G][B];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint32_t m = __builtin_amdgcn_readlane(bm.meta_v, g0 + j);
            const char *xp = xh + ((m & 0x3FFFu) << 4);
#pragma unroll
            for (int b = 0; b < B; ++b) xv[j][b] = *(const u32x4 *)(xp + b * bm.xb_bytes);
        }
        if constexpr (IL) {
#pragma unroll
            for (int j = 0; j < G; ++j) dn[g0 + j] = issue_unit(*q, g0 + j, lane);
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint32_t m = __builtin_amdgcn_readlane(bm.meta_v, g0 + j);
#pragma unroll
            for (int b = 0; b < B; ++b) acc[b] = dot8(d[g0 + j], xv[j][b], acc[b]);
            if (m & 0x4000u) {
                const uint32_t slot = m >> 16;
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const float sum = wave_sum_last(acc[b]);
                    if (lane == 63) part[slot + b] = sum;
                    acc[b] = 0.0f;
                }
            }
        }
    }
}

// Matrix-core path: one unit (16 row-parts x 512 K) per block.  Load t of
// lane l reads 16 bytes of row l % 16 at K offset 8 (l / 16) + 32 t: the A
// operand of v_mfma_f32_16x16x32_bf16.  Lanes past the end of their row read
// an out-of-range offset (value 0, no traffic); rows past the tile's last
// valid row fall outside the buffer's range the same way.
__device__ __forceinline__ void load_tile(const KArgs &a, StreamState &S, u32x4 (&d)[TILE_LOADS], BlockMeta &bm,
                                          uint32_t lane) {
    TileDesc td;
    td.valid = false;
    if (!S.done_all) td = unit_desc_tile(S.h, S.runs, S.u, S.u_beg, S.u_end, S.w, a.nb);
    const bool valid = !S.done_all && td.valid;
    const uint64_t ptr = valid ? td.ptr : (uint64_t)(uintptr_t)a.ist.W;
    const uint32_t plo = __builtin_amdgcn_readfirstlane((uint32_t)ptr);
    const uint32_t phi = __builtin_amdgcn_readfirstlane((uint32_t)(ptr >> 32));
    const uint32_t nrec = __builtin_amdgcn_readfirstlane(valid ? td.nrec : 0u);
    const void *base = (const void *)(uintptr_t)(((uint64_t)phi << 32) | plo);
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)nrec, (int)RSRC_W3);
    const uint32_t q = lane >> 4;
    const uint32_t lane_off = (lane & 15u) * (uint32_t)(valid ? td.rstride : 0) + q * 16u;
    const int32_t kv = (valid ? td.kval : 0) - 8 * (int32_t)q;  // K elements from this lane's first position
#pragma unroll
    for (int t = 0; t < TILE_LOADS; ++t) {
        const uint32_t off = 32 * t < kv ? lane_off + 64u * (uint32_t)t : 0x80000000u;
        d[t] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, WEIGHT_AUX);
    }
    bm.xb_bytes = S.h.xb_bytes;
    bm.x_off = S.h.x_off;
    bm.part_off = S.h.part_off;
    bm.xoff = valid ? td.xoff : 0u;
    bm.rows = valid ? td.rows : 0;
    bm.slot0 = valid ? td.slot0 : 0;
    bm.slot_stride = valid ? td.slot_stride : 0;
    bm.seg_end = valid && td.seg_end;
    stream_advance(S, bm, 1);
}

__device__ __forceinline__ void consume_tile(const u32x4 (&d)[TILE_LOADS], const BlockMeta &bm, f32x4 &acc,
                                             const char *lds, uint32_t lane, int32_t nb) {
    const uint32_t q = lane >> 4, j = lane & 15u;
    const uint32_t jr = (int32_t)j < nb ? j : (uint32_t)(nb - 1);  // batch rows past nb: results unused
    const char *xp = lds + bm.x_off + jr * (uint32_t)bm.xb_bytes + bm.xoff + q * 16u;
#pragma unroll
    for (int t = 0; t < TILE_LOADS; ++t) {
        const u32x4 xv = *(const u32x4 *)(xp + 64 * t);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, d[t]), __builtin_bit_cast(bf16x8, xv),
                                                      acc, 0, 0, 0);
    }
    if (bm.seg_end) {
        // lane l holds rows 4 (l / 16) + r, batch row l % 16
        float *part = (float *)(lds + bm.part_off);
        const float av[4] = {acc[0], acc[1], acc[2], acc[3]};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int32_t row = 4 * (int32_t)q + r;
            if (row < bm.rows && (int32_t)j < nb) part[bm.slot0 + row * bm.slot_stride + (int32_t)j] = av[r];
        }
        acc = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    }
}

template <int B, bool TILE>
struct Acc;
template <int B>
struct Acc<B, false> {
    float v[B];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int b = 0; b < B; ++b) v[b] = 0.0f;
    }
};
template <int B>
struct Acc<B, true> {
    f32x4 v;
    __device__ __forceinline__ void zero() { v = (f32x4){0.0f, 0.0f, 0.0f, 0.0f}; }
};

template <bool TILE, int R>
constexpr int block_loads() { return TILE ? TILE_LOADS : ring_depth(R); }

template <int B, bool TILE, int R>
__device__ __forceinline__ void load_any(const KArgs &a, StreamState &S, u32x4 (&d)[block_loads<TILE, R>()],
                                         BlockMeta &bm, uint32_t lane) {
    if constexpr (TILE) load_tile(a, S, d, bm, lane);
    else load_block<B, ring_depth(R)>(a, S, d, bm, lane);
}
template <int B, bool TILE, int R>
__device__ __forceinline__ void consume_any(const KArgs &a, const u32x4 (&d)[block_loads<TILE, R>()],
                                            const BlockMeta &bm, Acc<B, TILE> &acc, const char *lds, uint32_t lane) {
    if constexpr (TILE) consume_tile(d, bm, acc.v, lds, lane, a.nb);
    else consume_block<B, ring_depth(R)>(d, bm, acc.v, lds, lane);
}

// Whether the streaming waves hold a phase's last refill until the control
// wave has issued the phase's stores (a third barrier per phase).
template <bool TILE, int R>
constexpr bool epi_barrier() { return EPI_BARRIER != 0 && (TILE || !ring_interleaved(R)); }

// Whether all waves share the epilogue's output rows (burst ring 0 only: at
// the third barrier a streaming wave has just one older block in flight, so
// waiting for its own stores costs little).
template <int B, bool TILE, int R>
constexpr bool epi_share() {
    // (the interleaved ring at batch 4 would spill: its streaming waves hold
    // three blocks of weights across the epilogue)
    return (R == 0 && EPI_BARRIER == 1 && (EPI_SHARE == 2 || (EPI_SHARE >= 1 && TILE))) ||
           (EPI_SHARE == 3 && !TILE && ring_interleaved(R) && B <= 3);
}
// Whether all waves share the input copies of a phase (the matrix-core path):
// one more barrier per phase (the flags have been seen), after which every
// wave issues its share of the copies and waits for them -- on that path a
// streaming wave then has only one block of weight loads in flight, issued
// well before.
template <bool TILE, int R>
constexpr bool in_share() {
    return IN_SHARE && ((TILE && R == 0) || (IN_SHARE == 2 && !TILE && ring_interleaved(R)));
}

template <int B, bool CHAIN>
__device__ __forceinline__ void issue_source_loads(const KArgs &a, int32_t nsrc, int32_t xb, const char *lds,
                                                   char *xh, uint32_t lane, int32_t w, int32_t nw, bool zero_tail);
template <int B, bool CHAIN, bool TILE>
__device__ __forceinline__ void epilogue(const KArgs &a, const RunHdr &h, const Run *runs, int32_t g, const float *part,
                                         const float *epi, float *carry, uint32_t lane, int32_t wsel, int32_t nw,
                                         bool with_argmax);
template <bool TILE>
__device__ __forceinline__ void argmax_shared(const KArgs &a, const RunHdr &h, const Run *runs, int32_t g,
                                              const float *part, float *carry, char *lds, uint32_t lane, int32_t w);

// A streaming wave's part of phase p's input copies (when the phase's header
// asks for shared copies): after the barrier that follows the control wave's
// wait for the flags, copy every WAVES-th 1 KB of the inputs and wait for
// those copies (and this wave's older weight loads).
template <int B, bool CHAIN>
__device__ __forceinline__ void share_inputs(const KArgs &a, const StreamState &S, int32_t p, char *lds,
                                             uint32_t lane, int32_t w) {
    const RunHdr &hh = *(const RunHdr *)run_buf_s(S, p);
    if (!hh.share_in) return;
    wg_barrier();  // the control wave has seen phase p-1's flags
    issue_source_loads<B, CHAIN>(a, MAX_SRC, hh.xb_bytes / 2, lds, lds + hh.x_off, lane, w, WAVES, false);
    __builtin_amdgcn_s_waitcnt(0);
}

// Vector path with interleaved refills.  Slot k's refill is prepared (run
// list read, addresses computed) right after slot k is consumed and issued,
// one load per unit, while slot k+1 is consumed; NS - 2 blocks are fully
// in flight beyond the one being consumed, plus the one being issued.  At a
// phase end the prepared refill waits for the next phase's x-hat barrier, so
// the control wave's stores, flag store, flag polls and input loads meet an
// idle memory pipeline.
template <int B, bool CHAIN, int R>
__device__ __forceinline__ void stream_wave_il(const KArgs &a, int32_t g, int32_t w, char *lds) {
    constexpr int NS = ring_slots(R), D = ring_depth(R);
    static_assert(NS >= 2, "at least two block buffers");
    const uint32_t lane = lane_id();
    StreamState S;
    S.desc = lds + LDS_DESC_OFF;
    S.dmask = desc_bufs(R) - 1;
    S.g = g;
    S.w = w;
    S.p1 = a.p1;
    S.done_all = false;
    wg_barrier();  // run lists of the first phases are in LDS
    if (abort_flag_get()) return;  // an earlier run's wait gave up: nothing runs
    stream_begin_phase(S, a.p0);
    u32x4 d[NS][D];
    BlockMeta m[NS];
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    uint64_t *tl = (uint64_t *)(lds + LDS_TRACE_OFF);  // trace slots
    const bool tw = a.trace && w == 0 && lane == 0;
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) load_block<B, D>(a, S, d[k], m[k], lane);
    PendLoads pq = prepare_block<B, D>(a, S, m[NS - 1], lane);
    if constexpr (in_share<false, R>()) share_inputs<B, CHAIN>(a, S, a.p0, lds, lane, w);
    if (((const RunHdr *)run_buf_s(S, a.p0))->has_norm) norm_all<B>(lds, w, lane);
    wg_barrier();  // x-hat of the first phase is ready
    bool ok = abort_flag_get() == 0;
    int32_t p = a.p0;
    if (tw) tl[(p & 1) * 6 + 0] = wall_clock64();
    int32_t nblk = 0;  // blocks of phase p consumed (trace only)
    while (ok && p < a.p1) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            consume_block<B, D, true>(d[k], m[k], acc, lds, lane, &pq, d[(k + NS - 1) % NS]);
            if (tw && nblk < 3) tl[(p & 1) * 6 + 3 + nblk] = wall_clock64();
            ++nblk;
            const bool end = ok && m[k].last;
            if (end) {
                if (tw) tl[(p & 1) * 6 + 2] = wall_clock64();
                wg_barrier();  // partials of phase p are complete
                if constexpr (epi_share<B, false, R>()) {
                    // this wave's share of the phase's output rows and argmax
                    // keys; its stores (and its weight loads in flight)
                    // complete before the barrier after which the flag is set
                    const RunHdr &hh = *(const RunHdr *)run_buf_s(S, p);
                    const Run *rr = (const Run *)((const char *)&hh + sizeof(RunHdr));
                    epilogue<B, CHAIN, false>(a, hh, rr, g, (const float *)(lds + hh.part_off),
                                              (const float *)(lds + hh.epi_off), (float *)(lds + hh.carry_off), lane,
                                              w, WAVES, false);
                    argmax_shared<false>(a, hh, rr, g, (const float *)(lds + hh.part_off),
                                         (float *)(lds + hh.carry_off), lds, lane, w);
                    __builtin_amdgcn_s_waitcnt(0);
                    wg_barrier();  // every wave's stores have completed
                }
            }
            pq = prepare_block<B, D>(a, S, m[k], lane);
            if (end) nblk = 0;
            if (end && ++p < a.p1) {
                if (tw) tl[(p & 1) * 6 + 1] = wall_clock64();
                if constexpr (in_share<false, R>()) share_inputs<B, CHAIN>(a, S, p, lds, lane, w);
                if (((const RunHdr *)run_buf_s(S, p))->has_norm) norm_all<B>(lds, w, lane);
                wg_barrier();  // x-hat of phase p is ready
                ok = abort_flag_get() == 0;
                if (tw) tl[(p & 1) * 6 + 0] = wall_clock64();
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // no load of this wave is left in flight when it ends
}

template <int B, bool CHAIN, bool TILE, int R>
__device__ __forceinline__ void stream_wave(const KArgs &a, int32_t g, int32_t w, char *lds) {
    constexpr int NS = TILE ? 2 : ring_slots(R);
    const uint32_t lane = lane_id();
    StreamState S;
    S.desc = lds + LDS_DESC_OFF;
    S.dmask = desc_bufs_k(TILE, R) - 1;
    S.g = g;
    S.w = w;
    S.p1 = a.p1;
    S.done_all = false;
    wg_barrier();  // run lists of the first phases are in LDS
    if (abort_flag_get()) return;  // an earlier run's wait gave up: nothing runs
    stream_begin_phase(S, a.p0);
    u32x4 d[NS][block_loads<TILE, R>()];
    BlockMeta m[NS];
    Acc<B, TILE> acc;
    acc.zero();

    // A ring of NS block buffers: NS - 1 blocks are always in flight beyond the
    // one being consumed, and a buffer is refilled as soon as it has been
    // consumed.  When a block ends a phase, the refill is issued before
    // waiting for the next phase's x-hat, so the weight stream keeps running
    // through the device-wide phase boundary, and the next phase's first
    // blocks (loaded long before) are consumed as soon as x-hat is ready.
    // The loop has no early exit and no global stores: past the final phase
    // it only meets empty blocks (no barriers, no partial writes), which keeps
    // the compiler's vmcnt bookkeeping exact.
    uint64_t *tl = (uint64_t *)(lds + LDS_TRACE_OFF);  // trace slots
    const bool tw = a.trace && w == 0 && lane == 0;
#pragma unroll
    for (int k = 0; k < NS; ++k) load_any<B, TILE, R>(a, S, d[k], m[k], lane);
    if constexpr (in_share<TILE, R>()) share_inputs<B, CHAIN>(a, S, a.p0, lds, lane, w);
    if (((const RunHdr *)run_buf_s(S, a.p0))->has_norm) norm_all<B>(lds, w, lane);
    wg_barrier();  // x-hat of the first phase is ready
    bool ok = abort_flag_get() == 0;
    int32_t p = a.p0;
    if (tw) tl[(p & 1) * 6 + 0] = wall_clock64();
    int32_t nblk = 0;  // blocks of phase p consumed (trace only)
    while (ok && p < a.p1) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            consume_any<B, TILE, R>(a, d[k], m[k], acc, lds, lane);
            if (tw && nblk < 3) tl[(p & 1) * 6 + 3 + nblk] = wall_clock64();
            ++nblk;
            const bool end = ok && m[k].last;
            if (end) {
                if (tw) tl[(p & 1) * 6 + 2] = wall_clock64();
                wg_barrier();  // partials of phase p are complete
                if constexpr (epi_share<B, TILE, R>()) {
                    // this wave's share of the phase's output rows; its stores
                    // (and its one older block of weight loads) complete
                    // before the third barrier
                    const RunHdr &hh = *(const RunHdr *)run_buf_s(S, p);
                    const Run *rr = (const Run *)((const char *)&hh + sizeof(RunHdr));
                    epilogue<B, CHAIN, TILE>(a, hh, rr, g, (const float *)(lds + hh.part_off),
                                             (const float *)(lds + hh.epi_off), (float *)(lds + hh.carry_off), lane,
                                             w, WAVES, false);
                    argmax_shared<TILE>(a, hh, rr, g, (const float *)(lds + hh.part_off), (float *)(lds + hh.carry_off),
                                        lds, lane, w);
                    __builtin_amdgcn_s_waitcnt(0);
                } else if constexpr (!TILE && R == 0 && !CHAIN) {
                    // single-stage calls: argmax keys from every wave (in
                    // chains at batch 1 the larger kernel measured slower)
                    const RunHdr &hh = *(const RunHdr *)run_buf_s(S, p);
                    const Run *rr = (const Run *)((const char *)&hh + sizeof(RunHdr));
                    argmax_shared<false>(a, hh, rr, g, (const float *)(lds + hh.part_off), (float *)(lds + hh.carry_off),
                                         lds, lane, w);
                }
                if (epi_barrier<TILE, R>()) wg_barrier();  // the control wave has issued phase p's stores
            }
            load_any<B, TILE, R>(a, S, d[k], m[k], lane);
            if (end) nblk = 0;
            if (end && ++p < a.p1) {
                if (tw) tl[(p & 1) * 6 + 1] = wall_clock64();
                if constexpr (in_share<TILE, R>()) share_inputs<B, CHAIN>(a, S, p, lds, lane, w);
                if (((const RunHdr *)run_buf_s(S, p))->has_norm) norm_all<B>(lds, w, lane);
                wg_barrier();  // x-hat of phase p is ready
                ok = abort_flag_get() == 0;
                if (tw) tl[(p & 1) * 6 + 0] = wall_clock64();
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // no load of this wave is left in flight when it ends
}

// --------------------------------------------------------------- control wave
__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *(const u32x4 *)p; }

// Buffer resource over 2 GB from base; a null base gets an empty range, so
// loads through it return 0 and stores are dropped without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, base ? 0x7FFFFFFF : 0, (int)RSRC_W3);
}

// A pointer every lane holds the same value of (read from a run list in LDS,
// which all lanes build alike), moved to scalar registers.  Without this the
// compiler must assume a per-lane value: a buffer access through it becomes a
// loop over the distinct values, and a load in such a loop waits for every
// load issued before it.
template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (T *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int32_t uniform_i32(int32_t v) { return (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)v); }
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

#define WGN_GAS __attribute__((address_space(1)))
#define WGN_LAS __attribute__((address_space(3)))

// Copy n8 16-byte chunks of global memory into LDS (lane i of iteration it
// moves chunk it*64+i to dst + (it*64+i)*16).  Asynchronous: the caller waits.
template <int AUX>
__device__ __forceinline__ void copy_to_lds(const uint16_t *src, char *dst, int32_t n8, uint32_t lane) {
    for (int32_t it = 0; it * 64 < n8; ++it) {
        if (it * 64 + (int32_t)lane < n8)
            __builtin_amdgcn_global_load_lds((const WGN_GAS void *)(src + ((size_t)it * 64 + lane) * 8),
                                             (WGN_LAS void *)(dst + it * 1024), 16, 0, AUX);
    }
}

// LDS bytes of the gain/shift area of one source (gain, then shift; padded).
__device__ __forceinline__ int32_t prm_bytes(const DevSource &src) { return nchunks_of(src.K) * UNIT * 2 * 2; }

// Issued before the device-wide wait (nothing here depends on an earlier
// phase, so its latency overlaps the wait): the norm gains and shifts of the
// phase's normalised sources are copied into their LDS areas, as the phase's
// source table (already in LDS) lists them.
__device__ void prefetch_params(const DevPhase &ph, char *lds, uint32_t lane) {
    const SrcInfo *T = (const SrcInfo *)(lds + LDS_SRC_OFF);
#pragma unroll
    for (int32_t si = 0; si < MAX_SRC; ++si) {
        if (si >= ph.nsrc) break;
        const int32_t n8 = uniform_i32(T[si].K) >> 3;
        const uint16_t *gamma = uniform_ptr(T[si].gamma), *beta = uniform_ptr(T[si].beta);
        char *gp = lds + uniform_i32(T[si].prm);
        if (gamma) copy_to_lds<0>(gamma, gp, n8, lane);
        if (beta) copy_to_lds<0>(beta, gp + uniform_i32(T[si].prm_half), n8, lane);
    }
}

// The phase's source table and normalisation job list, written to LDS
// (LDS_SRC_OFF, LDS_NORM_OFF) by the control wave.
template <bool CHAIN>
__device__ void write_phase_info(const KArgs &a, int32_t p, char *lds, uint32_t lane) {
    if (CHAIN && a.phinfo) {
        // precomputed (the table, then the jobs): asynchronous copies
        constexpr int32_t nt = MAX_SRC * (int)sizeof(SrcInfo);
        const uint16_t *src = (const uint16_t *)(a.phinfo + (size_t)p * PHASE_INFO_BYTES);
        copy_to_lds<0>(src, lds + LDS_SRC_OFF, nt / 16, lane);
        copy_to_lds<0>(src + nt / 2, lds + LDS_NORM_OFF, (int)sizeof(NormHdr) / 16, lane);
        return;
    }
    // every lane computes the same tables
    make_phase_info<CHAIN>(a, p, (SrcInfo *)(lds + LDS_SRC_OFF), *(NormHdr *)(lds + LDS_NORM_OFF));
}

// Staging of the phase's inputs as BF16 x-hat in LDS (FP32 statistics): all
// input chunks are requested at once (one memory round trip) together with the
// epilogue's bias/residual values, then the statistics and the normalisation
// run out of LDS.
// Copy the phase's inputs (every batch row of every source, from the source
// table in LDS) into x-hat with coherent LDS-DMA loads, 1 KB per wave
// instruction.  The copies are numbered across sources and batch rows and
// wave w of nw issues every nw-th one; the zero padding of each row's last
// unit is written by the wave with zero_tail.  Asynchronous: the caller waits.
template <int B, bool CHAIN>
__device__ __forceinline__ void issue_source_loads(const KArgs &a, int32_t nsrc, int32_t xb, const char *lds,
                                                   char *xh, uint32_t lane, int32_t w, int32_t nw,
                                                   bool zero_tail) {
    const SrcInfo *T = (const SrcInfo *)(lds + LDS_SRC_OFF);
    const int32_t nb = a.nb;
    // every entry is read at once (one LDS round trip), then the copies issued
    const uint16_t *x[MAX_SRC];
    int64_t xs[MAX_SRC];
    int32_t K[MAX_SRC], lo[MAX_SRC];
#pragma unroll
    for (int j = 0; j < MAX_SRC; ++j) {
        x[j] = T[j].x;
        xs[j] = T[j].x_stride;
        K[j] = T[j].K;
        lo[j] = T[j].lds_off;
    }
    int32_t base = 0;  // copies numbered so far
#pragma unroll
    for (int j = 0; j < MAX_SRC; ++j) {
        if (j >= nsrc) break;
        const uint16_t *src = uniform_ptr(x[j]);
        const int64_t stride = uniform_i64(xs[j]);
        const int32_t n8 = uniform_i32(K[j]) >> 3;
        const int32_t padded8 = nchunks_of(uniform_i32(K[j])) * (UNIT / 8);
        const int32_t off = uniform_i32(lo[j]);
        const int32_t nit = (n8 + 63) >> 6;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (b >= nb) break;
            char *dst = xh + ((size_t)b * xb + off) * 2;
            const uint16_t *sb = src + (int64_t)b * stride;
            int32_t it = w - base % nw;
            if (it < 0) it += nw;
            for (; it < nit; it += nw)
                if (it * 64 + (int32_t)lane < n8)
                    __builtin_amdgcn_global_load_lds((const WGN_GAS void *)(sb + ((size_t)it * 64 + lane) * 8),
                                                     (WGN_LAS void *)(dst + it * 1024), 16, 0, COH);
            base += nit;
            if (zero_tail)
                for (int32_t i = n8 + lane; i < padded8; i += 64) *(u32x4 *)(dst + i * 16) = (u32x4){0u, 0u, 0u, 0u};
        }
    }
}

// While the streaming waves stream, stage the epilogue's inputs of this
// workgroup's rows into LDS.  Row-part rp's record (epi_rec(nb) floats) holds
// the bias, then the residual of each batch row, then the addend of a fused
// residual add of another stage (its FP32 row sums plus its bias).
template <int B, bool CHAIN>
__device__ void stage_epilogue_inputs(const KArgs &a, const RunHdr &h, const Run *runs, float *epi, uint32_t lane) {
    const int32_t nb = a.nb;
    const LaneSplit ls = lane_split(nb, lane);
    const int32_t nruns = uniform_i32(h.nruns);
    for (int32_t ri = 0; ri < nruns; ++ri) {
        const Run &r = runs[ri];
        const uint16_t *bias = uniform_ptr(r.bias);
        const uint16_t *res = uniform_ptr(r.residual);
        const float *pf = uniform_ptr(r.post_F);
        if ((!bias && !res && !pf) || (uniform_i32(r.carry) & CARRY_OUT) || !ls.active) continue;
        const int64_t res_stride = uniform_i64(r.res_stride);
        const int32_t row0 = uniform_i32(r.row0), nrows = uniform_i32(r.nrows), rp_base = uniform_i32(r.rp_base),
                      parts = uniform_i32(r.parts), N = uniform_i32(r.N);
        const uint16_t *pbias = uniform_ptr(r.post_bias);
        const __amdgpu_buffer_rsrc_t rb = rsrc_of(bias), rr = rsrc_of(res), rf = rsrc_of(pf), rpb = rsrc_of(pbias);
        for (int32_t i = ls.i0; i < nrows; i += ls.step) {
            const int32_t n = row0 + i;
            float *e = epi + (size_t)(rp_base + i * parts) * epi_rec(nb);
            // All four loads are issued unconditionally (an absent input has
            // an empty buffer range and reads 0), so they are in flight
            // together.  Bias and post bias are constants (cached loads);
            // residual and addend come from earlier phases (coherent loads).
            const uint32_t bv = __builtin_amdgcn_raw_buffer_load_b16(rb, n * 2, 0, 0);
            const uint32_t rv =
                __builtin_amdgcn_raw_buffer_load_b16(rr, (int)(((int64_t)ls.b * res_stride + n) * 2), 0, COH);
            const uint32_t fv = __builtin_amdgcn_raw_buffer_load_b32(rf, (int)(((int64_t)ls.b * N + n) * 4), 0, COH);
            const uint32_t pv = __builtin_amdgcn_raw_buffer_load_b16(rpb, n * 2, 0, 0);
            if (ls.b == 0) e[0] = bf2f(bv);
            e[1 + ls.b] = bf2f(rv);
            if (pf) e[1 + nb + ls.b] = __uint_as_float(fv) + bf2f(pv);
        }
    }
}

// Merge the per-workgroup argmax keys of one ARGMAX stage (called by the last
// workgroup to arrive) and write the index / maximum outputs.
__device__ void argmax_merge(const KArgs &a, int32_t am_slot, void *y, float *maxval, uint32_t lane) {
    const int32_t nb = a.nb;
    for (int b = 0; b < nb; ++b) {
        uint64_t best = 0;
        for (int32_t gg = lane; gg < a.G; gg += 64) {
            uint64_t k = __hip_atomic_load(&a.am_part[((size_t)am_slot * a.G + gg) * nb + b], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            best = k > best ? k : best;
        }
        best = wave_max_u64(best);
        if (lane == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(0xFFFFFFFFu - (uint32_t)best, rsrc_of(y), b * 4, 0, COH);
            if (maxval)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(unorderable((uint32_t)(best >> 32))),
                                                      rsrc_of(maxval), b * 4, 0, COH);
        }
    }
}

// Row sums of one output row (both parts of a SwiGLU row): the partial slots
// in wave order, after the carry of earlier K windows; kept in the carry when
// this window does not end the row.
template <bool TILE>
__device__ __forceinline__ void row_sums(const RunHdr &h, const Run &r, int32_t i, int32_t b, int32_t nb,
                                         const float *part, float *carry, float (&acc)[2]) {
    const int32_t parts = r.parts, nch = r.nchunks, cy = r.carry;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
        if (pt >= parts) break;
        const int32_t rp = r.rp_base + i * parts + pt;
        const int32_t a0 = first_unit_of_rowpart(r, i, pt, TILE);
        const int32_t span = first_wave_hdr(h, a0 + nch - 1) - first_wave_hdr(h, a0) + 1;
        const float *pp = part + (size_t)rp * h.jmax * nb + b;
        float s = (cy & CARRY_IN) ? carry[rp * nb + b] + pp[0] : pp[0];
        for (int32_t j = 1; j < span; ++j) s += pp[j * nb];
        if (cy & CARRY_OUT) carry[rp * nb + b] = s;
        acc[pt] = s;
    }
}

// Sum the partial slots of every output row, then either carry the sums to
// the next K window or apply the epilogue and store the outputs.  Lane l
// serves batch row l % P of every (64 / P)-th output row of the phase (all of
// its stages at once; P = batch rounded up to a power of two).  Argmax stages
// are reduced afterwards, one at a time.
template <int B, bool CHAIN, bool TILE>
__device__ __forceinline__ void epilogue(const KArgs &a, const RunHdr &h, const Run *runs, int32_t g, const float *part,
                         const float *epi, float *carry, uint32_t lane, int32_t wsel, int32_t nw, bool with_argmax) {
    const int32_t nb = a.nb;
    const LaneSplit ls = lane_split(nb, lane);
    const int32_t b = ls.b;
    // row starts are read from the LDS header: indexing the register copy with
    // a per-lane index would move it to scratch memory
    const int32_t *rstart = ((const RunHdr *)((const char *)runs - sizeof(RunHdr)))->rstart;
    // this wave's share of the output rows: wave wsel of nw (none for nw = 0)
    const int32_t total = ls.active && nw > 0 ? rstart[MAX_RUNS] : 0;
    const int32_t kstep = ls.step * (nw > 0 ? nw : 1);
    for (int32_t k = ls.i0 + ls.step * wsel; k < total; k += kstep) {
        int32_t ri = 0;
#pragma unroll
        for (int32_t j = 1; j < MAX_RUNS; ++j) ri += rstart[j] <= k ? 1 : 0;
        const Run &r = runs[ri];
        const int32_t epi_kind = r.epi;
        if (epi_kind == EPI_ARGMAX) continue;
        const int32_t i = k - rstart[ri];
        const int32_t n = r.row0 + i;
        float acc[2];
        row_sums<TILE>(h, r, i, b, nb, part, carry, acc);
        if (r.carry & CARRY_OUT) continue;
        if (epi_kind == EPI_F32) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[0]), rsrc_of(r.y),
                                                  (int)(((int64_t)b * r.y_stride + n) * 4), 0, COH);
            continue;
        }
        const float *ep = epi + (size_t)(r.rp_base + i * r.parts) * epi_rec(nb);
        const float z = acc[0] + (r.bias ? ep[0] : 0.0f);
        float e;
        if (epi_kind == EPI_GELU_TANH) {
            e = gelu_tanh(z);
            // the pre-activation, kept for the backward pass of the GELU
            if (r.logits)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(z), rsrc_of(r.logits),
                                                      (int)(((int64_t)b * r.N + n) * 4), 0, COH);
        }
        else if (epi_kind == EPI_SWIGLU) e = silu(z) * acc[1];
        else e = z;
        if (r.residual) e += ep[1 + b];
        const uint16_t o = f2bf(e);
        __builtin_amdgcn_raw_buffer_store_b16(o, rsrc_of(r.y), (int)(((int64_t)b * r.y_stride + n) * 2), 0, COH);
        if (r.post_y)
            __builtin_amdgcn_raw_buffer_store_b16(f2bf(bf2f(o) + ep[1 + nb + b]), rsrc_of(r.post_y),
                                                  (int)(((int64_t)b * r.post_stride + n) * 2), 0, COH);
    }
    for (int32_t ri = 0; with_argmax && ri < h.nruns; ++ri) {
        const Run &r = runs[ri];
        if (r.epi != EPI_ARGMAX) continue;
        const int32_t nrows = ls.active ? r.nrows : 0;
        const int32_t N = uniform_i32(r.N), row0 = uniform_i32(r.row0);
        float *logits = uniform_ptr(r.logits);
        uint64_t best = 0;
        for (int32_t i = ls.i0; i < nrows; i += ls.step) {
            const int32_t n = row0 + i;
            float acc[2];
            row_sums<TILE>(h, r, i, b, nb, part, carry, acc);
            if (r.carry & CARRY_OUT) continue;
            const float z = acc[0];
            if (logits)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(z), rsrc_of(logits),
                                                      (int)(((int64_t)b * N + n) * 4), 0, 0);
            const uint64_t key = ((uint64_t)orderable(z) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)n);
            best = key > best ? key : best;
        }
        if (r.carry & CARRY_OUT) continue;
        const int32_t am_slot = r.am_slot;
        // maximum over the lanes serving the same batch row
        for (int32_t o = ls.P; o < 64; o <<= 1) {
            const uint64_t t = __shfl_xor(best, o);
            best = t > best ? t : best;
        }
        if ((int32_t)lane < nb)
            __hip_atomic_store(&a.am_part[((size_t)am_slot * a.G + g) * nb + lane], best, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        // the partial keys are agent-scope atomic stores; once they have
        // completed, the ticket tells the last workgroup to merge them
        __builtin_amdgcn_s_waitcnt(0);
        uint32_t old = 0;
        if (lane == 0)
            old = __hip_atomic_fetch_add(&a.tickets[am_slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0);
        if (old == (uint32_t)(a.G - 1)) {
            argmax_merge(a, am_slot, uniform_ptr(r.y), uniform_ptr(r.maxval), lane);
            if (lane == 0)
                __hip_atomic_store(&a.tickets[am_slot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Argmax stages of a phase, with every wave of the workgroup taking part:
// each wave reduces its share of the rows to one key per batch row, posts it
// in LDS (the normalisation statistics area, idle at this point of a phase),
// and after a barrier the control wave combines the waves' keys in wave order
// and publishes the workgroup's key as in the single-wave epilogue.  All
// waves pass the same two barriers per argmax stage.
template <bool TILE>
__device__ __forceinline__ void argmax_shared(const KArgs &a, const RunHdr &h, const Run *runs, int32_t g,
                                              const float *part, float *carry, char *lds, uint32_t lane, int32_t w) {
    static_assert(WAVES * MAX_BATCH * 8 <= WAVES * STATS_ROWS * 16, "argmax keys fit the statistics area");
    uint64_t *keys = (uint64_t *)(lds + LDS_STATS_OFF);
    const int32_t nb = a.nb;
    const LaneSplit ls = lane_split(nb, lane);
    const int32_t b = ls.b;
    const int32_t nr = uniform_i32(h.nruns);
    for (int32_t ri = 0; ri < nr; ++ri) {
        const Run &r = runs[ri];
        if (uniform_i32(r.epi) != EPI_ARGMAX) continue;
        const bool co = (uniform_i32(r.carry) & CARRY_OUT) != 0;
        const int32_t nrows = ls.active ? r.nrows : 0;
        const int32_t N = uniform_i32(r.N), row0 = uniform_i32(r.row0);
        float *logits = uniform_ptr(r.logits);
        uint64_t best = 0;
        for (int32_t i = ls.i0 + ls.step * w; i < nrows; i += ls.step * WAVES) {
            const int32_t n = row0 + i;
            float acc[2];
            row_sums<TILE>(h, r, i, b, nb, part, carry, acc);
            if (co) continue;
            const float z = acc[0];
            if (logits)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(z), rsrc_of(logits),
                                                      (int)(((int64_t)b * N + n) * 4), 0, 0);
            const uint64_t key = ((uint64_t)orderable(z) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)n);
            best = key > best ? key : best;
        }
        // maximum over the lanes serving the same batch row
        for (int32_t o = ls.P; o < 64; o <<= 1) {
            const uint64_t t = __shfl_xor(best, o);
            best = t > best ? t : best;
        }
        if (!co && (int32_t)lane < nb) keys[w * nb + (int32_t)lane] = best;
        wg_barrier();  // every wave's keys are posted
        if (w == STREAM_WAVES && !co) {
            const int32_t am_slot = uniform_i32(r.am_slot);
            uint64_t k = 0;
            if ((int32_t)lane < nb)
                for (int32_t ww = 0; ww < WAVES; ++ww) {
                    const uint64_t t = keys[ww * nb + (int32_t)lane];
                    k = t > k ? t : k;
                }
            if ((int32_t)lane < nb)
                __hip_atomic_store(&a.am_part[((size_t)am_slot * a.G + g) * nb + lane], k, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            // the partial keys are agent-scope atomic stores; once they have
            // completed, the ticket tells the last workgroup to merge them
            __builtin_amdgcn_s_waitcnt(0);
            uint32_t old = 0;
            if (lane == 0)
                old = __hip_atomic_fetch_add(&a.tickets[am_slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            old = __shfl(old, 0);
            if (old == (uint32_t)(a.G - 1)) {
                argmax_merge(a, am_slot, uniform_ptr(r.y), uniform_ptr(r.maxval), lane);
                if (lane == 0)
                    __hip_atomic_store(&a.tickets[am_slot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        wg_barrier();  // the keys area may be reused
    }
}

// Write phase q's run list for workgroup g into its LDS buffer: a copy of the
// precomputed list for chains (asynchronous: memory to LDS), else built here.
template <bool CHAIN, bool TILE, int R>
__device__ void build_runs(const KArgs &a, int32_t q, int32_t g, char *desc, uint32_t lane) {
    char *buf = desc + (q & (desc_bufs_k(TILE, R) - 1)) * RUN_BUF_STRIDE;
    if (CHAIN && a.runimg) {
        copy_to_lds<0>((const uint16_t *)(a.runimg + ((size_t)q * a.G + g) * RUN_BUF_STRIDE), buf, RUN_BUF_STRIDE / 16,
                       lane);
        return;
    }
    // every lane computes the same list; the runs go straight into LDS
    // the header is built in place too: its tables are indexed at run time,
    // which a register copy could only do through scratch memory
    make_runs<CHAIN>(a, q, g, TILE, *(RunHdr *)buf, (Run *)(buf + sizeof(RunHdr)));
}

// A later phase's precomputed run list and phase info, read into registers
// while the streaming waves consume and written to LDS after the flag store.
constexpr int RL_CHUNKS = RUN_BUF_STRIDE / 16, PI_CHUNKS = PHASE_INFO_BYTES / 16;
static_assert(RL_CHUNKS <= 128 && PI_CHUNKS <= 64, "two reads per lane for a run list, one for a phase info");
struct AheadRegs {
    u32x4 rl0, rl1, pi;
};
__device__ __forceinline__ void ahead_load(const KArgs &a, int32_t q_rl, int32_t q_pi, int32_t g, uint32_t lane,
                                           AheadRegs &r) {
    if (q_rl < a.p1) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.runimg + ((size_t)q_rl * a.G + g) * RUN_BUF_STRIDE), (short)0, RUN_BUF_STRIDE, (int)RSRC_W3);
        r.rl0 = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(lane * 16), 0, 0);
        r.rl1 = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((64 + lane) * 16), 0, 0);  // past the end: 0
    }
    if (q_pi < a.p1) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.phinfo + (size_t)q_pi * PHASE_INFO_BYTES), (short)0, PHASE_INFO_BYTES, (int)RSRC_W3);
        r.pi = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(lane * 16), 0, 0);
    }
}
template <bool TILE, int R>
__device__ __forceinline__ void ahead_store(const KArgs &a, int32_t q_rl, int32_t q_pi, char *lds, uint32_t lane,
                                            const AheadRegs &r) {
    if (q_rl < a.p1) {
        char *buf = lds + LDS_DESC_OFF + (q_rl & (desc_bufs_k(TILE, R) - 1)) * RUN_BUF_STRIDE;
        *(u32x4 *)(buf + lane * 16) = r.rl0;
        if ((int32_t)lane + 64 < RL_CHUNKS) *(u32x4 *)(buf + (64 + lane) * 16) = r.rl1;
    }
    if (q_pi < a.p1 && (int32_t)lane < PI_CHUNKS) {
        constexpr int32_t nt = MAX_SRC * (int)sizeof(SrcInfo) / 16;
        char *dst = (int32_t)lane < nt ? lds + LDS_SRC_OFF + lane * 16 : lds + LDS_NORM_OFF + (lane - nt) * 16;
        *(u32x4 *)dst = r.pi;
    }
}

// ------------------------------------------------------- attention phases
// Run by the control wave in place of a product phase's input copies and
// normalisation; the phase streams no weights, so the streaming waves only
// meet its barriers (its weights-ahead walk continues past it).  q, k_new and
// v_new were written earlier in the same launch: read at the coherent level.

// Maximum / sum over the 64 lanes by DPP (rows, then the row broadcasts into
// lane 63), read back from lane 63 into a scalar register: every lane gets
// the same value, with no LDS permute on the path.
__device__ __forceinline__ float wave_max_bcast(float v) {
    const int ninf = (int)0xFF800000u;
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x142, 0xA, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x143, 0xC, 0xF, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sum_last(v)), 63));
}

// Position of batch row b's new token, read through the scalar cache (a
// value written before the launch): no vector-memory round trip.
__device__ __forceinline__ int32_t attn_last(const DevAttn &A, int32_t b) {
    const int32_t p0 = WGN_CONST_PTR(int32_t, A.pos)[b];
    return (p0 >= 0 && p0 < A.slots) ? p0 : -1;
}
// Slots per chunk of a row whose last valid slot is last >= 0: its valid
// length split over the row's nchunk partials, in whole passes (the same in
// both phases, so the merge finds the chunks the scores phase filled).
template <int PASS>
__device__ __forceinline__ int32_t attn_chunk(const DevAttn &A, int32_t last) {
    const int32_t c = (last + A.nchunk) / A.nchunk;  // ceil((last + 1) / nchunk)
    return (c + PASS - 1) / PASS * PASS;
}

// The scores item of this workgroup and the first pass of its cache rows,
// copied into LDS (stage: 4 key then 4 value copies of 1 KB, lane l's 16
// bytes at l * 16) before the wait for the previous phase: the cache does not
// depend on it, and the copies hold no registers across the wait.  Row r of
// 16 lanes takes slots t + 4 i + r (i < 4), lane col of a row holds
// dimensions 8 col .. 8 col + 7; slots past the chunk or the last valid slot
// re-read the last valid one (never beyond it) and get weight 0.  The new
// token's slot is read here too and replaced after the wait.
template <int NL>
__device__ __forceinline__ void attn_prefetch(const DevAttn &A, int32_t nb, int32_t g, uint32_t lane, char *stage) {
    const int32_t r = (int32_t)(lane >> 4);
    const uint32_t lo = (lane & 15u) * 16u;
    const int32_t items = nb * A.hkv * A.nchunk;
    if (g >= items) return;
    const int32_t pair = g / A.nchunk, c = g - pair * A.nchunk;
    const int32_t last = attn_last(A, pair / A.hkv);
    if (last < 0) return;  // no valid slot: nothing is scored
    const int32_t t0 = c * attn_chunk<4 * NL>(A, last);
    if (t0 > last) return;
    const char *kc = (const char *)(A.k_cache + (size_t)pair * A.slots * ATTN_D);
    const char *vc = (const char *)(A.v_cache + (size_t)pair * A.slots * ATTN_D);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const size_t off = (size_t)min(t0 + 4 * i + r, last) * ATTN_D * 2 + lo;
        __builtin_amdgcn_global_load_lds((const WGN_GAS void *)(kc + off), (WGN_LAS void *)(stage + i * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const WGN_GAS void *)(vc + off), (WGN_LAS void *)(stage + (4 + i) * 1024), 16, 0,
                                         0);
    }
}

// Scores phase: this workgroup's (batch row, key/value head, chunk) item
// (one per workgroup as planned; further items, if any, load their rows
// here).  Online softmax per query head over the passes; the four rows of
// the wave are combined through LDS (cmb: [row][head][D] FP32, then m and l
// per (row, head)) in row order, and one partial is written: acc[G][D],
// m[G], l[G].
template <int NL>
__device__ __forceinline__ void attn_scores(const DevAttn &A, int32_t nb, int32_t g, int32_t G, uint32_t lane,
                                            float *cmb, const char *stage) {
    const int32_t grp = A.hq / A.hkv, E = attn_part_floats(grp);
    const int32_t r = (int32_t)(lane >> 4), col = (int32_t)(lane & 15);
    const int32_t items = nb * A.hkv * A.nchunk;
    const uint32_t lo = (uint32_t)col * 16u;  // this lane's byte offset inside a 256-byte row
    for (int32_t it = g; it < items; it += G) {
        const int32_t pair = it / A.nchunk, c = it - pair * A.nchunk;
        const int32_t b = pair / A.hkv, kh = pair - b * A.hkv;
        const int32_t last = attn_last(A, b);
        if (last < 0) continue;  // no valid slot: the merge writes zeros
        const int32_t chunk = attn_chunk<4 * NL>(A, last);
        const int32_t t0 = c * chunk;
        if (t0 > last) continue;  // past the valid slots: the merge skips this chunk
        const int32_t t1 = min(t0 + chunk, last + 1);
        const __amdgpu_buffer_rsrc_t rkc = rsrc_of(A.k_cache + (size_t)pair * A.slots * ATTN_D);
        const __amdgpu_buffer_rsrc_t rvc = rsrc_of(A.v_cache + (size_t)pair * A.slots * ATTN_D);
        // the group's query rows into LDS (4 heads of 256 bytes per copy),
        // requested with the new key and value: one round trip for all
        const char *qg = (const char *)(A.q + (size_t)b * A.q_stride + (size_t)kh * grp * ATTN_D);
        char *qs = (char *)cmb + ATTN_Q_OFF;
#pragma unroll
        for (int i = 0; i < ATTN_MAX_GROUP / 4; ++i)
            if (4 * i + r < grp)
                __builtin_amdgcn_global_load_lds((const WGN_GAS void *)(qg + (size_t)(4 * i + r) * ATTN_D * 2 + lo),
                                                 (WGN_LAS void *)(qs + i * 1024), 16, 0, COH);
        const __amdgpu_buffer_rsrc_t rkn = rsrc_of(A.k_new + (size_t)b * A.k_stride + (size_t)kh * ATTN_D);
        const __amdgpu_buffer_rsrc_t rvn = rsrc_of(A.v_new + (size_t)b * A.v_stride + (size_t)kh * ATTN_D);
        const u32x4 kn = __builtin_amdgcn_raw_buffer_load_b128(rkn, (int)lo, 0, COH);
        const u32x4 vn = __builtin_amdgcn_raw_buffer_load_b128(rvn, (int)lo, 0, COH);
        // the group's query heads HS at a time (registers), each sweep over
        // every pass of the chunk; the first pass comes from the staged copies
        constexpr int HS = 4;
        __builtin_amdgcn_s_waitcnt(0);  // query rows (and the staged cache rows) have landed
        for (int32_t h0 = 0; h0 < grp; h0 += HS) {
            u32x4 qv[HS];
            float m[HS], l[HS], acc[HS][8];
#pragma unroll
            for (int h = 0; h < HS; ++h) {
                const int32_t hh = h0 + h < grp ? h0 + h : 0;  // in range; heads past the group are never used
                qv[h] = *(const u32x4 *)(qs + hh * ATTN_D * 2 + lo);
                m[h] = -INFINITY;
                l[h] = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[h][j] = 0.0f;
            }
            for (int32_t t = t0; t < t1; t += 4 * NL) {
                u32x4 kd[NL], vd[NL];
                if (it == g && t == t0) {
                    __builtin_amdgcn_s_waitcnt(0);  // the copies into stage have landed
#pragma unroll
                    for (int i = 0; i < NL; ++i) {
                        kd[i] = *(const u32x4 *)(stage + i * 1024 + lane * 16);
                        vd[i] = *(const u32x4 *)(stage + (4 + i) * 1024 + lane * 16);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < NL; ++i) {
                        const uint32_t sl = (uint32_t)min(t + 4 * i + r, last);
                        kd[i] = __builtin_amdgcn_raw_buffer_load_b128(rkc, (int)(sl * ATTN_D * 2u + lo), 0, 0);
                        vd[i] = __builtin_amdgcn_raw_buffer_load_b128(rvc, (int)(sl * ATTN_D * 2u + lo), 0, 0);
                    }
                }
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    if (min(t + 4 * i + r, last) == last) {  // the new token: from k_new / v_new
                        kd[i] = kn;
                        vd[i] = vn;
                    }
                }
#pragma unroll
                for (int h = 0; h < HS; ++h) {
                    if (h0 + h >= grp) break;
                    float sc[NL], mx = m[h];
#pragma unroll
                    for (int i = 0; i < NL; ++i) {
                        const float sv = group_sum(dot8(kd[i], qv[h], 0.0f), 16) * A.scale_log2;
                        sc[i] = t + 4 * i + r < t1 ? sv : -INFINITY;
                        mx = fmaxf(mx, sc[i]);
                    }
                    if (mx != -INFINITY) {  // this row has seen a valid slot
                        const float alpha = __builtin_amdgcn_exp2f(m[h] - mx);
                        float pw[NL], lw = 0.0f;
#pragma unroll
                        for (int i = 0; i < NL; ++i) {
                            pw[i] = __builtin_amdgcn_exp2f(sc[i] - mx);
                            lw += pw[i];
                        }
                        l[h] = l[h] * alpha + lw;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            float e0 = acc[h][2 * j] * alpha, e1 = acc[h][2 * j + 1] * alpha;
#pragma unroll
                            for (int i = 0; i < NL; ++i) {
                                const uint32_t vw = j == 0 ? vd[i].x : j == 1 ? vd[i].y : j == 2 ? vd[i].z : vd[i].w;
                                e0 += pw[i] * bf2f(vw & 0xFFFFu);
                                e1 += pw[i] * bf2f(vw >> 16);
                            }
                            acc[h][2 * j] = e0;
                            acc[h][2 * j + 1] = e1;
                        }
                        m[h] = mx;
                    }
                }
                // the append (first sweep): the row holding the new token's
                // slot stores it (no workgroup reads that slot from the cache
                // in this launch)
                if (h0 == 0) {
#pragma unroll
                    for (int i = 0; i < NL; ++i) {
                        if (t + 4 * i + r == last) {
                            __builtin_amdgcn_raw_buffer_store_b128(kd[i], rkc, (int)((uint32_t)last * ATTN_D * 2u + lo),
                                                                   0, 0);
                            __builtin_amdgcn_raw_buffer_store_b128(vd[i], rvc, (int)((uint32_t)last * ATTN_D * 2u + lo),
                                                                   0, 0);
                        }
                    }
                }
            }
            // this sweep's rows into LDS, to be combined in row order below
#pragma unroll
            for (int h = 0; h < HS; ++h) {
                if (h0 + h >= grp) break;
                const int32_t hh = h0 + h;
                float *dst = cmb + ((r * ATTN_MAX_GROUP + hh) * ATTN_D + col * 8);
                *(f32x4 *)dst = (f32x4){acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
                *(f32x4 *)(dst + 4) = (f32x4){acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
                if (col == 0) {
                    cmb[4 * ATTN_MAX_GROUP * ATTN_D + r * ATTN_MAX_GROUP + hh] = m[h];
                    cmb[4 * ATTN_MAX_GROUP * ATTN_D + 4 * ATTN_MAX_GROUP + r * ATTN_MAX_GROUP + hh] = l[h];
                }
            }
        }
        const __amdgpu_buffer_rsrc_t rp = rsrc_of(A.part + ((size_t)pair * A.nchunk + c) * E);
#pragma unroll
        for (int k = 0; k < ATTN_MAX_GROUP / 2; ++k) {
            const int32_t q4 = (int32_t)lane + 64 * k;  // float4 group: head q4 / 32, dimensions 4 (q4 % 32) ..
            if (q4 >= grp * (ATTN_D / 4)) break;
            const int32_t h = q4 >> 5, d0 = (q4 & 31) * 4;
            float mr[4], lr[4], M = -INFINITY;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                mr[rr] = cmb[4 * ATTN_MAX_GROUP * ATTN_D + rr * ATTN_MAX_GROUP + h];
                lr[rr] = cmb[4 * ATTN_MAX_GROUP * ATTN_D + 4 * ATTN_MAX_GROUP + rr * ATTN_MAX_GROUP + h];
                M = fmaxf(M, mr[rr]);  // finite: row 0 holds slot t0 <= last
            }
            f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
            float L = 0.0f;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float f = __builtin_amdgcn_exp2f(mr[rr] - M);
                o += f * *(const f32x4 *)(cmb + ((rr * ATTN_MAX_GROUP + h) * ATTN_D + d0));
                L += f * lr[rr];
            }
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rp, (h * ATTN_D + d0) * 4, 0, COH);
            if (d0 == 0) {
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(M), rp, (grp * ATTN_D + h) * 4, 0, COH);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(L), rp, (grp * ATTN_D + grp + h) * 4, 0, COH);
            }
        }

    }
}

// Merge phase: items (batch row, query head, SL-dimension slice) spread over
// the workgroups.  Lane i folds the partials of chunks i, i + 64, ... in that
// order (running maximum), then the wave combines its lanes in a fixed order;
// lanes 0 .. SL/2 - 1 store the SL BF16 outputs.  A row with no valid slot
// gets 0.
template <int SL, int PASS>
__device__ __forceinline__ void attn_merge(const DevAttn &A, int32_t nb, int32_t g, int32_t G, uint32_t lane,
                                           int32_t last_g) {
    constexpr int NSL = ATTN_D / SL;
    const int32_t grp = A.hq / A.hkv, E = attn_part_floats(grp);
    const int32_t items = nb * A.hq * NSL;
    for (int32_t it = g; it < items; it += G) {
        const int32_t b = it / (A.hq * NSL), rem = it - b * A.hq * NSL;
        const int32_t hq = rem / NSL, ds = rem - hq * NSL;
        const int32_t kh = hq / grp, hi = hq - kh * grp, pair = b * A.hkv + kh;
        const int32_t last = it == g ? last_g : attn_last(A, b);
        const int32_t nvalid = last < 0 ? 0 : last / attn_chunk<PASS>(A, last) + 1;  // chunks holding a valid slot
        const __amdgpu_buffer_rsrc_t rp = rsrc_of(A.part + (size_t)pair * A.nchunk * E);
        float mm = -INFINITY, ll = 0.0f, aa[SL];
#pragma unroll
        for (int j = 0; j < SL; ++j) aa[j] = 0.0f;
        for (int32_t i0 = (int32_t)lane; i0 < nvalid; i0 += 128) {
            // the partials of chunks i0 and i0 + 64, both requested before
            // either is folded (one round trip), folded in that order
            float mi[2], li[2];
            u32x4 av[2][SL / 4];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bool ok = i0 + 64 * u < nvalid;
                const int32_t base = (ok ? i0 + 64 * u : i0) * E;  // in range; unused when !ok
                mi[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, (base + grp * ATTN_D + hi) * 4, 0, COH));
                li[u] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rp, (base + grp * ATTN_D + grp + hi) * 4, 0, COH));
#pragma unroll
                for (int k = 0; k < SL / 4; ++k)
                    av[u][k] = __builtin_amdgcn_raw_buffer_load_b128(rp, (base + hi * ATTN_D + ds * SL + 4 * k) * 4,
                                                                     0, COH);
                if (!ok) {
                    mi[u] = -INFINITY;
                    li[u] = 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float M = fmaxf(mm, mi[u]);  // finite: chunk i0 is valid
                const float f0 = __builtin_amdgcn_exp2f(mm - M), f1 = __builtin_amdgcn_exp2f(mi[u] - M);
                ll = ll * f0 + li[u] * f1;
#pragma unroll
                for (int k = 0; k < SL / 4; ++k) {
                    const f32x4 v = __builtin_bit_cast(f32x4, av[u][k]);
                    aa[4 * k] = aa[4 * k] * f0 + v.x * f1;
                    aa[4 * k + 1] = aa[4 * k + 1] * f0 + v.y * f1;
                    aa[4 * k + 2] = aa[4 * k + 2] * f0 + v.z * f1;
                    aa[4 * k + 3] = aa[4 * k + 3] * f0 + v.w * f1;
                }
                mm = M;
            }
        }
        const float M = wave_max_bcast(mm);
        const float f = mm == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mm - M);
        const float L = wave_sum_bcast(ll * f);
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < SL / 2; ++j) {
            const float o0 = wave_sum_bcast(aa[2 * j] * f), o1 = wave_sum_bcast(aa[2 * j + 1] * f);
            const uint32_t w2 = L > 0.0f ? f2bf2(o0 / L, o1 / L) : 0u;
            word = lane == (uint32_t)j ? w2 : word;
        }
        if (lane < (uint32_t)(SL / 2))
            __builtin_amdgcn_raw_buffer_store_b32(
                word, rsrc_of(A.out + (size_t)b * A.out_stride + (size_t)hq * ATTN_D + ds * SL),
                (int)(lane * 4u), 0, COH);
    }
}

__device__ __forceinline__ const DevAttn attn_of(const KArgs &a, int32_t att) {
    return WGN_CONST_PTR(DevAttn, a.att)[(att - 1) >> 1];
}
__device__ __forceinline__ bool attn_is_scores(int32_t att) { return ((att - 1) & 1) == 0; }

template <int B, bool CHAIN, bool TILE, int R, bool ATT>
__device__ __forceinline__ void control_wave(const KArgs &a, int32_t g, char *lds) {
    const uint32_t lane = lane_id();
    char *desc = lds + LDS_DESC_OFF;
    // A wait of an earlier run that gave up leaves the error word set and the
    // flags and tickets of that run behind: until wgn_chain_check has cleared
    // them, every launch exits at once and writes nothing.
    const uint32_t prior = a.persistent ? __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    if (a.trace && lane < 12) ((uint64_t *)(lds + LDS_TRACE_OFF))[lane] = 0;
    const uint32_t flag_val =
        a.persistent ? __hip_atomic_load(a.run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u : 0u;
    // Run lists: phase q's list is written at the end of iteration
    // q - AH, after the flag store, into one of NBUF LDS buffers (the one an
    // earlier phase used, which every wave has finished with by then); AH is
    // the ring's block buffers + 2 (4 for two buffers).  With two buffers a
    // streaming wave may, right after phase q's partials barrier, load phase
    // q+2's block and read phase q+3's list header; that list was written
    // before the x-hat barrier of phase q.  A phase's source table and
    // normalisation jobs are written at the end of the iteration before it.
    // (This schedule is modelled and checked on the host by
    // tests/test_schedule.py.)  From batch 2 up, chains read precomputed
    // lists and tables into registers while the streaming waves consume, so
    // none of this is on the path between a phase's flags and its x-hat; at
    // batch 1 the flags arrive later than the lists are built here, and the
    // reads would only add latency to the flag stores.
    constexpr int AH = desc_ahead(R), NBUF = desc_bufs_k(TILE, R);
    static_assert(NBUF <= path_desc_bufs(TILE), "the planner leaves room for this many run lists");
    for (int32_t q = a.p0; q < a.p1 && q < a.p0 + AH; ++q) build_runs<CHAIN, TILE, R>(a, q, g, desc, lane);
    write_phase_info<CHAIN>(a, a.p0, lds, lane);
    if (lane == 0) abort_flag_set(prior != 0u ? 1 : 0);
    __builtin_amdgcn_s_waitcnt(0);  // copied lists and tables have landed
    wg_barrier();
    if (prior != 0u) return;  // the streaming waves see the abort flag after this barrier
    const bool pre = CHAIN && a.runimg && a.phinfo;
    for (int32_t p = a.p0; p < a.p1; ++p) {
        const DevPhase ph = phase_of<CHAIN>(a, p);
        char *xh = lds + ph.x_off;
        const float *part = (const float *)(lds + ph.part_off);
        float *epi = (float *)(lds + ph.epi_off);
        float *carry = (float *)(lds + ph.carry_off);
        trace_point(a, p, g, 0, lane);
        const char *rb = desc + (p & (NBUF - 1)) * RUN_BUF_STRIDE;
        const RunHdr &h = *(const RunHdr *)rb;  // in LDS (a register copy passed by reference would go to scratch)
        const Run *runs = (const Run *)(rb + sizeof(RunHdr));
        // the gains do not depend on the previous phase: request them before
        // waiting for it (and an attention item's first cache rows)
        prefetch_params(ph, lds, lane);
        // (a merge item's descriptor and position are read here too: two
        // dependent scalar-cache misses off the path after the wait)
        int32_t att_last = -1;
        if constexpr (ATT) {
            if (ph.att) {
                const DevAttn A = attn_of(a, ph.att);
                if (attn_is_scores(ph.att))
                    attn_prefetch<attn_pass(B) / 4>(A, a.nb, g, lane, lds + ph.part_off + ATTN_STAGE_OFF);
                else if (g < a.nb * A.hq * (ATTN_D / attn_slice(B))) att_last = attn_last(A, g / (A.hq * (ATTN_D / attn_slice(B))));
            }
        }
        if (a.persistent && p > a.p0 && ph.wait) {
            // every workgroup's flag of phase p-1 must carry this run's value
            const __amdgpu_buffer_rsrc_t rf = rsrc_of(a.flags + (size_t)(p - 1) * flag_row(a.G));
            const uint64_t t0 = wall_clock64();
            bool timed_out = false;
            if (POLL_DELAY > 0) __builtin_amdgcn_s_sleep(POLL_DELAY);
            if (FLAG_WORDS == 1) {
                for (;;) {
                    bool ok = true;
                    for (int32_t i = (int32_t)lane * 4; i < a.G; i += 256) {
                        const u32x4 f = __builtin_amdgcn_raw_buffer_load_b128(rf, i * 4, 0, COH);
                        const uint32_t ff[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) ok &= (i + e >= a.G) || ff[e] == flag_val;
                    }
                    if (__all(ok)) break;
                    if (wall_clock64() - t0 > a.wait_ticks) {
                        timed_out = true;
                        break;
                    }
                    // every workgroup polls the same few lines: spacing the
                    // reads out keeps them from slowing the flag stores
                    if (POLL_GAP > 0) __builtin_amdgcn_s_sleep(POLL_GAP);
                }
            } else {
                // lane l watches flags l, l + 64, ... and re-reads only those
                // it has not seen yet
                const int32_t mine = a.G > (int32_t)lane ? (a.G - (int32_t)lane + 63) / 64 : 0;
                const uint32_t need = mine >= 32 ? 0xFFFFFFFFu : (1u << mine) - 1u;
                uint32_t seen = 0;
                for (;;) {
                    for (int32_t k = 0; k < mine; ++k)
                        if (!(seen & (1u << k)) &&
                            __builtin_amdgcn_raw_buffer_load_b32(rf, ((int32_t)lane + 64 * k) * FLAG_WORDS * 4, 0, COH) ==
                                flag_val)
                            seen |= 1u << k;
                    if (__all((seen & need) == need)) break;
                    if (wall_clock64() - t0 > a.wait_ticks) {
                        timed_out = true;
                        break;
                    }
                }
            }
            if (timed_out) {
                if (lane == 0) {
                    abort_flag_set(1);
                    __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                // meet the streaming waves at this phase's barriers (input
                // copies, norm steps, x-hat); they then see the abort flag and
                // exit
                if (in_share<TILE, R>() && h.share_in) wg_barrier();
                if (h.has_norm) {
                    // the barriers of norm_all
                    wg_barrier();
                    if constexpr (!norm_one_wave<B>()) wg_barrier();
                }
                wg_barrier();
                __builtin_amdgcn_s_waitcnt(0);  // the gain copies issued before the wait
                return;
            }
        }
        trace_point(a, p, g, 1, lane);
        if (in_share<TILE, R>() && h.share_in) {
            wg_barrier();  // the flags have been seen: every wave copies its share of the inputs
            issue_source_loads<B, CHAIN>(a, ph.nsrc, ph.xb, lds, xh, lane, STREAM_WAVES, WAVES, true);
        } else {
            issue_source_loads<B, CHAIN>(a, ph.nsrc, ph.xb, lds, xh, lane, 0, 1, true);
        }
        if constexpr (ATT) {
            if (ph.att) {
                if (attn_is_scores(ph.att))
                    attn_scores<attn_pass(B) / 4>(attn_of(a, ph.att), a.nb, g, a.G, lane, (float *)(lds + ph.part_off),
                                lds + ph.part_off + ATTN_STAGE_OFF);
                else attn_merge<attn_slice(B), attn_pass(B)>(attn_of(a, ph.att), a.nb, g, a.G, lane, att_last);
                // The phase streams no weights, but its empty blocks still
                // read x-hat (and multiply it by zero weights): zeros, not
                // whatever an earlier phase left in LDS, which read as BF16
                // may be a NaN pattern.
                for (int32_t i = (int32_t)lane; i < a.nb * ph.xb / 8; i += 64)
                    *(u32x4 *)(xh + i * 16) = (u32x4){0u, 0u, 0u, 0u};
            }
        }
        stage_epilogue_inputs<B, CHAIN>(a, h, runs, epi, lane);
        __builtin_amdgcn_s_waitcnt(0);  // inputs, gains and epilogue values have landed
        if (h.has_norm) norm_all<B>(lds, STREAM_WAVES, lane);
        trace_point(a, p, g, 2, lane);
        wg_barrier();  // x-hat ready
        // later phases' run list and tables, read while the streaming waves consume
        AheadRegs ahead;
        if (pre) {
            ahead_load(a, p + AH, p + 1, g, lane, ahead);
        } else if constexpr (build_in_window(TILE, R)) {
            // phase p + AH's run list and phase p + 1's tables, built while
            // the streaming waves consume (phase p's own list and tables are
            // not touched: its norm is done and the ring has 8 lists)
            if (p + AH < a.p1) build_runs<CHAIN, TILE, R>(a, p + AH, g, desc, lane);
            if (p + 1 < a.p1) write_phase_info<CHAIN>(a, p + 1, lds, lane);
        }
        wg_barrier();  // partials complete
        trace_point(a, p, g, 3, lane);
        if (a.trace && lane < 6) {
            uint64_t *tl = (uint64_t *)(lds + LDS_TRACE_OFF);
            a.trace[((size_t)p * a.G + g) * TRACE_POINTS + 6 + lane] = tl[(p & 1) * 6 + lane];
            if (lane >= 3) tl[(p & 1) * 6 + lane] = 0;  // per-block slots: cleared for phase p + 2
        }
        if constexpr (epi_share<B, TILE, R>()) {
            // every wave stores its share of the rows and waits for its own
            // stores; after the barrier all of them have completed
            epilogue<B, CHAIN, TILE>(a, h, runs, g, part, epi, carry, lane, STREAM_WAVES, WAVES, false);
            argmax_shared<TILE>(a, h, runs, g, part, carry, lds, lane, STREAM_WAVES);
            __builtin_amdgcn_s_waitcnt(0);
            trace_point(a, p, g, 4, lane);
            wg_barrier();  // every wave's stores have completed: the streaming waves may refill
        } else {
            if constexpr (!TILE && R == 0 && !CHAIN) {
                epilogue<B, CHAIN, TILE>(a, h, runs, g, part, epi, carry, lane, 0, 1, false);
                argmax_shared<false>(a, h, runs, g, part, carry, lds, lane, STREAM_WAVES);
            } else {
                epilogue<B, CHAIN, TILE>(a, h, runs, g, part, epi, carry, lane, 0, 1, true);
            }
            trace_point(a, p, g, 4, lane);
            if (epi_barrier<TILE, R>() && EPI_BARRIER == 1) wg_barrier();  // stores issued: the streaming waves may refill
        }
        if (a.persistent) {
            // outputs are written through (coherent stores); once they have
            // completed, publish this workgroup's flag for phase p
            __builtin_amdgcn_s_waitcnt(0);
            if (lane == 0)
                __builtin_amdgcn_raw_buffer_store_b32(flag_val, rsrc_of(a.flags + (size_t)p * flag_row(a.G)),
                                                      g * FLAG_WORDS * 4, 0, COH);
        }
        if (epi_barrier<TILE, R>() && EPI_BARRIER == 2) wg_barrier();  // flag issued too
        trace_point(a, p, g, 5, lane);
        if (pre) {
            ahead_store<TILE, R>(a, p + AH, p + 1, lds, lane, ahead);
        } else if constexpr (!build_in_window(TILE, R)) {
            if (p + AH < a.p1) build_runs<CHAIN, TILE, R>(a, p + AH, g, desc, lane);
            if (p + 1 < a.p1) write_phase_info<CHAIN>(a, p + 1, lds, lane);
        }
    }
    if (a.persistent) {
        // The last workgroup to finish advances the run counter, so the next
        // run (or graph replay) publishes flags with a new value; every other
        // workgroup is past all of its waits by then.
        __builtin_amdgcn_s_waitcnt(0);
        uint32_t old = 0;
        if (lane == 0)
            old = __hip_atomic_fetch_add(&a.tickets[a.n_argmax], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0);
        if (old == (uint32_t)(a.G - 1) && lane == 0) {
            __hip_atomic_store(a.run, flag_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.tickets[a.n_argmax], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int B, bool CHAIN, bool TILE, int R, bool ATT>
__global__ __launch_bounds__(THREADS, 1) void chain_kernel(KArgs a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int32_t g = blockIdx.x;
    const int32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w < STREAM_WAVES) {
        if constexpr (!TILE && ring_interleaved(R)) stream_wave_il<B, CHAIN, R>(a, g, w, lds);
        else stream_wave<B, CHAIN, TILE, R>(a, g, w, lds);
    }
    else control_wave<B, CHAIN, TILE, R, ATT>(a, g, lds);
}

// ------------------------------------------------------------- touch pass
// Optional prefetch of a later launch's weights into the memory-side
// Infinity Cache (256 MB), run on a second stream while the current launch
// streams its own weights: the side-stream prefetch of "Making small PyTorch
// ops faster on a laptop GPU", section "Prefetching the next layer while this
// one runs", with the GPU's last-level cache in the place of L2.  Plain
// (allocating) 128-bit loads of the leading frac_q16 / 65536 of every range;
// the values only meet in a register, so the pass writes no memory at all.
__global__ __launch_bounds__(256) void touch_kernel(const TouchRange *r, int32_t n, uint32_t frac_q16) {
    const uint64_t nt = (uint64_t)gridDim.x * 256;
    const uint64_t tid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (int32_t i = 0; i < n; ++i) {
        const TouchRange t = r[i];
        const uint64_t n16 = ((t.bytes >> 4) * frac_q16) >> 16;
        const u32x4 *q = (const u32x4 *)t.p;
        uint64_t j = tid;
        for (; j + 3 * nt < n16; j += 4 * nt) {
            const u32x4 v0 = q[j], v1 = q[j + nt], v2 = q[j + 2 * nt], v3 = q[j + 3 * nt];
            acc ^= (v0.x ^ v0.y ^ v0.z ^ v0.w) ^ (v1.x ^ v1.y ^ v1.z ^ v1.w) ^ (v2.x ^ v2.y ^ v2.z ^ v2.w) ^
                   (v3.x ^ v3.y ^ v3.z ^ v3.w);
        }
        for (; j < n16; j += nt) {
            const u32x4 v = q[j];
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    __asm__ volatile("" ::"v"(acc));  // keeps the loads; nothing is stored
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

template <int B, bool CHAIN, bool TILE, int R, bool ATT = false>
static hipError_t launch_chain_b(const KArgs &a, int32_t grid, size_t lds, hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
        // 160 KB of LDS per workgroup on gfx950, minus the kernel's static LDS
        hipError_t e = hipFuncSetAttribute((const void *)chain_kernel<B, CHAIN, TILE, R, ATT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((chain_kernel<B, CHAIN, TILE, R, ATT>), dim3(grid), dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

// Chains with attention phases run kernels of their own (ATT), so that the
// kernels of chains without them stay as they are.
template <int B, bool ATT>
static hipError_t launch_chain_ring(int32_t ring, const KArgs &a, int32_t grid, size_t lds, hipStream_t s) {
    switch (ring) {
    case 0: return launch_chain_b<B, true, false, 0, ATT>(a, grid, lds, s);
    case 1: return launch_chain_b<B, true, false, 1, ATT>(a, grid, lds, s);
    case 2: return launch_chain_b<B, true, false, 2, ATT>(a, grid, lds, s);
    default: return hipErrorInvalidValue;
    }
}

// Chains run any ring on the vector path; single-stage calls (no program in
// memory) and the matrix-core path use ring 0.
hipError_t launch_chain(int32_t batch, bool tile, int32_t ring, const KArgs &a, int32_t grid, size_t lds,
                        hipStream_t s) {
    const bool att = a.att != nullptr;
    if (tile) {
        if (batch > MAX_BATCH) return hipErrorInvalidValue;
        if (att) return launch_chain_b<MAX_BATCH, true, true, 0, true>(a, grid, lds, s);
        return a.phases ? launch_chain_b<MAX_BATCH, true, true, 0>(a, grid, lds, s)
                        : launch_chain_b<MAX_BATCH, false, true, 0>(a, grid, lds, s);
    }
    if (!a.phases) {
        switch (batch) {
        case 1: return launch_chain_b<1, false, false, 0>(a, grid, lds, s);
        case 2: return launch_chain_b<2, false, false, 0>(a, grid, lds, s);
        case 3: return launch_chain_b<3, false, false, 0>(a, grid, lds, s);
        case 4: return launch_chain_b<4, false, false, 0>(a, grid, lds, s);
        default: return hipErrorInvalidValue;
        }
    }
    if (att) {
        switch (batch) {
        case 1: return launch_chain_ring<1, true>(ring, a, grid, lds, s);
        case 2: return launch_chain_ring<2, true>(ring, a, grid, lds, s);
        case 3: return launch_chain_ring<3, true>(ring, a, grid, lds, s);
        case 4: return launch_chain_ring<4, true>(ring, a, grid, lds, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (batch) {
    case 1: return launch_chain_ring<1, false>(ring, a, grid, lds, s);
    case 2: return launch_chain_ring<2, false>(ring, a, grid, lds, s);
    case 3: return launch_chain_ring<3, false>(ring, a, grid, lds, s);
    case 4: return launch_chain_ring<4, false>(ring, a, grid, lds, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_touch(const TouchRange *r, int32_t n, uint32_t frac_q16, int32_t blocks, hipStream_t s) {
    hipLaunchKernelGGL(touch_kernel, dim3(blocks), dim3(256), 0, s, r, n, frac_q16);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const uint16_t *x, int64_t xs, const uint16_t *g, float eps, uint16_t *y, int64_t ys,
                               int32_t rows, int32_t K, bool f16, hipStream_t s) {
    dim3 grid((rows + 3) / 4), block(256);
    if (f16) hipLaunchKernelGGL(rmsnorm_rows_kernel<true>, grid, block, 0, s, x, xs, g, eps, y, ys, rows, K);
    else hipLaunchKernelGGL(rmsnorm_rows_kernel<false>, grid, block, 0, s, x, xs, g, eps, y, ys, rows, K);
    return hipGetLastError();
}

}  // namespace wgn

// ------------------------------------------------ fixed scratch (no allocation)
// Device memory that the allocation-free LM-head entry point uses in place of
// a caller's workspace: the argmax ticket (offset 0) and the per-workgroup
// (value, index) keys (offset 256), SCRATCH_BYTES at most -- 256 workgroups x
// 16 batch rows x 8 bytes plus the ticket area.  Every GPU the library runs on
// holds its own copy until the process ends; calls on one GPU share it.
namespace wgn {

static __device__ __align__(256) char scratch[SCRATCH_BYTES];

// Clears the ticket area (the only part that must start at zero; every call
// leaves it at zero again).  A kernel, not a memset, so that a caller may
// capture it into a graph.
__global__ void scratch_clear_kernel(uint32_t *p, int32_t n) {
    if ((int32_t)threadIdx.x < n) p[threadIdx.x] = 0u;
}

hipError_t scratch_address(void **out, hipStream_t s) {
    constexpr int MAX_DEV = 64;
    static std::mutex mu;
    static void *ptr[MAX_DEV];
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!ptr[dev]) {
        // the array's name is a host-side stand-in: its device address on
        // this GPU comes from the runtime, once, with this device current
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(scratch_clear_kernel, dim3(1), dim3(64), 0, s, (uint32_t *)p, 64);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return hipSuccess;
}

}  // namespace wgn
