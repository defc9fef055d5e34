// wgn_bwd.hip -- backward pass of a chain of LayerNorm -> Linear(+bias) ->
// GELU-tanh blocks: one persistent launch for all blocks, last block first.
//
// "Making small PyTorch ops faster on a laptop GPU", section "It works in
// training too": the backward pass visits the layers in reverse order, so the
// weights worth fetching ahead while layer i's gradient is computed are those
// of layer i-1.  Here each workgroup, once its tile of block i is done,
// issues the loads of its tile of block i-1 (weights, pre-activations, x-hat,
// block input) and only then waits for block i to finish device-wide
// (prefetch on); with prefetch off it issues them after the wait.  The
// arithmetic is the same either way, so the gradients are bit-identical.
//
// Per block (N outputs, K inputs, batch B <= 16) an item is a tile of 64
// weight rows x 64 columns, and a workgroup handles tiles g, g + T, ... of
// every block (T workgroups):
//   * gy of the tile's rows: the gradient of the mean-square loss (or the
//     caller's output gradient) for the last block; else the LayerNorm
//     backward of the following block at this block's output elements, from
//     the following block's published partials: its gxh at these elements
//     is the sum of its row blocks' partials (added in row-block order), and
//     its row sums of gamma gxh and gamma gxh u are sums of per-tile shares
//     (linear in the partials, added in a fixed order), so every workgroup
//     that needs them gets the same bits;
//   * gz = R(gy * GELU'(z)) from the FP32 pre-activation the forward kept;
//   * the tile's share of gxh = gz W (its 64 rows), and its shares of the two
//     row sums over its 64 columns, are published (system-coherent stores);
//     then the workgroup's flag tells that it is done with the block -- one
//     hand-over per block, no atomics;
//   * gW = R(gz^T xh) and gb come last: nothing waits for them.
// Every wait is bounded and reports through an error word.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wgn_bwd.h"
#include "wgn_numerics.h"

namespace wgn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int BWD_COH = 17;                   // sc0|sc1: data exchanged between workgroups
constexpr int BWD_NT = 2;                     // nt: weights are read once
// Gradient stores keep the default policy: they complete at L2 (written back
// later), so a later wait for this wave's loads -- which also waits for its
// earlier stores -- is not held up by a write to HBM.
constexpr int BWD_WB = 0;
constexpr uint32_t BWD_RSRC_W3 = 0x00020000u; // raw buffer descriptor
constexpr int TR = BWD_TILE_ROWS, TC = BWD_TILE_COLS, NBM = BWD_MAX_BATCH;
constexpr int WROW = TC + 8;                  // LDS row of the weight tile: 16 bytes of padding

static_assert(BWD_THREADS == 256 && TR == 64 && TC == 64 && NBM * 16 == BWD_THREADS,
              "thread layout of an item");

// The block table is written by the host before the launch and only read
// here: read through the constant address space, its fields come in with
// scalar loads (a vector load of a field would be followed by a wait for
// every memory operation of the wave still in flight, prefetches included).
typedef __attribute__((address_space(4))) const BwdLayer CLayer;
__device__ __forceinline__ CLayer *table(const BwdArgs &a) { return (CLayer *)(a.layers); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void *p) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)p, (short)0, (int)0x7FFFFFF0, (int)BWD_RSRC_W3);
}
__device__ __forceinline__ f32x4 coh_load4(const float *base, uint32_t idx) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(brsrc(base), idx * 4, 0, BWD_COH));
}
__device__ __forceinline__ f32x2 coh_load2(const float *base, uint32_t idx) {
    return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(brsrc(base), idx * 4, 0, BWD_COH));
}
__device__ __forceinline__ void coh_store4(float *base, uint32_t idx, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), brsrc(base), idx * 4, 0, BWD_COH);
}
__device__ __forceinline__ void coh_store2(float *base, uint32_t idx, f32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), brsrc(base), idx * 4, 0, BWD_COH);
}
__device__ __forceinline__ float lo_bf(uint32_t v) { return bf2f(v & 0xFFFFu); }
__device__ __forceinline__ float hi_bf(uint32_t v) { return bf2f(v >> 16); }

// Forward data of one item, held in registers from the moment its loads are
// issued until the item runs.  Thread t serves rows t/8 and t/8 + 32 of the
// weight tile, gz rows t%64 of batch rows t/64 + 4h, and four columns
// 4 (t%16) .. of batch row t/16 for the partial.
struct ItemData {
    u32x4 w[2];    // W[n0 + t/8 + 32 h][k0 + 8 (t%8) .. +8]
    float z[4];    // pre[b][n0 + t%64] for b = t/64 + 4 h
    u32x2 xh;      // xh[t/16][k0 + 4 (t%16) .. +4]
    u32x2 xin;     // x[t/16][k0 + 4 (t%16) .. +4]: the block input, for u
    u32x2 gam;     // gamma[k0 + 4 (t%16) .. +4]
    float mu, rs;  // statistics of batch row t/16
};

__device__ __forceinline__ ItemData load_item(CLayer &L, int32_t B, int32_t item) {
    const int32_t t = (int32_t)threadIdx.x;
    const int32_t r = item / L.ncb, c = item - r * L.ncb;
    const int32_t n0 = r * TR, k0 = c * TC;
    ItemData d;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int32_t n = n0 + (t >> 3) + 32 * h, k = k0 + 8 * (t & 7);
        d.w[h] = (u32x4){0u, 0u, 0u, 0u};
        if (n < L.N && k < L.K)
            d.w[h] = __builtin_amdgcn_raw_buffer_load_b128(brsrc(L.W), (uint32_t)(n * L.K + k) * 2u, 0, BWD_NT);
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int32_t n = n0 + (t & 63), b = (t >> 6) + 4 * h;
        d.z[h] = (n < L.N && b < B) ? L.pre[b * L.N + n] : 0.0f;
    }
    const int32_t b = t >> 4, k = k0 + 4 * (t & 15);
    const bool ok = b < B && k < L.K;
    d.xh = ok ? *(const u32x2 *)(L.xh + (int64_t)b * L.K + k) : (u32x2){0u, 0u};
    d.xin = ok ? *(const u32x2 *)(L.x + (int64_t)b * L.x_stride + k) : (u32x2){0u, 0u};
    d.gam = (L.gamma && k < L.K) ? *(const u32x2 *)(L.gamma + k) : (u32x2){0x3F803F80u, 0x3F803F80u};
    d.mu = b < B ? L.stats[2 * b] : 0.0f;
    d.rs = b < B ? L.stats[2 * b + 1] : 0.0f;
    return d;
}

struct Smem {
    uint16_t w[TR][WROW];   // the weight tile
    float gz[NBM][TR];      // gz of the tile's rows (zero outside)
    uint16_t xh[NBM][TC];   // x-hat of the tile's columns
    float gzT[TR][NBM];     // the same, batch rows contiguous
    float gx[NBM][TR];      // gxh of the following block at this tile's rows
    float gxu[NBM][TR];     // gxh u there (for its gain gradient)
    uint16_t gy[NBM][TR];   // gy of the tile's rows (stored after the flag)
    float pr[16][TC];       // partials of the row groups (row group x batch row)
    float red[16][NBM][2];  // per-thread-group shares of the row sums
    float S[NBM][2];        // row sums of gamma gxh and gamma gxh u of the following block
    uint32_t flag;
};

// The following block U's gxh at its input elements n0 .. n0 + 63 (its
// column block n0 / 64), every batch row, into sm.gx: the sum of U's row
// blocks' partials in row-block order; and U's row sums into sm.S: the sum
// of U's per-tile shares, each thread group adding tiles t/16, t/16 + 16, ..
// in order, then the 16 groups in order.
// The forward data of U's LayerNorm backward at this thread's elements
// (batch rows t/64 + 4h of element n0 + t%64), loaded with the gather.
struct LnPre {
    float x[4], mu[4], rs[4], gam;
};

__device__ LnPre gather_following(const BwdArgs &a, CLayer &U, int32_t ui, int32_t n0, Smem &sm) {
    const int32_t t = (int32_t)threadIdx.x, B = a.B;
    LnPre lp;
    {
        const int32_t n = n0 + (t & 63);
        lp.gam = (U.gamma && n < U.K) ? bf2f(U.gamma[n]) : 1.0f;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int32_t b = (t >> 6) + 4 * h;
            const bool ok = b < B && n < U.K;
            lp.x[h] = ok ? bf2f(U.x[(int64_t)b * U.x_stride + n]) : 0.0f;
            lp.mu[h] = b < B ? U.stats[2 * b] : 0.0f;
            lp.rs[h] = b < B ? U.stats[2 * b + 1] : 0.0f;
        }
    }
    const float *part = a.part[ui & 1];
    const float *q = a.q[ui & 1];
    {
        const int32_t b = t >> 4, kq = 4 * (t & 15), k = n0 + kq;
        f32x4 g = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        if (b < B && k < U.K) {
            for (int32_t r0 = 0; r0 < U.nrb; r0 += 12) {
                f32x4 v[12];
#pragma unroll
                for (int j = 0; j < 12; ++j)
                    if (r0 + j < U.nrb) v[j] = coh_load4(part, (uint32_t)(((r0 + j) * B + b) * U.K + k));
#pragma unroll
                for (int j = 0; j < 12; ++j)
                    if (r0 + j < U.nrb) g = r0 + j == 0 ? v[j] : g + v[j];
            }
        }
        *(f32x4 *)&sm.gx[b][kq] = g;
    }
    {
        const int32_t b = t & 15, grp = t >> 4, items = U.nrb * U.ncb;
        f32x2 s = (f32x2){0.0f, 0.0f};
        if (b < B) {
            for (int32_t j0 = grp; j0 < items; j0 += 16 * 8) {
                f32x2 v[8];
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    if (j0 + 16 * m < items) v[m] = coh_load2(q, (uint32_t)(((j0 + 16 * m) * B + b) * 2));
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    if (j0 + 16 * m < items) s += v[m];
            }
        }
        *(f32x2 *)&sm.red[grp][b][0] = s;
    }
    __syncthreads();
    if (t < B) {
        f32x2 s = *(const f32x2 *)&sm.red[0][t][0];
        for (int grp = 1; grp < 16; ++grp) s += *(const f32x2 *)&sm.red[grp][t][0];
        sm.S[t][0] = s.x;
        sm.S[t][1] = s.y;
    }
    return lp;
}

// LayerNorm backward of block U at its input element n0 + t%64 of batch row
// b = t/64 + 4h, from sm.gx, sm.S and the thread's LnPre:
// (gamma gxh - S1 / K - u S2 / K) / sigma, u = (x - mu) / sigma.
__device__ __forceinline__ float ln_back(CLayer &U, const Smem &sm, const LnPre &lp, int h) {
    const int32_t t = (int32_t)threadIdx.x, b = (t >> 6) + 4 * h;
    const float u = (lp.x[h] - lp.mu[h]) * lp.rs[h];
    const float K1 = (float)U.K;
    return lp.rs[h] * (lp.gam * sm.gx[b][t & 63] - sm.S[b][0] / K1 - u * (sm.S[b][1] / K1));
}

// Bounded wait until every tile workgroup's flag has reached `target` (the
// flags count finished blocks, last block first).  false: the wait gave up
// (or another workgroup's did); the error word is set.
__device__ bool wait_flags(const BwdArgs &a, uint32_t target, Smem &sm) {
    const int32_t t = (int32_t)threadIdx.x;  // wave 0 polls
    if (t < 64) {
        const uint64_t t0 = wall_clock64();
        const __amdgpu_buffer_rsrc_t rf = brsrc(a.flags);
        // a bound of 0 gives up at once (how tests force the time-out path)
        uint32_t good = a.wait_ticks > 0 ? 1u : 0u;
        while (good) {
            bool ok = true;
            for (int32_t i = t * 4; i < a.tile_wgs; i += 256) {
                const u32x4 f = __builtin_amdgcn_raw_buffer_load_b128(rf, (uint32_t)i * 4u, 0, BWD_COH);
                ok &= f.x >= target && (i + 1 >= a.tile_wgs || f.y >= target) &&
                      (i + 2 >= a.tile_wgs || f.z >= target) && (i + 3 >= a.tile_wgs || f.w >= target);
            }
            if (__all(ok)) break;
            if (__hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
                wall_clock64() - t0 > a.wait_ticks) {
                good = 0u;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (t == 0) {
            if (!good) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sm.flag = good;
        }
    }
    __syncthreads();
    const bool ok = sm.flag != 0u;
    __syncthreads();  // the flag word is reused
    return ok;
}

// This workgroup is done with block li: its flag becomes n - li.
__device__ __forceinline__ void set_flag(const BwdArgs &a, int32_t li) {
    __builtin_amdgcn_s_waitcnt(0);  // the partials and shares are written through
    __syncthreads();
    if (threadIdx.x == 0)
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(a.n - li), brsrc(a.flags), blockIdx.x * 4u, 0, BWD_COH);
}

__device__ __forceinline__ void stamp(uint64_t *tr, int p) {
    if (tr && threadIdx.x == 0) tr[p] = wall_clock64();
}

// First part of an item: gy, gz, the tile's partial of gxh and its shares of
// the row sums (published), and, for the first column block, the gain and
// shift gradients of the following block at the tile's rows.
// tr: this item's trace slots (null: not traced).
__device__ void run_a(const BwdArgs &a, CLayer &L, CLayer &U, bool last, int32_t li, int32_t item,
                      const ItemData &d, Smem &sm, uint64_t *tr) {
    const int32_t t = (int32_t)threadIdx.x;
    const int32_t B = a.B, N = L.N, K = L.K;
    const int32_t r = item / L.ncb, c = item - r * L.ncb;
    const int32_t n0 = r * TR, k0 = c * TC;
    __syncthreads();  // the previous item is done with the LDS
#pragma unroll
    for (int h = 0; h < 2; ++h) *(u32x4 *)&sm.w[(t >> 3) + 32 * h][8 * (t & 7)] = d.w[h];
    *(u32x2 *)&sm.xh[t >> 4][4 * (t & 15)] = d.xh;
    LnPre lp;
    if (!last) lp = gather_following(a, U, li + 1, n0, sm);
    __syncthreads();

    // gy and gz of the tile's rows; for the following block's gain
    // gradient also gxh u at these elements
    const int32_t rho = t & 63, n = n0 + rho;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int32_t b = (t >> 6) + 4 * h;
        float gzv = 0.0f;
        if (b < B && n < N) {
            uint16_t gyb;
            if (!last) {
                gyb = f2bf(ln_back(U, sm, lp, h));
                sm.gxu[b][rho] = sm.gx[b][rho] * ((lp.x[h] - lp.mu[h]) * lp.rs[h]);
            } else if (a.g_out) {
                gyb = a.g_out[(int64_t)b * a.g_stride + n];
            } else {
                // mean-square loss over the B x N output: 2 y / (B N), in FP64, one rounding
                const double v = (double)bf2f(a.y[(int64_t)b * a.y_stride + n]) * (2.0 / ((double)B * (double)N));
                gyb = f64_to_bf16(v);
            }
            const uint16_t gzb = f2bf(bf2f(gyb) * gelu_tanh_grad(d.z[h]));
            sm.gy[b][rho] = gyb;
            gzv = bf2f(gzb);
        }
        sm.gz[b][rho] = gzv;
        sm.gzT[rho][b] = gzv;
    }
    __syncthreads();
    stamp(tr, 2);

    // this tile's rows' share of gxh = gz W and its shares of the row sums
    // over its columns.  Every thread works: with the batch rounded up to a
    // power of two (Bp), the 64 rows are split into 16 / Bp row groups, each
    // summed in row order, then the groups are added in group order.
    {
        const int32_t Bp = B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : 16;
        const int32_t RG = 16 / Bp, RPG = TR / RG;
        const int32_t kq = 4 * (t & 15), b = (t >> 4) & (Bp - 1), rg = (t >> 4) / Bp;
        f32x4 p = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        if (b < B && k0 + kq < K) {
            for (int32_t rr0 = rg * RPG; rr0 < (rg + 1) * RPG; rr0 += 4) {
                const f32x4 g4 = *(const f32x4 *)&sm.gz[b][rr0];
                u32x2 wv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) wv[j] = *(const u32x2 *)&sm.w[rr0 + j][kq];
                const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    p.x = fmaf(gg[j], lo_bf(wv[j].x), p.x);
                    p.y = fmaf(gg[j], hi_bf(wv[j].x), p.y);
                    p.z = fmaf(gg[j], lo_bf(wv[j].y), p.z);
                    p.w = fmaf(gg[j], hi_bf(wv[j].y), p.w);
                }
            }
        }
        *(f32x4 *)&sm.pr[t >> 4][kq] = p;
        __syncthreads();
        if (rg == 0) {
            for (int32_t g2 = 1; g2 < RG; ++g2) p += *(const f32x4 *)&sm.pr[g2 * Bp + b][kq];
            if (b < B && k0 + kq < K) coh_store4(a.part[li & 1], (uint32_t)((r * B + b) * K + k0 + kq), p);
        }
        const float pp[4] = {p.x, p.y, p.z, p.w};
        const float xs[4] = {lo_bf(d.xin.x), hi_bf(d.xin.x), lo_bf(d.xin.y), hi_bf(d.xin.y)};
        const float gs[4] = {lo_bf(d.gam.x), hi_bf(d.gam.x), lo_bf(d.gam.y), hi_bf(d.gam.y)};
        float q1 = 0.0f, q2 = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float gu = gs[e] * pp[e];
            q1 += gu;
            q2 += gu * ((xs[e] - d.mu) * d.rs);
        }
        // the 16 lanes of one batch row hold the tile's 64 columns
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) {
            q1 += __shfl_xor(q1, o);
            q2 += __shfl_xor(q2, o);
        }
        if (rg == 0 && (t & 15) == 0 && b < B) coh_store2(a.q[li & 1], (uint32_t)((item * B + b) * 2), (f32x2){q1, q2});
    }
    stamp(tr, 3);
}

// Second part of an item: what no workgroup waits for -- the weight and bias
// gradients of the tile (sums over the batch rows in order), and a share of
// the row block's gy and gz stores and of the following block's gain and
// shift gradients at the row block's rows (its gxh is in sm.gx): the tiles
// of one row block take rows c, c + ncb, ... each, so that no tile carries
// more of this than another.
__device__ void run_b(const BwdArgs &a, CLayer &L, CLayer &U, bool last, int32_t item, Smem &sm) {
    const int32_t t = (int32_t)threadIdx.x;
    const int32_t B = a.B, N = L.N, K = L.K;
    const int32_t r = item / L.ncb, c = item - r * L.ncb;
    const int32_t n0 = r * TR, k0 = c * TC;
    {
        const int32_t rho = t & 63, n = n0 + rho;
        if (n < N && rho % L.ncb == c) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int32_t b = (t >> 6) + 4 * h;
                if (b < B) {
                    if (L.gy) L.gy[b * N + n] = sm.gy[b][rho];
                    if (L.gz) L.gz[b * N + n] = f2bf(sm.gz[b][rho]);
                }
            }
            if (!last && t < TR && (U.ggamma || U.gbeta)) {
                float sg = 0.0f, sb = 0.0f;
                for (int32_t b = 0; b < B; ++b) {
                    sg += sm.gxu[b][rho];
                    sb += sm.gx[b][rho];
                }
                if (U.ggamma) U.ggamma[n] = f2bf(sg);
                if (U.gbeta) U.gbeta[n] = f2bf(sb);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int32_t rr = (t >> 3) + 32 * h, kc = 8 * (t & 7), nn = n0 + rr, k = k0 + kc;
        if (nn < N && k < K) {
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
            for (int32_t b0 = 0; b0 < B; b0 += 4) {
                // four batch rows at a time: their gz (one read) and x-hat
                const f32x4 g4 = *(const f32x4 *)&sm.gzT[rr][b0];
                const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
                u32x4 xv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) xv[j] = *(const u32x4 *)&sm.xh[b0 + j][kc];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (b0 + j < B) {
                        const uint32_t xx[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            acc[2 * e] = fmaf(gg[j], lo_bf(xx[e]), acc[2 * e]);
                            acc[2 * e + 1] = fmaf(gg[j], hi_bf(xx[e]), acc[2 * e + 1]);
                        }
                    }
                }
            }
            u32x4 o;
            o.x = (uint32_t)f2bf(acc[0]) | ((uint32_t)f2bf(acc[1]) << 16);
            o.y = (uint32_t)f2bf(acc[2]) | ((uint32_t)f2bf(acc[3]) << 16);
            o.z = (uint32_t)f2bf(acc[4]) | ((uint32_t)f2bf(acc[5]) << 16);
            o.w = (uint32_t)f2bf(acc[6]) | ((uint32_t)f2bf(acc[7]) << 16);
            __builtin_amdgcn_raw_buffer_store_b128(o, brsrc(L.gW), (uint32_t)(nn * K + k) * 2u, 0, BWD_WB);
        }
    }
    if (c == 0 && L.gb && t < TR && n0 + t < N) {
        const int32_t rr = t;
        float s = 0.0f;
        for (int32_t b = 0; b < B; ++b) s += sm.gzT[rr][b];
        L.gb[n0 + rr] = f2bf(s);
    }
}

__global__ __launch_bounds__(BWD_THREADS) void bwd_kernel(BwdArgs a) {
    __shared__ __align__(16) Smem sm;
    const int32_t g = (int32_t)blockIdx.x, T = a.tile_wgs;
    ItemData cur;
    bool have = false;
    for (int32_t li = a.n - 1; li >= 0; --li) {
        CLayer &L = table(a)[li];
        const int32_t items = L.nrb * L.ncb;
        if (g < items) {
            const bool last = li == a.n - 1;
            CLayer &U = last ? L : table(a)[li + 1];
            uint64_t *tr = a.trace ? a.trace + ((size_t)li * T + g) * BWD_TRACE_POINTS : nullptr;
            stamp(tr, 0);
            bool waited = last;
            if (!have) {
                if (!waited && !a.prefetch) {
                    if (!wait_flags(a, (uint32_t)(a.n - li - 1), sm)) return;
                    waited = true;
                }
                cur = load_item(L, a.B, g);
            }
            if (!waited && !wait_flags(a, (uint32_t)(a.n - li - 1), sm)) return;
            stamp(tr, 1);
            for (int32_t j = g; j < items; j += T) {
                run_a(a, L, U, last, li, j, cur, sm, j == g ? tr : nullptr);
                if (j + T >= items) {
                    set_flag(a, li);
                    stamp(tr, 4);
                }
                // the next tile's loads go out now, before this tile's weight
                // gradients; for the next block in backward order (its tile of
                // block i-1 while block i finishes) only with prefetch on
                have = false;
                ItemData next;
                if (j + T < items) {
                    next = load_item(L, a.B, j + T);
                    have = true;
                } else if (a.prefetch && li > 0) {
                    CLayer &P = table(a)[li - 1];
                    if (g < P.nrb * P.ncb) {
                        next = load_item(P, a.B, g);
                        have = true;
                    }
                }
                if (j == g) stamp(tr, 5);
                run_b(a, L, U, last, j, sm);
                if (j == g) stamp(tr, 6);
                if (have) cur = next;
            }
        } else {
            set_flag(a, li);  // no tile of this block
        }
    }
    if (!a.g_in && !table(a)[0].ggamma && !table(a)[0].gbeta) return;  // scalar loads
    // the first block's LayerNorm backward: the chain-input gradient and the
    // first block's gain and shift gradients, one column block per workgroup
    CLayer &L = table(a)[0];
    if (!wait_flags(a, (uint32_t)a.n, sm)) return;
    const int32_t t = (int32_t)threadIdx.x;
    for (int32_t cb = g; cb < L.ncb; cb += T) {
        const int32_t n0 = cb * TC;
        __syncthreads();
        const LnPre lp = gather_following(a, L, 0, n0, sm);
        __syncthreads();
        const int32_t rho = t & 63, n = n0 + rho;
        if (a.g_in && n < L.K)
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int32_t b = (t >> 6) + 4 * h;
                if (b < a.B) a.g_in[(int64_t)b * a.gin_stride + n] = f2bf(ln_back(L, sm, lp, h));
            }
        if (t < TC && n < L.K && (L.ggamma || L.gbeta)) {
            float sg = 0.0f, sb = 0.0f;
            float xv[NBM];
#pragma unroll
            for (int b = 0; b < NBM; ++b)
                xv[b] = b < a.B ? (bf2f(L.x[(int64_t)b * L.x_stride + n]) - L.stats[2 * b]) * L.stats[2 * b + 1] : 0.0f;
            for (int32_t b = 0; b < a.B; ++b) {
                const float gg = sm.gx[b][rho];
                sg += gg * xv[b];
                sb += gg;
            }
            if (L.ggamma) L.ggamma[n] = f2bf(sg);
            if (L.gbeta) L.gbeta[n] = f2bf(sb);
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
    __syncthreads();
    return t;
}

// Per (block, batch row): the LayerNorm statistics of the block input and its
// x-hat in BF16, in binary64 with one rounding (the forward's definition:
// mean, biased variance about the mean, (x - mu) r gamma + beta with
// r = (var + eps)^-1/2).  Workgroup 0 also clears the run's counters.
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdLayer *layers, int32_t B, uint32_t *zero,
                                                       int32_t nzero) {
#pragma clang fp contract(off)
    __shared__ double red[4];
    const int32_t t = (int32_t)threadIdx.x;
    if (blockIdx.x == 0)
        for (int32_t i = t; i < nzero; i += 256) zero[i] = 0u;
    const int32_t li = (int32_t)blockIdx.x / B, b = (int32_t)blockIdx.x - li * B;
    const BwdLayer L = layers[li];
    const uint16_t *xr = L.x + (int64_t)b * L.x_stride;
    const int32_t K = L.K, n8 = K >> 3;
    double s = 0.0;
    for (int32_t i = t; i < n8; i += 256) {
        const u32x4 v = *(const u32x4 *)(xr + (int64_t)i * 8);
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) s += (double)bf2f(vv[e] & 0xFFFFu) + (double)bf2f(vv[e] >> 16);
    }
    const double mu = block_sum(s, red) / (double)K;
    double ss = 0.0;
    for (int32_t i = t; i < n8; i += 256) {
        const u32x4 v = *(const u32x4 *)(xr + (int64_t)i * 8);
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double lo = (double)bf2f(vv[e] & 0xFFFFu) - mu, hi = (double)bf2f(vv[e] >> 16) - mu;
            ss += lo * lo;
            ss += hi * hi;
        }
    }
    const double rr = 1.0 / sqrt(block_sum(ss, red) / (double)K + (double)L.eps);
    if (t == 0) {
        L.stats[2 * b] = (float)mu;
        L.stats[2 * b + 1] = (float)rr;
    }
    uint16_t *yr = L.xh + (int64_t)b * K;
    for (int32_t i = t; i < n8; i += 256) {
        const u32x4 v = *(const u32x4 *)(xr + (int64_t)i * 8);
        const u32x4 gv = L.gamma ? *(const u32x4 *)(L.gamma + (int64_t)i * 8)
                                 : (u32x4){0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
        const u32x4 bv = L.beta ? *(const u32x4 *)(L.beta + (int64_t)i * 8) : (u32x4){0u, 0u, 0u, 0u};
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w}, gg[4] = {gv.x, gv.y, gv.z, gv.w}, bb[4] = {bv.x, bv.y, bv.z, bv.w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            double q[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const double xv = (double)bf2f((vv[e] >> (16 * h)) & 0xFFFFu);
                q[h] = (xv - mu) * rr * (double)bf2f((gg[e] >> (16 * h)) & 0xFFFFu) +
                       (double)bf2f((bb[e] >> (16 * h)) & 0xFFFFu);
            }
            o[e] = (uint32_t)f64_to_bf16(q[0]) | ((uint32_t)f64_to_bf16(q[1]) << 16);
        }
        *(u32x4 *)(yr + (int64_t)i * 8) = (u32x4){o[0], o[1], o[2], o[3]};
    }
}

}  // namespace

hipError_t launch_bwd_prep(const BwdLayer *layers, int32_t n, int32_t B, uint32_t *zero, int32_t nzero,
                           hipStream_t s) {
    if (n < 1 || B < 1 || B > BWD_MAX_BATCH) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)(n * B)), dim3(256), 0, s, layers, B, zero, nzero);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs &a, int32_t grid, hipStream_t s) {
    if (grid < 1 || a.n < 1 || a.B < 1 || a.B > BWD_MAX_BATCH) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_kernel, dim3((unsigned)grid), dim3(BWD_THREADS), 0, s, a);
    return hipGetLastError();
}

int32_t bwd_resident_grid() {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, bwd_kernel, BWD_THREADS, 0) != hipSuccess) return 0;
    return cus * per;
}

}  // namespace wgn
