// wgn_bwd.hip -- backward pass of a chain of LayerNorm -> Linear(+bias) ->
// GELU-tanh blocks: one persistent launch for all blocks, last block first.
//
// "Making small PyTorch ops faster on a laptop GPU", section "It works in
// training too": the backward pass visits the layers in reverse order, so the
// weights worth fetching ahead while layer i's gradient is computed are those
// of layer i-1.  Here each workgroup, once its last tile of block i is done,
// issues the loads of its tile of block i-1 (weights, pre-activations, x-hat)
// and only then waits for block i to finish device-wide (prefetch on); with
// prefetch off it issues them after the wait.  The arithmetic is the same
// either way, so the gradients are bit-identical.
//
// Per block (N outputs, K inputs, batch B <= 16) an item is a tile of 32
// weight rows x 64 columns:
//   * gz = R(gy * GELU'(z)) for the tile's rows, from the FP32 pre-activation
//     the forward kept; gy is the gradient of the mean-square loss (or the
//     caller's output gradient) for the last block, else the LayerNorm
//     backward of the following block at this block's output element;
//   * gW = R(gz^T xh) for the tile (x-hat in BF16 from the prep pass), and gb
//     from the tiles of the first column block;
//   * the tile's share of gxh = gz W (its 32 rows) goes to a partial buffer;
//     the last tile of a column block to take the column block's ticket adds
//     the row blocks in order (a fixed FP32 order), keeps gxh, the column
//     block's sums of gamma gxh and gamma gxh u, writes the gain and shift
//     gradients and counts the column block as done.
// Workgroups exchange data at the system-coherent level (sc0|sc1 stores and
// loads) and publish it with a counter only after their stores completed;
// every wait is bounded and reports through an error word.
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
constexpr int BWD_NT = 2;                     // nt: weights are read once, gradients written once
constexpr uint32_t BWD_RSRC_W3 = 0x00020000u; // raw buffer descriptor
constexpr int TR = BWD_TILE_ROWS, TC = BWD_TILE_COLS, NBM = BWD_MAX_BATCH;
constexpr int WROW = TC + 8;                  // LDS row of the weight tile: 16 bytes of padding

static_assert(BWD_THREADS == 256 && TR * TC == BWD_THREADS * 8 && NBM * 16 == BWD_THREADS,
              "thread layout of an item");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void *p) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)p, (short)0, (int)0x7FFFFFF0, (int)BWD_RSRC_W3);
}
__device__ __forceinline__ f32x4 coh_load4(const float *base, uint32_t idx) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(brsrc(base), idx * 4, 0, BWD_COH));
}
__device__ __forceinline__ f32x2 coh_load2(const float *base, uint32_t idx) {
    return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(brsrc(base), idx * 4, 0, BWD_COH));
}
__device__ __forceinline__ float coh_load(const float *base, uint32_t idx) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(brsrc(base), idx * 4, 0, BWD_COH));
}
__device__ __forceinline__ void coh_store4(float *base, uint32_t idx, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), brsrc(base), idx * 4, 0, BWD_COH);
}
__device__ __forceinline__ void coh_store2(float *base, uint32_t idx, f32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), brsrc(base), idx * 4, 0, BWD_COH);
}

// Forward data of one item, held in registers from the moment its loads are
// issued until the item runs.
struct ItemData {
    u32x4 w;       // W[n0 + t/8][k0 + 8 (t%8) .. +8]
    float z0, z1;  // pre[b][n0 + t%32] for b = t/32 and t/32 + 8
    u32x2 xh;      // xh[t/16][k0 + 4 (t%16) .. +4]
};

__device__ __forceinline__ ItemData load_item(const BwdLayer &L, int32_t B, int32_t item) {
    const int32_t t = (int32_t)threadIdx.x;
    const int32_t r = item / L.ncb, c = item - r * L.ncb;
    const int32_t n0 = r * TR, k0 = c * TC;
    ItemData d;
    d.w = (u32x4){0u, 0u, 0u, 0u};
    {
        const int32_t n = n0 + (t >> 3), k = k0 + 8 * (t & 7);
        if (n < L.N && k < L.K)
            d.w = __builtin_amdgcn_raw_buffer_load_b128(brsrc(L.W), (uint32_t)(n * L.K + k) * 2u, 0, BWD_NT);
    }
    {
        const int32_t n = n0 + (t & 31), b = t >> 5;
        d.z0 = (n < L.N && b < B) ? L.pre[b * L.N + n] : 0.0f;
        d.z1 = (n < L.N && b + 8 < B) ? L.pre[(b + 8) * L.N + n] : 0.0f;
    }
    {
        const int32_t b = t >> 4, k = k0 + 4 * (t & 15);
        d.xh = (b < B && k < L.K) ? *(const u32x2 *)(L.xh + (int64_t)b * L.K + k) : (u32x2){0u, 0u};
    }
    return d;
}

struct Smem {
    uint16_t w[TR][WROW];   // the weight tile
    float gz[NBM][TR];      // gz of the tile's rows (zero outside)
    uint16_t xh[NBM][TC];   // x-hat of the tile's columns
    float cg[NBM][TC];      // finisher: gxh of the column block
    float cgu[NBM][TC];     // finisher: gxh * u
    float S[NBM][2];        // totals of gamma gxh and gamma gxh u of the following block
    uint32_t flag;
};

// LayerNorm backward of block U at its input element n of batch row b:
// (gamma gxh - S1 / K - u S2 / K) / sigma, u = (x - mu) / sigma.
__device__ __forceinline__ float ln_back(const BwdLayer &U, int32_t b, int32_t n, float S1, float S2) {
    const float g = coh_load(U.gxh, (uint32_t)(b * U.K + n));
    const float mu = U.stats[2 * b], rs = U.stats[2 * b + 1];
    const float u = (bf2f(U.x[(int64_t)b * U.x_stride + n]) - mu) * rs;
    const float gam = U.gamma ? bf2f(U.gamma[n]) : 1.0f;
    const float K1 = (float)U.K;
    return rs * (gam * g - S1 / K1 - u * (S2 / K1));
}

// Sums of the column blocks of block U per batch row, in column-block order.
__device__ __forceinline__ void load_totals(const BwdLayer &U, int32_t B, Smem &sm) {
    const int32_t t = (int32_t)threadIdx.x;
    if (t < B) {
        float s1 = 0.0f, s2 = 0.0f;
        for (int32_t c = 0; c < U.ncb; ++c) {
            const f32x2 v = coh_load2(U.s12, (uint32_t)((c * B + t) * 2));
            s1 += v.x;
            s2 += v.y;
        }
        sm.S[t][0] = s1;
        sm.S[t][1] = s2;
    }
}

// Bounded wait until block j has all its column blocks done.  false: the
// wait gave up (or another workgroup's did); the error word is set.
__device__ bool wait_done(const BwdArgs &a, int32_t j, uint32_t target, Smem &sm) {
    if (threadIdx.x == 0) {
        const uint64_t t0 = wall_clock64();
        uint32_t ok = 1u;
        while (__hip_atomic_load(&a.done[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (__hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
                wall_clock64() - t0 > a.wait_ticks) {
                __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0u;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        sm.flag = ok;
    }
    __syncthreads();
    const bool ok = sm.flag != 0u;
    __syncthreads();  // the flag word is reused
    return ok;
}

__device__ void run_item(const BwdArgs &a, const BwdLayer &L, const BwdLayer &U, bool last, int32_t li, int32_t item,
                         const ItemData &d, Smem &sm) {
    const int32_t t = (int32_t)threadIdx.x;
    const int32_t B = a.B, N = L.N, K = L.K;
    const int32_t r = item / L.ncb, c = item - r * L.ncb;
    const int32_t n0 = r * TR, k0 = c * TC;
    __syncthreads();  // the previous item is done with the LDS
    *(u32x4 *)&sm.w[t >> 3][8 * (t & 7)] = d.w;
    *(u32x2 *)&sm.xh[t >> 4][4 * (t & 15)] = d.xh;
    if (!last) load_totals(U, B, sm);
    __syncthreads();

    // gy and gz of the tile's rows
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int32_t rho = t & 31, b = (t >> 5) + 8 * h, n = n0 + rho;
        float gzv = 0.0f;
        if (b < B && n < N) {
            uint16_t gyb;
            if (!last) {
                gyb = f2bf(ln_back(U, b, n, sm.S[b][0], sm.S[b][1]));
            } else if (a.g_out) {
                gyb = a.g_out[(int64_t)b * a.g_stride + n];
            } else {
                // mean-square loss over the B x N output: 2 y / (B N), in FP64, one rounding
                const double v = (double)bf2f(a.y[(int64_t)b * a.y_stride + n]) * (2.0 / ((double)B * (double)N));
                gyb = f64_to_bf16(v);
            }
            const uint16_t gzb = f2bf(bf2f(gyb) * gelu_tanh_grad(h ? d.z1 : d.z0));
            if (c == 0) {
                if (L.gy) L.gy[b * N + n] = gyb;
                if (L.gz) L.gz[b * N + n] = gzb;
            }
            gzv = bf2f(gzb);
        }
        sm.gz[b][rho] = gzv;
    }
    __syncthreads();

    // weight gradient of the tile: sum over the batch rows in order
    {
        const int32_t rho = t >> 3, kc = 8 * (t & 7), n = n0 + rho, k = k0 + kc;
        if (n < N && k < K) {
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
            for (int32_t b = 0; b < B; ++b) {
                const float g = sm.gz[b][rho];
                const u32x4 xv = *(const u32x4 *)&sm.xh[b][kc];
                const uint32_t xx[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] = fmaf(g, bf2f(xx[e] & 0xFFFFu), acc[2 * e]);
                    acc[2 * e + 1] = fmaf(g, bf2f(xx[e] >> 16), acc[2 * e + 1]);
                }
            }
            u32x4 o;
            o.x = (uint32_t)f2bf(acc[0]) | ((uint32_t)f2bf(acc[1]) << 16);
            o.y = (uint32_t)f2bf(acc[2]) | ((uint32_t)f2bf(acc[3]) << 16);
            o.z = (uint32_t)f2bf(acc[4]) | ((uint32_t)f2bf(acc[5]) << 16);
            o.w = (uint32_t)f2bf(acc[6]) | ((uint32_t)f2bf(acc[7]) << 16);
            __builtin_amdgcn_raw_buffer_store_b128(o, brsrc(L.gW), (uint32_t)(n * K + k) * 2u, 0, BWD_NT);
        }
        if (c == 0 && L.gb && t < TR && n0 + t < N) {
            float s = 0.0f;
            for (int32_t b = 0; b < B; ++b) s += sm.gz[b][t];
            L.gb[n0 + t] = f2bf(s);
        }
    }

    // this tile's rows' share of gxh = gz W, summed over the rows in order
    {
        const int32_t b = t >> 4, kq = 4 * (t & 15);
        if (b < B && k0 + kq < K) {
            f32x4 s = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
            for (int32_t rho = 0; rho < TR; ++rho) {
                const float g = sm.gz[b][rho];
                const u32x2 wv = *(const u32x2 *)&sm.w[rho][kq];
                s.x = fmaf(g, bf2f(wv.x & 0xFFFFu), s.x);
                s.y = fmaf(g, bf2f(wv.x >> 16), s.y);
                s.z = fmaf(g, bf2f(wv.y & 0xFFFFu), s.z);
                s.w = fmaf(g, bf2f(wv.y >> 16), s.w);
            }
            coh_store4(a.part, (uint32_t)((r * B + b) * K + k0 + kq), s);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the partial is written through
    __syncthreads();
    if (t == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&a.tickets[c], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t fin = old == (uint32_t)(L.nrb - 1) ? 1u : 0u;
        if (fin) __hip_atomic_store(&a.tickets[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.flag = fin;
    }
    __syncthreads();
    if (sm.flag == 0u) return;

    // ---- the column block's finisher: add the row blocks in order
    {
        const int32_t b = t >> 4, kq = 4 * (t & 15), k = k0 + kq;
        const bool ok = b < B && k < K;
        float p1 = 0.0f, p2 = 0.0f;
        f32x4 g = (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, gu_u = g;
        if (ok) {
            for (int32_t r0 = 0; r0 < L.nrb; r0 += 8) {
                f32x4 v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (r0 + j < L.nrb) v[j] = coh_load4(a.part, (uint32_t)(((r0 + j) * B + b) * K + k));
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (r0 + j < L.nrb) g = r0 + j == 0 ? v[j] : g + v[j];
            }
            coh_store4(L.gxh, (uint32_t)(b * K + k), g);
            const float mu = L.stats[2 * b], rs = L.stats[2 * b + 1];
            const u32x2 xv = *(const u32x2 *)(L.x + (int64_t)b * L.x_stride + k);
            const u32x2 gv = L.gamma ? *(const u32x2 *)(L.gamma + k) : (u32x2){0x3F803F80u, 0x3F803F80u};
            const float xs[4] = {bf2f(xv.x & 0xFFFFu), bf2f(xv.x >> 16), bf2f(xv.y & 0xFFFFu), bf2f(xv.y >> 16)};
            const float gs[4] = {bf2f(gv.x & 0xFFFFu), bf2f(gv.x >> 16), bf2f(gv.y & 0xFFFFu), bf2f(gv.y >> 16)};
            const float gg[4] = {g.x, g.y, g.z, g.w};
            float uu[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uu[e] = (xs[e] - mu) * rs;
                const float gu = gs[e] * gg[e];
                p1 += gu;
                p2 += gu * uu[e];
            }
            gu_u = (f32x4){gg[0] * uu[0], gg[1] * uu[1], gg[2] * uu[2], gg[3] * uu[3]};
        }
        *(f32x4 *)&sm.cg[b][kq] = g;
        *(f32x4 *)&sm.cgu[b][kq] = gu_u;
        // the 16 lanes of one batch row hold the column block's 64 columns
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) {
            p1 += __shfl_xor(p1, o);
            p2 += __shfl_xor(p2, o);
        }
        if ((t & 15) == 0 && b < B) coh_store2(L.s12, (uint32_t)((c * B + b) * 2), (f32x2){p1, p2});
    }
    __syncthreads();
    if (t < TC && k0 + t < K && (L.ggamma || L.gbeta)) {
        float sg = 0.0f, sb = 0.0f;
        for (int32_t b = 0; b < B; ++b) {
            sg += sm.cgu[b][t];
            sb += sm.cg[b][t];
        }
        if (L.ggamma) L.ggamma[k0 + t] = f2bf(sg);
        if (L.gbeta) L.gbeta[k0 + t] = f2bf(sb);
    }
    __builtin_amdgcn_s_waitcnt(0);  // gxh, the sums and the ticket reset are written through
    __syncthreads();
    if (t == 0) __hip_atomic_fetch_add(&a.done[li], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(BWD_THREADS) void bwd_kernel(BwdArgs a) {
    __shared__ __align__(16) Smem sm;
    const int32_t G = (int32_t)gridDim.x, g = (int32_t)blockIdx.x;
    ItemData cur;
    bool have = false;
    for (int32_t li = a.n - 1; li >= 0; --li) {
        const BwdLayer L = a.layers[li];
        const int32_t items = L.nrb * L.ncb;
        if (g >= items) continue;
        const bool last = li == a.n - 1;
        const BwdLayer U = last ? L : a.layers[li + 1];
        bool waited = last;
        if (!have) {
            if (!waited && !a.prefetch) {
                if (!wait_done(a, li + 1, (uint32_t)U.ncb, sm)) return;
                waited = true;
            }
            cur = load_item(L, a.B, g);
        }
        if (!waited && !wait_done(a, li + 1, (uint32_t)U.ncb, sm)) return;
        for (int32_t j = g; j < items; j += G) {
            run_item(a, L, U, last, li, j, cur, sm);
            // The next item's loads go out once this item's stores have
            // completed (a store wait would otherwise wait for them too).
            have = false;
            if (j + G < items) {
                cur = load_item(L, a.B, j + G);
                have = true;
            } else if (a.prefetch && li > 0) {
                // the next block in backward order: its weight tile is
                // requested now, before the wait for this block to finish
                const BwdLayer P = a.layers[li - 1];
                if (g < P.nrb * P.ncb) {
                    cur = load_item(P, a.B, g);
                    have = true;
                }
            }
        }
    }
    if (!a.g_in) return;
    // gradient of the chain input: LayerNorm backward of the first block
    const BwdLayer L = a.layers[0];
    if (!wait_done(a, 0, (uint32_t)L.ncb, sm)) return;
    load_totals(L, a.B, sm);
    __syncthreads();
    const int32_t total = a.B * L.K;
    for (int32_t e = g * BWD_THREADS + (int32_t)threadIdx.x; e < total; e += G * BWD_THREADS) {
        const int32_t b = e / L.K, k = e - b * L.K;
        a.g_in[(int64_t)b * a.gin_stride + k] = f2bf(ln_back(L, b, k, sm.S[b][0], sm.S[b][1]));
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
