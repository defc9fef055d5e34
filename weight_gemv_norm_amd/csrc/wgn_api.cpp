// wgn_api.cpp -- host side of libwgn.so: argument validation, grouping of a
// stage list into phases, device-program layout, launches.
//
// Everything here runs before a kernel is enqueued; a failed check returns a
// negative status and enqueues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "wgn.h"
#include "wgn_attn.h"
#include "wgn_bwd.h"
#include "wgn_gemm.h"
#include "wgn_loader.h"

namespace wgn {
hipError_t launch_chain(int32_t batch, bool tile, int32_t ring, const KArgs &a, int32_t grid, size_t lds,
                        hipStream_t s);
hipError_t launch_rmsnorm_rows(const uint16_t *x, int64_t xs, const uint16_t *g, float eps, uint16_t *y, int64_t ys,
                               int32_t rows, int32_t K, bool f16, hipStream_t s);
hipError_t launch_touch(const TouchRange *r, int32_t n, uint32_t frac_q16, int32_t blocks, hipStream_t s);
size_t gemv_int4_lds_bytes(int32_t batch, int32_t K);
hipError_t launch_gemv_int4(const uint16_t *x, int64_t xs, int32_t batch, int32_t K, const uint8_t *W4,
                            const uint16_t *sc, const uint16_t *zr, int32_t N, uint16_t *y, int64_t ys,
                            int32_t cus, hipStream_t s);
hipError_t scratch_address(void **out, hipStream_t s);
hipError_t launch_stream_read(const void *src, uint64_t n16, int32_t grid, int32_t threads, int32_t depth,
                              uint32_t *sink, hipStream_t s);
}  // namespace wgn

using namespace wgn;

#ifndef WGN_PRE_B1
#define WGN_PRE_B1 0
#endif
namespace {

thread_local char g_last_hip_error[256] = "";

// Record a failing HIP call's error for wgn_last_hip_error().
hipError_t note(hipError_t e, const char *what) {
    if (e != hipSuccess)
        std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
    return e;
}

constexpr size_t LDS_BUDGET = 160 * 1024 - 256;  // gfx950 LDS per workgroup, minus static use
constexpr int32_t VERSION = 1;

struct DevInfo {
    bool ok = false;
    int32_t cus = 0;
};

DevInfo device_info() {
    static std::mutex mu;
    static DevInfo cache[16];
    static bool have[16] = {false};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return DevInfo{};
    std::lock_guard<std::mutex> lk(mu);
    if (!have[dev]) {
        hipDeviceProp_t prop;
        DevInfo d;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
            d.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            d.cus = prop.multiProcessorCount;
        }
        cache[dev] = d;
        have[dev] = true;
    }
    return cache[dev];
}

inline bool a16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool a4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline bool a2(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }
inline size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

wgn_status check_stage(const wgn_stage &s, int32_t batch, int32_t max_batch = MAX_BATCH) {
    if (batch < 1 || batch > max_batch) return WGN_E_ARG;
    if (s.N < 1 || s.K < 8 || (s.K & 7)) return WGN_E_ARG;
    if (s.K > (1 << 24)) return WGN_E_UNSUPPORTED;  // 16 rows x K x 2 bytes must fit 32-bit buffer offsets
    if (!s.W || !s.x || !s.y) return WGN_E_ARG;
    if (s.norm < NORM_NONE || s.norm > NORM_LAYER) return WGN_E_ARG;
    if (s.epi < EPI_NONE || s.epi > EPI_ARGMAX) return WGN_E_ARG;
    if (s.epi == EPI_SWIGLU && !s.W_up) return WGN_E_ARG;
    if (s.epi != EPI_SWIGLU && s.W_up) return WGN_E_ARG;
    if (s.epi == EPI_SWIGLU && s.bias) return WGN_E_UNSUPPORTED;
    if (s.epi == EPI_ARGMAX && s.residual) return WGN_E_ARG;
    if (s.maxval && s.epi != EPI_ARGMAX) return WGN_E_ARG;
    if (s.logits && s.epi != EPI_ARGMAX && s.epi != EPI_GELU_TANH) return WGN_E_ARG;
    if (s.norm != NORM_LAYER && s.beta) return WGN_E_ARG;
    if (s.norm == NORM_NONE && s.gamma) return WGN_E_ARG;
    if (s.norm != NORM_NONE && !(s.eps >= 0.0f)) return WGN_E_ARG;
    if (batch > 1 && s.x_stride < s.K) return WGN_E_ARG;
    if (batch > 1 && s.epi != EPI_ARGMAX && s.y_stride < s.N) return WGN_E_ARG;
    if (batch > 1 && s.residual && s.res_stride < s.N) return WGN_E_ARG;
    if (!a16(s.W) || (s.W_up && !a16(s.W_up))) return WGN_E_ALIGN;
    if (!a16(s.x) || (s.x_stride & 7)) return WGN_E_ALIGN;
    if ((s.gamma && !a16(s.gamma)) || (s.beta && !a16(s.beta))) return WGN_E_ALIGN;
    if ((s.bias && !a2(s.bias)) || (s.residual && !a2(s.residual))) return WGN_E_ALIGN;
    if (s.epi == EPI_ARGMAX) {
        if (!a4(s.y) || (s.logits && !a4(s.logits)) || (s.maxval && !a4(s.maxval))) return WGN_E_ALIGN;
    } else if (!a2(s.y) || (s.logits && !a4(s.logits))) {
        return WGN_E_ALIGN;
    }
    return WGN_OK;
}

// Byte ranges a stage reads (activations) and writes.
struct Range {
    uintptr_t lo, hi;
};
inline bool overlap(const Range &a, const Range &b) { return a.lo < b.hi && b.lo < a.hi; }
inline Range rng(const void *p, size_t bytes) {
    uintptr_t u = reinterpret_cast<uintptr_t>(p);
    return Range{u, u + bytes};
}

void stage_ranges(const wgn_stage &s, int32_t B, std::vector<Range> &reads, std::vector<Range> &writes,
                  std::vector<Range> &consts) {
    reads.clear();
    writes.clear();
    consts.clear();
    reads.push_back(rng(s.x, ((size_t)(B - 1) * s.x_stride + s.K) * 2));
    if (s.residual) reads.push_back(rng(s.residual, ((size_t)(B - 1) * s.res_stride + s.N) * 2));
    if (s.epi == EPI_ARGMAX) {
        writes.push_back(rng(s.y, (size_t)B * 4));
        if (s.logits) writes.push_back(rng(s.logits, (size_t)B * s.N * 4));
        if (s.maxval) writes.push_back(rng(s.maxval, (size_t)B * 4));
    } else {
        writes.push_back(rng(s.y, ((size_t)(B - 1) * s.y_stride + s.N) * 2));
        if (s.logits) writes.push_back(rng(s.logits, (size_t)B * s.N * 4));
    }
    consts.push_back(rng(s.W, (size_t)s.N * s.K * 2));
    if (s.W_up) consts.push_back(rng(s.W_up, (size_t)s.N * s.K * 2));
    if (s.gamma) consts.push_back(rng(s.gamma, (size_t)s.K * 2));
    if (s.beta) consts.push_back(rng(s.beta, (size_t)s.K * 2));
    if (s.bias) consts.push_back(rng(s.bias, (size_t)s.N * 2));
}

bool any_overlap(const std::vector<Range> &a, const std::vector<Range> &b) {
    for (const Range &x : a)
        for (const Range &y : b)
            if (overlap(x, y)) return true;
    return false;
}

bool same_source(const DevSource &s, const wgn_stage &st) {
    return s.x == (const uint16_t *)st.x && s.x_stride == st.x_stride && s.K == st.K && s.norm == st.norm &&
           s.gamma == (const uint16_t *)st.gamma && s.beta == (const uint16_t *)st.beta &&
           (st.norm == NORM_NONE || s.eps == st.eps);
}

// A stage pointer into the workspace's FP32 row-sum area (what = 0: the
// stage's own output y; 1: its fused residual add's addend post_F).
struct FFix {
    int32_t stage;
    size_t off;
    int32_t what;
};

// Host image of a device program.
struct Program {
    int32_t B = 1, G = 1;
    bool tile = false;                   // matrix-core streaming path
    std::vector<DevPhase> phases;
    std::vector<DevStage> stages;
    std::vector<DevSource> sources;
    std::vector<int32_t> rowb;
    std::vector<int32_t> phase_of_stage;
    std::vector<int32_t> group_end;      // per phase: one past the last phase of its launch group
    std::vector<int32_t> part_bytes;     // per phase: bytes of its partial-slot area
    std::vector<FFix> f_fix;             // pointers into the FP32 row-sum area, set at creation
    size_t f_bytes = 0;                  // bytes of that workspace area
    int32_t n_argmax = 0;
    std::vector<DevAttn> attn;           // attention items (part set at creation)
    size_t attn_part_bytes = 0;          // workspace bytes of the partials (shared by all items)
    size_t lds_end = 0;                  // dynamic LDS bytes of the largest phase (set with tile)
    size_t lds_total() const { return lds_end; }
    static size_t al16(size_t v) { return (v + 15) & ~size_t(15); }
};

// LDS bytes of the gain/shift area of one source (gain then shift, padded to
// whole units), matching the device's layout.
inline size_t prm_bytes_of(int32_t K) { return (size_t)nchunks_of(K) * UNIT * 2 * 2; }

DevStage make_dev_stage(const wgn_stage &s) {
    DevStage d;
    std::memset(&d, 0, sizeof d);
    d.W = (const uint16_t *)s.W;
    d.W_up = (const uint16_t *)s.W_up;
    d.bias = (const uint16_t *)s.bias;
    d.residual = (const uint16_t *)s.residual;
    d.y = s.y;
    d.logits = s.logits;
    d.maxval = s.maxval;
    d.res_stride = s.res_stride;
    d.y_stride = s.y_stride;
    d.N = s.N;
    d.K = s.K;
    d.epi = s.epi;
    d.nchunks = nchunks_of(s.K);
    d.parts = s.epi == EPI_SWIGLU ? 2 : 1;
    d.am_slot = -1;
    return d;
}

DevSource make_dev_source(const wgn_stage &s) {
    DevSource d;
    std::memset(&d, 0, sizeof d);
    d.x = (const uint16_t *)s.x;
    d.gamma = (const uint16_t *)s.gamma;
    d.beta = (const uint16_t *)s.beta;
    d.x_stride = s.x_stride;
    d.K = s.K;
    d.norm = s.norm;
    d.eps = s.eps;
    return d;
}

// Cost-balanced split of a phase's rows over G workgroups (cost = weight bytes).
void balance_rows(const std::vector<DevStage> &st, int32_t s0, int32_t ns, int32_t G, std::vector<int32_t> &out) {
    int64_t total = 0;
    for (int32_t i = 0; i < ns; ++i) total += (int64_t)st[s0 + i].N * st[s0 + i].parts * st[s0 + i].K;
    int32_t nrows = 0;
    for (int32_t i = 0; i < ns; ++i) nrows += st[s0 + i].N;
    const size_t base = out.size();
    out.resize(base + G + 1);
    // walk rows once, assigning boundary g when the cumulative cost reaches g*total/G
    int32_t g = 0, row = 0;
    int64_t cum = 0;
    for (int32_t i = 0; i < ns && g <= G; ++i) {
        const int64_t c = (int64_t)st[s0 + i].parts * st[s0 + i].K;
        for (int32_t r = 0; r < st[s0 + i].N; ++r, ++row) {
            while (g <= G && cum >= (total * g) / G) out[base + g++] = row;
            cum += c;
        }
    }
    while (g <= G) out[base + g++] = nrows;
    out[base + G] = nrows;
}

// Exact partial-slot demand of a phase under its workgroup partition: the
// largest number of waves any row-part segment spans (slots per row-part) and
// the largest number of row-parts any workgroup owns.
struct PhaseStats {
    int32_t jmax = 1, max_rp = 0;
};

PhaseStats phase_stats(const std::vector<DevStage> &st, const std::vector<int32_t> &rowb, const DevPhase &ph,
                       int32_t G, bool tile) {
    PhaseStats S;
    // The spans depend only on the workgroup's row count in each stage, and a
    // partition has few distinct such tuples: each is evaluated once (a large
    // single stage, e.g. an LM head, would otherwise cost a loop over every
    // row of every workgroup on each call).
    std::vector<std::vector<int32_t>> seen;
    for (int32_t g = 0; g < G; ++g) {
        const int32_t r0 = ph.rb_off >= 0 ? rowb[ph.rb_off + g] : even_row_begin(g, ph.nrows, G);
        const int32_t r1 = ph.rb_off >= 0 ? rowb[ph.rb_off + g + 1] : even_row_begin(g + 1, ph.nrows, G);
        int32_t U = 0, rp = 0;
        std::vector<int32_t> key;
        key.reserve(ph.nstages);
        for (int32_t i = 0; i < ph.nstages; ++i) {
            const DevStage &d = st[ph.stage0 + i];
            const StageSpan sp = stage_span(d, r0, r1, 0, 0);
            U += units_of(sp.nrows, d.parts, d.nchunks, tile);
            rp += sp.nrows * d.parts;
            key.push_back(sp.nrows);
        }
        S.max_rp = std::max(S.max_rp, rp);
        if (std::find(seen.begin(), seen.end(), key) != seen.end()) continue;
        seen.push_back(key);
        int32_t u_base = 0;
        for (int32_t i = 0; i < ph.nstages; ++i) {
            const DevStage &d = st[ph.stage0 + i];
            const StageSpan sp = stage_span(d, r0, r1, 0, 0);
            const int32_t nseg = (tile ? (sp.nrows + TILE_ROWS - 1) / TILE_ROWS : sp.nrows) * d.parts;
            for (int32_t sg = 0; sg < nseg; ++sg) {
                const int32_t a0 = u_base + sg * d.nchunks;
                const int32_t span =
                    first_wave(a0 + d.nchunks - 1, U, STREAM_WAVES) - first_wave(a0, U, STREAM_WAVES) + 1;
                S.jmax = std::max(S.jmax, span);
            }
            u_base += nseg * d.nchunks;
        }
    }
    return S;
}

// Place a phase's LDS areas after the fixed ones; false if they do not fit.
bool layout_phase(const Program &P, DevPhase &ph, const PhaseStats &S, bool carry, size_t &end_out,
                  int32_t &part_bytes) {
    const size_t nb = (size_t)P.B;
    size_t prm = 0;
    bool epi_in = false;
    for (int32_t i = 0; i < ph.nsrc; ++i)
        if (P.sources[ph.src0 + i].norm != NORM_NONE) prm += prm_bytes_of(P.sources[ph.src0 + i].K);
    for (int32_t i = 0; i < ph.nstages; ++i) {
        const DevStage &d = P.stages[ph.stage0 + i];
        if ((d.bias || d.residual || d.post_y) && !(d.carry & CARRY_OUT)) epi_in = true;
    }
    const size_t x = al256(nb * (size_t)ph.xb * 2);
    const size_t part = ph.att ? (size_t)ATTN_CMB_BYTES : Program::al16((size_t)S.max_rp * S.jmax * nb * 4);
    const size_t epi = epi_in ? Program::al16((size_t)S.max_rp * epi_rec((int32_t)nb) * 4) : 0;
    const size_t cy = carry ? Program::al16((size_t)S.max_rp * nb * 4) : 0;
    size_t o = lds_dyn_off(path_desc_bufs(P.tile));
    ph.x_off = (int32_t)o;
    o += x;
    ph.part_off = (int32_t)o;
    o += part;
    ph.prm_off = (int32_t)o;
    o += Program::al16(prm);
    ph.epi_off = (int32_t)o;
    o += epi;
    ph.carry_off = (int32_t)o;
    o += cy;
    ph.jmax = S.jmax;
    end_out = o;
    part_bytes = (int32_t)part;
    return o <= LDS_BUDGET && o < (1u << 18);
}

// x-hat row stride (elements) of a phase: its sources back to back, each
// padded to whole units; on the matrix-core path one extra 16-byte step keeps
// the 16 batch rows read by one instruction in distinct LDS banks.
int32_t xb_of(Program &P, DevPhase &ph) {
    int32_t xb = 0;
    for (int32_t i = 0; i < ph.nsrc; ++i) {
        P.sources[ph.src0 + i].lds_off = xb;
        xb += nchunks_of(P.sources[ph.src0 + i].K) * UNIT;
    }
    return P.tile ? xb + 8 : xb;
}

// Phase selection of the matrix-core path.
bool use_tile(int32_t B, int32_t path) { return path == 2 || (path == 0 && B > MAX_BATCH_VALU); }

// A stage as the planner places it: a caller's stage, possibly rewritten.
struct PStage {
    wgn_stage s;
    int32_t user = -1;          // caller index whose output this stage writes
    bool product_only = false;  // writes FP32 row sums to the workspace (EPI_F32)
    int32_t post = -1;          // caller index of a stage whose residual add runs in this epilogue
    size_t f_off = 0;           // workspace offset of those FP32 sums
};

// Cross-stage rewrite ("hoisting"): a stage S whose input vector no stage of
// the chain writes and whose epilogue is a plain residual add, with the
// residual being the output of an earlier stage D, is split in two.  Its
// product runs in the phase before D's (it depends on nothing) and leaves FP32
// row sums in the workspace; its residual add runs in D's epilogue on D's
// freshly rounded output.  The result is the same function (one rounding of
// residual + sums), and the dependency D -> S -> (readers of S) loses a
// device-wide phase boundary.  In a decoder block this is the attention
// output projection, whose residual is the previous block's output.
void find_hoists(const wgn_stage *st, int32_t n, int32_t B, std::vector<int32_t> &into, std::vector<int32_t> &post_of) {
    into.assign(n, -1);
    post_of.assign(n, -1);
    std::vector<std::vector<Range>> R(n), Wr(n), C(n);
    for (int32_t i = 0; i < n; ++i) stage_ranges(st[i], B, R[i], Wr[i], C[i]);
    for (int32_t s = 0; s < n; ++s) {
        const wgn_stage &S = st[s];
        if (S.epi != EPI_NONE || !S.residual) continue;
        const Range rx = rng(S.x, ((size_t)(B - 1) * S.x_stride + S.K) * 2);
        const Range rres = rng(S.residual, ((size_t)(B - 1) * S.res_stride + S.N) * 2);
        const Range ry = rng(S.y, ((size_t)(B - 1) * S.y_stride + S.N) * 2);
        bool x_written = false;
        for (int32_t t = 0; t < n && !x_written; ++t)
            for (const Range &w : Wr[t]) x_written |= overlap(w, rx);
        if (x_written) continue;
        int32_t D = -1;
        for (int32_t t = s - 1; t >= 0 && D < 0; --t)
            for (const Range &w : Wr[t])
                if (overlap(w, rres)) D = t;
        if (D < 0) continue;
        const wgn_stage &Ds = st[D];
        if (Ds.epi == EPI_ARGMAX || Ds.y != S.residual || Ds.N != S.N || post_of[D] >= 0 || into[D] >= 0) continue;
        if (B > 1 && Ds.y_stride != S.res_stride) continue;
        bool ok = !overlap(ry, rng(Ds.x, ((size_t)(B - 1) * Ds.x_stride + Ds.K) * 2));
        if (Ds.residual) ok &= !overlap(ry, rng(Ds.residual, ((size_t)(B - 1) * Ds.res_stride + Ds.N) * 2));
        for (int32_t t = D + 1; t < s && ok; ++t) {
            for (const Range &r : R[t]) ok &= !overlap(r, ry);
            for (const Range &w : Wr[t]) ok &= !overlap(w, ry) && !overlap(w, rres);
        }
        if (!ok) continue;
        into[s] = D;
        post_of[D] = s;
    }
}

// Checks of one attention item of a chain, and the byte ranges it reads and
// writes (caches included).
wgn_status check_attn(const wgn_attn_stage &s, int32_t B, std::vector<Range> &reads, std::vector<Range> &writes) {
    reads.clear();
    writes.clear();
    if (!s.q || !s.k_new || !s.v_new || !s.k_cache || !s.v_cache || !s.pos || !s.out) return WGN_E_ARG;
    if (s.q_heads < 1 || s.kv_heads < 1 || s.slots < 1 || s.q_heads % s.kv_heads) return WGN_E_ARG;
    if (!std::isfinite(s.scale)) return WGN_E_ARG;
    if (s.head_dim != ATTN_D || s.q_heads / s.kv_heads > ATTN_MAX_GROUP) return WGN_E_UNSUPPORTED;
    // 32-bit buffer offsets: one (batch row, head) cache row set, and the partials
    if ((int64_t)s.slots * ATTN_D * 2 >= (1ll << 31)) return WGN_E_UNSUPPORTED;
    const int64_t qn = (int64_t)s.q_heads * ATTN_D, kn = (int64_t)s.kv_heads * ATTN_D;
    if (B > 1 && (s.q_stride < qn || s.k_stride < kn || s.v_stride < kn || s.out_stride < qn)) return WGN_E_ARG;
    if (!a16(s.q) || !a16(s.k_new) || !a16(s.v_new) || !a16(s.k_cache) || !a16(s.v_cache) || !a16(s.out) ||
        !a4(s.pos))
        return WGN_E_ALIGN;
    if ((s.q_stride & 7) || (s.k_stride & 7) || (s.v_stride & 7) || (s.out_stride & 7)) return WGN_E_ALIGN;
    const size_t cache = (size_t)B * s.kv_heads * s.slots * ATTN_D * 2;
    const Range rk = rng(s.k_cache, cache), rv = rng(s.v_cache, cache);
    const Range ro = rng(s.out, ((size_t)(B - 1) * s.out_stride + qn) * 2);
    const Range rin[4] = {rng(s.q, ((size_t)(B - 1) * s.q_stride + qn) * 2),
                          rng(s.k_new, ((size_t)(B - 1) * s.k_stride + kn) * 2),
                          rng(s.v_new, ((size_t)(B - 1) * s.v_stride + kn) * 2), rng(s.pos, (size_t)B * 4)};
    if (overlap(rk, rv) || overlap(ro, rk) || overlap(ro, rv)) return WGN_E_ARG;
    for (const Range &x : rin)
        if (overlap(x, rk) || overlap(x, rv) || overlap(x, ro)) return WGN_E_ARG;
    for (const Range &x : rin) reads.push_back(x);
    reads.push_back(rk);
    reads.push_back(rv);
    writes.push_back(ro);
    writes.push_back(rk);
    writes.push_back(rv);
    return WGN_OK;
}

// Device descriptor of an attention item over G workgroups: about one scores
// item per workgroup, each (batch row, key/value head) with nchunk chunks of
// whole passes (the kernel splits each row's valid length over them).
DevAttn make_dev_attn(const wgn_attn_stage &s, int32_t B, int32_t G) {
    DevAttn d;
    std::memset(&d, 0, sizeof d);
    d.q = (const uint16_t *)s.q;
    d.k_new = (const uint16_t *)s.k_new;
    d.v_new = (const uint16_t *)s.v_new;
    d.k_cache = (uint16_t *)s.k_cache;
    d.v_cache = (uint16_t *)s.v_cache;
    d.pos = s.pos;
    d.out = (uint16_t *)s.out;
    d.q_stride = s.q_stride;
    d.k_stride = s.k_stride;
    d.v_stride = s.v_stride;
    d.out_stride = s.out_stride;
    d.hq = s.q_heads;
    d.hkv = s.kv_heads;
    d.slots = s.slots;
    const int32_t pairs = B * s.kv_heads;
    const int32_t per = std::max(1, G / pairs);
    d.nchunk = std::min(per, (s.slots + attn_pass(B) - 1) / attn_pass(B));
    d.scale_log2 = (float)((double)s.scale * 1.4426950408889634);  // log2(e)
    return d;
}

size_t attn_part_bytes_of(const DevAttn &d, int32_t B) {
    return (size_t)B * d.hkv * d.nchunk * attn_part_floats(d.hq / d.hkv) * sizeof(float);
}

wgn_status plan(const wgn_stage *stages, int32_t n, int32_t B, int32_t G, int32_t path, bool fuse, Program &P,
                const wgn_attn_stage *att = nullptr, const int32_t *att_before = nullptr, int32_t n_att = 0) {
    if (!stages || n < 1 || G < 1) return WGN_E_ARG;
    if (n_att < 0 || (n_att > 0 && (!att || !att_before))) return WGN_E_ARG;
    for (int32_t k = 0; k < n_att; ++k)
        if (att_before[k] < 0 || att_before[k] > n || (k > 0 && att_before[k] < att_before[k - 1])) return WGN_E_ARG;
    // the hoists assume an attention output that no stage writes
    if (n_att > 0) fuse = false;
    for (int32_t i = 0; i < n; ++i) {
        wgn_status st = check_stage(stages[i], B);
        if (st != WGN_OK) return st;
    }
    if (path < 0 || path > 2) return WGN_E_ARG;
    const bool tile = use_tile(B, path);
    if (!tile && B > MAX_BATCH_VALU) return WGN_E_UNSUPPORTED;
    // weights and norm parameters must not be written by any stage
    std::vector<Range> r, w, c, allw;
    for (int32_t i = 0; i < n; ++i) {
        stage_ranges(stages[i], B, r, w, c);
        allw.insert(allw.end(), w.begin(), w.end());
    }
    for (int32_t k = 0; k < n_att; ++k) {
        const wgn_status st = check_attn(att[k], B, r, w);
        if (st != WGN_OK) return st;
        allw.insert(allw.end(), w.begin(), w.end());
    }
    for (int32_t i = 0; i < n; ++i) {
        stage_ranges(stages[i], B, r, w, c);
        if (any_overlap(c, allw)) return WGN_E_ARG;
    }
    std::vector<int32_t> into, post_of;
    if (fuse) find_hoists(stages, n, B, into, post_of);
    else into.assign(n, -1), post_of.assign(n, -1);

    // Group the stages (hoisted ones removed) into phase lists, then place the
    // hoisted products; a product that finds no room, or whose phase then does
    // not fit in LDS, undoes its hoist and the plan starts over.
  replan:
    std::vector<PStage> ps;
    std::vector<std::vector<int32_t>> lists;
    std::vector<int32_t> list_att;  // per list: -1, or the attention item it stands for
    for (;;) {
        ps.clear();
        lists.clear();
        list_att.clear();
        std::vector<int32_t> phase_of_ps;
        std::vector<Range> ph_reads, ph_writes;
        std::vector<int32_t> pos(n, -1);
        int32_t next_att = 0;
        auto place_attn = [&](int32_t before) {
            for (; next_att < n_att && att_before[next_att] == before; ++next_att) {
                lists.emplace_back();
                list_att.push_back(next_att);
            }
        };
        for (int32_t i = 0; i < n; ++i) {
            place_attn(i);
            if (into[i] >= 0) continue;
            PStage p;
            p.s = stages[i];
            p.user = i;
            p.post = post_of[i];
            stage_ranges(stages[i], B, r, w, c);
            if (p.post >= 0) {
                const wgn_stage &S = stages[p.post];
                w.push_back(rng(S.y, ((size_t)(B - 1) * S.y_stride + S.N) * 2));
            }
            bool conflict = lists.empty() || list_att.back() >= 0 || any_overlap(r, ph_writes) ||
                            any_overlap(w, ph_reads) || any_overlap(w, ph_writes);
            if (!conflict) {
                std::vector<DevSource> srcs;
                for (int32_t q : lists.back()) {
                    bool have = false;
                    for (const DevSource &d : srcs) have |= same_source(d, ps[q].s);
                    if (!have) srcs.push_back(make_dev_source(ps[q].s));
                }
                bool have = false;
                for (const DevSource &d : srcs) have |= same_source(d, stages[i]);
                if ((!have && (int32_t)srcs.size() >= MAX_SRC) || (int32_t)lists.back().size() >= MAX_RUNS)
                    conflict = true;
            }
            if (conflict) {
                lists.emplace_back();
                list_att.push_back(-1);
                ph_reads.clear();
                ph_writes.clear();
            }
            pos[i] = (int32_t)ps.size();
            lists.back().push_back((int32_t)ps.size());
            phase_of_ps.push_back((int32_t)lists.size() - 1);
            ps.push_back(p);
            ph_reads.insert(ph_reads.end(), r.begin(), r.end());
            ph_writes.insert(ph_writes.end(), w.begin(), w.end());
        }
        place_attn(n);
        bool undone = false;
        for (int32_t s = 0; s < n; ++s) {
            if (into[s] < 0) continue;
            const int32_t D = into[s];
            bool placed = false;
            for (int32_t q = phase_of_ps[pos[D]] - 1; q >= 0 && !placed; --q) {
                std::vector<DevSource> srcs;
                for (int32_t k : lists[q]) {
                    bool have = false;
                    for (const DevSource &d : srcs) have |= same_source(d, ps[k].s);
                    if (!have) srcs.push_back(make_dev_source(ps[k].s));
                }
                bool have = false;
                for (const DevSource &d : srcs) have |= same_source(d, stages[s]);
                if ((!have && (int32_t)srcs.size() >= MAX_SRC) || (int32_t)lists[q].size() >= MAX_RUNS) continue;
                PStage p;
                p.s = stages[s];
                p.user = s;
                p.s.epi = EPI_NONE;
                p.s.residual = nullptr;
                p.s.res_stride = 0;
                p.s.bias = nullptr;
                p.product_only = true;
                lists[q].push_back((int32_t)ps.size());
                ps.push_back(p);
                placed = true;
            }
            if (!placed) {
                into[s] = -1;
                post_of[D] = -1;
                undone = true;
            }
        }
        if (!undone) break;
    }
    // workspace areas of the FP32 row sums
    P = Program();
    P.B = B;
    P.G = G;
    P.tile = tile;
    P.lds_end = (size_t)lds_dyn_off(path_desc_bufs(tile));
    P.phase_of_stage.assign(n, -1);
    for (PStage &p : ps) {
        if (!p.product_only) continue;
        p.f_off = P.f_bytes;
        P.f_bytes += al256((size_t)B * p.s.N * 4);
    }
    for (PStage &p : ps) {
        if (p.post < 0) continue;
        for (const PStage &q : ps)
            if (q.product_only && q.user == p.post) p.f_off = q.f_off;
    }

    wgn_status fail = WGN_OK;
    auto push_phase = [&](DevPhase &ph, const PhaseStats &S, bool carry) -> bool {
        size_t end = 0;
        int32_t pb = 0;
        if (!layout_phase(P, ph, S, carry, end, pb)) return false;
        P.lds_end = std::max(P.lds_end, end);
        P.phases.push_back(ph);
        P.part_bytes.push_back(pb);
        return true;
    };
    for (int32_t k = 0; k < n_att; ++k) {
        P.attn.push_back(make_dev_attn(att[k], B, G));
        P.attn_part_bytes = std::max(P.attn_part_bytes, attn_part_bytes_of(P.attn.back(), B));
    }
    for (size_t li = 0; li < lists.size(); ++li) {
        const std::vector<int32_t> &lst = lists[li];
        if (list_att[li] >= 0) {
            // attention: a scores phase and a merge phase, no weights
            for (int32_t kind = 0; kind < 2 && fail == WGN_OK; ++kind) {
                DevPhase ph;
                std::memset(&ph, 0, sizeof ph);
                ph.stage0 = (int32_t)P.stages.size();
                ph.src0 = (int32_t)P.sources.size();
                ph.rb_off = -1;
                // one unit of x-hat per batch row, zeroed by the kernel: the
                // phase's empty blocks read it against zero weights
                ph.xb = P.tile ? UNIT + 8 : UNIT;
                ph.wait = P.phases.empty() ? 0 : 1;
                ph.att = 2 * list_att[li] + 1 + kind;
                const int32_t first = (int32_t)P.phases.size();
                if (!push_phase(ph, phase_stats(P.stages, P.rowb, ph, G, tile), false)) fail = WGN_E_UNSUPPORTED;
                else P.group_end.push_back(first + 1);
            }
            if (fail != WGN_OK) break;
            continue;
        }
        DevPhase cur;
        std::memset(&cur, 0, sizeof cur);
        cur.stage0 = (int32_t)P.stages.size();
        cur.src0 = (int32_t)P.sources.size();
        std::vector<int32_t> users;
        for (int32_t k : lst) {
            const PStage &p = ps[k];
            int32_t src_idx = -1;
            for (int32_t q = cur.src0; q < (int32_t)P.sources.size(); ++q)
                if (same_source(P.sources[q], p.s)) src_idx = q - cur.src0;
            if (src_idx < 0) {
                P.sources.push_back(make_dev_source(p.s));
                src_idx = (int32_t)P.sources.size() - 1 - cur.src0;
            }
            DevStage d = make_dev_stage(p.s);
            d.src = src_idx;
            if (p.s.epi == EPI_ARGMAX) d.am_slot = P.n_argmax++;
            if (p.product_only) {
                d.epi = EPI_F32;
                d.y = nullptr;
                d.y_stride = p.s.N;
                P.f_fix.push_back({(int32_t)P.stages.size(), p.f_off, 0});
            }
            if (p.post >= 0) {
                const wgn_stage &S = stages[p.post];
                d.post_y = S.y;
                d.post_stride = S.y_stride;
                d.post_bias = (const uint16_t *)S.bias;
                P.f_fix.push_back({(int32_t)P.stages.size(), p.f_off, 1});
                users.push_back(p.post);
            }
            P.stages.push_back(d);
            if (p.user >= 0 && !p.product_only) users.push_back(p.user);
        }
        cur.nstages = (int32_t)P.stages.size() - cur.stage0;
        cur.nsrc = (int32_t)P.sources.size() - cur.src0;
        int32_t nrows = 0;
        for (int32_t i = 0; i < cur.nstages; ++i) {
            DevStage &d = P.stages[cur.stage0 + i];
            d.row_off = nrows;
            nrows += d.N;
        }
        cur.nrows = nrows;
        cur.xb = xb_of(P, cur);
        cur.rb_off = (int32_t)P.rowb.size();
        balance_rows(P.stages, cur.stage0, cur.nstages, G, P.rowb);
        cur.wait = P.phases.empty() ? 0 : 1;
        const int32_t first = (int32_t)P.phases.size();
        DevPhase whole = cur;
        if (push_phase(whole, phase_stats(P.stages, P.rowb, whole, G, tile), false)) {
            P.group_end.push_back(first + 1);
            for (int32_t u : users) P.phase_of_stage[u] = first;
            continue;
        }
        // A hoisted product made this phase too large: undo that hoist.
        bool undo = false;
        for (int32_t k : lst)
            if (ps[k].product_only) {
                post_of[into[ps[k].user]] = -1;
                into[ps[k].user] = -1;
                undo = true;
            }
        if (undo) goto replan;
        // The inputs do not fit in LDS: stream the phase in K windows.  Only a
        // phase with one un-normalised input can be windowed (a norm needs the
        // whole vector for its statistics).
        const DevSource src0 = P.sources[cur.src0];
        if (cur.nsrc != 1 || src0.norm != NORM_NONE) {
            fail = WGN_E_UNSUPPORTED;
            break;
        }
        const std::vector<DevStage> orig(P.stages.begin() + cur.stage0, P.stages.end());
        std::vector<FFix> fix_keep;
        for (const FFix &f : P.f_fix)
            if (f.stage < cur.stage0) fix_keep.push_back(f);
        std::vector<FFix> fix_here;
        for (const FFix &f : P.f_fix)
            if (f.stage >= cur.stage0) fix_here.push_back(f);
        const int32_t nch = nchunks_of(src0.K);
        bool done = false;
        for (int32_t nw = nch - 1; nw >= 1 && !done; --nw) {
            const int32_t S = (nch + nw - 1) / nw;
            P.stages.resize(cur.stage0);
            P.sources.resize(cur.src0);
            P.f_fix = fix_keep;
            std::vector<DevPhase> win;
            PhaseStats worst;
            for (int32_t s = 0; s < S; ++s) {
                const int32_t c0 = s * nw, cn = std::min(nw, nch - c0);
                DevPhase ph = cur;
                ph.stage0 = (int32_t)P.stages.size();
                ph.src0 = (int32_t)P.sources.size();
                ph.nsrc = 1;
                ph.wait = s == 0 ? cur.wait : 0;
                DevSource sw = src0;
                sw.x = src0.x + (size_t)c0 * UNIT;
                sw.K = std::min(nw * UNIT, src0.K - c0 * UNIT);
                P.sources.push_back(sw);
                for (size_t oi = 0; oi < orig.size(); ++oi) {
                    DevStage d = orig[oi];
                    d.c0 = c0;
                    d.nchunks = cn;
                    d.carry = (s > 0 ? CARRY_IN : 0) | (s < S - 1 ? CARRY_OUT : 0);
                    if (s < S - 1) {
                        d.bias = nullptr;    // bias, residual and fused adds enter in the last window only
                        d.residual = nullptr;
                        d.am_slot = -1;
                        d.post_y = nullptr;
                    } else {
                        for (const FFix &f : fix_here)
                            if (f.stage == cur.stage0 + (int32_t)oi)
                                P.f_fix.push_back({(int32_t)P.stages.size(), f.off, f.what});
                    }
                    P.stages.push_back(d);
                }
                ph.xb = xb_of(P, ph);
                const PhaseStats st = phase_stats(P.stages, P.rowb, ph, G, tile);
                worst.jmax = std::max(worst.jmax, st.jmax);
                worst.max_rp = std::max(worst.max_rp, st.max_rp);
                win.push_back(ph);
            }
            // every window uses one layout: x-hat sized by the first (widest)
            // window, epilogue inputs by the last
            DevPhase probe = win[S - 1];
            probe.xb = win[0].xb;
            size_t end = 0;
            int32_t pb = 0;
            if (!layout_phase(P, probe, worst, true, end, pb)) continue;
            for (DevPhase &ph : win) {
                ph.xb = probe.xb;
                ph.x_off = probe.x_off;
                ph.part_off = probe.part_off;
                ph.prm_off = probe.prm_off;
                ph.epi_off = probe.epi_off;
                ph.carry_off = probe.carry_off;
                ph.jmax = probe.jmax;
                P.phases.push_back(ph);
                P.part_bytes.push_back(pb);
            }
            P.lds_end = std::max(P.lds_end, end);
            const int32_t last = first + S - 1;
            for (int32_t s = 0; s < S; ++s) P.group_end.push_back(last + 1);
            for (int32_t u : users) P.phase_of_stage[u] = last;
            done = true;
        }
        if (!done) {
            fail = WGN_E_UNSUPPORTED;
            break;
        }
    }
    if (fail != WGN_OK) return fail;
    return WGN_OK;
}

struct WsLayout {
    // ctr..am_part is the synchronisation area (flags, run counter, tickets, error word)
    size_t phases, stages, sources, rowb, runimg, phinfo, att, touch, ctr, run, tickets, err, am_part, fsum, attp,
        trace, total;
};

WsLayout ws_layout(const Program &P, bool trace) {
    WsLayout L;
    size_t o = 0;
    L.phases = o;
    o += al256(P.phases.size() * sizeof(DevPhase));
    L.stages = o;
    o += al256(P.stages.size() * sizeof(DevStage));
    L.sources = o;
    o += al256(P.sources.size() * sizeof(DevSource));
    L.rowb = o;
    o += al256(P.rowb.size() * sizeof(int32_t));
    L.runimg = o;  // every (phase, workgroup) run list, as the kernel would build it
    o += al256(P.phases.size() * (size_t)P.G * RUN_BUF_STRIDE);
    L.phinfo = o;  // every phase's source table and normalisation jobs
    o += al256(P.phases.size() * (size_t)PHASE_INFO_BYTES);
    L.att = o;     // attention items
    o += al256(P.attn.size() * sizeof(DevAttn));
    L.touch = o;   // weight ranges of every launch group, for a prefetch plan's touch pass
    o += al256(P.phases.size() * (size_t)MAX_TOUCH * sizeof(TouchRange));
    L.ctr = o;
    o += al256(P.phases.size() * (size_t)flag_row(P.G) * sizeof(uint32_t));
    L.run = o;
    o += 256;
    L.tickets = o;
    o += al256((size_t)(P.n_argmax + 1) * sizeof(uint32_t));
    L.err = o;
    o += 256;
    L.am_part = o;
    o += al256((size_t)P.n_argmax * P.G * P.B * sizeof(uint64_t));
    L.fsum = o;
    o += P.f_bytes;
    L.attp = o;    // attention partials
    o += al256(P.attn_part_bytes);
    L.trace = o;
    if (trace) o += al256(P.phases.size() * (size_t)P.G * TRACE_POINTS * sizeof(uint64_t));
    L.total = o;
    return L;
}

int32_t resolve_grid(const wgn_chain_opts *opts) {
    int32_t g = opts ? opts->grid : 0;
    if (g > 0) return g;
    DevInfo d = device_info();
    return d.cus > 0 ? d.cus : 256;
}

// ------------------------------------------------- single-stage launches
struct SingleLaunch {
    KArgs a;
    int32_t G;
    bool tile;
    size_t lds;
    size_t ws;
};

// Geometry of a one-stage, one-phase launch (rows split evenly); false if its
// LDS areas do not fit (such a stage needs K windows, i.e. a chain).
bool single_geometry(const wgn_stage &s, int32_t B, int32_t cus, SingleLaunch &L) {
    std::memset(&L.a, 0, sizeof L.a);
    L.tile = use_tile(B, 0);
    const int32_t parts = s.epi == EPI_SWIGLU ? 2 : 1;
    const int32_t nch = nchunks_of(s.K);
    const int64_t units = (int64_t)units_of(s.N, parts, nch, L.tile);
    // about two units per streaming wave
    const int64_t per_wg = 2 * STREAM_WAVES;
    int64_t g = (units + per_wg - 1) / per_wg;
    g = std::max<int64_t>(1, std::min<int64_t>(g, cus));
    g = std::min<int64_t>(g, s.N);
    L.G = (int32_t)g;
    Program P;
    P.B = B;
    P.G = L.G;
    P.tile = L.tile;
    P.lds_end = (size_t)lds_dyn_off(path_desc_bufs(L.tile));
    P.stages.push_back(make_dev_stage(s));
    P.sources.push_back(make_dev_source(s));
    DevPhase &ph = L.a.iph;
    std::memset(&ph, 0, sizeof ph);
    ph.stage0 = 0;
    ph.nstages = 1;
    ph.src0 = 0;
    ph.nsrc = 1;
    ph.nrows = s.N;
    ph.wait = 0;
    ph.rb_off = -1;
    ph.xb = xb_of(P, ph);
    const PhaseStats S = phase_stats(P.stages, P.rowb, ph, L.G, L.tile);
    size_t end = 0;
    int32_t pb = 0;
    const bool fits = layout_phase(P, ph, S, false, end, pb);
    L.lds = end;
    L.ws = s.epi == EPI_ARGMAX ? 256 + al256((size_t)L.G * B * sizeof(uint64_t)) : 0;
    L.a.ist = P.stages[0];
    L.a.ist.src = 0;
    L.a.ist.row_off = 0;
    L.a.ist.am_slot = s.epi == EPI_ARGMAX ? 0 : -1;
    L.a.isrc = P.sources[0];
    L.a.p0 = 0;
    L.a.p1 = 1;
    L.a.persistent = 0;
    L.a.G = L.G;
    L.a.nb = B;
    L.a.wait_ticks = WAIT_TICKS;
    L.a.n_argmax = s.epi == EPI_ARGMAX ? 1 : 0;
    return fits;
}

}  // namespace

// =================================================================== C ABI
struct wgn_chain {
    Program P;
    KArgs a;
    bool trace;
    int32_t mode;
    int32_t ring;           // block-buffer ring of the vector path's streaming waves
    size_t lds;
    void *ws;
    WsLayout L;
    // mode 1: first phase of each launch, the number of weight ranges its
    // touch pass reads (table in the workspace), and the events that fork a
    // plan's touch passes off the main stream and join them back
    std::vector<int32_t> launch0, touch_n;
    std::vector<hipEvent_t> ev;
    ~wgn_chain() {
        for (hipEvent_t e : ev)
            if (e) (void)hipEventDestroy(e);
    }
};

namespace {
int32_t opts_path(const wgn_chain_opts *opts) { return opts ? opts->path : 0; }
bool opts_fuse(const wgn_chain_opts *opts) { return !(opts && opts->no_fuse); }

// The vector path's ring for a chain, by the shape that was measured fastest
// with each (decode step at batch 1-4, LayerNorm chain, decode step with
// attention phases): phases that give a streaming wave fewer than 4 units on
// average want many phases in flight (ring 1), at batch 1 up to 12 (a decode
// step with attention phases, 10: 1,445 against 1,487 us with ring 0);
// otherwise batch 2-4 streams best with interleaved refills (ring 2) and
// batch 1 with two large bursts (ring 0: the decode step, 29 units).
int32_t auto_ring(const Program &P) {
    if (P.tile || P.phases.empty()) return 0;
    double units = 0.0;
    for (const DevPhase &ph : P.phases)
        for (int32_t si = ph.stage0; si < ph.stage0 + ph.nstages; ++si) {
            const DevStage &st = P.stages[si];
            units += (double)st.N * st.parts * st.nchunks;
        }
    const double per_wave = units / ((double)P.phases.size() * P.G * STREAM_WAVES);
    if (per_wave < 4.0 || (P.B == 1 && per_wave < 12.0)) return 1;
    return P.B >= 2 ? 2 : 0;
}

// Whether a chain's phases are small: under 128 KB of weights per workgroup
// per phase on average (the LayerNorm chain, a decode step with attention
// phases; not the decode step's 58 phases of 200 KB and more).
bool small_phases(const Program &P) {
    if (P.phases.empty()) return false;
    double bytes = 0.0;
    for (const DevStage &st : P.stages) bytes += (double)st.N * st.parts * st.K * 2.0;
    return bytes / ((double)P.phases.size() * P.G) < 128.0 * 1024.0;
}

// Point the stages' FP32 row-sum pointers into the workspace area at base.
void patch_fsum(Program &P, char *base) {
    for (const FFix &f : P.f_fix) {
        if (f.what == 0) P.stages[f.stage].y = base + f.off;
        else P.stages[f.stage].post_F = (const float *)(base + f.off);
    }
}
}  // namespace


// ------------------------------------------------------------ decode attention
namespace {
struct AttLayout {
    int32_t top = 0;
    int32_t count[ATT_MAX_LEVELS + 1] = {};
    size_t part_off[ATT_MAX_LEVELS] = {};
    size_t tick_off[ATT_MAX_LEVELS + 1] = {};
    size_t total = 0;
};

// Shape checks shared by the workspace query and the call.
wgn_status att_shape(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t slots, int32_t head_dim,
                     AttLayout &L) {
    if (batch < 1 || batch > 65535 || q_heads < 1 || kv_heads < 1 || kv_heads > 65535 || slots < 1)
        return WGN_E_ARG;
    if (q_heads % kv_heads) return WGN_E_ARG;
    if (head_dim != ATT_D || q_heads / kv_heads > ATT_MAX_GROUP || slots > ATT_MAX_SLOTS) return WGN_E_UNSUPPORTED;
    L.top = att_levels(slots, L.count);
    if (L.top < 0) return WGN_E_UNSUPPORTED;
    const size_t entry = (size_t)att_entry_floats(q_heads / kv_heads) * sizeof(float);
    const size_t heads = (size_t)batch * kv_heads;
    size_t off = 0;
    for (int32_t l = 0; l < L.top; ++l) {
        L.part_off[l] = off;
        off += al256(heads * L.count[l] * entry);
    }
    for (int32_t l = 1; l <= L.top; ++l) {
        L.tick_off[l] = off;
        off += al256(heads * L.count[l] * sizeof(uint32_t));
    }
    L.total = std::max<size_t>(off, 256);
    return WGN_OK;
}
}  // namespace

extern "C" {

const char *wgn_status_string(int32_t s) {
    switch (s) {
    case WGN_OK: return "ok";
    case WGN_E_ARG: return "invalid argument";
    case WGN_E_ALIGN: return "misaligned pointer or stride";
    case WGN_E_UNSUPPORTED: return "unsupported request";
    case WGN_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case WGN_E_HIP: return "HIP runtime error";
    case WGN_E_DEVICE: return "no usable gfx950 device";
    case WGN_E_TIMEOUT: return "in-kernel wait timed out";
    default: return "unknown status";
    }
}

int32_t wgn_version(void) { return VERSION; }

const char *wgn_last_hip_error(void) { return g_last_hip_error; }

int32_t wgn_device_cu_count(void) { return device_info().cus; }

int32_t wgn_first_wave_of_unit(int32_t u, int32_t units, int32_t waves) {
    if (units <= 0 || waves <= 0 || u < 0 || u >= units) return -1;
    return first_wave(u, units, waves);
}

size_t wgn_gemv_norm_workspace_bytes(const wgn_stage *stage, int32_t batch) {
    if (!stage || check_stage(*stage, batch) != WGN_OK) return 0;
    SingleLaunch L;
    DevInfo d = device_info();
    if (!single_geometry(*stage, batch, d.cus > 0 ? d.cus : 256, L)) return 0;
    return L.ws;
}

wgn_status wgn_gemv_norm(const wgn_stage *stage, int32_t batch, void *workspace, size_t ws_bytes,
                         wgn_stream stream) {
    if (!stage) return WGN_E_ARG;
    wgn_status st = check_stage(*stage, batch);
    if (st != WGN_OK) return st;
    DevInfo d = device_info();
    if (!d.ok) return WGN_E_DEVICE;
    SingleLaunch L;
    if (!single_geometry(*stage, batch, d.cus, L)) return WGN_E_UNSUPPORTED;
    if (L.ws) {
        if (!workspace || ws_bytes < L.ws || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return WGN_E_WORKSPACE;
        L.a.tickets = (uint32_t *)workspace;
        L.a.err = (uint32_t *)((char *)workspace + 64);
        L.a.am_part = (uint64_t *)((char *)workspace + 256);
    }
    L.a.ist.W = (const uint16_t *)stage->W;
    hipError_t e = note(launch_chain(batch, L.tile, 0, L.a, L.G, L.lds, (hipStream_t)stream), "gemv_norm launch");
    return e == hipSuccess ? WGN_OK : WGN_E_HIP;
}

// ------------------------------------------------ batched product (wgn_gemm.hip)
namespace wgn {

// One launch of the batched path: stages [first, first + n) of a stage list,
// which read the same input with the same normalisation.
struct GemmGroup {
    GemmLaunch L;
    int32_t first = 0, n = 0;
    bool swiglu = false;
    bool norm = false;  // x-hat is written into the workspace first
    int32_t norm_stage = -1;  // the first normalised stage: its input and norm make the x-hat
    size_t lds = 0, ws = 0;
    size_t counters = 0;  // bytes of tickets and keys at the start of the workspace
    size_t off_ticket[GEMM_MAX_GROUP] = {}, off_part[GEMM_MAX_GROUP] = {};
    size_t off_keys = 0, off_xhat = 0;
};

// Workgroups of a batched launch per compute unit, and the fewest windows a
// workgroup streams (fewer would mostly add contributions to be summed).
#ifndef WGN_GEMM_WG_PER_CU
#define WGN_GEMM_WG_PER_CU 1
#endif
constexpr int32_t GEMM_MIN_UNITS = 4;
// Tiles per workgroup of the launch from which a stage's tiles become whole
// workgroups of their own.
constexpr int32_t GEMM_TILES_WHOLE = 4;

// Whether two normalised stages read the same x-hat: the same input, length
// and normalisation.
bool same_norm_input(const wgn_stage &a, const wgn_stage &b) {
    return a.x == b.x && a.x_stride == b.x_stride && a.K == b.K && a.norm == b.norm && a.gamma == b.gamma &&
           a.beta == b.beta && std::memcmp(&a.eps, &b.eps, sizeof a.eps) == 0;
}

// Whether stage st[j] may join the launch of stages st[i..j): the same
// epilogue family (one kernel instance), no argmax, and if it is normalised,
// the same x-hat as the launch's other normalised stages (one norm pass per
// launch).  Stages without normalisation read their own inputs.
bool may_join(const wgn_stage *st, int32_t i, int32_t j) {
    const wgn_stage &b = st[j];
    if ((st[i].epi == EPI_SWIGLU) != (b.epi == EPI_SWIGLU) || st[i].epi == EPI_ARGMAX || b.epi == EPI_ARGMAX)
        return false;
    if (b.norm == NORM_NONE) return true;
    for (int32_t k = i; k < j; ++k)
        if (st[k].norm != NORM_NONE) return same_norm_input(st[k], b);
    return true;
}

// The first normalised stage of st[0..n), or -1.
int32_t first_normalised(const wgn_stage *st, int32_t n) {
    for (int32_t i = 0; i < n; ++i)
        if (st[i].norm != NORM_NONE) return i;
    return -1;
}

// Work partition and workspace of stages st[0..n) as one launch at batch B:
// a stage's units are the 64-element windows of its 64-row tiles; the
// launch's cus x WGN_GEMM_WG_PER_CU workgroups are shared among the stages in
// proportion to their units (each workgroup then streams the same number of
// windows), with at least GEMM_MIN_UNITS windows per workgroup; a stage with
// GEMM_TILES_WHOLE or more tiles per workgroup gives each tile a workgroup.  base: bytes
// kept for counters at the start of the workspace (at least the launch's
// own); launches that share a workspace use the largest, so no launch's data
// lies where another keeps its tickets.  False if a stage is outside the path
// (argmax with a bias, a weight matrix or input rows past 32-bit byte
// offsets).
bool gemm_plan(const wgn_stage *st, int32_t n, int32_t B, int32_t cus, GemmGroup &G, size_t base = 0) {
    if (n < 1 || n > GEMM_MAX_GROUP) return false;
    const int32_t nt = (B + 15) / 16;
    const int32_t P = st[0].epi == EPI_SWIGLU ? 2 : 1;
    int64_t units = 0;
    for (int32_t i = 0; i < n; ++i) {
        const wgn_stage &s = st[i];
        if (s.epi == EPI_ARGMAX && s.bias) return false;
        if ((int64_t)s.N * s.K * 2 > 0x7FFFFFF0LL) return false;
        // the input rows are read through a 32-bit buffer range too
        const int64_t xs = s.norm != NORM_NONE ? s.K : (B > 1 ? s.x_stride : s.K);
        if (((int64_t)(B - 1) * xs + s.K) * 2 > 0x7FFFFFF0LL) return false;
        units += (int64_t)((s.N + GEMM_TILE_ROWS - 1) / GEMM_TILE_ROWS) * ((s.K + GEMM_KWIN - 1) / GEMM_KWIN);
    }
    const int64_t target = (int64_t)std::max(cus, 1) * WGN_GEMM_WG_PER_CU;
    std::memset(&G.L, 0, sizeof G.L);
    G.n = n;
    G.L.n = n;
    G.swiglu = P == 2;
    G.norm_stage = first_normalised(st, n);
    G.norm = G.norm_stage >= 0;
    size_t o = 0;
    for (int32_t i = 0; i < n; ++i) {
        G.off_ticket[i] = o;
        o += al256((size_t)((st[i].N + GEMM_TILE_ROWS - 1) / GEMM_TILE_ROWS + 1) * sizeof(uint32_t));
    }
    if (st[0].epi == EPI_ARGMAX) {
        G.off_keys = o;
        o += al256((size_t)B * sizeof(uint64_t));
    }
    o = std::max(o, base);
    G.counters = o;
    if (G.norm) {
        G.off_xhat = o;
        o += al256((size_t)B * st[G.norm_stage].K * 2);
    }
    int32_t wgs_total = 0;
    for (int32_t i = 0; i < n; ++i) {
        const wgn_stage &s = st[i];
        const int32_t ntiles = (s.N + GEMM_TILE_ROWS - 1) / GEMM_TILE_ROWS;
        const int32_t nwin = (s.K + GEMM_KWIN - 1) / GEMM_KWIN;
        const int64_t U = (int64_t)ntiles * nwin;
        const int64_t share = (target * U + units / 2) / units;
        // A stage with many more tiles than workgroups (an LM head) keeps one
        // tile per workgroup: the hardware then runs two at a time on each
        // compute unit, one's epilogue under the other's stream, which beats
        // refilling one workgroup's pipeline for every tile.
        const int32_t wgs = ntiles >= GEMM_TILES_WHOLE * target
                                ? ntiles
                                : (int32_t)std::max<int64_t>(1, std::min(share, U / GEMM_MIN_UNITS));
        if (gemm_tiles_shared(ntiles, nwin, wgs)) {
            // contributor slots of the shared tiles: at most wgs + ntiles - 1
            // (consecutive tiles' slots never overlap), addressed with 32-bit offsets
            const size_t part = (size_t)(wgs + ntiles) * 4 * P * nt * GEMM_FRAG_BYTES;
            if (part > 0x7FFFFFF0u) return false;
            G.off_part[i] = o;
            o += part;
        }
        GemmArgs &a = G.L.s[i];
        a.W = (const uint16_t *)s.W;
        a.W_up = (const uint16_t *)s.W_up;
        a.x = (const uint16_t *)s.x;
        a.x_stride = B > 1 ? s.x_stride : s.K;
        a.bias = (const uint16_t *)s.bias;
        a.residual = (const uint16_t *)s.residual;
        a.res_stride = s.residual && B > 1 ? s.res_stride : s.N;
        a.y = s.y;
        a.y_stride = B > 1 ? s.y_stride : s.N;
        a.logits = s.logits;
        a.maxval = s.maxval;
        a.N = s.N;
        a.K = s.K;
        a.B = B;
        a.epi = s.epi;
        a.ntiles = ntiles;
        a.nwin = nwin;
        a.wgs = wgs;
        G.L.start[i] = wgs_total;
        wgs_total += wgs;
    }
    G.L.start[n] = wgs_total;
    G.ws = o;
    G.lds = gemm_lds_bytes(nt * 16);
    return true;
}

// Enqueue one planned launch: the counter clear (clear = true), the norm pass
// (if any, once for all its stages), then the product.
hipError_t gemm_run(const wgn_stage *st, int32_t B, const GemmGroup &G0, char *ws, hipStream_t stream, bool clear) {
    if (clear) {
        hipError_t e = launch_zero_words((uint32_t *)ws, (int32_t)(G0.counters / 4), stream);
        if (e != hipSuccess) return e;
    }
    GemmLaunch L = G0.L;
    const uint16_t *x = nullptr;
    if (G0.norm) {
        const wgn_stage &s = st[G0.norm_stage];
        uint16_t *xh = (uint16_t *)(ws + G0.off_xhat);
        hipError_t e = launch_norm_rows64((const uint16_t *)s.x, B > 1 ? s.x_stride : s.K, (const uint16_t *)s.gamma,
                                          (const uint16_t *)s.beta, s.eps, s.norm == NORM_LAYER, xh, B, s.K, stream);
        if (e != hipSuccess) return e;
        x = xh;
    }
    for (int32_t i = 0; i < G0.n; ++i) {
        GemmArgs &a = L.s[i];
        a.tickets = (uint32_t *)(ws + G0.off_ticket[i]);
        a.keys = a.epi == EPI_ARGMAX ? (uint64_t *)(ws + G0.off_keys) : nullptr;
        a.part = G0.off_part[i] ? (float *)(ws + G0.off_part[i]) : nullptr;
        if (x && st[i].norm != NORM_NONE) {
            a.x = x;
            a.x_stride = a.K;
        }
    }
    return launch_gemm(L, G0.swiglu, G0.lds, stream);
}

// Checks of a stage on the batched path that need the plan: outputs must not
// overlap the stage's inputs (x, residual, weights) or each other.
bool gemm_outputs_disjoint(const wgn_stage &s, int32_t B) {
    std::vector<Range> reads, writes, consts;
    stage_ranges(s, B, reads, writes, consts);
    for (const Range &w : writes) {
        for (const Range &r : reads)
            if (overlap(w, r)) return false;
        for (const Range &c : consts)
            if (overlap(w, c)) return false;
    }
    for (size_t i = 0; i < writes.size(); ++i)
        for (size_t k = i + 1; k < writes.size(); ++k)
            if (overlap(writes[i], writes[k])) return false;
    return true;
}

// Whether stages a and b may run in one launch: neither writes what the other
// reads or writes (they run at the same time).
bool independent(const wgn_stage &a, const wgn_stage &b, int32_t B) {
    std::vector<Range> ra, wa, ca, rb, wb, cb;
    stage_ranges(a, B, ra, wa, ca);
    stage_ranges(b, B, rb, wb, cb);
    for (const Range &w : wa) {
        for (const Range &r : rb)
            if (overlap(w, r)) return false;
        for (const Range &w2 : wb)
            if (overlap(w, w2)) return false;
        for (const Range &c : cb)
            if (overlap(w, c)) return false;
    }
    for (const Range &w : wb) {
        for (const Range &r : ra)
            if (overlap(w, r)) return false;
        for (const Range &c : ca)
            if (overlap(w, c)) return false;
    }
    return true;
}

// The launches of a stage list on the batched path, in list order: runs of
// consecutive stages of one epilogue family that are independent of each
// other (at most GEMM_MAX_GROUP) share a launch, provided the normalised ones
// among them read the same x-hat (one norm pass per launch); stages without
// normalisation may read any input.  All launches use one counter area (the largest), so the
// workspace need is the largest launch's with that base.  False if a stage is
// outside the path.
bool plan_batched(const wgn_stage *st, int32_t n, int32_t B, int32_t cus, std::vector<GemmGroup> &groups,
                  size_t &need, size_t &counters) {
    groups.clear();
    counters = 0;
    for (int32_t i = 0; i < n;) {
        int32_t j = i + 1;
        while (j < n && j - i < GEMM_MAX_GROUP && may_join(st, i, j)) {
            bool ok = true;
            for (int32_t k = i; k < j && ok; ++k) ok = independent(st[k], st[j], B);
            if (!ok) break;
            ++j;
        }
        GemmGroup G;
        if (!gemm_plan(st + i, j - i, B, cus, G)) return false;
        G.first = i;
        counters = std::max(counters, G.counters);
        groups.push_back(G);
        i = j;
    }
    need = 0;
    for (GemmGroup &G : groups) {
        const int32_t first = G.first;
        gemm_plan(st + first, G.n, B, cus, G, counters);
        G.first = first;
        need = std::max(need, G.ws);
    }
    return true;
}

}  // namespace wgn

size_t wgn_gemm_norm_workspace_bytes(const wgn_stage *stage, int32_t batch) {
    if (!stage || check_stage(*stage, batch, GEMM_MAX_BATCH) != WGN_OK) return 0;
    GemmGroup G;
    DevInfo d = device_info();
    if (!gemm_plan(stage, 1, batch, d.cus > 0 ? d.cus : 256, G)) return 0;
    return G.ws;
}

wgn_status wgn_gemm_norm(const wgn_stage *stage, int32_t batch, void *workspace, size_t ws_bytes,
                         wgn_stream stream) {
    if (!stage) return WGN_E_ARG;
    wgn_status st = check_stage(*stage, batch, GEMM_MAX_BATCH);
    if (st != WGN_OK) return st;
    if (!gemm_outputs_disjoint(*stage, batch)) return WGN_E_ARG;
    DevInfo d = device_info();
    GemmGroup G;
    if (!gemm_plan(stage, 1, batch, d.cus > 0 ? d.cus : 256, G)) return WGN_E_UNSUPPORTED;
    if (!workspace || ws_bytes < G.ws || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return WGN_E_WORKSPACE;
    if (!d.ok) return WGN_E_DEVICE;
    hipError_t e = note(gemm_run(stage, batch, G, (char *)workspace, (hipStream_t)stream, true), "gemm_norm launch");
    return e == hipSuccess ? WGN_OK : WGN_E_HIP;
}

size_t wgn_lmhead_argmax_workspace_bytes(int32_t batch) {
    if (batch < 1 || batch > MAX_BATCH) return 0;
    DevInfo d = device_info();
    int32_t G = d.cus > 0 ? d.cus : 256;
    return 256 + al256((size_t)G * batch * sizeof(uint64_t));
}

wgn_status wgn_lmhead_argmax(const void *h, int64_t h_stride, int32_t batch, int32_t K, const void *gamma,
                             float eps, const void *W_lm, int32_t V, int32_t *idx_out, float *max_out,
                             float *logits_out, void *workspace, size_t ws_bytes, wgn_stream stream) {
    wgn_stage s;
    std::memset(&s, 0, sizeof s);
    s.N = V;
    s.K = K;
    s.W = W_lm;
    s.norm = gamma ? NORM_RMS : NORM_NONE;
    s.eps = eps;
    s.gamma = gamma;
    s.epi = EPI_ARGMAX;
    s.x = h;
    s.x_stride = h_stride;
    s.y = idx_out;
    s.logits = logits_out;
    s.maxval = max_out;
    return wgn_gemv_norm(&s, batch, workspace, ws_bytes, stream);
}

wgn_status wgn_lmhead_argmax_static(const void *h, int64_t h_stride, int32_t batch, int32_t K, const void *gamma,
                                    float eps, const void *W_lm, int32_t V, int32_t *idx_out, float *max_out,
                                    float *logits_out, wgn_stream stream) {
    // every argument check of the workspace form, before the scratch is touched
    wgn_stage s;
    std::memset(&s, 0, sizeof s);
    s.N = V;
    s.K = K;
    s.W = W_lm;
    s.norm = gamma ? NORM_RMS : NORM_NONE;
    s.eps = eps;
    s.gamma = gamma;
    s.epi = EPI_ARGMAX;
    s.x = h;
    s.x_stride = h_stride;
    s.y = idx_out;
    s.logits = logits_out;
    s.maxval = max_out;
    wgn_status st = check_stage(s, batch);
    if (st != WGN_OK) return st;
    DevInfo d = device_info();
    if (!d.ok) return WGN_E_DEVICE;
    SingleLaunch L;
    if (!single_geometry(s, batch, d.cus, L)) return WGN_E_UNSUPPORTED;
    if (L.ws > SCRATCH_BYTES) return WGN_E_WORKSPACE;  // more workgroups x batch rows than the fixed scratch holds
    void *ws = nullptr;
    if (note(scratch_address(&ws, (hipStream_t)stream), "fixed scratch address") != hipSuccess) return WGN_E_HIP;
    return wgn_gemv_norm(&s, batch, ws, SCRATCH_BYTES, stream);
}

wgn_status wgn_rmsnorm_rows(const void *x, int64_t x_stride, const void *gamma, float eps, void *y,
                            int64_t y_stride, int32_t rows, int32_t K, int32_t dtype, wgn_stream stream) {
    if (!x || !gamma || !y || rows < 0 || K < 8 || (K & 7)) return WGN_E_ARG;
    if (dtype != WGN_BF16 && dtype != WGN_FP16) return WGN_E_ARG;
    if (!(eps >= 0.0f)) return WGN_E_ARG;
    if (rows > 1 && (x_stride < K || y_stride < K)) return WGN_E_ARG;
    if (!a16(x) || !a16(gamma) || !a16(y) || (x_stride & 7) || (y_stride & 7)) return WGN_E_ALIGN;
    {
        Range rx = rng(x, ((size_t)(rows > 0 ? rows - 1 : 0) * x_stride + K) * 2);
        Range ry = rng(y, ((size_t)(rows > 0 ? rows - 1 : 0) * y_stride + K) * 2);
        if (overlap(rx, ry)) return WGN_E_ARG;
    }
    if (rows == 0) return WGN_OK;
    DevInfo d = device_info();
    if (!d.ok) return WGN_E_DEVICE;
    hipError_t e = note(launch_rmsnorm_rows((const uint16_t *)x, x_stride, (const uint16_t *)gamma, eps,
                                            (uint16_t *)y, y_stride, rows, K, dtype == WGN_FP16, (hipStream_t)stream),
                        "rmsnorm_rows launch");
    return e == hipSuccess ? WGN_OK : WGN_E_HIP;
}

size_t wgn_chain_workspace_bytes(const wgn_stage *stages, int32_t n_stages, int32_t batch,
                                 const wgn_chain_opts *opts) {
    return wgn_chain_attn_workspace_bytes(stages, n_stages, nullptr, nullptr, 0, batch, opts);
}

size_t wgn_chain_attn_workspace_bytes(const wgn_stage *stages, int32_t n_stages, const wgn_attn_stage *attn,
                                      const int32_t *attn_before, int32_t n_attn, int32_t batch,
                                      const wgn_chain_opts *opts) {
    Program P;
    if (plan(stages, n_stages, batch, resolve_grid(opts), opts_path(opts), opts_fuse(opts), P, attn, attn_before,
             n_attn) != WGN_OK)
        return 0;
    return ws_layout(P, opts && opts->trace).total;
}

wgn_status wgn_chain_create(const wgn_stage *stages, int32_t n_stages, int32_t batch, const wgn_chain_opts *opts,
                            void *workspace, size_t ws_bytes, wgn_stream stream, wgn_chain **out) {
    return wgn_chain_create_attn(stages, n_stages, nullptr, nullptr, 0, batch, opts, workspace, ws_bytes, stream,
                                 out);
}

wgn_status wgn_chain_create_attn(const wgn_stage *stages, int32_t n_stages, const wgn_attn_stage *attn,
                                 const int32_t *attn_before, int32_t n_attn, int32_t batch,
                                 const wgn_chain_opts *opts, void *workspace, size_t ws_bytes, wgn_stream stream,
                                 wgn_chain **out) {
    if (!out) return WGN_E_ARG;
    *out = nullptr;
    if (opts) {
        if (opts->mode < 0 || opts->mode > 1 || opts->grid < 0 || opts->grid > MAX_GRID || opts->trace < 0 ||
            opts->trace > 1 ||
            opts->path < 0 || opts->path > 2 || opts->no_fuse < 0 || opts->no_fuse > 1 || opts->ring < 0 ||
            opts->ring > NUM_RINGS)
            return WGN_E_ARG;
        for (int i = 0; i < 2; ++i)
            if (opts->reserved[i]) return WGN_E_ARG;
    }
    wgn_chain *c = new (std::nothrow) wgn_chain();
    if (!c) return WGN_E_ARG;
    wgn_status st = plan(stages, n_stages, batch, resolve_grid(opts), opts_path(opts), opts_fuse(opts), c->P, attn,
                         attn_before, n_attn);
    if (st != WGN_OK) {
        delete c;
        return st;
    }
    DevInfo d = device_info();
    if (!d.ok) {
        delete c;
        return WGN_E_DEVICE;
    }
    // the persistent kernel needs every workgroup resident at once (one per
    // compute unit: each takes the whole LDS)
    if ((!opts || opts->mode == 0) && c->P.G > d.cus) {
        delete c;
        return WGN_E_ARG;
    }
    c->trace = opts && opts->trace;
    c->L = ws_layout(c->P, c->trace);
    if (!workspace || ws_bytes < c->L.total || (reinterpret_cast<uintptr_t>(workspace) & 255u)) {
        delete c;
        return WGN_E_WORKSPACE;
    }
    c->mode = opts ? opts->mode : 0;
    c->ring = opts && opts->ring > 0 ? opts->ring - 1 : auto_ring(c->P);
    if (c->P.tile) c->ring = 0;
    c->ws = workspace;
    c->lds = c->P.lds_total();
    patch_fsum(c->P, (char *)workspace + c->L.fsum);
    // host image of the program, then one upload
    std::vector<char> img(c->L.ctr, 0);
    std::memcpy(img.data() + c->L.phases, c->P.phases.data(), c->P.phases.size() * sizeof(DevPhase));
    std::memcpy(img.data() + c->L.stages, c->P.stages.data(), c->P.stages.size() * sizeof(DevStage));
    std::memcpy(img.data() + c->L.sources, c->P.sources.data(), c->P.sources.size() * sizeof(DevSource));
    std::memcpy(img.data() + c->L.rowb, c->P.rowb.data(), c->P.rowb.size() * sizeof(int32_t));
    for (DevAttn &d : c->P.attn) d.part = (float *)((char *)workspace + c->L.attp);
    if (!c->P.attn.empty())
        std::memcpy(img.data() + c->L.att, c->P.attn.data(), c->P.attn.size() * sizeof(DevAttn));
    {
        // Run lists and phase tables are functions of (phase, workgroup)
        // alone: build them here, with the kernel's own code over the host
        // copy of the program, instead of on the kernel's critical path.
        KArgs h;
        std::memset(&h, 0, sizeof h);
        h.phases = c->P.phases.data();
        h.stages = c->P.stages.data();
        h.sources = c->P.sources.data();
        h.rowb = c->P.rowb.data();
        h.G = c->P.G;
        h.nb = c->P.B;
        for (int32_t q = 0; q < (int32_t)c->P.phases.size(); ++q) {
            for (int32_t g = 0; g < c->P.G; ++g) {
                char *buf = img.data() + c->L.runimg + ((size_t)q * c->P.G + g) * RUN_BUF_STRIDE;
                make_runs<true>(h, q, g, c->P.tile, *(RunHdr *)buf, (Run *)(buf + sizeof(RunHdr)));
            }
            char *pi = img.data() + c->L.phinfo + (size_t)q * PHASE_INFO_BYTES;
            make_phase_info<true>(h, q, (SrcInfo *)pi, *(NormHdr *)(pi + MAX_SRC * sizeof(SrcInfo)));
        }
    }
    // launch groups (mode 1) and the distinct weight matrices each reads
    for (int32_t p = 0; p < (int32_t)c->P.phases.size(); p = c->P.group_end[p]) {
        const int32_t li = (int32_t)c->launch0.size();
        c->launch0.push_back(p);
        TouchRange *t = (TouchRange *)(img.data() + c->L.touch) + (size_t)li * MAX_TOUCH;
        int32_t n = 0;
        for (int32_t q = p; q < c->P.group_end[p]; ++q) {
            const DevPhase &ph = c->P.phases[q];
            for (int32_t si = ph.stage0; si < ph.stage0 + ph.nstages; ++si) {
                const DevStage &st = c->P.stages[si];
                const uint64_t bytes = (uint64_t)st.N * (uint64_t)st.K * 2u;
                for (const uint16_t *w : {st.W, st.W_up}) {
                    if (!w || bytes == 0) continue;
                    bool seen = false;
                    for (int32_t k = 0; k < n; ++k) seen |= t[k].p == (const void *)w;
                    if (!seen && n < MAX_TOUCH) t[n++] = TouchRange{(const void *)w, bytes};
                }
            }
        }
        c->touch_n.push_back(n);
    }
    if (c->mode == 1) {
        c->ev.assign(c->launch0.size() + 1, nullptr);
        for (hipEvent_t &e : c->ev)
            if (note(hipEventCreateWithFlags(&e, hipEventDisableTiming), "plan events") != hipSuccess) {
                delete c;
                return WGN_E_HIP;
            }
    }
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    if (note(hipMemcpyAsync(ws, img.data(), img.size(), hipMemcpyHostToDevice, s), "chain upload") != hipSuccess ||
        note(hipMemsetAsync(ws + c->L.ctr, 0, c->L.am_part - c->L.ctr, s), "chain counters") != hipSuccess ||
        note(hipStreamSynchronize(s), "chain create sync") != hipSuccess) {
        delete c;
        return WGN_E_HIP;
    }
    KArgs &a = c->a;
    std::memset(&a, 0, sizeof a);
    a.phases = (const DevPhase *)(ws + c->L.phases);
    a.stages = (const DevStage *)(ws + c->L.stages);
    a.sources = (const DevSource *)(ws + c->L.sources);
    a.rowb = (const int32_t *)(ws + c->L.rowb);
    // precomputed lists from batch 2 up, and at batch 1 for chains of small
    // phases; with large phases at batch 1 the kernel builds them while it
    // waits for flags that arrive later anyway (measured on one box: decode
    // step 742 us built in place against 759 precomputed; LayerNorm chain 544
    // against 440, decode step with attention phases 1,564 against 1,494)
    if (c->P.B > 1 || c->P.tile || WGN_PRE_B1 || small_phases(c->P)) {
        a.runimg = ws + c->L.runimg;
        a.phinfo = ws + c->L.phinfo;
    }
    a.flags = (uint32_t *)(ws + c->L.ctr);
    a.run = (uint32_t *)(ws + c->L.run);
    a.tickets = (uint32_t *)(ws + c->L.tickets);
    a.err = (uint32_t *)(ws + c->L.err);
    a.am_part = (uint64_t *)(ws + c->L.am_part);
    a.trace = c->trace ? (uint64_t *)(ws + c->L.trace) : nullptr;
    a.att = c->P.attn.empty() ? nullptr : (const DevAttn *)(ws + c->L.att);
    a.p0 = 0;
    a.p1 = (int32_t)c->P.phases.size();
    a.persistent = c->mode == 0 ? 1 : 0;
    a.G = c->P.G;
    a.n_argmax = c->P.n_argmax;
    a.nb = c->P.B;
    a.wait_ticks = WAIT_TICKS;
    a.ist.W = (const uint16_t *)stages[0].W;  // address used by empty (zero-length) loads
    *out = c;
    return WGN_OK;
}

wgn_status wgn_chain_run(const wgn_chain *c, wgn_stream stream) {
    if (!c) return WGN_E_ARG;
    hipStream_t s = (hipStream_t)stream;
    if (c->mode == 0) {
        hipError_t e = note(launch_chain(c->P.B, c->P.tile, c->ring, c->a, c->P.G, c->lds, s), "chain launch");
        return e == hipSuccess ? WGN_OK : WGN_E_HIP;
    }
    // one launch per phase; the K windows of one phase share a launch (their
    // running sums live in LDS)
    KArgs a = c->a;
    for (int32_t p = 0; p < (int32_t)c->P.phases.size(); p = c->P.group_end[p]) {
        a.p0 = p;
        a.p1 = c->P.group_end[p];
        hipError_t e = note(launch_chain(c->P.B, c->P.tile, c->ring, a, c->P.G, c->lds, s), "chain phase launch");
        if (e != hipSuccess) return WGN_E_HIP;
    }
    return WGN_OK;
}

namespace {
bool plan_fields_ok(const wgn_plan &pl) {
    if (pl.prefetch < 0 || pl.prefetch > 1) return false;
    if (!pl.prefetch) return true;
    return pl.distance >= 1 && pl.distance <= 4 && pl.blocks >= 1 && pl.blocks <= 1024 && pl.frac_pct >= 1 &&
           pl.frac_pct <= 100;
}
}  // namespace

wgn_status wgn_chain_run_plan(const wgn_chain *c, const wgn_plan *plan, wgn_stream stream, wgn_stream side) {
    if (!c || !plan || !plan_fields_ok(*plan)) return WGN_E_ARG;
    if (!plan->prefetch) return wgn_chain_run(c, stream);
    if (c->mode != 1) return WGN_E_UNSUPPORTED;
    if (!side || side == stream) return WGN_E_ARG;
    hipStream_t s = (hipStream_t)stream, sd = (hipStream_t)side;
    const TouchRange *tab = (const TouchRange *)((const char *)c->ws + c->L.touch);
    const uint32_t frac = (uint32_t)(((uint64_t)plan->frac_pct << 16) / 100u);
    const int32_t nl = (int32_t)c->launch0.size(), d = plan->distance;
    KArgs a = c->a;
    bool forked = false;
    for (int32_t li = 0; li < nl; ++li) {
        // while launch li runs, the side stream reads launch li+d's weights;
        // it starts once everything before launch li is done
        if (li + d < nl && c->touch_n[li + d] > 0) {
            if (note(hipEventRecord(c->ev[li], s), "plan fork") != hipSuccess ||
                note(hipStreamWaitEvent(sd, c->ev[li], 0), "plan fork wait") != hipSuccess ||
                note(launch_touch(tab + (size_t)(li + d) * MAX_TOUCH, c->touch_n[li + d], frac, plan->blocks, sd),
                     "touch launch") != hipSuccess)
                return WGN_E_HIP;
            forked = true;
        }
        a.p0 = c->launch0[li];
        a.p1 = c->P.group_end[a.p0];
        if (note(launch_chain(c->P.B, c->P.tile, c->ring, a, c->P.G, c->lds, s), "chain phase launch") != hipSuccess)
            return WGN_E_HIP;
    }
    if (forked && (note(hipEventRecord(c->ev[nl], sd), "plan join") != hipSuccess ||
                   note(hipStreamWaitEvent(s, c->ev[nl], 0), "plan join wait") != hipSuccess))
        return WGN_E_HIP;
    return WGN_OK;
}

namespace {
// Two-sided 95 % Student t quantile for df degrees of freedom.
double t975(int df) {
    static const double t[] = {12.706, 4.303, 3.182, 2.776, 2.571, 2.447, 2.365, 2.306, 2.262, 2.228,
                               2.201,  2.179, 2.160, 2.145, 2.131, 2.120, 2.110, 2.101, 2.093, 2.086,
                               2.080,  2.074, 2.069, 2.064, 2.060, 2.056, 2.052, 2.048, 2.045, 2.042};
    if (df < 1) return 1e9;
    if (df <= 30) return t[df - 1];
    return df <= 60 ? 2.000 : df <= 120 ? 1.980 : 1.960;
}
}  // namespace

wgn_status wgn_chain_plan_tune(const wgn_chain *c, wgn_stream stream, wgn_stream side, int32_t reps,
                               wgn_plan *out) {
    if (!c || !out || reps < 3 || reps > 200) return WGN_E_ARG;
    if (c->mode != 1) return WGN_E_UNSUPPORTED;
    if (!side || side == stream) return WGN_E_ARG;
    std::vector<wgn_plan> cand;
    wgn_plan plain{};
    cand.push_back(plain);
    for (int32_t d : {1, 2})
        for (int32_t blocks : {16, 64, 256})
            for (int32_t frac : {50, 100}) {
                wgn_plan p{};
                p.prefetch = 1;
                p.distance = d;
                p.blocks = blocks;
                p.frac_pct = frac;
                cand.push_back(p);
            }
    const size_t nc = cand.size();
    hipStream_t s = (hipStream_t)stream;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (note(hipEventCreate(&e0), "tune events") != hipSuccess) return WGN_E_HIP;
    if (note(hipEventCreate(&e1), "tune events") != hipSuccess) {
        (void)hipEventDestroy(e0);
        return WGN_E_HIP;
    }
    std::vector<std::vector<double>> t(nc, std::vector<double>((size_t)reps, 0.0));
    wgn_status st = WGN_OK;
    for (int32_t w = 0; w < 2 && st == WGN_OK; ++w) st = wgn_chain_run(c, stream);  // warm-up
    if (st == WGN_OK) st = wgn_chain_run_plan(c, &cand[1], stream, side);
    for (int32_t r = 0; r < reps && st == WGN_OK; ++r) {
        // every round times each candidate once, in a rotated order, so
        // slow drifts of the clock or the memory affect all of them alike
        for (size_t k = 0; k < nc && st == WGN_OK; ++k) {
            const size_t ci = (k + (size_t)r) % nc;
            float ms = 0.0f;
            if (note(hipEventRecord(e0, s), "tune record") != hipSuccess) st = WGN_E_HIP;
            if (st == WGN_OK) st = wgn_chain_run_plan(c, &cand[ci], stream, side);
            if (st == WGN_OK && (note(hipEventRecord(e1, s), "tune record") != hipSuccess ||
                                 note(hipEventSynchronize(e1), "tune sync") != hipSuccess ||
                                 note(hipEventElapsedTime(&ms, e0, e1), "tune elapsed") != hipSuccess))
                st = WGN_E_HIP;
            t[ci][(size_t)r] = ms * 1000.0;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st != WGN_OK) return st;
    // speedup of candidate k in round r: plain time / candidate time (paired
    // by round); keep the best mean only if its 95 % interval clears +1 %
    double plain_mean = 0.0;
    for (double v : t[0]) plain_mean += v;
    plain_mean /= reps;
    size_t best = 0;
    double best_mean = 0.0, best_lo = 0.0, best_us = plain_mean;
    for (size_t k = 1; k < nc; ++k) {
        double m = 0.0, ss = 0.0, us = 0.0;
        for (int32_t r = 0; r < reps; ++r) {
            m += t[0][(size_t)r] / t[k][(size_t)r];
            us += t[k][(size_t)r];
        }
        m /= reps;
        for (int32_t r = 0; r < reps; ++r) {
            const double dv = t[0][(size_t)r] / t[k][(size_t)r] - m;
            ss += dv * dv;
        }
        const double sd = std::sqrt(ss / (reps - 1));
        const double lo = m - t975(reps - 1) * sd / std::sqrt((double)reps);
        if (best == 0 || m > best_mean) {
            best = k;
            best_mean = m;
            best_lo = lo;
            best_us = us / reps;
        }
    }
    *out = best_lo > 1.01 ? cand[best] : plain;
    out->plain_us = (float)plain_mean;
    out->best_us = (float)best_us;
    out->speedup_lo = (float)best_lo;
    out->candidates = (int32_t)(nc - 1);
    if (!(best_lo > 1.01)) {
        // report which candidate came closest, with prefetch left off
        out->distance = cand[best].distance;
        out->blocks = cand[best].blocks;
        out->frac_pct = cand[best].frac_pct;
    }
    return WGN_OK;
}

wgn_status wgn_chain_check(const wgn_chain *c, wgn_stream stream) {
    if (!c) return WGN_E_ARG;
    hipStream_t s = (hipStream_t)stream;
    if (note(hipStreamSynchronize(s), "chain check sync") != hipSuccess) return WGN_E_HIP;
    uint32_t err = 0;
    if (note(hipMemcpy(&err, (char *)c->ws + c->L.err, 4, hipMemcpyDeviceToHost), "chain check read") != hipSuccess)
        return WGN_E_HIP;
    if (!err) return WGN_OK;
    // an aborted run left flags and tickets behind: clear them (the run
    // counter is kept; flags from the aborted run are erased)
    char *w = (char *)c->ws;
    if (note(hipMemset(w + c->L.ctr, 0, c->L.run - c->L.ctr), "chain reset flags") != hipSuccess ||
        note(hipMemset(w + c->L.tickets, 0, c->L.am_part - c->L.tickets), "chain reset tickets") != hipSuccess)
        return WGN_E_HIP;
    return WGN_E_TIMEOUT;
}

wgn_status wgn_chain_set_wait_us(wgn_chain *c, int64_t us) {
    if (!c) return WGN_E_ARG;
    if (us > (int64_t)(WAIT_TICKS / 100) * 1000) return WGN_E_ARG;
    c->a.wait_ticks = us < 0 ? WAIT_TICKS : (uint64_t)us * 100u;  // the real-time clock runs at 100 MHz
    return WGN_OK;
}

int32_t wgn_chain_num_phases(const wgn_chain *c) { return c ? (int32_t)c->P.phases.size() : -1; }

int32_t wgn_chain_grid(const wgn_chain *c) { return c ? c->P.G : -1; }

int32_t wgn_chain_ring(const wgn_chain *c) { return c ? c->ring : -1; }

wgn_status wgn_chain_trace(const wgn_chain *c, wgn_stream stream, uint64_t *out, size_t n_out) {
    if (!c || !out) return WGN_E_ARG;
    if (!c->trace) return WGN_E_UNSUPPORTED;
    const size_t n = c->P.phases.size() * (size_t)c->P.G * TRACE_POINTS;
    if (n_out < n) return WGN_E_ARG;
    if (note(hipStreamSynchronize((hipStream_t)stream), "trace sync") != hipSuccess) return WGN_E_HIP;
    if (note(hipMemcpy(out, (char *)c->ws + c->L.trace, n * sizeof(uint64_t), hipMemcpyDeviceToHost),
             "trace read") != hipSuccess)
        return WGN_E_HIP;
    return WGN_OK;
}

wgn_status wgn_chain_stage_phases(const wgn_chain *c, int32_t *out) {
    if (!c || !out) return WGN_E_ARG;
    for (size_t i = 0; i < c->P.phase_of_stage.size(); ++i) out[i] = c->P.phase_of_stage[i];
    return WGN_OK;
}

void wgn_chain_destroy(wgn_chain *c) { delete c; }

namespace {

// Batch 17-128: the stages one launch (plus a norm pass) each, in list
// order, on the batched matrix-core path.  The counters at the start of the
// workspace are cleared first (it may hold a persistent chain's program).
wgn_status layer_chain_batched(const wgn_stage *stages, int32_t n_stages, int32_t batch, const wgn_chain_opts *opts,
                               const wgn_plan *plan, void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (!stages || n_stages < 1) return WGN_E_ARG;
    if ((plan && plan->prefetch) || (opts && (opts->trace || opts->path == 1))) return WGN_E_UNSUPPORTED;
    if (opts && (opts->path < 0 || opts->path > 3)) return WGN_E_ARG;
    DevInfo d = device_info();
    const int32_t cus = d.cus > 0 ? d.cus : 256;
    for (int32_t i = 0; i < n_stages; ++i) {
        wgn_status st = check_stage(stages[i], batch, GEMM_MAX_BATCH);
        if (st != WGN_OK) return st;
        if (!gemm_outputs_disjoint(stages[i], batch)) return WGN_E_ARG;
    }
    std::vector<GemmGroup> groups;
    size_t need = 0, counters = 0;
    if (!plan_batched(stages, n_stages, batch, cus, groups, need, counters)) return WGN_E_UNSUPPORTED;
    if (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return WGN_E_WORKSPACE;
    if (!d.ok) return WGN_E_DEVICE;
    char *ws = (char *)workspace;
    hipError_t e = note(launch_zero_words((uint32_t *)ws, (int32_t)(counters / 4), stream), "counter clear");
    for (size_t g = 0; g < groups.size() && e == hipSuccess; ++g)
        e = note(gemm_run(stages + groups[g].first, batch, groups[g], ws, stream, false), "batched launch");
    return e == hipSuccess ? WGN_OK : WGN_E_HIP;
}

}  // namespace

wgn_status wgn_layer_chain(const wgn_stage *stages, int32_t n_stages, int32_t batch, const wgn_chain_opts *opts,
                           const wgn_plan *plan, void *workspace, size_t ws_bytes, wgn_stream stream,
                           wgn_stream side) {
    if ((batch > MAX_BATCH && batch <= GEMM_MAX_BATCH) || (opts && opts->path == 3 && batch >= 1))
        return layer_chain_batched(stages, n_stages, batch, opts, plan, workspace, ws_bytes, (hipStream_t)stream);
    const bool prefetch = plan && plan->prefetch;
    if (prefetch && !(opts && opts->mode == 1)) return WGN_E_UNSUPPORTED;  // plans drive per-phase launches
    wgn_chain *c = nullptr;
    wgn_status st = wgn_chain_create(stages, n_stages, batch, opts, workspace, ws_bytes, stream, &c);
    if (st != WGN_OK) return st;
    st = prefetch ? wgn_chain_run_plan(c, plan, stream, side) : wgn_chain_run(c, stream);
    wgn_chain_destroy(c);
    return st;
}

wgn_status wgn_plan_tune(const wgn_stage *stages, int32_t n_stages, int32_t batch, wgn_plan *out, void *workspace,
                         size_t ws_bytes, wgn_stream stream, wgn_stream side) {
    if (!out) return WGN_E_ARG;
    wgn_chain_opts o;
    std::memset(&o, 0, sizeof o);
    o.mode = 1;  // the touch pass prefetches the weights of later launches
    wgn_chain *c = nullptr;
    wgn_status st = wgn_chain_create(stages, n_stages, batch, &o, workspace, ws_bytes, stream, &c);
    if (st != WGN_OK) return st;
    st = wgn_chain_plan_tune(c, stream, side, 15, out);
    wgn_chain_destroy(c);
    return st;
}

namespace {

// Workspace of the batched path for the stages (and an LM head of V rows over
// the hidden state the stages end with: the last stage's output width, RMSNorm
// prologue, argmax); false if a stage is outside the path.
bool batched_need(const wgn_stage *stages, int32_t n_stages, int32_t batch, int32_t V, size_t &need) {
    need = 0;
    if (!stages || n_stages < 1 || batch < 1 || batch > GEMM_MAX_BATCH) return false;
    std::vector<wgn_stage> all(stages, stages + n_stages);
    if (V > 0) {
        alignas(16) static const uint16_t dummy[8] = {};
        const int32_t kh = (stages[n_stages - 1].N + 7) / 8 * 8;
        wgn_stage s;
        std::memset(&s, 0, sizeof s);
        s.N = V;
        s.K = kh;
        s.W = s.x = s.gamma = dummy;
        s.norm = NORM_RMS;
        s.epi = EPI_ARGMAX;
        s.x_stride = kh;
        s.y = (void *)dummy;
        all.push_back(s);
    }
    for (const wgn_stage &s : all)
        if (check_stage(s, batch, GEMM_MAX_BATCH) != WGN_OK) return false;
    DevInfo d = device_info();
    std::vector<GemmGroup> groups;
    size_t counters = 0;
    return plan_batched(all.data(), (int32_t)all.size(), batch, d.cus > 0 ? d.cus : 256, groups, need, counters);
}

}  // namespace

size_t wgn_workspace_bytes(const wgn_stage *stages, int32_t n_stages, int32_t batch, int32_t V) {
    size_t batched = 0;
    const bool batched_ok = batched_need(stages, n_stages, batch, V, batched);
    if (batch > MAX_BATCH) return batched_ok ? batched : 0;
    size_t need = 0;
    if (n_stages > 0) {
        wgn_chain_opts o;
        std::memset(&o, 0, sizeof o);
        for (int32_t mode = 0; mode <= 1; ++mode) {
            o.mode = mode;
            const size_t b = wgn_chain_workspace_bytes(stages, n_stages, batch, &o);
            if (b == 0) return 0;  // the stages cannot be planned
            need = std::max(need, b);
        }
        for (int32_t i = 0; i < n_stages; ++i) need = std::max(need, wgn_gemv_norm_workspace_bytes(&stages[i], batch));
    }
    if (V > 0) need = std::max(need, wgn_lmhead_argmax_workspace_bytes(batch));
    if (batched_ok) need = std::max(need, batched);  // wgn_layer_chain with opts->path == 3
    return need;
}

int32_t wgn_plan_phases(const wgn_stage *stages, int32_t n_stages, int32_t batch, const wgn_chain_opts *opts,
                        int32_t *phase_of_stage) {
    Program P;
    const int32_t grid = opts && opts->grid > 0 ? opts->grid : 256;
    wgn_status st = plan(stages, n_stages, batch, grid, opts_path(opts), opts_fuse(opts), P);
    if (st != WGN_OK) return st;
    if (phase_of_stage)
        for (int32_t i = 0; i < n_stages; ++i) phase_of_stage[i] = P.phase_of_stage[i];
    return (int32_t)P.phases.size();
}

// Host emulation of the work partition of a planned chain: every unit of every
// phase must be streamed by exactly one wave of exactly one workgroup, with the
// right address; every partial slot must be written once and lie inside its
// phase's area; the epilogue must read exactly the slots the waves write; the
// LDS areas must be ordered and inside the budget.  Returns the number of
// violations (0 = consistent), or a negative status if planning failed.
int32_t wgn_partition_selftest(const wgn_stage *stages, int32_t n_stages, int32_t batch,
                               const wgn_chain_opts *opts) {
    Program P;
    const int32_t grid = opts && opts->grid > 0 ? opts->grid : 256;
    wgn_status st = plan(stages, n_stages, batch, grid, opts_path(opts), opts_fuse(opts), P);
    if (st == WGN_OK) patch_fsum(P, (char *)((uintptr_t)1 << 44));  // a fake workspace address
    if (st != WGN_OK) return st;
    const bool tile = P.tile;
    const int32_t nb = P.B;
    KArgs a;
    std::memset(&a, 0, sizeof a);
    a.phases = P.phases.data();
    a.stages = P.stages.data();
    a.sources = P.sources.data();
    a.rowb = P.rowb.data();
    a.G = P.G;
    a.nb = nb;
    int32_t bad = 0;
    if (P.lds_total() > LDS_BUDGET) ++bad;
    // both normalisation splits cover every (item, lane-in-item) once for
    // every item count the kernel uses (items = (source, batch row) pairs,
    // padded to a power of two, at most MAX_SRC x MAX_BATCH): the one-wave
    // split over min(items, WAVES) waves, no item spanning more than one
    // wave, and the spread split over WAVES waves, each item's statistics in
    // the waves and slots its combine step reads
    for (int32_t spread = 0; spread <= 1; ++spread) {
        for (int32_t nq = 1; nq <= MAX_SRC * MAX_BATCH; nq *= 2) {
            const int32_t nw = spread ? WAVES : std::min<int32_t>(nq, WAVES);
            std::vector<std::vector<int32_t>> cover(nq);
            for (int32_t w = 0; w < nw; ++w)
                for (uint32_t lane = 0; lane < 64; ++lane) {
                    const NormSplit S = norm_split(nq, w, lane, nw);
                    if (S.slot < 0 || S.slot >= STATS_ROWS || S.rslot < 0 || S.rslot >= STATS_ROWS) ++bad;
                    if (!S.active) continue;
                    if (w < S.w0 || w >= S.w1 || S.sub < 0 || S.sub >= S.lanes) ++bad;
                    if (S.w1 - S.w0 == 1 && S.slot != S.rslot) ++bad;
                    if (!spread && (S.w1 != S.w0 + 1 || S.lanes > 64)) ++bad;
                    cover[S.row].push_back(S.sub);
                }
            for (int32_t r = 0; r < nq; ++r) {
                std::sort(cover[r].begin(), cover[r].end());
                for (size_t i = 0; i < cover[r].size(); ++i)
                    if (cover[r][i] != (int32_t)i) ++bad;
                if (cover[r].empty()) ++bad;
            }
        }
    }
    for (int32_t p = 0; p < (int32_t)P.phases.size(); ++p) {
        const DevPhase &ph = P.phases[p];
        if (!(ph.x_off >= lds_dyn_off(path_desc_bufs(P.tile)) && ph.part_off >= ph.x_off + nb * ph.xb * 2 && ph.prm_off >= ph.part_off &&
              ph.epi_off >= ph.prm_off && ph.carry_off >= ph.epi_off && (size_t)ph.carry_off <= P.lds_total()))
            ++bad;
        if (P.group_end[p] <= p || P.group_end[p] > (int32_t)P.phases.size()) ++bad;
        std::vector<int32_t> row_owner(ph.nrows, 0);
        for (int32_t g = 0; g < P.G; ++g) {
            const PhaseGeo G = phase_geo<true>(a, p, g, tile);
            if (G.r0 > G.r1 || G.r0 < 0 || G.r1 > ph.nrows) {
                ++bad;
                continue;
            }
            for (int32_t r = G.r0; r < G.r1; ++r) row_owner[r]++;
            RunHdr h;
            Run runs[MAX_RUNS];
            make_runs<true>(a, p, g, tile, h, runs);
            const int32_t U = h.U;
            if (U != G.U) ++bad;
            for (int32_t u = 0; u < U; ++u)
                if (first_wave_hdr(h, u) != first_wave(u, U, STREAM_WAVES)) ++bad;
            std::vector<uint32_t> slot_writes;
            for (int32_t w = 0; w < STREAM_WAVES; ++w) {
                const int32_t ub = U > 0 ? wave_begin(w, U, STREAM_WAVES) : 0;
                const int32_t ue = U > 0 ? wave_begin(w + 1, U, STREAM_WAVES) : 0;
                for (int32_t v = ub; v < ue; ++v) {
                    if (tile) {
                        const TileDesc d = unit_desc_tile(h, runs, v, ub, ue, w, nb);
                        if (!d.valid || d.nrec == 0 || (d.nrec & 15u) || d.rows < 1 || d.rows > TILE_ROWS) {
                            ++bad;
                            continue;
                        }
                        if (d.seg_end)
                            for (int32_t row = 0; row < d.rows; ++row)
                                for (int32_t b = 0; b < nb; ++b)
                                    slot_writes.push_back((uint32_t)(d.slot0 + row * d.slot_stride + b));
                        if (d.xoff + UNIT * 2u > (uint32_t)ph.xb * 2u) ++bad;
                    } else {
                        const UnitDesc d = unit_desc_runs(h, runs, v, ub, ue, w, nb);
                        if ((d.meta & 0x8000u) == 0 || d.nbytes == 0 || (d.nbytes & 15u)) {
                            ++bad;
                            continue;
                        }
                        if (d.meta & 0x4000u)
                            for (int32_t b = 0; b < nb; ++b) slot_writes.push_back((d.meta >> 16) + (uint32_t)b);
                        if (((d.meta & 0x3FFFu) << 4) + UNIT * 2u > (uint32_t)ph.xb * 2u) ++bad;
                    }
                }
                // units just outside the wave's share are invalid
                if (tile ? unit_desc_tile(h, runs, ue, ub, ue, w, nb).valid
                         : unit_desc_runs(h, runs, ue, ub, ue, w, nb).nbytes != 0)
                    ++bad;
            }
            // every unit of every owned row-part, once, with the right address
            int32_t rp_base = 0, u_base = 0;
            if (h.nruns != ph.nstages) ++bad;
            std::vector<uint32_t> slot_reads;
            for (int32_t si = 0; si < ph.nstages && si < h.nruns; ++si) {
                const DevStage &sg = P.stages[ph.stage0 + si];
                const StageSpan sp = stage_span(sg, G.r0, G.r1, 0, 0);
                const Run &rn = runs[si];
                if (rn.stage != ph.stage0 + si || rn.nrows != sp.nrows || (sp.nrows && rn.row0 != sp.row0) ||
                    rn.u_base != u_base || rn.rp_base != rp_base || rn.epi != sg.epi || rn.y != sg.y ||
                    rn.c0 != sg.c0 || rn.carry != sg.carry)
                    ++bad;
                const int32_t ntiles = (sp.nrows + TILE_ROWS - 1) / TILE_ROWS;
                const int32_t nseg = (tile ? ntiles : sp.nrows) * sg.parts;
                for (int32_t sgi = 0; sgi < nseg; ++sgi) {
                    const int32_t grp = sgi / sg.parts, pt = sgi % sg.parts;
                    const uint16_t *Wp = pt == 0 ? sg.W : sg.W_up;
                    for (int32_t c = 0; c < sg.nchunks; ++c) {
                        const int32_t v = u_base + sgi * sg.nchunks + c;
                        const int32_t w = first_wave(v, U, STREAM_WAVES);
                        const int32_t ub = wave_begin(w, U, STREAM_WAVES), ue = wave_begin(w + 1, U, STREAM_WAVES);
                        if (v < ub || v >= ue) ++bad;
                        const uint32_t koff = (uint32_t)(sg.c0 + c) * UNIT * 2u;
                        if (tile) {
                            const TileDesc d = unit_desc_tile(h, runs, v, ub, ue, w, nb);
                            const int32_t rows = std::min(TILE_ROWS, sp.nrows - grp * TILE_ROWS);
                            const uint16_t *tp = Wp + (int64_t)(sp.row0 + grp * TILE_ROWS) * sg.K;
                            if (d.ptr != (uint64_t)(uintptr_t)tp + koff) ++bad;
                            if (d.rows != rows || d.nrec != (uint32_t)(rows * sg.K * 2) - koff) ++bad;
                            if (d.kval != sg.K - (sg.c0 + c) * UNIT || d.rstride != sg.K * 2) ++bad;
                        } else {
                            const UnitDesc d = unit_desc_runs(h, runs, v, ub, ue, w, nb);
                            const uint16_t *rowp = Wp + (int64_t)(sp.row0 + grp) * sg.K;
                            if (d.ptr != (uint64_t)(uintptr_t)rowp + koff) ++bad;
                            if (d.nbytes != (uint32_t)(sg.K * 2) - koff) ++bad;
                        }
                    }
                }
                // the epilogue walks rows; each row-part reads its slots
                for (int32_t i = 0; i < sp.nrows; ++i)
                    for (int32_t pt = 0; pt < sg.parts; ++pt) {
                        const int32_t rp = rp_base + i * sg.parts + pt;
                        const int32_t a0 = first_unit_of_rowpart(rn, i, pt, tile);
                        const int32_t span = first_wave(a0 + sg.nchunks - 1, U, STREAM_WAVES) -
                                             first_wave(a0, U, STREAM_WAVES) + 1;
                        if (span > ph.jmax) ++bad;
                        for (int32_t j = 0; j < span; ++j)
                            for (int32_t b = 0; b < nb; ++b)
                                slot_reads.push_back((uint32_t)((rp * ph.jmax + j) * nb + b));
                    }
                rp_base += sp.nrows * sg.parts;
                u_base += units_of(sp.nrows, sg.parts, sg.nchunks, tile);
            }
            if (u_base != U) ++bad;
            // the staged epilogue inputs and the K-window carry of every owned
            // row-part fit their areas
            bool staged = false, carried = false;
            for (int32_t si = 0; si < ph.nstages; ++si) {
                const DevStage &sg = P.stages[ph.stage0 + si];
                staged |= (sg.bias || sg.residual || sg.post_y) && !(sg.carry & CARRY_OUT);
                carried |= sg.carry != 0;
            }
            if (staged && (size_t)rp_base * epi_rec(nb) * 4 > (size_t)(ph.carry_off - ph.epi_off)) ++bad;
            if (carried && ph.carry_off + (size_t)rp_base * nb * 4 > P.lds_total()) ++bad;
            std::sort(slot_writes.begin(), slot_writes.end());
            std::sort(slot_reads.begin(), slot_reads.end());
            if (slot_writes != slot_reads) ++bad;
            if (std::adjacent_find(slot_writes.begin(), slot_writes.end()) != slot_writes.end()) ++bad;
            if (!slot_writes.empty() && (size_t)(slot_writes.back() + 1) * 4 > (size_t)P.part_bytes[p]) ++bad;
            if ((size_t)rp_base * nb * 4 > (size_t)(ph.prm_off - ph.part_off) && !slot_writes.empty() &&
                (size_t)rp_base * ph.jmax * nb * 4 > (size_t)P.part_bytes[p])
                ++bad;
        }
        for (int32_t r = 0; r < ph.nrows; ++r)
            if (row_owner[r] != 1) ++bad;
    }
    return bad;
}

size_t wgn_decode_attention_workspace_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t slots,
                                            int32_t head_dim) {
    AttLayout L;
    return att_shape(batch, q_heads, kv_heads, slots, head_dim, L) == WGN_OK ? L.total : 0;
}

wgn_status wgn_decode_attention(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                                const int32_t *pos, int32_t batch, int32_t q_heads, int32_t kv_heads,
                                int32_t slots, int32_t head_dim, float scale, void *out, void *workspace,
                                size_t ws_bytes, wgn_stream stream) {
    AttLayout L;
    wgn_status st = att_shape(batch, q_heads, kv_heads, slots, head_dim, L);
    if (st != WGN_OK) return st;
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !pos || !out) return WGN_E_ARG;
    if (!std::isfinite(scale)) return WGN_E_ARG;
    if (!a16(q) || !a16(k_new) || !a16(v_new) || !a16(k_cache) || !a16(v_cache) || !a16(out) || !a4(pos))
        return WGN_E_ALIGN;
    {
        const size_t cache = (size_t)batch * kv_heads * slots * ATT_D * 2;
        const Range rk = rng(k_cache, cache), rv = rng(v_cache, cache);
        const Range ro = rng(out, (size_t)batch * q_heads * ATT_D * 2);
        const Range rin[4] = {rng(q, (size_t)batch * q_heads * ATT_D * 2),
                              rng(k_new, (size_t)batch * kv_heads * ATT_D * 2),
                              rng(v_new, (size_t)batch * kv_heads * ATT_D * 2), rng(pos, (size_t)batch * 4)};
        if (overlap(rk, rv) || overlap(ro, rk) || overlap(ro, rv)) return WGN_E_ARG;
        for (const Range &x : rin)
            if (overlap(x, rk) || overlap(x, rv) || overlap(x, ro)) return WGN_E_ARG;
    }
    if (L.top > 0) {
        if (!workspace || ((uintptr_t)workspace & 255)) return WGN_E_WORKSPACE;
        if (ws_bytes < L.total) return WGN_E_WORKSPACE;
    }
    DevInfo d = device_info();
    if (!d.ok) return WGN_E_DEVICE;
    AttnArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = (const uint16_t *)q;
    a.k_new = (const uint16_t *)k_new;
    a.v_new = (const uint16_t *)v_new;
    a.k_cache = (uint16_t *)k_cache;
    a.v_cache = (uint16_t *)v_cache;
    a.pos = pos;
    a.out = (uint16_t *)out;
    for (int32_t l = 0; l < L.top; ++l) a.part[l] = (float *)((char *)workspace + L.part_off[l]);
    for (int32_t l = 1; l <= L.top; ++l) a.tick[l] = (uint32_t *)((char *)workspace + L.tick_off[l]);
    for (int32_t l = 0; l <= ATT_MAX_LEVELS; ++l) a.count[l] = L.count[l];
    a.top = L.top;
    a.slots = slots;
    a.hq = q_heads;
    a.hkv = kv_heads;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
    hipError_t e = note(launch_decode_attention(a, q_heads / kv_heads, batch, (hipStream_t)stream),
                        "decode_attention launch");
    return e == hipSuccess ? WGN_OK : WGN_E_HIP;
}

wgn_status wgn_gemv_int4(const void *x, int64_t x_stride, int32_t batch, int32_t K, const void *W4,
                         const void *scales, const void *zeros, int32_t N, void *y, int64_t y_stride,
                         wgn_stream stream) {
    if (!x || !W4 || !scales || !zeros || !y) return WGN_E_ARG;
    if (batch < 1 || batch > 8 || N < 1 || K < 128 || (K % 128)) return WGN_E_ARG;
    if ((batch > 1 && (x_stride < K || y_stride < N)) || x_stride < 0 || y_stride < 0) return WGN_E_ARG;
    if (!a16(x) || !a16(W4) || (x_stride & 7) || !a2(scales) || !a2(zeros) || !a2(y)) return WGN_E_ALIGN;
    if (gemv_int4_lds_bytes(batch, K) > 160 * 1024) return WGN_E_UNSUPPORTED;
    {
        const Range ry = rng(y, ((size_t)(batch - 1) * y_stride + N) * 2);
        const Range rin[4] = {rng(x, ((size_t)(batch - 1) * x_stride + K) * 2), rng(W4, (size_t)N * K / 2),
                              rng(scales, (size_t)N * (K / 128) * 2), rng(zeros, (size_t)N * (K / 128) * 2)};
        for (const Range &r : rin)
            if (overlap(r, ry)) return WGN_E_ARG;
    }
    DevInfo d = device_info();
    if (!d.ok) return WGN_E_DEVICE;
    hipError_t e = note(launch_gemv_int4((const uint16_t *)x, x_stride, batch, K, (const uint8_t *)W4,
                                         (const uint16_t *)scales, (const uint16_t *)zeros, N, (uint16_t *)y,
                                         batch > 1 ? y_stride : N, d.cus > 0 ? d.cus : 256, (hipStream_t)stream),
                        "gemv_int4 launch");
    return e == hipSuccess ? WGN_OK : WGN_E_HIP;
}

wgn_status wgn_stream_read(const void *src, size_t bytes, int32_t grid, int32_t threads, int32_t depth,
                           uint32_t *sink, wgn_stream stream) {
    if (!src || !sink || bytes == 0 || (bytes & 15)) return WGN_E_ARG;
    if (grid < 1 || grid > 65536 || threads < 64 || threads > 1024 || (threads & 63)) return WGN_E_ARG;
    if (depth != 1 && depth != 2 && depth != 4 && depth != 8 && depth != 16) return WGN_E_ARG;
    if (!a16(src) || !a4(sink)) return WGN_E_ALIGN;
    DevInfo d = device_info();
    if (!d.ok) return WGN_E_DEVICE;
    hipError_t e = note(launch_stream_read(src, (uint64_t)(bytes >> 4), grid, threads, depth, sink, (hipStream_t)stream),
                        "stream_read launch");
    return e == hipSuccess ? WGN_OK : WGN_E_HIP;
}

}  // extern "C"

// ------------------------------------------------------------ backward pass
struct wgn_backward {
    int32_t n = 0, B = 0, G = 0;
    void *ws = nullptr;
    size_t err_off = 0, ctr_off = 0;
    int32_t nctr = 0;
    wgn::BwdArgs a;
};

namespace {

using wgn::BwdLayer;

// Offsets of one backward run's workspace: the layer table, per-layer
// statistics and x-hat, two partial buffers and two share buffers (by block
// parity), then the counters: one flag per workgroup of the largest grid
// (the device's resident workgroups, at most the largest block's tiles)
// and the error word.
struct BwdLayout {
    std::vector<size_t> stats, xh;
    size_t descs = 0, part[2] = {0, 0}, q[2] = {0, 0}, ctr = 0, total = 0;
    int32_t max_items = 0, nctr = 0;
};

inline size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

wgn_status bwd_check_stages(const wgn_stage *stages, int32_t n, int32_t batch) {
    if (!stages || n < 1 || n > wgn::BWD_MAX_LAYERS) return WGN_E_ARG;
    if (batch < 1 || batch > wgn::BWD_MAX_BATCH) return WGN_E_ARG;
    for (int32_t i = 0; i < n; ++i) {
        const wgn_stage &s = stages[i];
        const wgn_status st = check_stage(s, batch, wgn::BWD_MAX_BATCH);
        if (st != WGN_OK) return st;
        if (s.norm != NORM_LAYER || s.epi != EPI_GELU_TANH || s.residual) return WGN_E_UNSUPPORTED;
        if (!s.logits) return WGN_E_ARG;  // the pre-activations the forward kept
        if ((int64_t)s.N * s.K >= ((int64_t)1 << 30)) return WGN_E_UNSUPPORTED;  // 32-bit byte offsets
        if (i > 0 && s.K != stages[i - 1].N) return WGN_E_ARG;
    }
    return WGN_OK;
}

BwdLayout bwd_layout(const wgn_stage *stages, int32_t n, int32_t B) {
    BwdLayout L;
    size_t o = 0;
    L.descs = o;
    o = up256(o + (size_t)n * sizeof(BwdLayer));
    size_t part = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t N = stages[i].N, K = stages[i].K;
        const int32_t nrb = (N + wgn::BWD_TILE_ROWS - 1) / wgn::BWD_TILE_ROWS;
        const int32_t ncb = (K + wgn::BWD_TILE_COLS - 1) / wgn::BWD_TILE_COLS;
        L.max_items = std::max(L.max_items, nrb * ncb);
        part = std::max(part, (size_t)nrb * B * K * 4);
        L.stats.push_back(o);
        o = up256(o + (size_t)B * 2 * 4);
        L.xh.push_back(o);
        o = up256(o + (size_t)B * K * 2);
    }
    for (int p = 0; p < 2; ++p) {
        L.part[p] = o;
        o = up256(o + part);
        L.q[p] = o;
        o = up256(o + (size_t)L.max_items * B * 2 * 4);
    }
    L.ctr = o;
    // flags of every workgroup (rounded up to 4: the polls read 16 bytes), the error word
    L.nctr = (L.max_items + 3) / 4 * 4 + 4;
    o = up256(o + (size_t)L.nctr * 4);
    L.total = o;
    return L;
}

// Byte ranges the backward pass writes (outputs) and reads (forward tensors);
// outputs may overlap neither each other nor anything read.
wgn_status bwd_check_ranges(const wgn_stage *st, int32_t n, int32_t B, const wgn_grad *gr, const void *g_out,
                            int64_t g_stride, const void *g_in, int64_t gin_stride, const void *ws, size_t ws_bytes) {
    std::vector<Range> w, r;
    auto rows = [&](const void *p, int64_t stride, int32_t len) {
        return rng(p, ((size_t)(B - 1) * (size_t)stride + (size_t)len) * 2);
    };
    for (int32_t i = 0; i < n; ++i) {
        const wgn_stage &s = st[i];
        const wgn_grad &g = gr[i];
        w.push_back(rng(g.gW, (size_t)s.N * s.K * 2));
        if (g.gbias) w.push_back(rng(g.gbias, (size_t)s.N * 2));
        if (g.ggamma) w.push_back(rng(g.ggamma, (size_t)s.K * 2));
        if (g.gbeta) w.push_back(rng(g.gbeta, (size_t)s.K * 2));
        if (g.gy) w.push_back(rng(g.gy, (size_t)B * s.N * 2));
        if (g.gz) w.push_back(rng(g.gz, (size_t)B * s.N * 2));
        r.push_back(rng(s.W, (size_t)s.N * s.K * 2));
        r.push_back(rows(s.x, s.x_stride, s.K));
        r.push_back(rng(s.logits, (size_t)B * s.N * 4));
        if (s.gamma) r.push_back(rng(s.gamma, (size_t)s.K * 2));
        if (s.beta) r.push_back(rng(s.beta, (size_t)s.K * 2));
    }
    const wgn_stage &last = st[n - 1];
    if (g_out) r.push_back(rows(g_out, g_stride, last.N));
    else r.push_back(rows(last.y, last.y_stride, last.N));
    if (g_in) w.push_back(rows(g_in, gin_stride, st[0].K));
    w.push_back(rng(ws, ws_bytes));
    std::sort(w.begin(), w.end(), [](const Range &a, const Range &b) { return a.lo < b.lo; });
    for (size_t i = 1; i < w.size(); ++i)
        if (w[i].lo < w[i - 1].hi) return WGN_E_ARG;
    for (const Range &q : r) {
        auto it = std::lower_bound(w.begin(), w.end(), q.hi, [](const Range &a, uintptr_t v) { return a.lo < v; });
        if (it != w.begin() && overlap(*(it - 1), q)) return WGN_E_ARG;
    }
    return WGN_OK;
}

}  // namespace

extern "C" {

size_t wgn_backward_workspace_bytes(const wgn_stage *stages, int32_t n_stages, int32_t batch) {
    if (bwd_check_stages(stages, n_stages, batch) != WGN_OK) return 0;
    return bwd_layout(stages, n_stages, batch).total;
}

wgn_status wgn_backward_create(const wgn_stage *stages, int32_t n, int32_t batch, const wgn_grad *grads,
                               const void *g_out, int64_t g_stride, void *g_in, int64_t gin_stride,
                               void *workspace, size_t ws_bytes, wgn_stream stream, wgn_backward **out) {
    if (!out) return WGN_E_ARG;
    *out = nullptr;
    wgn_status st = bwd_check_stages(stages, n, batch);
    if (st != WGN_OK) return st;
    if (!grads) return WGN_E_ARG;
    for (int32_t i = 0; i < n; ++i) {
        const wgn_stage &s = stages[i];
        const wgn_grad &g = grads[i];
        if (!g.gW) return WGN_E_ARG;
        if (!g.gbias != !s.bias) return WGN_E_ARG;
        if ((g.ggamma && !s.gamma) || (g.gbeta && !s.beta)) return WGN_E_ARG;
        if (!a16(g.gW)) return WGN_E_ALIGN;
        if (!a2(g.gbias) || !a2(g.ggamma) || !a2(g.gbeta) || !a2(g.gy) || !a2(g.gz)) return WGN_E_ALIGN;
    }
    const wgn_stage &last = stages[n - 1];
    if (g_out && batch > 1 && g_stride < last.N) return WGN_E_ARG;
    if (g_in && batch > 1 && gin_stride < stages[0].K) return WGN_E_ARG;
    if (!a2(g_out) || !a2(g_in)) return WGN_E_ALIGN;
    const BwdLayout L = bwd_layout(stages, n, batch);
    if (!workspace || ws_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return WGN_E_WORKSPACE;
    st = bwd_check_ranges(stages, n, batch, grads, g_out, g_stride, g_in, gin_stride, workspace, ws_bytes);
    if (st != WGN_OK) return st;
    DevInfo d = device_info();
    if (!d.ok) return WGN_E_DEVICE;

    char *ws = (char *)workspace;
    std::vector<BwdLayer> img((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
        const wgn_stage &s = stages[i];
        const wgn_grad &g = grads[i];
        BwdLayer &b = img[(size_t)i];
        std::memset(&b, 0, sizeof b);
        b.W = (const uint16_t *)s.W;
        b.x = (const uint16_t *)s.x;
        b.gamma = (const uint16_t *)s.gamma;
        b.beta = (const uint16_t *)s.beta;
        b.pre = s.logits;
        b.gW = (uint16_t *)g.gW;
        b.gb = (uint16_t *)g.gbias;
        b.ggamma = (uint16_t *)g.ggamma;
        b.gbeta = (uint16_t *)g.gbeta;
        b.gy = (uint16_t *)g.gy;
        b.gz = (uint16_t *)g.gz;
        b.stats = (float *)(ws + L.stats[(size_t)i]);
        b.xh = (uint16_t *)(ws + L.xh[(size_t)i]);
        b.x_stride = batch > 1 ? s.x_stride : s.K;
        b.eps = s.eps;
        b.N = s.N;
        b.K = s.K;
        b.nrb = (s.N + wgn::BWD_TILE_ROWS - 1) / wgn::BWD_TILE_ROWS;
        b.ncb = (s.K + wgn::BWD_TILE_COLS - 1) / wgn::BWD_TILE_COLS;
    }
    const int32_t resident = wgn::bwd_resident_grid();
    if (resident < 1) return WGN_E_HIP;
    hipStream_t s = (hipStream_t)stream;
    if (note(hipMemcpyAsync(ws + L.descs, img.data(), img.size() * sizeof(BwdLayer), hipMemcpyHostToDevice, s),
             "backward upload") != hipSuccess ||
        note(hipStreamSynchronize(s), "backward create sync") != hipSuccess)
        return WGN_E_HIP;
    wgn_backward *h = new (std::nothrow) wgn_backward;
    if (!h) return WGN_E_HIP;
    h->n = n;
    h->B = batch;
    h->G = std::min(L.max_items, resident);  // every workgroup resident at once
    h->ws = workspace;
    h->ctr_off = L.ctr;
    h->nctr = L.nctr;
    h->err_off = L.ctr + (size_t)(L.nctr - 4) * 4;
    wgn::BwdArgs &a = h->a;
    std::memset(&a, 0, sizeof a);
    a.layers = (const BwdLayer *)(ws + L.descs);
    a.n = n;
    a.B = batch;
    a.y = (const uint16_t *)last.y;
    a.y_stride = batch > 1 ? last.y_stride : last.N;
    a.g_out = (const uint16_t *)g_out;
    a.g_stride = batch > 1 ? g_stride : last.N;
    a.g_in = (uint16_t *)g_in;
    a.gin_stride = batch > 1 ? gin_stride : stages[0].K;
    for (int p = 0; p < 2; ++p) {
        a.part[p] = (float *)(ws + L.part[p]);
        a.q[p] = (float *)(ws + L.q[p]);
    }
    a.flags = (uint32_t *)(ws + L.ctr);
    a.err = (uint32_t *)(ws + h->err_off);
    a.tile_wgs = h->G;
    a.wait_ticks = WAIT_TICKS;
    *out = h;
    return WGN_OK;
}

wgn_status wgn_backward_run(const wgn_backward *h, int32_t prefetch, wgn_stream stream) {
    if (!h || (prefetch != 0 && prefetch != 1)) return WGN_E_ARG;
    hipStream_t s = (hipStream_t)stream;
    wgn::BwdArgs a = h->a;
    a.prefetch = prefetch;
    if (note(wgn::launch_bwd_prep(a.layers, h->n, h->B, a.flags, h->nctr, s), "backward prep launch") != hipSuccess ||
        note(wgn::launch_bwd(a, h->G, s), "backward launch") != hipSuccess)
        return WGN_E_HIP;
    return WGN_OK;
}

wgn_status wgn_backward_check(const wgn_backward *h, wgn_stream stream) {
    if (!h) return WGN_E_ARG;
    if (note(hipStreamSynchronize((hipStream_t)stream), "backward check sync") != hipSuccess) return WGN_E_HIP;
    uint32_t err = 0;
    if (note(hipMemcpy(&err, (const char *)h->ws + h->err_off, 4, hipMemcpyDeviceToHost), "backward check read") !=
        hipSuccess)
        return WGN_E_HIP;
    return err ? WGN_E_TIMEOUT : WGN_OK;
}

wgn_status wgn_backward_set_wait_us(wgn_backward *h, int64_t us) {
    if (!h) return WGN_E_ARG;
    if (us > (int64_t)(WAIT_TICKS / 100) * 1000) return WGN_E_ARG;
    h->a.wait_ticks = us < 0 ? WAIT_TICKS : (uint64_t)us * 100u;  // the real-time clock runs at 100 MHz
    return WGN_OK;
}

int32_t wgn_backward_grid(const wgn_backward *h) { return h ? h->G : -1; }

wgn_status wgn_backward_set_trace(wgn_backward *h, uint64_t *device_buf, size_t n_slots) {
    if (!h) return WGN_E_ARG;
    if (device_buf && n_slots < (size_t)h->n * h->G * wgn::BWD_TRACE_POINTS) return WGN_E_ARG;
    if (device_buf && (reinterpret_cast<uintptr_t>(device_buf) & 7u)) return WGN_E_ALIGN;
    h->a.trace = device_buf;
    return WGN_OK;
}

void wgn_backward_destroy(wgn_backward *h) { delete h; }

wgn_status wgn_chain_backward(const wgn_stage *stages, int32_t n, int32_t batch, const wgn_grad *grads,
                              const void *g_out, int64_t g_stride, void *g_in, int64_t gin_stride, int32_t prefetch,
                              void *workspace, size_t ws_bytes, wgn_stream stream) {
    if (prefetch != 0 && prefetch != 1) return WGN_E_ARG;
    wgn_backward *h = nullptr;
    wgn_status st = wgn_backward_create(stages, n, batch, grads, g_out, g_stride, g_in, gin_stride, workspace,
                                        ws_bytes, stream, &h);
    if (st != WGN_OK) return st;
    st = wgn_backward_run(h, prefetch, stream);
    wgn_backward_destroy(h);
    return st;
}

}  // extern "C"
