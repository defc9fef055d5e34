// wgn_loader.h -- where each streamed weight unit comes from.
//
// A streaming wave walks its share of every phase's units in a fixed order.
// Because weights never depend on activations, the walk can run ahead of the
// computation and across phase boundaries: the kernel issues the loads of the
// next block of units before it consumes the current block, so weight traffic
// of phase p+1 is already in flight while the workgroup waits for phase p to
// finish device-wide.  This is the prefetch-the-next-layer idea of "Making
// small PyTorch ops faster on a laptop GPU" (section "Prefetching the next
// layer while this one runs") moved inside one persistent kernel.
//
// make_runs() reduces a phase to the workgroup's "run list" (one entry per
// stage of the phase); unit_desc_runs() (vector path) and unit_desc_tile()
// (matrix-core path) map one unit index to its weight address and the data
// the wave needs to consume it.  On the device, the control wave builds run
// lists three phases ahead into LDS and the streaming waves evaluate the unit
// descriptors of their next block from them; the host planner's self-test
// runs the same functions for every unit to check the partition.
#pragma once
#include "wgn_prog.h"

#if defined(__HIP_DEVICE_COMPILE__)
// Program descriptors are read-only for the kernel's lifetime: reading them
// through the constant address space lets the compiler use scalar loads,
// which never wait behind the vector loads of the weight stream.
#define WGN_CONST_PTR(T, p) ((const __attribute__((address_space(4))) T *)(p))
#else
#define WGN_CONST_PTR(T, p) ((const T *)(p))
#endif

namespace wgn {

template <bool CHAIN>
WGN_HD DevPhase phase_of(const KArgs &a, int32_t p) {
    if constexpr (CHAIN) return WGN_CONST_PTR(DevPhase, a.phases)[p];
    else return a.iph;
}
template <bool CHAIN>
WGN_HD DevStage stage_of(const KArgs &a, int32_t i) {
    if constexpr (CHAIN) return WGN_CONST_PTR(DevStage, a.stages)[i];
    else return a.ist;
}
template <bool CHAIN>
WGN_HD DevSource source_of(const KArgs &a, int32_t i) {
    if constexpr (CHAIN) return WGN_CONST_PTR(DevSource, a.sources)[i];
    else return a.isrc;
}

// Geometry of one phase for one workgroup.
struct PhaseGeo {
    int32_t p;
    int32_t r0, r1;        // rows owned in the phase's row space
    int32_t U;             // units owned
    int32_t jmax;
    int32_t xb_bytes;      // LDS bytes per batch row of x-hat
    int32_t stage0, nstages, src0;
    int32_t x_off, part_off;
};

template <bool CHAIN>
WGN_HD PhaseGeo phase_geo(const KArgs &a, int32_t p, int32_t g, bool tile) {
    const DevPhase ph = phase_of<CHAIN>(a, p);
    PhaseGeo G;
    G.p = p;
    if (ph.rb_off >= 0) {
        G.r0 = WGN_CONST_PTR(int32_t, a.rowb)[ph.rb_off + g];
        G.r1 = WGN_CONST_PTR(int32_t, a.rowb)[ph.rb_off + g + 1];
    } else {
        G.r0 = even_row_begin(g, ph.nrows, a.G);
        G.r1 = even_row_begin(g + 1, ph.nrows, a.G);
    }
    G.jmax = ph.jmax;
    G.xb_bytes = ph.xb * 2;
    G.stage0 = ph.stage0;
    G.nstages = ph.nstages;
    G.src0 = ph.src0;
    G.x_off = ph.x_off;
    G.part_off = ph.part_off;
    int32_t U = 0;
    for (int32_t i = 0; i < ph.nstages; ++i) {
        const DevStage st = stage_of<CHAIN>(a, ph.stage0 + i);
        StageSpan sp = stage_span(st, G.r0, G.r1, 0, 0);
        U += units_of(sp.nrows, st.parts, st.nchunks, tile);
    }
    G.U = U;
    return G;
}

// Run list of phase p for workgroup g: one entry per stage of the phase, in
// order (nrows = 0 when the workgroup owns none of its rows; an argmax stage
// still takes part in the merge then).
template <bool CHAIN>
WGN_HD void make_runs(const KArgs &a, int32_t p, int32_t g, bool tile, RunHdr &h, Run *runs) {
    const PhaseGeo G = phase_geo<CHAIN>(a, p, g, tile);
    h.U = G.U;
    h.jmax = G.jmax;
    h.xb_bytes = G.xb_bytes;
    h.x_off = G.x_off;
    h.part_off = G.part_off;
    {
        const DevPhase ph = phase_of<CHAIN>(a, p);
        h.epi_off = ph.epi_off;
        h.carry_off = ph.carry_off;
        int32_t hn = 0;
        int64_t in_bytes = 0;
        for (int32_t i = 0; i < ph.nsrc; ++i) {
            const DevSource src = source_of<CHAIN>(a, ph.src0 + i);
            hn |= src.norm != NORM_NONE ? 1 : 0;
            in_bytes += (int64_t)src.K * a.nb * 2;
        }
        h.has_norm = hn;
        h.share_in = in_bytes >= SHARE_IN_MIN_BYTES ? 1 : 0;
        h.pad3 = 0;
    }
    for (int32_t w = 0; w <= STREAM_WAVES; ++w) h.wb[w] = G.U > 0 ? wave_begin(w, G.U, STREAM_WAVES) : 0;
    int32_t n = 0, u_base = 0, rp_base = 0, rows = 0;
    h.rstart[0] = 0;
    for (int32_t i = 0; i < G.nstages && n < MAX_RUNS; ++i) {
        const DevStage st = stage_of<CHAIN>(a, G.stage0 + i);
        const StageSpan sp = stage_span(st, G.r0, G.r1, 0, 0);
        Run r;
        r.W = st.W;
        r.W_up = st.W_up;
        r.K = st.K;
        r.nchunks = st.nchunks;
        r.parts = st.parts;
        r.row0 = sp.row0;
        r.nrows = sp.nrows;
        r.u_base = u_base;
        r.rp_base = rp_base;
        r.c0 = st.c0;
        r.carry = st.carry;
        r.xoff = (uint32_t)source_of<CHAIN>(a, G.src0 + st.src).lds_off * 2u;
        r.stage = G.stage0 + i;
        r.epi = st.epi;
        r.N = st.N;
        r.am_slot = st.am_slot;
        r.bias = st.bias;
        r.residual = st.residual;
        r.y = st.y;
        r.logits = st.logits;
        r.maxval = st.maxval;
        r.res_stride = st.res_stride;
        r.y_stride = st.y_stride;
        r.post_y = st.post_y;
        r.post_F = st.post_F;
        r.post_bias = st.post_bias;
        r.post_stride = st.post_stride;
        runs[n++] = r;
        u_base += units_of(sp.nrows, st.parts, st.nchunks, tile);
        rp_base += sp.nrows * st.parts;
        rows += sp.nrows;
        h.rstart[n] = rows;
    }
    for (int32_t i = n + 1; i <= MAX_RUNS; ++i) h.rstart[i] = rows;
    h.nruns = n;
}

struct UnitDesc {
    uint64_t ptr;          // address of the unit's first byte (row start + chunk offset)
    uint32_t nbytes;       // bytes of the row from ptr on (0 = invalid unit: loads return 0)
    uint32_t meta;         // pack_meta(...)
};

// Descriptor of WG-local unit v from a run list (the form the kernel uses).
// A phase's source table (as the control wave uses it) and normalisation job
// list (read by every wave), in source order; every normalised source gets
// its gain (and shift) area in the phase's parameter area, in order.
template <bool CHAIN>
WGN_HD void make_phase_info(const KArgs &a, int32_t p, SrcInfo *T, NormHdr &J) {
    const DevPhase ph = phase_of<CHAIN>(a, p);
    int32_t off = 0, nj = 0;
    for (int32_t si = 0; si < MAX_SRC; ++si) {
        SrcInfo t;
        t.x = nullptr;
        t.x_stride = 0;
        t.K = 0;
        t.norm = NORM_NONE;
        t.eps = 0.0f;
        t.lds_off = 0;
        t.prm = ph.prm_off;
        t.prm_half = 0;
        t.has_gamma = 0;
        t.has_beta = 0;
        t.gamma = nullptr;
        t.beta = nullptr;
        if (si < ph.nsrc) {
            const DevSource src = source_of<CHAIN>(a, ph.src0 + si);
            const bool normed = src.norm != NORM_NONE;
            const int32_t pb = nchunks_of(src.K) * UNIT * 2 * 2;  // gain and shift, padded
            t.x = src.x;
            t.x_stride = src.x_stride;
            t.K = src.K;
            t.norm = src.norm;
            t.eps = src.eps;
            t.lds_off = src.lds_off;
            t.prm = ph.prm_off + off;
            t.prm_half = pb / 2;
            t.has_gamma = normed && src.gamma != nullptr;
            t.has_beta = src.norm == NORM_LAYER && src.beta != nullptr;
            t.gamma = t.has_gamma ? src.gamma : nullptr;
            t.beta = t.has_beta ? src.beta : nullptr;
            if (normed) {
                NormJob &jb = J.job[nj++];
                jb.norm = src.norm;
                jb.K = src.K;
                jb.xoff = src.lds_off;
                jb.prm = t.prm;
                jb.prm_half = t.prm_half;
                jb.eps = src.eps;
                jb.has_gamma = t.has_gamma;
                jb.has_beta = t.has_beta;
                off += pb;
            }
        }
        T[si] = t;
    }
    for (int32_t j = nj; j < MAX_SRC; ++j) {
        NormJob &jb = J.job[j];
        jb.norm = NORM_NONE;
        jb.K = 0;
        jb.xoff = 0;
        jb.prm = 0;
        jb.prm_half = 0;
        jb.eps = 0.0f;
        jb.has_gamma = 0;
        jb.has_beta = 0;
    }
    J.njobs = nj;
    J.nb = a.nb;
    J.x_off = ph.x_off;
    J.xb = ph.xb;
}

WGN_HD UnitDesc unit_desc_runs(const RunHdr &h, const Run *runs, int32_t v, int32_t u_beg, int32_t u_end,
                               int32_t w, int32_t B) {
    UnitDesc d;
    d.ptr = 0;
    d.nbytes = 0;
    d.meta = 0;
    if (v < u_beg || v >= u_end) return d;
    for (int32_t i = 0; i < h.nruns; ++i) {
        const Run &r = runs[i];
        const int32_t per_row = r.parts * r.nchunks;
        if (v < r.u_base + r.nrows * per_row) {
            const int32_t local = v - r.u_base;
            const int32_t rk = local / per_row;
            const int32_t rem = local - rk * per_row;
            const int32_t part = rem / r.nchunks;
            const int32_t chunk = rem - part * r.nchunks;
            const uint32_t off = (uint32_t)(r.c0 + chunk) * (UNIT * 2u);
            const uint16_t *rowp = (part == 0 ? r.W : r.W_up) + (int64_t)(r.row0 + rk) * r.K;
            d.ptr = (uint64_t)(uintptr_t)rowp + off;
            d.nbytes = (uint32_t)r.K * 2u - off;
            const int32_t rp = r.rp_base + rk * r.parts + part;
            const int32_t ua = v - chunk;
            const int32_t j = ua < u_beg ? w - first_wave_hdr(h, ua) : 0;
            const uint32_t slot = (uint32_t)((rp * h.jmax + j) * B);
            const bool seg_end = (chunk == r.nchunks - 1) || (v == u_end - 1);
            d.meta = pack_meta(r.xoff + (uint32_t)chunk * (UNIT * 2u), seg_end, true, slot);
            return d;
        }
    }
    return d;
}

// Matrix-core unit: TILE_ROWS consecutive row-parts (one part of one stage) x
// 512 K elements.  Wave-uniform; lane l then loads row l % 16 at K offset
// 8 * (l / 16) + 32 t for t = 0..15.
struct TileDesc {
    uint64_t ptr;          // first byte of the tile's first row at this chunk
    uint32_t nrec;         // bytes from ptr to the end of the tile's last row (0 = invalid unit)
    int32_t kval;          // K elements of a row from this chunk on
    uint32_t xoff;         // LDS byte offset of the chunk inside a batch row of x-hat
    int32_t rows;          // valid rows of the tile (1..16)
    int32_t rstride;       // row stride in bytes (K * 2)
    int32_t slot0;         // partial slot of the tile's first row (floats, batch included)
    int32_t slot_stride;   // slot distance between consecutive rows of the tile
    bool seg_end;          // last unit of this wave's share of the tile's row-parts
    bool valid;
};

WGN_HD TileDesc unit_desc_tile(const RunHdr &h, const Run *runs, int32_t v, int32_t u_beg, int32_t u_end,
                               int32_t w, int32_t nb) {
    TileDesc d;
    d.ptr = 0;
    d.nrec = 0;
    d.kval = 0;
    d.xoff = 0;
    d.rows = 0;
    d.rstride = 0;
    d.slot0 = 0;
    d.slot_stride = 0;
    d.seg_end = false;
    d.valid = false;
    if (v < u_beg || v >= u_end) return d;
    for (int32_t i = 0; i < h.nruns; ++i) {
        const Run &r = runs[i];
        const int32_t per_tile = r.parts * r.nchunks;
        const int32_t ntiles = (r.nrows + TILE_ROWS - 1) / TILE_ROWS;
        if (v < r.u_base + ntiles * per_tile) {
            const int32_t local = v - r.u_base;
            const int32_t ti = local / per_tile;
            const int32_t rem = local - ti * per_tile;
            const int32_t part = rem / r.nchunks;
            const int32_t chunk = rem - part * r.nchunks;
            const int32_t rows = r.nrows - ti * TILE_ROWS < TILE_ROWS ? r.nrows - ti * TILE_ROWS : TILE_ROWS;
            const int32_t kc = (r.c0 + chunk) * UNIT;
            const uint16_t *base = (part == 0 ? r.W : r.W_up) + (int64_t)(r.row0 + ti * TILE_ROWS) * r.K;
            d.ptr = (uint64_t)(uintptr_t)base + (uint64_t)kc * 2u;
            d.nrec = (uint32_t)rows * (uint32_t)r.K * 2u - (uint32_t)kc * 2u;
            d.kval = r.K - kc;
            d.xoff = r.xoff + (uint32_t)chunk * (UNIT * 2u);
            d.rows = rows;
            d.rstride = r.K * 2;
            const int32_t rp0 = r.rp_base + ti * TILE_ROWS * r.parts + part;
            const int32_t ua = v - chunk;
            const int32_t j = ua < u_beg ? w - first_wave_hdr(h, ua) : 0;
            d.slot0 = (rp0 * h.jmax + j) * nb;
            d.slot_stride = r.parts * h.jmax * nb;
            d.seg_end = (chunk == r.nchunks - 1) || (v == u_end - 1);
            d.valid = true;
            return d;
        }
    }
    return d;
}

// First unit (WG-local index) of row i, part pt of a run.
WGN_HD int32_t first_unit_of_rowpart(const Run &r, int32_t i, int32_t pt, bool tile) {
    return tile ? r.u_base + ((i / TILE_ROWS) * r.parts + pt) * r.nchunks
                : r.u_base + (i * r.parts + pt) * r.nchunks;
}

}  // namespace wgn
