// wgn_prog.h -- device program layout and the work-partition rules, shared by
// the host planner (wgn_api.cpp) and the kernels (wgn_kernels.hip).
//
// Work decomposition of one phase (a set of mutually independent stages):
//  * rows of all stages in the phase form one "row space"; every workgroup (WG)
//    owns a contiguous, cost-balanced run of whole rows;
//  * a row of a SwiGLU stage has two "row-parts" (gate, up), other rows one;
//  * row-parts are streamed in "units" of 512 consecutive K elements:
//      - vector path (batch <= 4): a unit is one row-part's 512 elements =
//        64 lanes x 16 bytes, one 128-bit load per lane, fully coalesced;
//        a block of 8 to 20 units (the ring's depth) is as many independent
//        loads;
//      - matrix-core path (any batch, used for batch > 4): a unit is a tile of
//        16 consecutive row-parts x 512 elements, streamed as 16 loads in
//        which lane l reads 16 bytes of row l%16 (64 contiguous bytes per row
//        per load) -- exactly the A operand of v_mfma_f32_16x16x32_bf16; a
//        block is one such unit;
//  * the WG's units are split evenly over its streaming waves (a row-part may
//    be split across neighbouring waves); each wave reduces its part of a
//    row-part and writes the partial to an LDS slot indexed by (row-part,
//    wave - first wave of that row-part), and the WG's control wave sums the
//    slots in wave order.  The order of every FP32 sum is therefore fixed by
//    (grid, shape) alone and results are bit-reproducible;
//  * a phase whose inputs do not fit in LDS (the 8960-long down-projection
//    input at batch 16) is split into "K windows": consecutive phases over
//    the same rows, each streaming a window of the K chunks; partial row sums
//    are carried in LDS from one window to the next and only the last window
//    runs the epilogue.
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define WGN_HD __host__ __device__ inline
#else
#define WGN_HD inline
#endif

namespace wgn {

constexpr int UNIT = 512;            // K elements per unit (64 lanes x 8 BF16)
constexpr int MAX_SRC = 4;           // distinct normalised inputs per phase
#ifndef WGN_STREAM_WAVES
#define WGN_STREAM_WAVES 7
#endif
constexpr int STREAM_WAVES = WGN_STREAM_WAVES;  // weight-streaming waves per WG
constexpr int WAVES = STREAM_WAVES + 1;   // + one control wave
constexpr int THREADS = WAVES * 64;
constexpr int MAX_BATCH = 16;
constexpr int MAX_BATCH_VALU = 4;   // largest batch of the vector path
constexpr int TILE_ROWS = 16;        // row-parts per matrix-core unit
constexpr int TRACE_POINTS = 12;
constexpr int MAX_RUNS = 8;          // stages per phase (the planner splits larger phases)
#ifndef WGN_EPI_BARRIER
#define WGN_EPI_BARRIER 1
#endif
// 1: the streaming waves issue the loads that follow a phase's last block only
// after the control wave has issued the phase's output stores (which would
// otherwise queue behind them in the compute unit's memory pipeline)
constexpr int EPI_BARRIER = WGN_EPI_BARRIER;
#ifndef WGN_EPI_SHARE
#define WGN_EPI_SHARE 3
#endif
// Which kernels run the epilogue's output rows (and argmax keys) on all waves
// (each wave then waits for its own stores before a barrier, so the flag
// follows all of them): 0 none, 1 the matrix-core path, 2 that and the burst
// ring 0 at batch 1 (measured slower there), 3 the matrix-core path and the
// interleaved ring at batch 2-3.
constexpr int EPI_SHARE = WGN_EPI_SHARE;
#ifndef WGN_IN_SHARE
#define WGN_IN_SHARE 2
#endif
// All waves share the input copies of a phase whose inputs are at least
// SHARE_IN_MIN_BYTES per workgroup (below that the extra barrier and the
// streaming waves' wait for their newest weight loads cost more than the
// copies take): 1 on the matrix-core path, 2 also on the interleaved ring
// (batch 2-4); the burst rings keep one large block in flight at a phase
// start and copy on the control wave alone.
constexpr int IN_SHARE = WGN_IN_SHARE;
constexpr int SHARE_IN_MIN_BYTES = 32 * 1024;
// Block-buffer rings of the vector path's streaming waves (the matrix-core
// path always uses ring 0's two buffers).  A wave keeps slots - 1 blocks of
// `depth` units in flight beyond the one it consumes:
//   ring 0: 2 buffers x 20 units, a consumed buffer refilled in one burst;
//   ring 1: 5 buffers x 8 units, refilled in one burst;
//   ring 2: 4 buffers x 10 units, a consumed buffer's loads issued one per
//           unit while the next buffer is consumed (a phase's last refill
//           then goes out after the next phase's x-hat barrier, so that path
//           needs no third barrier).
// Measured on the decode step and the LayerNorm chain: ring 0 is fastest at
// batch 1 with large phases, ring 2 at batch 2-4 with large phases, ring 1
// when phases give each wave only a few units (many phases in flight).
constexpr int NUM_RINGS = 3;
constexpr int ring_slots(int r) { return r == 1 ? 5 : r == 2 ? 4 : 2; }
constexpr int ring_depth(int r) { return r == 1 ? 8 : r == 2 ? 10 : 20; }
constexpr bool ring_interleaved(int r) { return r == 2; }
constexpr int MAX_SLOTS = 5;
// Run lists resident in LDS at once (a ring of desc_bufs(r), a power of two,
// so the index is a mask), and how far ahead of its own iteration the control
// wave writes one: phase p+desc_ahead(r)'s list at the end of iteration p.  A
// streaming wave reads lists up to slots + 1 phases ahead of the phase it
// consumes, hence slots + 2 (checked by the host schedule model for every
// ring).  A larger look-ahead than needed costs: every list up to it is built
// before the first phase starts, and at batch 1 those are built in place.
constexpr int desc_bufs(int r) { return ring_slots(r) + 2 <= 4 ? 4 : 8; }
constexpr int desc_ahead(int r) { return ring_slots(r) + 2; }
constexpr int MAX_DESC_BUFS = 8;
#ifndef WGN_BUILD_WIN
#define WGN_BUILD_WIN 0
#endif
// Whether the control wave builds run lists (and the next phase's source
// table) in LDS while the streaming waves consume a phase, instead of right
// after the phase's completion flag.  Only where lists are built in place
// (no precomputed images) on the vector path's ring 0; the list of phase
// p + desc_ahead is then written during phase p, so its buffer must not be
// phase p's own: the ring has 8 buffers.
constexpr bool build_in_window(bool tile, int r) { return WGN_BUILD_WIN != 0 && !tile && r == 0; }
constexpr int desc_bufs_k(bool tile, int r) { return build_in_window(tile, r) ? MAX_DESC_BUFS : desc_bufs(r); }
static_assert(desc_bufs(0) <= MAX_DESC_BUFS && desc_bufs(1) <= MAX_DESC_BUFS && desc_bufs(2) <= MAX_DESC_BUFS &&
                  ring_slots(0) <= MAX_SLOTS && ring_slots(1) <= MAX_SLOTS && ring_slots(2) <= MAX_SLOTS,
              "ring tables out of range");
constexpr uint64_t WAIT_TICKS = 200000000ull;  // default wait bound: 2 s at the 100 MHz real-time clock

enum { NORM_NONE = 0, NORM_RMS = 1, NORM_LAYER = 2 };
enum { EPI_NONE = 0, EPI_GELU_TANH = 1, EPI_SWIGLU = 2, EPI_ARGMAX = 3,
       EPI_F32 = 4 };  // internal: store the FP32 row sums (a product whose epilogue runs elsewhere)

// A normalised input vector ("source") of a phase, staged as BF16 in LDS.
struct DevSource {
    const uint16_t *x;
    const uint16_t *gamma;
    const uint16_t *beta;
    int64_t x_stride;
    int32_t K;
    int32_t norm;
    float eps;
    int32_t lds_off;       // element offset inside one batch row of the LDS x-hat area
};

struct DevStage {
    const uint16_t *W;
    const uint16_t *W_up;
    const uint16_t *bias;
    const uint16_t *residual;
    void *y;
    float *logits;
    float *maxval;
    int64_t res_stride;
    int64_t y_stride;
    int32_t N, K;
    int32_t epi;
    int32_t src;           // source index inside the phase
    int32_t nchunks;       // ceil(K / UNIT)
    int32_t parts;         // 2 for SwiGLU, else 1
    int32_t row_off;       // first row of this stage in the phase's row space
    int32_t am_slot;       // argmax slot (ARGMAX only)
    int32_t c0;            // first K chunk streamed (K windows; 0 otherwise)
    int32_t carry;         // CARRY_IN | CARRY_OUT (K windows; 0 otherwise)
    // A fused residual add of another stage ("post"): after storing its own
    // output o, this stage also stores post_y = R(o + post_F + post_bias),
    // where post_F holds that stage's FP32 row sums from an earlier phase.
    void *post_y;
    const float *post_F;
    const uint16_t *post_bias;
    int64_t post_stride;
};
// K-window carry: CARRY_OUT = this window ends in the LDS carry instead of an
// epilogue; CARRY_IN = the row sums start from the carry.
enum { CARRY_IN = 1, CARRY_OUT = 2 };

struct DevPhase {
    int32_t stage0, nstages;
    int32_t src0, nsrc;
    int32_t nrows;         // rows in the phase's row space
    int32_t wait;          // wait for every WG to finish the previous phase
    int32_t xb;            // LDS x-hat elements per batch row
    int32_t rb_off;        // offset of this phase's G+1 row bounds; -1 = even split
    int32_t jmax;          // partial slots per row-part
    int32_t x_off;         // LDS byte offset of x-hat (row stride xb elements)
    int32_t part_off;      // LDS byte offset of the partial slots
    int32_t prm_off;       // LDS byte offset of the norm gains/shifts
    int32_t epi_off;       // LDS byte offset of the staged bias/residual values
    int32_t carry_off;     // LDS byte offset of the K-window carry (row-parts x batch FP32)
    int32_t att;           // 0: a product phase; 2k+1 / 2k+2: the scores / merge phase of attention k
};

// Attention of each batch row's new token over its key/value cache, as two
// phases of a chain that stream no weights ("Making small PyTorch ops faster
// on a laptop GPU", section "A full decode step is a different story": the
// new key and value appended, FP32 softmax, the cache split across blocks and
// the splits merged; "One Token, Kernel by Kernel", section "The fix: Part
// 10's split-KV kernel": (batch, head, slot, dimension) cache layout, the
// valid length read on the device, each key/value head read once for its
// group of query heads).
//  * scores phase: item (batch row, key/value head, chunk of the row's valid
//    slots), one per workgroup; the control wave scores its slots for every query
//    head of the group, keeps a running maximum and weight sum per head
//    (online softmax) and writes one partial: the weighted value sums, the
//    maxima and the weight sums.  The chunk holding the new token's slot
//    takes that key and value from k_new / v_new and appends them.
//  * merge phase: item (batch row, query head, 8 or 16 dimensions), spread
//    over the workgroups; the control wave merges the valid chunks' partials of
//    its head (lane i takes chunks i, i + 64, ...; then a wave reduction in a
//    fixed order) and stores 16 BF16 outputs.
// Both phases end with the usual completion flags, so the product that reads
// `out` waits for the merge like for any earlier phase.
constexpr int ATTN_D = 128;          // head dimension
constexpr int ATTN_MAX_GROUP = 8;    // query heads per key/value head
// Slots one wave scores per pass (4 rows of 16 lanes x pass / 4 loads): 8 at
// batch 1 (about twice the chunks, so nearly every workgroup holds a scores
// item, each with half the arithmetic), else 16.
constexpr int attn_pass(int batch) { return batch == 1 ? 8 : 16; }
// Output dimensions per merge item: 8 at batch 1 (192 items of the pages'
// 12 query heads, one round of 256 workgroups, fewer wave reductions each),
// else 16.
constexpr int attn_slice(int batch) { return batch == 1 ? 8 : 16; }
// Floats of one partial: acc[G][D], then m[G], then l[G]; padded to 16 bytes.
WGN_HD int32_t attn_part_floats(int32_t G) { return (G * (ATTN_D + 2) + 3) & ~3; }
// LDS of a scores phase: the combine of the four 16-lane rows of its wave
// ([row][head][D] FP32, then m and l per (row, head)), then the staged first
// pass of cache rows (4 key and 4 value copies of 1 KB), then the group's
// query rows ([head][D] BF16).
constexpr int ATTN_STAGE_OFF = 4 * ATTN_MAX_GROUP * (ATTN_D + 2) * 4;
constexpr int ATTN_Q_OFF = ATTN_STAGE_OFF + 8 * 1024;
constexpr int ATTN_CMB_BYTES = ATTN_Q_OFF + ATTN_MAX_GROUP * ATTN_D * 2;
struct DevAttn {
    const uint16_t *q;       // [B][q_stride]: q_heads x ATTN_D (written earlier in the launch)
    const uint16_t *k_new;   // [B][k_stride]: kv_heads x ATTN_D
    const uint16_t *v_new;   // [B][v_stride]
    uint16_t *k_cache;       // [B][kv_heads][slots][ATTN_D]
    uint16_t *v_cache;
    const int32_t *pos;      // [B]: slot of the new token (out of range: no valid slot, output 0)
    uint16_t *out;           // [B][out_stride]: q_heads x ATTN_D
    float *part;             // [B * kv_heads][nchunk][attn_part_floats(G)] partials
    int64_t q_stride, k_stride, v_stride, out_stride;
    int32_t hq, hkv, slots;
    int32_t nchunk;          // chunks (scores items, partials) per (batch row, key/value head); a row's
                             // valid slots are split over them in whole passes on the device
    float scale_log2;        // score scale times log2(e): weights are 2^(s - m)
};

// One contiguous byte range of weights read by the optional touch pass (the
// Infinity-Cache prefetch of a later launch's weights on a second stream).
struct TouchRange {
    const void *p;
    uint64_t bytes;        // a multiple of 16
};
constexpr int MAX_TOUCH = 2 * MAX_RUNS;  // weight matrices of one launch (W and W_up of each stage)

// Kernel arguments (passed by value).  A chain points at a program in device
// memory; a single-stage call carries its one phase/stage/source inline.
struct KArgs {
    const DevPhase *phases;
    const DevStage *stages;
    const DevSource *sources;
    const int32_t *rowb;
    uint32_t *flags;       // [nphases][G] completion flags (persistent mode)
    uint32_t *run;         // run counter: a run's flags carry the value run + 1
    uint32_t *tickets;     // [n_argmax] argmax tickets, then [1] done ticket
    uint64_t *am_part;     // [n_argmax][G][batch] packed (value, index) keys
    uint32_t *err;         // error word
    uint64_t *trace;       // [nphases][G][TRACE_POINTS] timestamps, or null
    const char *runimg;    // chains: [nphases][G] run lists, RUN_BUF_STRIDE bytes each (built on the host)
    const char *phinfo;    // chains: [nphases] phase infos, PHASE_INFO_BYTES each (built on the host)
    const DevAttn *att;    // chains with attention phases: [attention items], else null
    int32_t p0, p1;        // phases of this launch
    int32_t persistent;
    int32_t G;
    int32_t n_argmax;
    int32_t nb;            // batch rows
    uint64_t wait_ticks;   // bound of every in-kernel wait (100 MHz ticks)
    DevPhase iph;
    DevStage ist;
    DevSource isrc;
};

// ---------------------------------------------------------- partition rules
// Even split of U units over W waves.  With U >= W every wave gets at least one
// unit; with U < W waves 0..U-1 get one unit each and the rest none, so empty
// waves never sit inside a row-part (the epilogue sums one slot per wave that
// covers a row-part, and every such wave writes its slot).
WGN_HD int32_t wave_begin(int32_t w, int32_t U, int32_t W) {
    if (U < W) return w < U ? w : U;
    return (int32_t)(((int64_t)w * U) / W);
}
// The wave whose range [wave_begin(w), wave_begin(w+1)) holds unit u (0 <= u < U).
WGN_HD int32_t first_wave(int32_t u, int32_t U, int32_t W) {
    if (U < W) return u;
    return (int32_t)(((int64_t)(u + 1) * W + U - 1) / U) - 1;
}
WGN_HD int32_t even_row_begin(int32_t g, int32_t nrows, int32_t G) {
    return (int32_t)(((int64_t)g * nrows) / G);
}
WGN_HD int32_t nchunks_of(int32_t K) { return (K + UNIT - 1) / UNIT; }
// Units of nrows rows (row-parts per row: parts) with nch chunks each.
WGN_HD int32_t units_of(int32_t nrows, int32_t parts, int32_t nch, bool tile) {
    return (tile ? (nrows + TILE_ROWS - 1) / TILE_ROWS : nrows) * parts * nch;
}
// Completion flags: one per (phase, workgroup), FLAG_WORDS words apart.  With
// FLAG_WORDS = 1 the row is dense and one poll of all flags is one 16-byte
// load per lane; wider strides put fewer flags in one 64-byte line (writers
// sharing a line delay each other) at the cost of more lines per poll.
#ifndef WGN_FLAG_WORDS
#define WGN_FLAG_WORDS 1
#endif
constexpr int FLAG_WORDS = WGN_FLAG_WORDS;
WGN_HD int32_t flag_row(int32_t G) { return FLAG_WORDS == 1 ? (G + 3) & ~3 : G * FLAG_WORDS; }
constexpr int MAX_GRID = 2048;
// Fixed device scratch of the allocation-free LM-head call: the ticket area
// (256 bytes) and one 8-byte key per (workgroup, batch row) for up to 256
// workgroups and 16 batch rows.
constexpr size_t SCRATCH_BYTES = 256 + 256 * 16 * 8;

// Meta word of one streamed unit (wave-uniform):
//   bits  0..13  x-hat byte offset / 16
//   bit   14     last unit of this wave's share of its row-part
//   bit   15     unit is valid
//   bits 16..31  partial slot index (in floats, already multiplied by batch)
WGN_HD uint32_t pack_meta(uint32_t xoff_bytes, bool seg_end, bool valid, uint32_t slot) {
    return ((xoff_bytes >> 4) & 0x3FFFu) | (seg_end ? 0x4000u : 0u) | (valid ? 0x8000u : 0u) |
           (slot << 16);
}

// One stage's rows inside one workgroup's share of a phase, as the streaming
// waves need it (built once per phase, read from LDS on the hot path).
struct Run {
    const uint16_t *W;
    const uint16_t *W_up;
    int32_t K, nchunks, parts, row0;   // row0: stage-local first row; K: row length
    int32_t nrows, u_base, rp_base;    // WG-local first unit / row-part (nrows may be 0)
    int32_t c0, carry;                 // first K chunk of the window; CARRY_* bits
    uint32_t xoff;                     // LDS byte offset of the stage's source in a batch row
    int32_t stage;                     // global stage index
    // epilogue fields (read by the control wave)
    int32_t epi, N, am_slot;
    const uint16_t *bias;
    const uint16_t *residual;
    void *y;
    float *logits;
    float *maxval;
    int64_t res_stride, y_stride;
    void *post_y;
    const float *post_F;
    const uint16_t *post_bias;
    int64_t post_stride;
};
struct RunHdr {
    int32_t nruns, U, jmax, xb_bytes;  // xb_bytes: x-hat row stride
    int32_t x_off, part_off;           // LDS byte offsets of x-hat and the partial slots
    int32_t has_norm;                  // the phase normalises an input (all waves take part)
    int32_t epi_off;                   // LDS byte offset of the staged epilogue inputs
    int32_t wb[STREAM_WAVES + 1];      // wave_begin(w) for w = 0..STREAM_WAVES
    int32_t rstart[MAX_RUNS + 1];      // first WG-local output row of each run (cumulative nrows)
    int32_t carry_off;                 // LDS byte offset of the K-window carry
    int32_t share_in;                  // matrix-core path: all waves copy the phase's inputs
    int32_t pad3;                      // the runs that follow the header start 8-byte aligned
};
// Run lists are built on the host for chains and copied into LDS as bytes, so
// the host and device compilations must agree on the layout.
static_assert(sizeof(Run) == 160 && alignof(Run) == 8, "Run layout");
static_assert(sizeof(RunHdr) == 112, "RunHdr layout");
// Floats per row-part in the staged epilogue inputs: bias, then the residual
// of each batch row, then the addend of a fused residual add per batch row.
WGN_HD int32_t epi_rec(int32_t nb) { return 1 + 2 * nb; }

// first_wave() from a header's wave boundaries (compares only, no division).
WGN_HD int32_t first_wave_hdr(const RunHdr &h, int32_t u) {
    int32_t w = 0;
#pragma unroll
    for (int32_t i = 1; i < STREAM_WAVES; ++i) w += h.wb[i] <= u ? 1 : 0;
    return w;
}
constexpr int RUN_BUF_BYTES = (int)(sizeof(RunHdr) + MAX_RUNS * sizeof(Run));
// stride of the LDS run-list buffers and of the precomputed run lists (whole
// 16-byte chunks: they are copied 16 bytes per lane)
constexpr int RUN_BUF_STRIDE = (RUN_BUF_BYTES + 15) & ~15;
// Fixed part of the dynamic LDS: the run-list ring, then six streaming-wave
// trace timestamps.  The per-phase areas (x-hat, partials, gains, epilogue
// inputs, K-window carry) follow at offsets the plan gives each phase; areas
// of different phases may overlap, since the control wave writes phase p+1's
// areas only after it has finished reading phase p's, and the streaming waves
// touch x-hat and partials only between a phase's two barriers.
// A normalisation job of a phase (one per normalised source), posted in LDS
// by the control wave and run by all waves of the workgroup.
struct NormJob {
    int32_t norm, K;       // NORM_RMS / NORM_LAYER, input length
    int32_t xoff;          // element offset of the source inside a batch row of x-hat
    int32_t prm;           // LDS byte offset of the gain (the shift follows at prm + prm_half)
    int32_t prm_half;
    float eps;
    int32_t has_gamma, has_beta;
};
struct NormHdr {
    int32_t njobs, nb, x_off, xb;  // x-hat base (bytes) and row stride (elements)
    NormJob job[MAX_SRC];
};
WGN_HD int32_t wgn_clz(uint32_t v) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_clz(v);
#else
    int32_t n = 0;
    while (n < 32 && !(v & 0x80000000u)) {
        v <<= 1;
        ++n;
    }
    return n;
#endif
}
// How nw waves share the normalisation of nb batch rows (padded to a power of
// two P): a row over one or more whole waves when P <= nw, several rows per
// wave otherwise.  nw (a power of two) is WAVES: all waves of a workgroup
// normalise together.
struct NormSplit {
    int32_t row, sub, lanes;   // batch row, lane index inside the row's lanes, lanes per row
    int32_t lpr;               // lanes of this row inside this wave (group_sum width)
    int32_t slot;              // statistics slot of this wave for its row
    int32_t w0, w1, rslot;     // waves [w0, w1) holding the row's statistics, slot inside them
    bool active;
};
WGN_HD NormSplit norm_split(int32_t nb, int32_t w, uint32_t lane, int32_t nw) {
    // nw is a power of two, so every quotient below is a shift.  The two
    // cases are merged into one branch-free form: up = log2(rows per wave)
    // (0 when a row spans whole waves), dn = log2(waves per row) (0 when a
    // wave holds several rows).
    NormSplit S;
    const int32_t shift = nb <= 1 ? 0 : 32 - wgn_clz((uint32_t)(nb - 1));  // P = 1 << shift
    const int32_t lognw = 31 - wgn_clz((uint32_t)nw);
    const int32_t up = shift > lognw ? shift - lognw : 0;
    const int32_t dn = shift > lognw ? 0 : lognw - shift;
    S.lpr = 64 >> up;
    S.row = ((w << up) >> dn) + (int32_t)(lane >> (6 - up));
    S.w0 = (S.row >> up) << dn;
    S.w1 = S.w0 + (1 << dn);
    S.lanes = (64 >> up) << dn;
    S.sub = (w - S.w0) * 64 + (int32_t)(lane & (uint32_t)(S.lpr - 1));
    S.slot = (int32_t)(lane >> (6 - up));
    S.rslot = S.row & ((1 << up) - 1);
    S.active = S.row < nb;
    return S;
}


constexpr int LDS_TRACE_OFF = 0;
constexpr int LDS_NORM_OFF = LDS_TRACE_OFF + 2 * 6 * 8;  // 6 streaming-wave timestamps per phase parity
// partial statistics: [wave][normalisation item of that wave][sum, sum of squares], FP64;
// items are (source, batch row) pairs, at most MAX_SRC * MAX_BATCH = 64 over WAVES waves
constexpr int STATS_ROWS = 8;        // items one wave may hold
constexpr int LDS_STATS_OFF = (LDS_NORM_OFF + (int)sizeof(NormHdr) + 15) & ~15;
// The phase's sources as the control wave uses them after its wait, written
// by that wave before the wait (one LDS read then replaces dependent scalar
// loads of the source descriptors on the critical path).
struct SrcInfo {
    const uint16_t *x;
    int64_t x_stride;
    int32_t K, norm;
    float eps;
    int32_t lds_off;       // element offset inside one batch row of x-hat
    int32_t prm, prm_half; // gain at LDS byte offset prm (the phase's area), shift at prm + prm_half
    int32_t has_gamma, has_beta;
    const uint16_t *gamma; // null unless has_gamma
    const uint16_t *beta;  // null unless has_beta
};
static_assert(sizeof(SrcInfo) == 64 && offsetof(SrcInfo, K) == 16 && offsetof(SrcInfo, prm) == 32,
              "SrcInfo is read as 16-byte words");
static_assert(sizeof(NormHdr) == 144, "NormHdr layout");
// A phase's source table and normalisation job list, as one image (the
// source table, then the job list): precomputed for chains, copied to
// LDS_SRC_OFF and LDS_NORM_OFF.
constexpr int PHASE_INFO_BYTES = MAX_SRC * (int)sizeof(SrcInfo) + (int)sizeof(NormHdr);
static_assert(PHASE_INFO_BYTES % 16 == 0 && PHASE_INFO_BYTES <= 64 * 16, "phase info fits one 16-byte read per lane");
static_assert(MAX_SRC * MAX_BATCH <= WAVES * STATS_ROWS, "normalisation items must fit the statistics slots");
constexpr int LDS_SRC_OFF = (LDS_STATS_OFF + WAVES * STATS_ROWS * 16 + 15) & ~15;
// The run-list ring comes last among the fixed areas; its size depends on the
// streaming waves' ring, so the per-phase areas of a program start at
// lds_dyn_off(run lists): the matrix-core path always streams with ring 0
// (4 lists), the vector path leaves room for any ring.
constexpr int LDS_DESC_OFF = (LDS_SRC_OFF + MAX_SRC * (int)sizeof(SrcInfo) + 15) & ~15;
constexpr int lds_dyn_off(int nbufs) { return (LDS_DESC_OFF + nbufs * RUN_BUF_STRIDE + 255) & ~255; }
constexpr int path_desc_bufs(bool tile) { return tile ? desc_bufs(0) : MAX_DESC_BUFS; }

// Per-(WG, stage) geometry inside a phase.
struct StageSpan {
    int32_t row0, nrows;   // stage-local first row and count owned by this WG
    int32_t rp_base;       // WG-local row-part index of its first row-part
    int32_t u_base;        // WG-local unit index of its first unit
};

WGN_HD StageSpan stage_span(const DevStage &st, int32_t r0, int32_t r1, int32_t rp_base,
                            int32_t u_base) {
    StageSpan s;
    int32_t lo = r0 > st.row_off ? r0 : st.row_off;
    int32_t hi = r1 < st.row_off + st.N ? r1 : st.row_off + st.N;
    s.row0 = lo - st.row_off;
    s.nrows = hi > lo ? hi - lo : 0;
    s.rp_base = rp_base;
    s.u_base = u_base;
    return s;
}

}  // namespace wgn
