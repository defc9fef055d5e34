// wgn_gemm.h -- launch arguments of the batched product on the matrix cores
// (wgn_gemm.hip), shared by the host planner (wgn_api.cpp) and the kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wgn {

constexpr int GEMM_MAX_BATCH = 128;                      // batch rows of one call
constexpr int GEMM_TILE_ROWS = 64;                       // output rows per item (16 per wave)
constexpr int GEMM_THREADS = 256;                        // four waves
constexpr int GEMM_KWIN = 64;                            // K elements per window (2 steps of 32)
#ifndef WGN_GEMM_RING
#define WGN_GEMM_RING 4
#endif
constexpr int GEMM_RING = WGN_GEMM_RING;                 // windows in the LDS ring (all but one in flight)
constexpr int GEMM_FRAG_BYTES = 64 * 16;                 // one wave's 16 x 16 FP32 accumulator tile

// One stage's work: the units are the GEMM_KWIN-element windows of its row
// tiles of 64 rows, tile after tile (ntiles x nwin); workgroup g of the
// stage's wgs streams units [g U / wgs, (g + 1) U / wgs) through a ring of
// LDS windows.  A tile whose windows fall to several workgroups (its
// contributors) is summed by the last of them to finish (tickets[tile]): the
// others leave their accumulators in part[], and the sum runs in contributor
// order, so results do not depend on timing.
struct GemmArgs {
    const uint16_t *W, *W_up;     // [N][K] BF16
    const uint16_t *x;            // [B][x_stride] BF16: x-hat (normalised) or the raw input
    const uint16_t *bias;         // [N] or null
    const uint16_t *residual;     // [B][res_stride] or null
    void *y;                      // [B][y_stride] BF16; argmax: int32 [B]
    float *logits;                // argmax: optional FP32 [B][N]
    float *maxval;                // argmax: optional FP32 [B]
    float *part;                  // contributor slots of shared tiles (gemm_tiles_shared), else unused
    uint32_t *tickets;            // [ntiles + 1], zero between calls
    uint64_t *keys;               // argmax: packed (value, index) keys [B], zero between calls
    int64_t x_stride, res_stride, y_stride;
    int32_t N, K, B, epi;
    int32_t ntiles;               // row tiles of GEMM_TILE_ROWS
    int32_t nwin;                 // windows of GEMM_KWIN per tile: ceil(K / GEMM_KWIN)
    int32_t wgs;                  // workgroups of the stage, at most ntiles x nwin
};

// Whether some tile of a stage falls to more than one workgroup: unless every
// workgroup's range is a whole number of tiles.
inline bool gemm_tiles_shared(int32_t ntiles, int32_t nwin, int32_t wgs) {
    const int64_t U = (int64_t)ntiles * nwin;
    return wgs > 1 && nwin > 1 && !(U % wgs == 0 && (U / wgs) % nwin == 0);
}

// Stages of one launch: consecutive independent stages of one epilogue family
// (Q, K and V, and an O product that reads its own input) run as one grid;
// items [start[i], start[i+1]) belong to stage i.  All share the batch, so
// the same kernel instance (16-row batch groups, SwiGLU or not) serves them;
// the normalised ones read one x-hat.
constexpr int GEMM_MAX_GROUP = 4;
struct GemmLaunch {
    GemmArgs s[GEMM_MAX_GROUP];
    int32_t start[GEMM_MAX_GROUP + 1];
    int32_t n;
};

// A window of bpad = 16 nt batch rows is nt * 2 copies of 1 KB (8 rows of
// GEMM_KWIN elements each), spread over the four waves; a ring slot holds
// every wave's copies (the ones past the batch are never read).
constexpr int gemm_copies_per_wave(int nt) { return (nt * 2 + 3) / 4; }
constexpr uint32_t gemm_slot_bytes(int nt) { return (uint32_t)gemm_copies_per_wave(nt) * 4u * 1024u; }
static_assert(GEMM_KWIN * 2 * 8 == 1024, "one copy is 8 batch rows of a window");

// LDS bytes of a call: the ring of input windows (also the epilogue's
// staging area), the argmax merge area and a flag; at most lds_cap(), so
// that WGN_GEMM_OCC workgroups fit one compute unit's 160 KB.
inline size_t gemm_lds_bytes(int32_t bpad) {
    return (size_t)GEMM_RING * gemm_slot_bytes((bpad + 15) / 16) + (size_t)4 * GEMM_MAX_BATCH * 8 + 16;
}
// Workgroups per compute unit that registers and LDS are sized for (two: the
// hardware keeps two at a time where the grid has more than one per unit).
#ifndef WGN_GEMM_OCC
#define WGN_GEMM_OCC 2
#endif
inline constexpr size_t lds_cap() { return 160 * 1024 / WGN_GEMM_OCC; }

hipError_t launch_gemm(const GemmLaunch &L, bool swiglu, size_t lds, hipStream_t s);
// x-hat rows [rows][K] (row stride K) of RMSNorm (layer = false) or LayerNorm.
hipError_t launch_norm_rows64(const uint16_t *x, int64_t x_stride, const uint16_t *gamma, const uint16_t *beta,
                              float eps, bool layer, uint16_t *y, int32_t rows, int32_t K, hipStream_t s);
// A fill kernel, not hipMemsetAsync: the calls may be captured in a HIP graph.
hipError_t launch_zero_words(uint32_t *p, int32_t n, hipStream_t s);

}  // namespace wgn
