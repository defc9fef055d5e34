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
constexpr int GEMM_RING = 4;                             // windows in the LDS ring (3 in flight)
constexpr int GEMM_FRAG_BYTES = 64 * 16;                 // one wave's 16 x 16 FP32 accumulator tile

// One call's work: items = ntiles x nslices; item i is row tile i / nslices
// (rows 64 t ..) over K slice i % nslices (elements [s kslice, (s+1) kslice),
// kslice a multiple of GEMM_KWIN), streamed through a ring of LDS windows of
// GEMM_KWIN elements.  With nslices > 1 each item
// leaves its accumulators in part[] and the last item of a tile to finish
// (tickets[tile]) adds the slices in slice order and applies the epilogue.
struct GemmArgs {
    const uint16_t *W, *W_up;     // [N][K] BF16
    const uint16_t *x;            // [B][x_stride] BF16: x-hat (normalised) or the raw input
    const uint16_t *bias;         // [N] or null
    const uint16_t *residual;     // [B][res_stride] or null
    void *y;                      // [B][y_stride] BF16; argmax: int32 [B]
    float *logits;                // argmax: optional FP32 [B][N]
    float *maxval;                // argmax: optional FP32 [B]
    float *part;                  // partial accumulators (nslices > 1)
    uint32_t *tickets;            // [ntiles + 1], zero between calls
    uint64_t *keys;               // argmax: packed (value, index) keys [B], zero between calls
    int64_t x_stride, res_stride, y_stride;
    int32_t N, K, B, epi;
    int32_t ntiles, nslices, kslice;
};

// Stages of one launch: consecutive stages that read the same input with the
// same normalisation (Q, K and V) run as one grid; items [start[i],
// start[i+1]) belong to stage i.  All share the batch, so the same kernel
// instance (16-row batch groups, SwiGLU or not) serves them.
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
// that two workgroups fit one compute unit's 160 KB.
inline size_t gemm_lds_bytes(int32_t bpad) {
    return (size_t)GEMM_RING * gemm_slot_bytes((bpad + 15) / 16) + (size_t)4 * GEMM_MAX_BATCH * 8 + 16;
}
inline constexpr size_t lds_cap() { return 80 * 1024; }

hipError_t launch_gemm(const GemmLaunch &L, bool swiglu, size_t lds, hipStream_t s);
// x-hat rows [rows][K] (row stride K) of RMSNorm (layer = false) or LayerNorm.
hipError_t launch_norm_rows64(const uint16_t *x, int64_t x_stride, const uint16_t *gamma, const uint16_t *beta,
                              float eps, bool layer, uint16_t *y, int32_t rows, int32_t K, hipStream_t s);
// A fill kernel, not hipMemsetAsync: the calls may be captured in a HIP graph.
hipError_t launch_zero_words(uint32_t *p, int32_t n, hipStream_t s);

}  // namespace wgn
