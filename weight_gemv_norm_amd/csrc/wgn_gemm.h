// wgn_gemm.h -- launch arguments of the batched product on the matrix cores
// (wgn_gemm.hip), shared by the host planner (wgn_api.cpp) and the kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wgn {

constexpr int GEMM_MAX_BATCH = 128;                      // batch rows of one call
constexpr int GEMM_TILE_ROWS = 64;                       // output rows per item (16 per wave)
constexpr int GEMM_THREADS = 256;                        // four waves
constexpr int GEMM_KWIN = 128;                          // K elements per LDS window (4 steps of 32)
constexpr int GEMM_ROW_PAD = 16;                         // bytes after each batch row of the window
constexpr int GEMM_FRAG_BYTES = 64 * 16;                 // one wave's 16 x 16 FP32 accumulator tile

// One call's work: items = ntiles x nslices; item i is row tile i / nslices
// (rows 64 t ..) over K slice i % nslices (elements [s kslice, (s+1) kslice),
// kslice a multiple of GEMM_KWIN), streamed through LDS windows of GEMM_KWIN
// elements.  With nslices > 1 each item
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

// LDS bytes of a call: two x-hat windows (the one being multiplied and the
// next one being copied), the argmax merge area and a flag; at most
// lds_cap(), so that two workgroups fit one compute unit's 160 KB.
inline size_t gemm_lds_bytes(int32_t bpad) {
    return 2 * (size_t)bpad * ((size_t)GEMM_KWIN * 2 + GEMM_ROW_PAD) + (size_t)4 * GEMM_MAX_BATCH * 8 + 16;
}
inline constexpr size_t lds_cap() { return 80 * 1024; }

hipError_t launch_gemm(const GemmLaunch &L, bool swiglu, size_t lds, hipStream_t s);
// x-hat rows [rows][K] (row stride K) of RMSNorm (layer = false) or LayerNorm.
hipError_t launch_norm_rows64(const uint16_t *x, int64_t x_stride, const uint16_t *gamma, const uint16_t *beta,
                              float eps, bool layer, uint16_t *y, int32_t rows, int32_t K, hipStream_t s);
// A fill kernel, not hipMemsetAsync: the calls may be captured in a HIP graph.
hipError_t launch_zero_words(uint32_t *p, int32_t n, hipStream_t s);

}  // namespace wgn
