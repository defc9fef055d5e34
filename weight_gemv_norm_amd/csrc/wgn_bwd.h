// wgn_bwd.h -- launch arguments of the backward pass of a chain of
// LayerNorm -> Linear(+bias) -> GELU-tanh blocks (wgn_bwd.hip), shared by the
// host side (wgn_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wgn {

constexpr int BWD_MAX_BATCH = 16;
constexpr int BWD_TILE_ROWS = 64;     // weight rows of one item (16 per wave)
constexpr int BWD_TILE_COLS = 64;     // weight columns of one item (16 bytes per thread)
constexpr int BWD_THREADS = 256;
constexpr int BWD_MAX_LAYERS = 4096;

// One block, device view (forward order; the kernel walks them backwards).
// Forward tensors are read only; gradient outputs are written once per run.
struct BwdLayer {
    const uint16_t *W;       // [N][K] BF16
    const uint16_t *x;       // [B][x_stride] BF16 block input (the forward's saved activation)
    const uint16_t *gamma;   // [K] or null (1)
    const uint16_t *beta;    // [K] or null (0)
    const float *pre;        // [B][N] FP32 pre-activation written by the forward
    uint16_t *gW;            // [N][K] BF16
    uint16_t *gb;            // [N] BF16 or null
    uint16_t *ggamma;        // [K] BF16 or null
    uint16_t *gbeta;         // [K] BF16 or null
    uint16_t *gy;            // [B][N] BF16 or null: gradient reaching the block output
    uint16_t *gz;            // [B][N] BF16 or null: gradient of the pre-activation
    // workspace
    float *stats;            // [B][2]: mean and 1 / sigma of the input rows
    uint16_t *xh;            // [B][K] BF16 x-hat
    int64_t x_stride;
    float eps;
    int32_t N, K, nrb, ncb;  // row blocks of BWD_TILE_ROWS, column blocks of BWD_TILE_COLS
};

struct BwdArgs {
    const BwdLayer *layers;  // n of them
    int32_t n, B;
    const uint16_t *y;       // chain output [B][y_stride]: mean-square loss when g_out is null
    int64_t y_stride;
    const uint16_t *g_out;   // [B][g_stride] gradient of the chain output, or null
    int64_t g_stride;
    uint16_t *g_in;          // [B][gin_stride] gradient of the chain input, or null
    int64_t gin_stride;
    float *part[2];          // [max nrb][B][max K] row-block partials of gxh, by block parity
    float *q[2];             // [max tiles][B][2] per-tile shares of the LayerNorm row sums, by block parity
    uint32_t *flags;         // [tile_wgs]: blocks each workgroup is done with (zero at launch)
    uint32_t *err;           // set to 1 when a bounded wait gives up
    uint64_t wait_ticks;
    uint64_t *trace;         // null, or [n][grid][BWD_TRACE_POINTS] real-time clock stamps
    int32_t tile_wgs;        // the grid
    int32_t prefetch;        // 1: issue the next layer's weight loads before waiting for it
};
// Trace points of a workgroup's first tile of each block: 0 before the wait
// for the following block, 1 wait over, 2 gz of the tile ready, 3 the tile's
// partial and shares stored, 4 the workgroup's flag for the block set, 5 the
// next tile's loads issued, 6 the tile's weight-gradient work done.
constexpr int BWD_TRACE_POINTS = 7;

// Statistics and x-hat of every block input; also clears nzero counter words.
hipError_t launch_bwd_prep(const BwdLayer *layers, int32_t n, int32_t B, uint32_t *zero, int32_t nzero,
                           hipStream_t s);
hipError_t launch_bwd(const BwdArgs &a, int32_t grid, hipStream_t s);
// Workgroups of the backward kernel that fit the device at once.
int32_t bwd_resident_grid();

}  // namespace wgn
