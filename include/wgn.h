/*
 * wgn.h -- C ABI of libwgn.so, the MI355X (gfx950) decode-step weight stream.
 *
 * The library computes chains of norm-fused weight-matrix x activation-vector
 * products at batch 1..16, the way a batch-1 decode step spends nearly all of
 * its time ("One Token, Kernel by Kernel: A Decode Step on a Laptop GPU",
 * sections "TL;DR", "What one block launches" and "Step 2: every kernel class
 * on the roofline": the weight matrix-vector products dominate the step and
 * are bound by memory bandwidth).
 *
 * Conventions shared by every entry point
 *  - Storage: BF16 values as 16-bit IEEE bfloat16 bit patterns; weights are
 *    [N][K] row-major (K contiguous), activations are [batch][stride].
 *  - Arithmetic: the normalised input x-hat is computed in FP32 and rounded once
 *    to BF16; products accumulate in FP32 in an order fixed by the launch
 *    configuration (so repeated calls are bit-identical); every epilogue runs on
 *    the un-rounded FP32 accumulator and the stored output is rounded exactly
 *    once (round to nearest even).
 *  - Ownership: the caller owns every buffer (weights, activations, outputs,
 *    workspace).  The library never allocates device memory inside a call and
 *    keeps no hidden state other than its loaded kernels.
 *  - Streams: every call is asynchronous on the caller's stream (a hipStream_t
 *    passed as `wgn_stream`; NULL = the default stream) and reads no device
 *    value on the host, except wgn_chain_create (one upload) and
 *    wgn_chain_check (synchronises).
 *  - Errors: every check runs on the host before anything is enqueued; a failed
 *    check returns a negative wgn_status and enqueues nothing.  A failing HIP
 *    launch returns WGN_E_HIP.  NaN/Inf inputs are not checked.
 *  - Alignment: W, W_up, x, gamma and beta must be 16-byte aligned and x's row
 *    stride a multiple of 8 elements (they are read with 128-bit loads); other
 *    pointers need their element's natural alignment; K must be a multiple of 8.
 *  - Workspace: device memory of at least wgn_*_workspace_bytes() bytes,
 *    256-byte aligned, zero-filled once by the caller when allocated.  Calls
 *    leave its counters at zero, so it can be reused and graph-captured.
 *    Concurrent calls must not share a workspace.
 */
#ifndef WGN_H
#define WGN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *wgn_stream; /* a hipStream_t */

typedef enum wgn_status {
    WGN_OK = 0,
    WGN_E_ARG = -1,         /* null pointer, bad size, bad enum value */
    WGN_E_ALIGN = -2,       /* pointer or stride violates the alignment rules */
    WGN_E_UNSUPPORTED = -3, /* valid request this build does not implement */
    WGN_E_WORKSPACE = -4,   /* workspace missing, misaligned or too small */
    WGN_E_HIP = -5,         /* a HIP runtime call failed */
    WGN_E_DEVICE = -6,      /* no usable gfx950 device */
    WGN_E_TIMEOUT = -7      /* an in-kernel wait hit its bound (see wgn_chain_check) */
} wgn_status;

/* Normalisation prologue applied to a stage's input vector(s).
 *  RMS:   x-hat = x * (mean(x^2) + eps)^(-1/2) * gamma
 *         ("GPU Kernel Optimization" README, section "Architecture";
 *          "One Token, Kernel by Kernel", section "The setup")
 *  LAYER: x-hat = (x - mean) * (biased var + eps)^(-1/2) * gamma + beta
 *         ("Making small PyTorch ops faster on a laptop GPU", section
 *          "Beyond language models")
 *  NONE:  x-hat = x                                                        */
typedef enum wgn_norm_kind { WGN_NORM_NONE = 0, WGN_NORM_RMS = 1, WGN_NORM_LAYER = 2 } wgn_norm_kind;

/* Epilogue on the FP32 accumulator a = W . x-hat (+ bias):
 *  NONE:      y = R(residual + a)
 *  GELU_TANH: y = R(residual + 0.5 a (1 + tanh(sqrt(2/pi)(a + 0.044715 a^3))))
 *  SWIGLU:    y = R(residual + silu(a) * (W_up . x-hat)),  silu(z) = z / (1 + e^-z)
 *             ("One Token, Kernel by Kernel", section "The setup": SwiGLU MLP)
 *  ARGMAX:    logits = a (FP32, never rounded); y is int32 [batch]: the lowest
 *             index attaining each row's maximum ("One Token, Kernel by
 *             Kernel", sections "The setup" and "The whole step": LM head
 *             followed by a greedy argmax over the logits)
 * R() = round to nearest even BF16; residual is optional (NULL = 0).       */
typedef enum wgn_epi_kind {
    WGN_EPI_NONE = 0, WGN_EPI_GELU_TANH = 1, WGN_EPI_SWIGLU = 2, WGN_EPI_ARGMAX = 3
} wgn_epi_kind;

typedef enum wgn_dtype { WGN_BF16 = 0, WGN_FP16 = 1, WGN_FP32 = 2 } wgn_dtype;

/* One norm-fused product stage: y = R(residual + epi(W . norm(x) + bias)). */
typedef struct wgn_stage {
    int32_t N;            /* output rows (weight rows), >= 1                          */
    int32_t K;            /* input length, >= 8, multiple of 8                        */
    const void *W;        /* [N][K] BF16 row-major                                    */
    const void *W_up;     /* SWIGLU only: the "up" [N][K] BF16 matrix; else NULL      */
    const void *bias;     /* [N] BF16 added to the accumulator, or NULL (not SWIGLU)  */
    int32_t norm;         /* wgn_norm_kind                                            */
    float eps;            /* norm epsilon                                             */
    const void *gamma;    /* [K] BF16 gain (RMS, LAYER) or NULL = 1                   */
    const void *beta;     /* [K] BF16 shift (LAYER) or NULL = 0                       */
    int32_t epi;          /* wgn_epi_kind                                             */
    const void *x;        /* [batch][x_stride] BF16 input                             */
    int64_t x_stride;     /* elements between batch rows of x                         */
    const void *residual; /* [batch][res_stride] BF16 or NULL (not ARGMAX)            */
    int64_t res_stride;
    void *y;              /* [batch][y_stride] BF16 output; ARGMAX: int32 [batch]     */
    int64_t y_stride;     /* elements between batch rows of y (ignored for ARGMAX)    */
    float *logits;        /* ARGMAX: optional FP32 [batch][N] logits; GELU_TANH:      */
                          /* optional FP32 [batch][N] pre-activation (accumulator +   */
                          /* bias, before GELU) for the backward pass; else NULL      */
    float *maxval;        /* ARGMAX only: optional FP32 [batch] maxima, or NULL       */
} wgn_stage;

/* ---------------------------------------------------------------- info */
const char *wgn_status_string(int32_t status);
int32_t wgn_version(void);
/* Text of the last failing HIP call on this thread ("" if none): which call,
 * the runtime's message and code.  Valid until the next failure. */
const char *wgn_last_hip_error(void);
/* Number of compute units of the current device (0 if none). */
int32_t wgn_device_cu_count(void);

/* ---------------------------------------------------------- one stage */
/* Workspace bytes wgn_gemv_norm needs for this stage at this batch
 * (0 unless epi == ARGMAX). */
size_t wgn_gemv_norm_workspace_bytes(const wgn_stage *stage, int32_t batch);

/* One norm-fused product, one kernel launch: the normalisation of "GPU Kernel
 * Optimization" README, section "Architecture" (mean square, rsqrt and gain
 * multiply fused into one pass) feeding the weight-matrix x activation-vector
 * product that "One Token, Kernel by Kernel", section "What one block
 * launches", runs as a norm kernel followed by a matrix-vector kernel; here
 * both are one launch.  batch in [1, 16]; batch rows of
 * x, residual and y are independent.  The normalisation prologue is computed
 * by every workgroup from the whole input vector, so there is no separate
 * norm kernel.  Batches up to 4 use the vector (v_dot2) path, larger batches
 * the matrix-core path (v_mfma_f32_16x16x32_bf16, batch padded to 16 inside
 * the kernel; padded rows are never stored).  A stage whose batch x K inputs
 * do not fit in the 160 KB of LDS returns WGN_E_UNSUPPORTED here: a chain
 * (wgn_layer_chain, even of one stage) streams such a stage in K windows.
 * Returns WGN_OK or an error (nothing enqueued on error). */
wgn_status wgn_gemv_norm(const wgn_stage *stage, int32_t batch,
                         void *workspace, size_t ws_bytes, wgn_stream stream);

/* Final norm + LM head + argmax in one launch ("One Token, Kernel by Kernel",
 * section "The whole step").  h: [batch][h_stride] BF16; gamma: [K] BF16
 * (RMS gain) or NULL for no norm; W_lm: [V][K] BF16.  Writes idx_out[batch]
 * (int32, lowest index of the maximum), and optionally max_out[batch] and
 * logits_out[batch][V] (FP32). */
size_t wgn_lmhead_argmax_workspace_bytes(int32_t batch);
wgn_status wgn_lmhead_argmax(const void *h, int64_t h_stride, int32_t batch, int32_t K,
                             const void *gamma, float eps, const void *W_lm, int32_t V,
                             int32_t *idx_out, float *max_out, float *logits_out,
                             void *workspace, size_t ws_bytes, wgn_stream stream);

/* wgn_lmhead_argmax without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): the argmax ticket and per-workgroup keys
 * live in a fixed device array of the library (33,024 bytes per GPU, held
 * until the process ends), and the call allocates nothing.  Results are those
 * of wgn_lmhead_argmax bit for bit.  A launch needing more than the fixed
 * array (workgroups x batch rows x 8 bytes + 256; more than 256 compute
 * units at batch 16) returns WGN_E_WORKSPACE; other errors as
 * wgn_lmhead_argmax.  Every call on one GPU shares that array: calls that
 * overlap on one GPU (other streams, other threads) race and must not be
 * issued.  The first call on a GPU also enqueues one small clearing kernel. */
wgn_status wgn_lmhead_argmax_static(const void *h, int64_t h_stride, int32_t batch, int32_t K,
                                    const void *gamma, float eps, const void *W_lm, int32_t V,
                                    int32_t *idx_out, float *max_out, float *logits_out,
                                    wgn_stream stream);

/* ----------------------------------------- larger batches (matrix cores) */
/* Workspace bytes wgn_gemm_norm needs for this stage at this batch (0 if the
 * stage or the batch is outside the call). */
size_t wgn_gemm_norm_workspace_bytes(const wgn_stage *stage, int32_t batch);

/* One norm-fused product for batch in [1, 128] on the matrix cores: the batch
 * sweep of "One Token, Kernel by Kernel", section "Batching: when does decode
 * stop being memory-bound?", where every weight read serves all batch rows.
 * Same stage semantics and numeric contract as wgn_gemv_norm (FP32
 * accumulation, epilogue on the FP32 sum, one rounding to BF16; argmax over
 * FP32 logits, lowest index of the maximum).  Differences:
 *  - the RMSNorm prologue is a pass of its own that writes x-hat (BF16) into
 *    the workspace, then the product reads it (the unfused order of the same
 *    page: norm kernel, then the product);
 *  - a stage with few 64-row tiles is split over K; the last workgroup of a
 *    tile adds the slices in slice order, so results are reproducible;
 *  - a LayerNorm prologue and an argmax with a bias return WGN_E_UNSUPPORTED,
 *    as does a weight matrix of 2^31 bytes or more;
 *  - outputs (y, logits, maxval) must not overlap x, residual, the weights or
 *    each other (WGN_E_ARG).
 * Workspace: wgn_gemm_norm_workspace_bytes(stage, batch) bytes, 256-byte
 * aligned, any content: it starts with the call's tickets and argmax keys,
 * which the call clears first (a fill kernel, so the call can be captured in
 * a HIP graph), followed by x-hat and the partial sums of a K split.
 * Asynchronous on `stream`: the clear, the norm pass (if any) and the product
 * kernel; nothing is enqueued on error. */
wgn_status wgn_gemm_norm(const wgn_stage *stage, int32_t batch, void *workspace, size_t ws_bytes,
                         wgn_stream stream);

/* Standalone RMSNorm over `rows` rows of length K, FP16 or BF16 in and out,
 * FP32 statistics, one rounding ("GPU Kernel Optimization" README, section
 * "Architecture": one program per row).  y may not alias x. */
wgn_status wgn_rmsnorm_rows(const void *x, int64_t x_stride, const void *gamma, float eps,
                            void *y, int64_t y_stride, int32_t rows, int32_t K,
                            int32_t dtype, wgn_stream stream);

/* --------------------------------------------------------- 4-bit weights */
/* Product with 4-bit integer weights in groups of 128 along K, one launch
 * ("One Token, Kernel by Kernel", section "4-bit weights"; the pages give no
 * bit layout, this is the library's):
 *   W4     [N][K/2] bytes, byte j of a row holds the code of k = 2j in its
 *          low nibble and of k = 2j+1 in its high nibble (codes 0..15)
 *   scales, zeros  [N][K/128] BF16: the weight is w = scale * code + zero
 *   x      [batch][x_stride] BF16;  y [batch][y_stride] BF16
 *   y[b][n] = R( sum_k w[n][k] x[b][k] ), FP32 accumulation, one rounding.
 * batch in [1, 8]; K a multiple of 128 with batch * K * 2.125 bytes <= 160 KB
 * (x and its 32-input sums are staged in LDS), else WGN_E_UNSUPPORTED.  x and
 * W4 16-byte aligned, x_stride a multiple of 8; y may not overlap the inputs.
 * No workspace; asynchronous on `stream`; nothing is enqueued on error. */
wgn_status wgn_gemv_int4(const void *x, int64_t x_stride, int32_t batch, int32_t K, const void *W4,
                         const void *scales, const void *zeros, int32_t N, void *y, int64_t y_stride,
                         wgn_stream stream);

/* ------------------------------------------------------ decode attention */
/* Attention of one new token over a static key/value cache, in one launch
 * ("Making small PyTorch ops faster on a laptop GPU", section "A full decode
 * step is a different story": the new key and value are appended, the softmax
 * is FP32, the cache is split across workgroups and the last one to finish
 * merges; "One Token, Kernel by Kernel", section "The fix: Part 10's split-KV
 * kernel": cache layout (batch, head, slot, dimension), the valid length read
 * on the device, each key/value head read once for its group of query heads).
 *
 *   q       [batch][q_heads][head_dim]          BF16, read
 *   k_new   [batch][kv_heads][head_dim]         BF16, read (also v_new)
 *   k_cache [batch][kv_heads][slots][head_dim]  BF16, read; slot pos[b] of row
 *           b is overwritten with k_new (v_cache likewise with v_new)
 *   pos     [batch] int32 in device memory: the new token's slot.  Slots
 *           0 .. pos[b] are attended to; slots after it are never read.  A row
 *           whose pos is outside [0, slots) appends nothing and gets zeros.
 *   out     [batch][q_heads][head_dim] BF16: for query head h (key/value head
 *           h / (q_heads / kv_heads)), R(sum_t softmax_t(scale * q.k_t) v_t).
 *   All activation and cache pointers 16-byte aligned, pos 4-byte aligned;
 *   out, the caches and the inputs may not overlap.
 * head_dim must be 128 and q_heads / kv_heads at most 8 (WGN_E_UNSUPPORTED
 * otherwise); slots in [1, 2^24].  The workspace (size from the query below,
 * 256-byte aligned, zero-filled once at allocation) holds the partial results
 * and arrival counters; every call leaves the counters zero.  A cache of at
 * most 128 slots needs no workspace (NULL allowed).  Calls that share a
 * workspace must not run concurrently.  Asynchronous on `stream`; nothing is
 * enqueued when an argument check fails. */
size_t wgn_decode_attention_workspace_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads,
                                            int32_t slots, int32_t head_dim);
wgn_status wgn_decode_attention(const void *q, const void *k_new, const void *v_new,
                                void *k_cache, void *v_cache, const int32_t *pos,
                                int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t slots,
                                int32_t head_dim, float scale, void *out,
                                void *workspace, size_t ws_bytes, wgn_stream stream);

/* ------------------------------------------------------ read ceiling */
/* Plain streaming read of `bytes` of device memory (a measurement, not a step
 * of the method): the GPU's measured HBM read ceiling, against which the
 * weight stream's bandwidth is reported beside the rated peak ("One Token,
 * Kernel by Kernel", section "Step 2: every kernel class on the roofline": the
 * pages measure their card's read ceiling and quote both).  Each 16-byte chunk
 * of src is read once with a non-temporal 128-bit load; `grid` workgroups of
 * `threads` threads (a multiple of 64, at most 1024), each lane keeping `depth`
 * loads in flight (1, 2, 4, 8 or 16).  sink: one device uint32 that the kernel
 * writes only when the folded value of a lane's loads equals a fixed pattern
 * (it exists so the loads cannot be removed; its content is meaningless).
 * src 16-byte aligned, bytes a non-zero multiple of 16.  Asynchronous on
 * `stream`; nothing is enqueued on error. */
wgn_status wgn_stream_read(const void *src, size_t bytes, int32_t grid, int32_t threads, int32_t depth,
                           uint32_t *sink, wgn_stream stream);

/* --------------------------------------------------------------- chains */
/* A chain is a list of stages in dependency order (a stage may read earlier
 * stages' outputs), tuned and laid out once and then run many times, like the
 * stage-list wrapper of "Making small PyTorch ops faster on a laptop GPU",
 * section "Beyond language models".  Maximal runs of consecutive stages that
 * do not touch each other's outputs form one phase; phases are separated by
 * device-side completion counters inside one persistent kernel (mode 0) or by
 * kernel boundaries (mode 1).  Weights must not be written by any stage.
 * Every stage writes its own output buffer.
 *
 * Hoisting (default; opts.no_fuse = 1 turns it off): a stage whose input no
 * stage of the chain writes and whose epilogue is a plain residual add, the
 * residual being an earlier stage D's output, is split: its product runs in
 * the phase before D's and leaves FP32 row sums in the workspace, and its
 * residual add (one rounding of D's output + the sums + its bias) runs in D's
 * epilogue.  Same function, one device-wide phase boundary less per such
 * stage -- in a decoder block the attention output projection, whose residual
 * is the previous block's output ("One Token, Kernel by Kernel", section
 * "What one block launches": the residual add folded into a neighbouring
 * kernel).  wgn_chain_stage_phases reports the phase that writes each output.
 * A stage whose inputs do not fit in LDS (an un-normalised input of batch x K
 * BF16 over about 150 KB) is streamed in K windows over consecutive phases. */
typedef struct wgn_chain wgn_chain;

typedef struct wgn_chain_opts {
    int32_t mode;        /* 0: one persistent launch (default); 1: one launch per phase */
    int32_t grid;        /* workgroups; 0 = one per compute unit; mode 0: at most the   */
                         /* compute units (all resident at once), and at most 2048     */
    int32_t trace;       /* 1: record per-phase, per-workgroup timestamps (see below)  */
    int32_t path;        /* 0: auto (vector path for batch <= 4, matrix cores above);   */
                         /* 1: vector path (batch <= 4 only); 2: matrix-core path;     */
                         /* 3: wgn_layer_chain only: the stage-by-stage tiled products */
                         /* of wgn_gemm_norm at any batch in [1, 128] (always above 16) */
    int32_t no_fuse;     /* 1: keep every stage whole (no hoisting, see below)          */
    int32_t ring;        /* vector path's block-buffer ring: 0 auto; 1: 2 x 20 units,   */
                         /* burst refills; 2: 5 x 8 units, burst refills; 3: 4 x 10     */
                         /* units, refills interleaved with compute (same results)      */
    int32_t reserved[2]; /* must be zero                                               */
} wgn_chain_opts;

/* Workspace bytes for a chain over these stages (mode/grid as in opts, NULL = defaults). */
size_t wgn_chain_workspace_bytes(const wgn_stage *stages, int32_t n_stages, int32_t batch,
                                 const wgn_chain_opts *opts);

/* Validate, group into phases, lay the device program out in the workspace
 * (one host->device copy on `stream`, then a stream synchronisation) and
 * return a host handle.  The stage buffers must stay valid while the chain is
 * used.  Not for the hot loop. */
wgn_status wgn_chain_create(const wgn_stage *stages, int32_t n_stages, int32_t batch,
                            const wgn_chain_opts *opts, void *workspace, size_t ws_bytes,
                            wgn_stream stream, wgn_chain **out);

/* Decode attention as part of a chain: the operation of wgn_decode_attention
 * (same passages, same cache layout, append and outputs) run inside the
 * chain's launch, between the stages that write q, k_new and v_new and the
 * stage that reads out ("Making small PyTorch ops faster on a laptop GPU",
 * section "A full decode step is a different story"; "One Token, Kernel by
 * Kernel", sections "The fix: Part 10's split-KV kernel" and "Step 3: where
 * the 14.8 ms go": attention as a part of the one decode step).
 *   q       [batch][q_stride]   BF16, q_heads x head_dim per row (read)
 *   k_new   [batch][k_stride]   BF16, kv_heads x head_dim per row (read; v_new likewise)
 *   k_cache [batch][kv_heads][slots][head_dim] BF16: slot pos[b] of row b
 *           is overwritten with k_new (v_cache with v_new)
 *   pos     [batch] int32 in device memory (out of [0, slots): no append, zero output)
 *   out     [batch][out_stride] BF16, q_heads x head_dim per row (written)
 *   scale   the score scale (finite; 1/sqrt(head_dim) in the pages' model)
 * head_dim must be 128 and q_heads / kv_heads at most 8 (WGN_E_UNSUPPORTED
 * otherwise).  Pointers 16-byte aligned (pos 4-byte), strides multiples of 8
 * elements and at least the row length when batch > 1; out, the caches and
 * the inputs may not overlap.  The item runs as two phases without weights:
 * partial results per chunk of the cache, then their merge; the product phases
 * around them keep streaming weights ahead. */
typedef struct wgn_attn_stage {
    const void *q;
    int64_t q_stride;
    const void *k_new;
    int64_t k_stride;
    const void *v_new;
    int64_t v_stride;
    void *k_cache;
    void *v_cache;
    const int32_t *pos;
    void *out;
    int64_t out_stride;
    int32_t q_heads, kv_heads, slots, head_dim;
    float scale;
} wgn_attn_stage;

/* A chain of `stages` with attention items: item i runs after stages
 * [0, attn_before[i]) and before stage attn_before[i] (non-decreasing, in
 * [0, n_stages]).  Hoisting (opts.no_fuse = 0) is not applied to such a chain.
 * Otherwise as wgn_chain_workspace_bytes / wgn_chain_create; the workspace
 * also holds the attention partials.  A chain created here runs with
 * wgn_chain_run, wgn_chain_check and the other chain calls. */
size_t wgn_chain_attn_workspace_bytes(const wgn_stage *stages, int32_t n_stages, const wgn_attn_stage *attn,
                                      const int32_t *attn_before, int32_t n_attn, int32_t batch,
                                      const wgn_chain_opts *opts);
wgn_status wgn_chain_create_attn(const wgn_stage *stages, int32_t n_stages, const wgn_attn_stage *attn,
                                 const int32_t *attn_before, int32_t n_attn, int32_t batch,
                                 const wgn_chain_opts *opts, void *workspace, size_t ws_bytes,
                                 wgn_stream stream, wgn_chain **out);

/* Enqueue one run of the chain on `stream` (no host synchronisation). */
wgn_status wgn_chain_run(const wgn_chain *chain, wgn_stream stream);

/* Synchronise `stream` and report WGN_E_TIMEOUT if an in-kernel wait of an
 * earlier run hit its bound (the counters are then reset); else WGN_OK.
 * Once a wait has given up, the error word stays set and every later run of
 * the chain (also a graph replay) exits at once without writing anything,
 * until this call has reset the counters: a run never proceeds on the flags
 * an aborted run left behind. */
wgn_status wgn_chain_check(const wgn_chain *chain, wgn_stream stream);

/* Bound of every in-kernel wait of later runs of this chain, in microseconds
 * (a negative value restores the default of 2 s; 0 makes a wait give up at
 * its first poll that does not find every flag).  Each wait polls, so every
 * kernel still ends when the bound is hit; this is how tests force the
 * time-out path from the host.  WGN_E_ARG for a null chain or a bound above
 * the default.  Takes effect from the next wgn_chain_run. */
wgn_status wgn_chain_set_wait_us(wgn_chain *chain, int64_t us);

int32_t wgn_chain_num_phases(const wgn_chain *chain);
int32_t wgn_chain_grid(const wgn_chain *chain);
/* Ring the vector path's streaming waves use (0..2 = opts.ring - 1; the auto
 * choice takes ring 1 when phases give a streaming wave fewer than 4 units on
 * average, else ring 2 from batch 2 up and ring 0 at batch 1); -1 for null. */
int32_t wgn_chain_ring(const wgn_chain *chain);

/* Trace of the last run of a chain created with opts.trace = 1: for every
 * phase p and workgroup g, WGN_TRACE_POINTS timestamps of the device's 100 MHz
 * real-time clock at out[(p * grid + g) * WGN_TRACE_POINTS + i]:
 *   0 phase start, 1 previous phase complete device-wide, 2 x-hat staged,
 *   3 weight stream of the phase done, 4 outputs stored, 5 completion released
 *   (control wave); 6 first streaming wave passes the phase's x-hat barrier,
 *   7 it has issued its loads ahead of that barrier, 8 it has consumed its
 *   last block of the phase, 9..11 it has consumed its first, second, third
 *   block of the phase (0 if it has fewer).
 * Synchronises `stream`; n_out = number of uint64 slots available. */
#define WGN_TRACE_POINTS 12
wgn_status wgn_chain_trace(const wgn_chain *chain, wgn_stream stream, uint64_t *out, size_t n_out);
/* Phase index of each stage (array of n_stages). */
wgn_status wgn_chain_stage_phases(const wgn_chain *chain, int32_t *phase_of_stage);
void wgn_chain_destroy(wgn_chain *chain);

/* create + run + destroy in one call (the create step synchronises `stream`):
 * the chain of layers that read weights, each a norm-fused product, of "One
 * Token, Kernel by Kernel", sections "What one block launches" and "The whole
 * step", run with a plan as "Making small PyTorch ops faster on a laptop GPU",
 * section "Beyond language models", runs a stage list it has tuned once.
 * plan: NULL or plan->prefetch == 0 runs the chain plainly; a prefetch plan
 * (from wgn_plan_tune) needs opts->mode == 1 (WGN_E_UNSUPPORTED otherwise) and
 * runs its touch passes on `side` (see wgn_chain_run_plan); side is ignored
 * without one.  The workspace is sized by wgn_chain_workspace_bytes for the
 * same opts (wgn_workspace_bytes covers every mode).
 * batch in [17, 128], or opts->path == 3 at any batch: the stages run in list
 * order through the wgn_gemm_norm path, up to 4 consecutive independent
 * stages of one epilogue family in one launch (Q, K, V and an O product that
 * reads its own input), the normalised ones among them reading one x-hat made
 * by one norm pass (a plan must not prefetch, opts must not trace or force
 * the vector path: WGN_E_UNSUPPORTED); the workspace (wgn_workspace_bytes at
 * that batch) needs no zero fill, the call clears its counters first. */
wgn_status wgn_layer_chain(const wgn_stage *stages, int32_t n_stages, int32_t batch,
                           const wgn_chain_opts *opts, const struct wgn_plan *plan, void *workspace,
                           size_t ws_bytes, wgn_stream stream, wgn_stream side);

/* One workspace size that serves every call of the library on these stages at
 * this batch: a chain over them in either mode with default options, each
 * stage alone through wgn_gemv_norm, and -- when V > 0 -- wgn_lmhead_argmax
 * over V rows.  At batch 17-128 (and, at any batch, for opts->path == 3 of
 * wgn_layer_chain): wgn_layer_chain on the stages, each stage
 * through wgn_gemm_norm, and -- when V > 0 -- an RMSNorm + argmax stage of V
 * rows over the last stage's output (its N, rounded up to a multiple of 8)
 * through wgn_gemm_norm.  0 if the
 * stages cannot be planned (a call on them would return its error). */
size_t wgn_workspace_bytes(const wgn_stage *stages, int32_t n_stages, int32_t batch, int32_t V);

/* --------------------------------------------------------- backward pass */
/* Backward pass of a chain of LayerNorm -> Linear(+bias) -> GELU-tanh blocks
 * for small-batch training ("Making small PyTorch ops faster on a laptop GPU",
 * section "It works in training too": the backward visits the layers in
 * reverse, so the weights to fetch ahead while block i's gradient is computed
 * are those of block i-1; section "Beyond language models" for the block).
 *
 * stages: the forward stages as given to wgn_layer_chain (same order), each
 * norm = LAYER, epi = GELU_TANH, no residual, stage i's K equal to stage i-1's
 * N, and `logits` pointing at the FP32 [batch][N] pre-activation that the
 * forward wrote there (a GELU stage with logits set keeps it); stage x is the
 * block input and the last stage's y the chain output.  All forward tensors
 * are read only and must hold the forward's values.  batch in [1, 16].
 * Definition, per block, from the output gradient gy (BF16):
 *   gz = R(gy GELU'(z)), gb = R(sum_b gz), gW = R(sum_b gz xh),
 *   gxh = gz W, gx = R(LayerNorm backward of gxh), ggamma = R(sum_b gxh u),
 *   gbeta = R(sum_b gxh), with xh = R(LayerNorm(x)), u = (x - mean) / sigma;
 * gx of block i is gy of block i-1.  The last block's gy is g_out (BF16
 * [batch][g_stride]) or, when g_out is NULL, the gradient of the mean of the
 * squared chain output, R(2 y / (batch N)).  R() rounds to BF16. */
typedef struct wgn_grad {
    void *gW;      /* [N][K] BF16, required, 16-byte aligned                          */
    void *gbias;   /* [N] BF16: required when the stage has a bias, else NULL          */
    void *ggamma;  /* [K] BF16 or NULL; NULL when the stage has no gamma               */
    void *gbeta;   /* [K] BF16 or NULL; NULL when the stage has no beta                */
    void *gy;      /* [batch][N] BF16 or NULL: the gradient reaching the block output  */
    void *gz;      /* [batch][N] BF16 or NULL: the gradient of the pre-activation      */
} wgn_grad;
typedef struct wgn_backward wgn_backward;

/* Workspace bytes of a backward pass over these stages (0 if they do not
 * qualify: a create call would return its error). */
size_t wgn_backward_workspace_bytes(const wgn_stage *stages, int32_t n_stages, int32_t batch);

/* Validate, lay the block table out in the workspace (one host->device copy
 * on `stream`, then a stream synchronisation) and return a host handle.
 * grads[n_stages]: the outputs of each block.  g_in: NULL or BF16
 * [batch][gin_stride] for the gradient of the chain input.  Outputs may
 * overlap neither each other, nor any tensor read, nor the workspace
 * (WGN_E_ARG).  The buffers must stay valid while the handle is used.
 * WGN_E_UNSUPPORTED for a stage that is not a LayerNorm + GELU block (or
 * whose N x K reaches 2^30).  Not for the hot loop. */
wgn_status wgn_backward_create(const wgn_stage *stages, int32_t n_stages, int32_t batch,
                               const wgn_grad *grads, const void *g_out, int64_t g_stride,
                               void *g_in, int64_t gin_stride, void *workspace, size_t ws_bytes,
                               wgn_stream stream, wgn_backward **out);

/* Enqueue one backward pass on `stream`: a prep launch (LayerNorm statistics
 * and x-hat of every block input; it also clears the run's counters) and one
 * persistent launch that walks the blocks from the last to the first, then
 * writes g_in.  prefetch = 1: each workgroup requests its weight tile of the
 * next block in backward order (block i-1 while block i runs) before it waits
 * for block i to finish; 0: only after the wait.  Results are bit-identical
 * either way and between runs.  No host synchronisation; graph-capturable. */
wgn_status wgn_backward_run(const wgn_backward *bw, int32_t prefetch, wgn_stream stream);

/* Synchronise `stream`; WGN_E_TIMEOUT if an in-kernel wait of the last run
 * hit its bound (its outputs are then incomplete), else WGN_OK.  Each run
 * starts from cleared counters. */
wgn_status wgn_backward_check(const wgn_backward *bw, wgn_stream stream);

/* Bound of the in-kernel waits of later runs in microseconds (negative: the
 * default of 2 s; 0: every wait gives up at once, so tests can force the
 * time-out path from the host).  WGN_E_ARG above the default. */
wgn_status wgn_backward_set_wait_us(wgn_backward *bw, int64_t us);
/* Workgroups of the persistent launch (all resident at once); -1 for NULL. */
int32_t wgn_backward_grid(const wgn_backward *bw);
/* Later runs record timestamps of the device's 100 MHz real-time clock into
 * the device buffer (NULL stops): for block i and workgroup g, at
 * buf[(i * grid + g) * WGN_BWD_TRACE_POINTS + p], of the workgroup's first
 * tile of the block: p = 0 before the wait for block i+1, 1 wait over, 2 the
 * tile's gz ready, 3 the tile's partial and row-sum shares stored, 4 the
 * workgroup's flag for block i set, 5 its next tile's loads issued, 6 the
 * tile's weight-gradient work done.  n_slots must cover n_stages x grid x
 * WGN_BWD_TRACE_POINTS (WGN_E_ARG). */
#define WGN_BWD_TRACE_POINTS 7
wgn_status wgn_backward_set_trace(wgn_backward *bw, uint64_t *device_buf, size_t n_slots);
void wgn_backward_destroy(wgn_backward *bw);

/* create + run + destroy in one call (the create step synchronises `stream`). */
wgn_status wgn_chain_backward(const wgn_stage *stages, int32_t n_stages, int32_t batch,
                              const wgn_grad *grads, const void *g_out, int64_t g_stride,
                              void *g_in, int64_t gin_stride, int32_t prefetch, void *workspace,
                              size_t ws_bytes, wgn_stream stream);

/* -------------------------------------------------------- prefetch plans */
/* Optional prefetch of later launches' weights into the GPU's memory-side
 * Infinity Cache by a touch pass on a second stream, for chains created with
 * one launch per phase (opts.mode = 1).  While launch i runs on `stream`, the
 * pass reads the leading frac_pct % of every weight matrix of launch
 * i + distance on `side`, with `blocks` workgroups of 256 threads ("Making
 * small PyTorch ops faster on a laptop GPU", section "Prefetching the next
 * layer while this one runs").  The pass only reads, so a run's outputs are
 * bit-identical with and without a plan.  A persistent chain (mode 0) issues
 * its next phases' weight loads from inside its kernel and takes no plan. */
typedef struct wgn_plan {
    int32_t prefetch;   /* 0: plain run (other fields ignored); 1: touch pass    */
    int32_t distance;   /* launches ahead, 1..4                                   */
    int32_t blocks;     /* workgroups of the touch pass, 1..1024                  */
    int32_t frac_pct;   /* leading share of each weight matrix touched, 1..100    */
    float plain_us;     /* set by wgn_plan_tune: mean time of a plain run         */
    float best_us;      /* set by wgn_plan_tune: mean time of the best candidate  */
    float speedup_lo;   /* set by wgn_plan_tune: lower end of the 95 % confidence */
                        /* interval of (plain time / best candidate's time)       */
    int32_t candidates; /* set by wgn_plan_tune: candidates measured              */
} wgn_plan;

/* Enqueue one run of a chain with a plan (no host synchronisation).  With
 * prefetch = 1 the run forks `side` off `stream` before each launch (event
 * record + wait) and ends with `stream` waiting for `side`, so later work on
 * `stream` sees the whole run.  The weight ranges of each launch are laid out
 * in the workspace by wgn_chain_create (at most 16 matrices per launch).
 * Errors: WGN_E_ARG for a null chain or plan, fields out of range, or a null
 * `side` or side == stream when prefetch = 1; WGN_E_UNSUPPORTED for a mode-0
 * chain with prefetch = 1; WGN_E_HIP if a launch or event call fails. */
wgn_status wgn_chain_run_plan(const wgn_chain *chain, const wgn_plan *plan, wgn_stream stream, wgn_stream side);

/* Time plain runs of a mode-1 chain against the touch-pass candidates
 * (distance 1 and 2, blocks 16, 64 and 256, frac 50 and 100 %) in `reps`
 * interleaved rounds (3..200), and write the plan to keep: the candidate with
 * the best mean speedup if the lower end of its 95 % confidence interval
 * clears 1.01, else prefetch = 0 with the closest candidate's settings and
 * figures ("Making small PyTorch ops faster on a laptop GPU", section
 * "Measuring instead of predicting": one plan per chain here, timed on the
 * chain's own weights).  Synchronises `stream`; the runs overwrite the
 * chain's outputs.  Not for the hot loop.  Errors: WGN_E_ARG (null chain or
 * out, reps out of range, null or equal streams), WGN_E_UNSUPPORTED (mode-0
 * chain), WGN_E_HIP. */
wgn_status wgn_chain_plan_tune(const wgn_chain *chain, wgn_stream stream, wgn_stream side, int32_t reps,
                               wgn_plan *out);

/* The same tuning for a stage list ("Making small PyTorch ops faster on a
 * laptop GPU", section "Beyond language models": a list of stages is tuned
 * once and the plan kept): plans a one-launch-per-phase chain over the stages
 * in `workspace` (at least wgn_workspace_bytes(stages, n, batch, 0) bytes,
 * zero-filled), tunes it in 15 rounds as wgn_chain_plan_tune and writes the
 * plan to keep to *out.  Synchronises `stream`; overwrites the stages'
 * outputs.  Errors as wgn_chain_create and wgn_chain_plan_tune. */
wgn_status wgn_plan_tune(const wgn_stage *stages, int32_t n_stages, int32_t batch, wgn_plan *out,
                         void *workspace, size_t ws_bytes, wgn_stream stream, wgn_stream side);

/* --------------------------------------------------------- host helpers */
/* The first wave of `waves` whose even share of `units` work units contains
 * unit `u` (exported so the partition rule can be tested on the host). */
int32_t wgn_first_wave_of_unit(int32_t u, int32_t units, int32_t waves);

/* Plan a chain on the host only (no device needed; grid and path from opts,
 * NULL or grid 0 = 256 workgroups) and return its number of phases, or a
 * negative wgn_status.  If phase_of_stage is not NULL it receives, per stage,
 * the phase that writes its output (for a stage streamed in K windows, the
 * last window). */
int32_t wgn_plan_phases(const wgn_stage *stages, int32_t n_stages, int32_t batch,
                        const wgn_chain_opts *opts, int32_t *phase_of_stage);

/* Plan a chain on the host only (no device needed) for opts->grid workgroups
 * (0 or NULL opts: 256) on the path opts->path selects, and emulate every
 * workgroup and wave of its work partition: each weight unit must be streamed
 * exactly once with the right address, each partial-sum slot written once and
 * read by the epilogue, each row owned by one workgroup, every LDS area inside
 * the budget.  Returns the number of violations (0 = consistent) or a
 * negative wgn_status if planning failed. */
int32_t wgn_partition_selftest(const wgn_stage *stages, int32_t n_stages, int32_t batch,
                               const wgn_chain_opts *opts);

#ifdef __cplusplus
}
#endif
#endif /* WGN_H */
