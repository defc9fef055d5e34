/*
 * wgn_oracle.c -- plain, slow, obviously-correct CPU oracle for the decode-step
 * weight stream.  TEST INFRASTRUCTURE ONLY: nothing in the product library
 * links, includes or calls this file.  It shares no code, header, table or
 * helper with the HIP path.
 *
 * What it computes (all arithmetic in IEEE binary64, sums in sequential k order):
 *
 *   RMSNorm   xh_k = R( x_k * (sum_j x_j^2 / K + eps)^(-1/2) * g_k )
 *             -- "GPU Kernel Optimization" (fused RMSNorm README), section
 *                "Architecture": mean of squares, reciprocal square root, then
 *                the per-channel weight.  Also "One Token, Kernel by Kernel",
 *                section "The setup": the model is RMSNorm-normalised.
 *   LayerNorm xh_k = R( (x_k - mu) * (var + eps)^(-1/2) * gamma_k + beta_k ),
 *             mu = mean, var = biased variance
 *             -- "Making small PyTorch ops faster on a laptop GPU", section
 *                "Beyond language models": the LayerNorm -> Linear -> GELU chain.
 *   product   a_n = sum_k W[n][k] * xh_k   (W is [N][K] row-major)
 *             -- "One Token, Kernel by Kernel", section "What one block
 *                launches": one matrix-vector product per weight matrix at
 *                batch 1, BF16 inputs and a wide accumulator.
 *   epilogue  y = R( residual + epi(a + bias) ),
 *             epi in { identity, GELU-tanh, SwiGLU: silu(a_gate) * a_up }
 *             -- same page, "The setup" (SwiGLU MLP) and "What one block
 *                launches" (the residual add is folded into a neighbouring
 *                kernel); GELU from "Beyond language models" on the first page.
 *   LM head   logits_v = sum_k W[v][k] * xh_k (never rounded),
 *             idx = lowest v attaining the maximum
 *             -- "One Token, Kernel by Kernel", sections "The setup" (greedy
 *                argmax of the last logits) and "The whole step" (LM head
 *                151,936 x 1,536 followed by an argmax).
 *   attention out = R( softmax_t(scale * q . k_t) . v ) over cache slots
 *             0 .. pos after the new key/value are written at slot pos;
 *             query head h reads key/value head h / (q_heads / kv_heads)
 *             -- "Making small PyTorch ops faster on a laptop GPU", section "A
 *                full decode step is a different story", and "One Token, Kernel
 *                by Kernel", section "The fix: Part 10's split-KV kernel".
 *   4-bit     y = R( sum_k (s_g q_k + z_g) x_k ), 4-bit codes q in groups of 128
 *             -- "One Token, Kernel by Kernel", section "4-bit weights".
 *   backward  of one block y = R(GELU(z)), z = xh W^T + bias, xh = R(LayerNorm(x)),
 *             given the output gradient gy (BF16), in this order:
 *               gz  = R( gy * GELU'(z) )
 *               gb  = R( sum_b gz ),  gW[n][k] = R( sum_b gz[b][n] xh[b][k] )
 *               gxh = sum_n gz[b][n] W[n][k]                (not rounded)
 *               u = (x - mu) / sigma,  gu = gamma * gxh
 *               gx  = R( (gu - mean_k gu - u * mean_k(gu u)) / sigma )
 *               ggamma = R( sum_b gxh u ),  gbeta = R( sum_b gxh )
 *             and the mean-square loss of the last output, g = R( 2 y / (batch N) )
 *             -- "Making small PyTorch ops faster on a laptop GPU", sections "It
 *                works in training too" (the example step's loss is the mean of
 *                the squared FP32 output; the backward visits the layers in
 *                reverse) and "Beyond language models" (the LayerNorm -> Linear
 *                -> GELU block).  The rounding points are a reading: BF16 at
 *                every tensor the unfused pipeline would store (gz, the
 *                parameter gradients, gx), wide arithmetic inside.
 *
 * R() is round-to-nearest-even to BF16 (FP16 for the standalone FP16 norm rows),
 * taken directly from the binary64 value (one rounding).  x-hat is rounded to
 * BF16 before the product: that is the tensor the unfused pipeline stores
 * between its norm kernel and its GEMV kernel.
 *
 * Threading: OpenMP over output rows only; every row's sum is sequential, so
 * results are bit-identical for any thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- encodings */

/* BF16 bits -> value: the upper half of an IEEE binary32. */
double wgo_bf16_to_f64(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Encode a value that is exactly representable in binary32 and take its upper
 * 16 bits (exact when the value is representable in BF16). */
static uint16_t top16_of_float(double v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Round a binary64 value to the nearest BF16 value, ties to even.
 * BF16: 8 significant bits, exponent range as binary32, subnormal spacing 2^-133. */
uint16_t wgo_f64_to_bf16(double v)
{
    if (isnan(v)) return (uint16_t)0x7FC0;
    if (isinf(v)) return v > 0 ? (uint16_t)0x7F80 : (uint16_t)0xFF80;
    if (v == 0.0) return signbit(v) ? (uint16_t)0x8000 : (uint16_t)0x0000;
    int ex;
    (void)frexp(v, &ex);          /* |v| = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;               /* floor(log2|v|) */
    if (e < -126) e = -126;       /* subnormal range: fixed spacing */
    double ulp = ldexp(1.0, e - 7);
    double q = rint(v / ulp);     /* default rounding mode: nearest, ties to even */
    double r = q * ulp;
    const double maxbf = ldexp(255.0, 127 - 7);   /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > maxbf) return v > 0 ? (uint16_t)0x7F80 : (uint16_t)0xFF80;
    if (r == 0.0) return signbit(v) ? (uint16_t)0x8000 : (uint16_t)0x0000;
    return top16_of_float(r);
}

/* FP16 bits -> value. */
double wgo_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1, E = (h >> 10) & 0x1F, M = h & 0x3FF;
    double v;
    if (E == 0x1F) v = M ? NAN : INFINITY;
    else if (E == 0) v = ldexp((double)M, -24);
    else v = ldexp(1024.0 + M, E - 25);
    return s ? -v : v;
}

/* Round a binary64 value to the nearest FP16 value, ties to even.
 * FP16: 11 significant bits, min normal 2^-14, subnormal spacing 2^-24, max 65504. */
uint16_t wgo_f64_to_f16(double v)
{
    if (isnan(v)) return (uint16_t)0x7E00;
    uint16_t sbit = signbit(v) ? 0x8000 : 0;
    if (isinf(v)) return sbit | 0x7C00;
    if (v == 0.0) return sbit;
    double a = fabs(v);
    int ex;
    (void)frexp(a, &ex);
    int e = ex - 1;
    if (e < -14) e = -14;
    double ulp = ldexp(1.0, e - 10);
    double r = rint(a / ulp) * ulp;
    if (r > 65504.0) return sbit | 0x7C00;
    if (r == 0.0) return sbit;
    (void)frexp(r, &ex);
    e = ex - 1;
    if (e < -14) {                                /* subnormal */
        return sbit | (uint16_t)(r / ldexp(1.0, -24));
    }
    uint16_t E = (uint16_t)(e + 15);
    uint16_t M = (uint16_t)((r / ldexp(1.0, e) - 1.0) * 1024.0);
    return sbit | (uint16_t)(E << 10) | M;
}

/* ------------------------------------------------------------ elementwise */

double wgo_gelu_tanh(double z)
{
    /* tanh approximation of GELU: 0.5 z (1 + tanh( sqrt(2/pi) (z + 0.044715 z^3) )) */
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

double wgo_silu(double z)
{
    return z / (1.0 + exp(-z));
}

/* ------------------------------------------------------------------ norms */

enum { WGO_NORM_NONE = 0, WGO_NORM_RMS = 1, WGO_NORM_LAYER = 2 };
enum { WGO_EPI_NONE = 0, WGO_EPI_GELU_TANH = 1, WGO_EPI_SWIGLU = 2 };

/* Normalise one BF16 vector of length K and round the result to BF16.
 * norm = NONE copies x.  gamma may be NULL (unit gain); beta may be NULL (zero). */
void wgo_norm_bf16(int norm, const uint16_t *x, const uint16_t *gamma,
                   const uint16_t *beta, int64_t K, double eps, uint16_t *xh)
{
    if (norm == WGO_NORM_NONE) {
        memcpy(xh, x, (size_t)K * sizeof(uint16_t));
        return;
    }
    if (norm == WGO_NORM_RMS) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = wgo_bf16_to_f64(x[k]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k) {
            double g = gamma ? wgo_bf16_to_f64(gamma[k]) : 1.0;
            xh[k] = wgo_f64_to_bf16(wgo_bf16_to_f64(x[k]) * r * g);
        }
        return;
    }
    /* LayerNorm: mean, then biased variance about the mean (two passes). */
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += wgo_bf16_to_f64(x[k]);
    double mu = s / (double)K;
    double sv = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double d = wgo_bf16_to_f64(x[k]) - mu;
        sv += d * d;
    }
    double r = 1.0 / sqrt(sv / (double)K + eps);
    for (int64_t k = 0; k < K; ++k) {
        double g = gamma ? wgo_bf16_to_f64(gamma[k]) : 1.0;
        double b = beta ? wgo_bf16_to_f64(beta[k]) : 0.0;
        xh[k] = wgo_f64_to_bf16((wgo_bf16_to_f64(x[k]) - mu) * r * g + b);
    }
}

/* Un-rounded statistics helper used by the pin tests: returns the binary64
 * normalised value before the final rounding (gain applied). */
void wgo_norm_f64(int norm, const uint16_t *x, const uint16_t *gamma,
                  const uint16_t *beta, int64_t K, double eps, double *out)
{
    if (norm == WGO_NORM_NONE) {
        for (int64_t k = 0; k < K; ++k) out[k] = wgo_bf16_to_f64(x[k]);
        return;
    }
    if (norm == WGO_NORM_RMS) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) { double v = wgo_bf16_to_f64(x[k]); ss += v * v; }
        double r = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            out[k] = wgo_bf16_to_f64(x[k]) * r * (gamma ? wgo_bf16_to_f64(gamma[k]) : 1.0);
        return;
    }
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += wgo_bf16_to_f64(x[k]);
    double mu = s / (double)K, sv = 0.0;
    for (int64_t k = 0; k < K; ++k) { double d = wgo_bf16_to_f64(x[k]) - mu; sv += d * d; }
    double r = 1.0 / sqrt(sv / (double)K + eps);
    for (int64_t k = 0; k < K; ++k)
        out[k] = (wgo_bf16_to_f64(x[k]) - mu) * r * (gamma ? wgo_bf16_to_f64(gamma[k]) : 1.0)
                 + (beta ? wgo_bf16_to_f64(beta[k]) : 0.0);
}

/* ---------------------------------------------------------------- product */

static int g_threads = 1;

void wgo_set_threads(int n) { g_threads = n < 1 ? 1 : n; }

int wgo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* acc[n] = sum_k W[n][k] * xh[k] for rows n in [0, N), sequential in k. */
void wgo_matvec(const uint16_t *W, int64_t N, int64_t K, const uint16_t *xh, double *acc)
{
    double *xv = (double *)malloc((size_t)K * sizeof(double));
    for (int64_t k = 0; k < K; ++k) xv[k] = wgo_bf16_to_f64(xh[k]);
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(g_threads)
#endif
    for (int64_t n = 0; n < N; ++n) {
        const uint16_t *row = W + n * K;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += wgo_bf16_to_f64(row[k]) * xv[k];
        acc[n] = s;
    }
    free(xv);
}

/* Same product for selected rows only (sampled parity at full size). */
void wgo_matvec_rows(const uint16_t *W, int64_t K, const int64_t *rows, int64_t nrows,
                     const uint16_t *xh, double *acc)
{
    for (int64_t i = 0; i < nrows; ++i) {
        const uint16_t *row = W + rows[i] * K;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += wgo_bf16_to_f64(row[k]) * wgo_bf16_to_f64(xh[k]);
        acc[i] = s;
    }
}

/* ------------------------------------------------------------------ stage */

/*
 * One norm-fused product stage over `batch` activation rows.
 *   x        [batch][x_stride] BF16, K used
 *   W, W_up  [N][K] BF16 (W_up only for SwiGLU)
 *   bias     [N] BF16 or NULL (added to the first accumulator)
 *   residual [batch][res_stride] BF16 or NULL
 *   y        [batch][y_stride] BF16 out
 *   xh_out   [batch][K] BF16 out (the rounded normalised input), may be NULL
 *   acc_out  [batch][N] binary64 out (epilogue input a+bias, or the gate value for
 *            SwiGLU), may be NULL
 */
void wgo_stage(int norm, int epi, int64_t N, int64_t K, int64_t batch,
               const uint16_t *x, int64_t x_stride,
               const uint16_t *gamma, const uint16_t *beta, double eps,
               const uint16_t *W, const uint16_t *W_up, const uint16_t *bias,
               const uint16_t *residual, int64_t res_stride,
               uint16_t *y, int64_t y_stride, uint16_t *xh_out, double *acc_out)
{
    uint16_t *xh = (uint16_t *)malloc((size_t)K * sizeof(uint16_t));
    double *a = (double *)malloc((size_t)N * sizeof(double));
    double *u = (epi == WGO_EPI_SWIGLU) ? (double *)malloc((size_t)N * sizeof(double)) : NULL;
    for (int64_t b = 0; b < batch; ++b) {
        wgo_norm_bf16(norm, x + b * x_stride, gamma, beta, K, eps, xh);
        if (xh_out) memcpy(xh_out + b * K, xh, (size_t)K * sizeof(uint16_t));
        wgo_matvec(W, N, K, xh, a);
        if (u) wgo_matvec(W_up, N, K, xh, u);
        for (int64_t n = 0; n < N; ++n) {
            double z = a[n] + (bias ? wgo_bf16_to_f64(bias[n]) : 0.0);
            double e;
            if (epi == WGO_EPI_GELU_TANH) e = wgo_gelu_tanh(z);
            else if (epi == WGO_EPI_SWIGLU) e = wgo_silu(z) * u[n];
            else e = z;
            if (residual) e += wgo_bf16_to_f64(residual[b * res_stride + n]);
            y[b * y_stride + n] = wgo_f64_to_bf16(e);
            if (acc_out) acc_out[b * N + n] = z;
        }
    }
    free(xh); free(a); free(u);
}

/*
 * Final RMSNorm + LM head + greedy argmax.
 *   h [batch][h_stride] BF16, g [K] BF16, W [V][K] BF16
 *   idx [batch] (lowest index attaining the maximum), maxv [batch],
 *   logits [batch][V] binary64 (may be NULL)
 */
void wgo_lmhead_argmax(int norm, const uint16_t *h, int64_t h_stride, const uint16_t *g,
                       double eps, const uint16_t *W, int64_t V, int64_t K, int64_t batch,
                       int32_t *idx, double *maxv, double *logits)
{
    uint16_t *xh = (uint16_t *)malloc((size_t)K * sizeof(uint16_t));
    double *l = (double *)malloc((size_t)V * sizeof(double));
    for (int64_t b = 0; b < batch; ++b) {
        wgo_norm_bf16(norm, h + b * h_stride, g, NULL, K, eps, xh);
        wgo_matvec(W, V, K, xh, l);
        int64_t best = 0;
        for (int64_t v = 1; v < V; ++v)
            if (l[v] > l[best]) best = v;        /* strict: ties keep the lowest index */
        idx[b] = (int32_t)best;
        maxv[b] = l[best];
        if (logits) memcpy(logits + b * V, l, (size_t)V * sizeof(double));
    }
    free(xh); free(l);
}

/* Standalone RMSNorm over FP16 rows: y = R16( x * (mean x^2 + eps)^(-1/2) * g ). */
void wgo_rmsnorm_rows_f16(const uint16_t *x, int64_t x_stride, const uint16_t *g, double eps,
                          uint16_t *y, int64_t y_stride, int64_t rows, int64_t K)
{
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(g_threads)
#endif
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * x_stride;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) { double v = wgo_f16_to_f64(xr[k]); ss += v * v; }
        double inv = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            y[r * y_stride + k] = wgo_f64_to_f16(wgo_f16_to_f64(xr[k]) * inv * wgo_f16_to_f64(g[k]));
    }
}

/* ------------------------------------------------------- decode attention */
/*
 * Attention of one new token over a static key/value cache, grouped-query.
 *   -- "Making small PyTorch ops faster on a laptop GPU", section "A full
 *      decode step is a different story": the new key and value are appended
 *      to the cache, then the softmax is taken over every cached position.
 *   -- "One Token, Kernel by Kernel", section "The fix: Part 10's split-KV
 *      kernel": cache layout (batch, head, slot, dimension); the valid
 *      positions are 0 .. pos, read per row; each key/value head serves a
 *      group of query heads (12 query heads over 2 key/value heads in the
 *      page's model, section "The setup").
 *
 *   q [batch][q_heads][d], k_new, v_new [batch][kv_heads][d]     BF16
 *   k_cache, v_cache [batch][kv_heads][slots][d]                 BF16, updated
 *   pos [batch]   slot of the new token.  A row whose pos lies outside
 *                 [0, slots) appends nothing and its output is zero (the
 *                 pages define no such case; this is the library's rule).
 *   Query head h reads key/value head h / (q_heads / kv_heads).
 *     s_t   = scale * sum_j q_j k_tj,  t = 0 .. pos
 *     out_j = R( sum_t e^(s_t - m) v_tj / sum_t e^(s_t - m) ),  m = max_t s_t
 *   out_f64 (may be NULL) receives the values before rounding.
 */
void wgo_decode_attention(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                          uint16_t *k_cache, uint16_t *v_cache, const int32_t *pos,
                          int64_t batch, int64_t q_heads, int64_t kv_heads, int64_t slots, int64_t d,
                          double scale, uint16_t *out, double *out_f64)
{
    const int64_t group = q_heads / kv_heads;
    /* the append comes first: the new token attends to itself */
    for (int64_t b = 0; b < batch; ++b) {
        if (pos[b] < 0 || pos[b] >= slots) continue;
        for (int64_t g = 0; g < kv_heads; ++g) {
            const int64_t row = ((b * kv_heads + g) * slots + pos[b]) * d;
            memcpy(k_cache + row, k_new + (b * kv_heads + g) * d, (size_t)d * sizeof(uint16_t));
            memcpy(v_cache + row, v_new + (b * kv_heads + g) * d, (size_t)d * sizeof(uint16_t));
        }
    }
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(g_threads)
#endif
    for (int64_t bh = 0; bh < batch * q_heads; ++bh) {
        const int64_t b = bh / q_heads, h = bh % q_heads, g = h / group;
        uint16_t *o = out + bh * d;
        double *of = out_f64 ? out_f64 + bh * d : NULL;
        if (pos[b] < 0 || pos[b] >= slots) {
            for (int64_t j = 0; j < d; ++j) { o[j] = 0; if (of) of[j] = 0.0; }
            continue;
        }
        const int64_t n = pos[b] + 1;
        const uint16_t *qh = q + bh * d;
        const uint16_t *K = k_cache + (b * kv_heads + g) * slots * d;
        const uint16_t *Vc = v_cache + (b * kv_heads + g) * slots * d;
        double *s = (double *)malloc((size_t)n * sizeof(double));
        double m = -INFINITY;
        for (int64_t t = 0; t < n; ++t) {
            double dot = 0.0;
            for (int64_t j = 0; j < d; ++j)
                dot += wgo_bf16_to_f64(qh[j]) * wgo_bf16_to_f64(K[t * d + j]);
            s[t] = scale * dot;
            if (s[t] > m) m = s[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < n; ++t) { s[t] = exp(s[t] - m); l += s[t]; }
        for (int64_t j = 0; j < d; ++j) {
            double a = 0.0;
            for (int64_t t = 0; t < n; ++t) a += s[t] * wgo_bf16_to_f64(Vc[t * d + j]);
            const double v = a / l;
            o[j] = wgo_f64_to_bf16(v);
            if (of) of[j] = v;
        }
        free(s);
    }
}

/* ------------------------------------------------------- 4-bit weights */
/*
 * Product with 4-bit integer weights in groups of 128 along K.
 *   -- "One Token, Kernel by Kernel", section "4-bit weights": every linear
 *      layer quantised to 4-bit integers in groups of 128.  The pages give no
 *      bit layout; the reading used here: row n of W4 holds K/2 bytes, byte j
 *      carries k = 2j in its low nibble and k = 2j+1 in its high nibble; each
 *      (row, group of 128) has a BF16 scale s and a BF16 zero z, and the
 *      weight is w = s * q + z for the code q in 0..15.
 *   y[b][n] = R( sum_k w[n][k] * x[b][k] ),  sequential in k, binary64.
 *   x [batch][x_stride] BF16; y [batch][N] BF16.
 */
void wgo_matvec_int4(const uint8_t *W4, const uint16_t *scales, const uint16_t *zeros, int64_t N, int64_t K,
                     const uint16_t *x, int64_t x_stride, int64_t batch, uint16_t *y, double *acc_out)
{
    const int64_t ng = K / 128;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(g_threads)
#endif
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < batch; ++b) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const uint8_t byte = W4[n * (K / 2) + k / 2];
                const int q = (k & 1) ? (byte >> 4) : (byte & 15);
                const double w = wgo_bf16_to_f64(scales[n * ng + k / 128]) * (double)q
                               + wgo_bf16_to_f64(zeros[n * ng + k / 128]);
                acc += w * wgo_bf16_to_f64(x[b * x_stride + k]);
            }
            y[b * N + n] = wgo_f64_to_bf16(acc);
            if (acc_out) acc_out[b * N + n] = acc;
        }
    }
}

/* ---------------------------------------------------------------- backward */

/* Derivative of the GELU-tanh form above: with a = c (z + 0.044715 z^3) and
 * t = tanh(a), d/dz = 0.5 (1 + t) + 0.5 z (1 - t^2) c (1 + 3 * 0.044715 z^2). */
double wgo_gelu_tanh_grad(double z)
{
    const double c = sqrt(2.0 / M_PI);
    const double t = tanh(c * (z + 0.044715 * z * z * z));
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * z * z);
}

/* Gradient of loss = mean over [batch][N] of y^2 (y read as BF16, squared and
 * averaged in wide precision): g = R(2 y / (batch N)). */
void wgo_mean_square_grad(const uint16_t *y, int64_t y_stride, int64_t N, int64_t batch,
                          uint16_t *g, int64_t g_stride)
{
    const double s = 2.0 / ((double)batch * (double)N);
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t n = 0; n < N; ++n)
            g[b * g_stride + n] = wgo_f64_to_bf16(wgo_bf16_to_f64(y[b * y_stride + n]) * s);
}

static double rnd_bf16(int rnd, double v) { return rnd ? wgo_bf16_to_f64(wgo_f64_to_bf16(v)) : v; }

/*
 * Backward of one LayerNorm -> Linear(+bias) -> GELU-tanh block (definition in
 * the header).  x [batch][x_stride] BF16 block input; W [N][K]; bias [N] or
 * NULL; gamma, beta [K] or NULL (1, 0); gy [batch][gy_stride] gradient of the
 * block output (binary64 values; BF16 values between rounded blocks).  rnd = 1 rounds at the stated points; rnd = 0 keeps every
 * value in binary64 (also xh, so that the result is the exact derivative of the
 * unrounded block).  Outputs (binary64; BF16 values when rnd = 1):
 * gx [batch][K], gW [N][K], gb [N] (NULL skips), ggamma and gbeta [K] (NULL
 * skips), gz [batch][N] (NULL skips).  gz_in [batch][N] (or NULL): when given,
 * the products and the norm backward use it in place of the computed gz (gz
 * itself is still computed and returned in gz_out).  Sums run in ascending
 * index order.
 */
void wgo_block_backward(int64_t N, int64_t K, int64_t batch,
                        const uint16_t *x, int64_t x_stride,
                        const uint16_t *gamma, const uint16_t *beta, double eps,
                        const uint16_t *W, const uint16_t *bias,
                        const double *gy, int64_t gy_stride, const double *gz_in, int rnd,
                        double *gx, double *gW, double *gb, double *ggamma, double *gbeta,
                        double *gz_out)
{
    double *u = (double *)malloc((size_t)(batch * K) * sizeof(double));
    double *xh = (double *)malloc((size_t)(batch * K) * sizeof(double));
    double *sig = (double *)malloc((size_t)batch * sizeof(double));
    double *gz = (double *)malloc((size_t)(batch * N) * sizeof(double));
    double *gxh = (double *)malloc((size_t)(batch * K) * sizeof(double));
    /* forward again: LayerNorm statistics, u, xh */
    for (int64_t b = 0; b < batch; ++b) {
        const uint16_t *xb = x + b * x_stride;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += wgo_bf16_to_f64(xb[k]);
        const double mu = s / (double)K;
        double sv = 0.0;
        for (int64_t k = 0; k < K; ++k) { double d = wgo_bf16_to_f64(xb[k]) - mu; sv += d * d; }
        sig[b] = sqrt(sv / (double)K + eps);
        for (int64_t k = 0; k < K; ++k) {
            u[b * K + k] = (wgo_bf16_to_f64(xb[k]) - mu) / sig[b];
            const double v = u[b * K + k] * (gamma ? wgo_bf16_to_f64(gamma[k]) : 1.0)
                             + (beta ? wgo_bf16_to_f64(beta[k]) : 0.0);
            xh[b * K + k] = rnd_bf16(rnd, v);
        }
    }
    /* pre-activation, then gz = gy * GELU'(z) */
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(g_threads)
#endif
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < batch; ++b) {
            double z = 0.0;
            for (int64_t k = 0; k < K; ++k) z += wgo_bf16_to_f64(W[n * K + k]) * xh[b * K + k];
            if (bias) z += wgo_bf16_to_f64(bias[n]);
            gz[b * N + n] = rnd_bf16(rnd, gy[b * gy_stride + n] * wgo_gelu_tanh_grad(z));
        }
    }
    if (gz_out) memcpy(gz_out, gz, (size_t)(batch * N) * sizeof(double));
    /* a caller that compares against a computation which rounded gz itself
     * hands that rounding decision in: the steps below then start from it */
    if (gz_in) memcpy(gz, gz_in, (size_t)(batch * N) * sizeof(double));
    /* bias and weight gradients: sums over the batch */
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(g_threads)
#endif
    for (int64_t n = 0; n < N; ++n) {
        if (gb) {
            double s = 0.0;
            for (int64_t b = 0; b < batch; ++b) s += gz[b * N + n];
            gb[n] = rnd_bf16(rnd, s);
        }
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t b = 0; b < batch; ++b) s += gz[b * N + n] * xh[b * K + k];
            gW[n * K + k] = rnd_bf16(rnd, s);
        }
    }
    /* gradient of the normalised input: gxh = gz W (sum over the output rows) */
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(g_threads)
#endif
    for (int64_t k = 0; k < K; ++k)
        for (int64_t b = 0; b < batch; ++b) {
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n) s += gz[b * N + n] * wgo_bf16_to_f64(W[n * K + k]);
            gxh[b * K + k] = s;
        }
    /* LayerNorm backward */
    for (int64_t b = 0; b < batch; ++b) {
        double m1 = 0.0, m2 = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double gu = (gamma ? wgo_bf16_to_f64(gamma[k]) : 1.0) * gxh[b * K + k];
            m1 += gu;
            m2 += gu * u[b * K + k];
        }
        m1 /= (double)K;
        m2 /= (double)K;
        for (int64_t k = 0; k < K; ++k) {
            const double gu = (gamma ? wgo_bf16_to_f64(gamma[k]) : 1.0) * gxh[b * K + k];
            gx[b * K + k] = rnd_bf16(rnd, (gu - m1 - u[b * K + k] * m2) / sig[b]);
        }
    }
    for (int64_t k = 0; k < K; ++k) {
        double sg = 0.0, sb = 0.0;
        for (int64_t b = 0; b < batch; ++b) {
            sg += gxh[b * K + k] * u[b * K + k];
            sb += gxh[b * K + k];
        }
        if (ggamma) ggamma[k] = rnd_bf16(rnd, sg);
        if (gbeta) gbeta[k] = rnd_bf16(rnd, sb);
    }
    free(u); free(xh); free(sig); free(gz); free(gxh);
}
