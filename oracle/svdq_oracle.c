/*
 * svdq_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU oracle for the SVDQuant W4A4 linear layer.  Only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * it; the library never links or calls it, and it shares no code, header or
 * table with the library.  Built with gcc -O2 -ffp-contract=off -fopenmp
 * (OpenMP only distributes independent output rows).
 *
 * What the method computes, from "Bringing Nunchaku 4-bit Diffusion
 * Inference to Diffusers" (Hugging Face blog), section "Background: SVDQuant
 * and Nunchaku": activation outliers are moved into the weights by a
 * per-channel smoothing, the hardest part of each weight matrix is kept in a
 * small 16-bit low-rank branch, and the remaining residual is quantized to
 * 4 bits; both weights and activations are 4-bit (W4A4).  Section "Native
 * loading in Diffusers" fixes rank 32 and a bfloat16 compute dtype.  The
 * exact formulas below are readings of that prose (listed with their
 * justification in the design notes of the repository):
 *
 *   smoothing   lambda_k = sqrt(max|X_k| / max_n |W_nk|)   (1 if either is 0)
 *               s_k      = fl32(1 / lambda_k)
 *   low rank    What_kn = W_nk / s_k;  top-r SVD What ~ U S V^T
 *               down[j][k] = bf16(s_k * (U S)_kj)   (r x K, smoothing folded)
 *               up[n][j]   = bf16(V_nj)             (N x r)
 *   residual    R_kn = (W_nk - sum_j down[j][k]*up[n][j]) / s_k   (fp64)
 *               quantized from fl32(R) per (n, 64-group along k)
 *   activation  xhat_mk = fl32(X_mk * s_k), quantized per (m, 64-group)
 *               h_mj    = sum_k X_mk * down[j][k]
 *   output      y_mn = sum_g sx_mg sw_ng sum_{k in g} qx_mk qw_nk
 *                      + sum_j h_mj up[n][j] + b_n     [optionally GELU-tanh]
 *
 * INT4 group quantizer (symmetric, 64 wide): a = max|v|; scale = fl32(a/7)
 * (0 if a == 0; rounded upward instead of to nearest when a/7 is below the
 * smallest normal fp32); q = round-half-even of the exact real quotient
 * v/scale, clamped to [-7, 7] (the clamp never acts).  The 4-bit code is
 * sign-magnitude, the same layout as an E2M1 code: bit 3 = sign of v (kept
 * for zero), bits 0-2 = |q|.  Nibbles: byte i = code[2i] | code[2i+1] << 4.
 *
 * MXFP4 block quantizer (OCP Microscaling v1.0 conversion; 32 wide):
 * X = floor(log2 a) - 2, clamped to [-127, 127], stored as E8M0 X + 127;
 * t = v * 2^-X rounded to the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to
 * the even grid index, |t| > 6 saturating to 6; code = sign << 3 | index,
 * the sign kept for zero.
 *
 * Every routine is the definition written out; none is blocked or reordered.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

#define ORACLE_INT4 0
#define ORACLE_MXFP4 1

/* ------------------------------------------------------------------ dtypes */

static double bf16_val(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ----------------------------------------------------------- INT4 groups */

/* One symmetric INT4 group: returns scale, writes the integers q in [-7, 7]
 * and (when `code` is not NULL) their sign-magnitude 4-bit codes. */
float oracle_quant_group_int4(const float *v, int n, int8_t *q, uint8_t *code)
{
    float a = 0.0f;
    for (int i = 0; i < n; ++i) {
        float t = fabsf(v[i]);
        if (t > a) a = t;
    }
    if (a == 0.0f) {
        for (int i = 0; i < n; ++i) {
            q[i] = 0;
            if (code) code[i] = (uint8_t)(signbit(v[i]) ? 8 : 0);
        }
        return 0.0f;
    }
    /* fl32(a / 7): the fp64 quotient rounded to fp32 is the correctly rounded
     * fp32 quotient (53 >= 2*24 + 2, so double rounding cannot bite). */
    float scale = (float)((double)a / 7.0);
    /* Below the normal range the quotient is rounded upward instead, so that
     * a <= 7 * scale holds for every group and no code is ever clamped. */
    if (scale < FLT_MIN && (double)scale * 7.0 < (double)a)
        scale = nextafterf(scale, INFINITY);
    double S = (double)scale;
    for (int i = 0; i < n; ++i) {
        double x = (double)v[i];
        double ax = fabs(x);
        /* |x| against the tie points (j + 1/2) * S, each exact in fp64. */
        int m = 8;
        for (int j = 0; j < 8; ++j) {
            double tie = ((double)j + 0.5) * S;
            if (ax < tie) { m = j; break; }
            if (ax == tie) { m = (j % 2 == 0) ? j : j + 1; break; }
        }
        if (m > 7) m = 7;
        q[i] = (int8_t)(x < 0 ? -m : m);
        if (code) code[i] = (uint8_t)((signbit(v[i]) ? 8 : 0) | m);
    }
    return scale;
}

/* ---------------------------------------------------------- MXFP4 blocks */

static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* One MXFP4 block: returns the E8M0 byte, writes E2M1 codes (one per byte). */
uint8_t oracle_quant_block_mxfp4(const float *v, int n, uint8_t *code)
{
    float a = 0.0f;
    for (int i = 0; i < n; ++i) {
        float t = fabsf(v[i]);
        if (t > a) a = t;
    }
    int X;
    if (a == 0.0f) {
        X = -127;
    } else {
        int e;
        frexp((double)a, &e);          /* a = f * 2^e, f in [0.5, 1) */
        X = (e - 1) - 2;               /* floor(log2 a) - emax(E2M1) */
    }
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    for (int i = 0; i < n; ++i) {
        double t = ldexp((double)v[i], -X);     /* exact */
        double at = fabs(t);
        int idx;
        if (at >= 6.0) {
            idx = 7;
        } else {
            idx = 0;
            for (int j = 0; j < 7; ++j) {
                double mid = 0.5 * (E2M1_GRID[j] + E2M1_GRID[j + 1]);
                if (at < mid) { idx = j; break; }
                if (at == mid) { idx = (j % 2 == 0) ? j : j + 1; break; }
                idx = j + 1;
            }
        }
        int sign = signbit(v[i]) ? 1 : 0;
        code[i] = (uint8_t)((sign << 3) | idx);
    }
    return (uint8_t)(X + 127);
}

double oracle_e2m1_value(uint8_t code)
{
    double m = E2M1_GRID[code & 7];
    return (code & 8) ? -m : m;
}

double oracle_e8m0_value(uint8_t e)
{
    if (e == 0xFF) return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* --------------------------------------------------------------- nibbles */

/* Two 4-bit codes per byte, element 2i in the low nibble. */
void oracle_pack_nibbles(const uint8_t *code, int n, uint8_t *out)
{
    for (int i = 0; i < n / 2; ++i)
        out[i] = (uint8_t)((code[2 * i] & 0x0F) | ((code[2 * i + 1] & 0x0F) << 4));
}

/* Sign-magnitude INT4 code -> integer. */
static int int4_of_nibble(int nib) { return (nib & 8) ? -(nib & 7) : (nib & 7); }

int oracle_int4_value(uint8_t code) { return int4_of_nibble(code & 15); }

/* Twice the E2M1 value of a code (an integer in [-12, 12]). */
static int e2m1_twice(int code)
{
    const int m = (int)(2.0 * E2M1_GRID[code & 7]);
    return (code & 8) ? -m : m;
}

static int nibble_at(const uint8_t *row, int k)
{
    uint8_t b = row[k >> 1];
    return (k & 1) ? (b >> 4) : (b & 0x0F);
}

/* Quantize one row of `K` values into codes (K/2 bytes) and scales. */
static void quant_row(const float *v, int K, int prec, uint8_t *codes, void *scales)
{
    if (prec == ORACLE_INT4) {
        int8_t q[64];
        uint8_t c[64];
        float *sc = (float *)scales;
        for (int g = 0; g < K / 64; ++g) {
            sc[g] = oracle_quant_group_int4(v + 64 * g, 64, q, c);
            oracle_pack_nibbles(c, 64, codes + 32 * g);
        }
    } else {
        uint8_t c[32];
        uint8_t *sc = (uint8_t *)scales;
        for (int b = 0; b < K / 32; ++b) {
            sc[b] = oracle_quant_block_mxfp4(v + 32 * b, 32, c);
            oracle_pack_nibbles(c, 32, codes + 16 * b);
        }
    }
}

/* -------------------------------------------------------------- smoothing */

/* s_k = fl32(1 / sqrt(max|X_k| / max_n|W_nk|)), 1 when either max is 0. */
void oracle_smooth(const uint16_t *W, const float *act_absmax, int N, int K, float *s)
{
    for (int k = 0; k < K; ++k) {
        double mw = 0.0;
        for (int n = 0; n < N; ++n) {
            double w = fabs(bf16_val(W[(size_t)n * K + k]));
            if (w > mw) mw = w;
        }
        double mx = (double)act_absmax[k];
        if (mx == 0.0 || mw == 0.0) {
            s[k] = 1.0f;
        } else {
            double lambda = sqrt(mx / mw);
            s[k] = (float)(1.0 / lambda);
        }
    }
}

/* --------------------------------------------------------------- residual */

/* R_kn = (W_nk - sum_j down[j][k] up[n][j]) / s_k  (fp64, j ascending),
 * then fl32(R) quantized per (n, group along k). */
void oracle_residual(const uint16_t *W, const float *s, const uint16_t *down,
                     const uint16_t *up, int N, int K, int r, int prec,
                     uint8_t *wq, void *wscale, float *R_out /* may be NULL */)
{
    int G = (prec == ORACLE_INT4) ? K / 64 : K / 32;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        float *row = (float *)malloc(sizeof(float) * (size_t)K);
        for (int k = 0; k < K; ++k) {
            double acc = 0.0;
            for (int j = 0; j < r; ++j)
                acc += bf16_val(down[(size_t)j * K + k]) * bf16_val(up[(size_t)n * r + j]);
            double R = (bf16_val(W[(size_t)n * K + k]) - acc) / (double)s[k];
            row[k] = (float)R;
        }
        if (R_out) memcpy(R_out + (size_t)n * K, row, sizeof(float) * (size_t)K);
        if (prec == ORACLE_INT4)
            quant_row(row, K, prec, wq + (size_t)n * (K / 2), (float *)wscale + (size_t)n * G);
        else
            quant_row(row, K, prec, wq + (size_t)n * (K / 2), (uint8_t *)wscale + (size_t)n * G);
        free(row);
    }
}

/* ------------------------------------------------------------- activation */

/* xhat = fl32(X * s) quantized per row/group; h = X . down^T in fp64. */
void oracle_quant_act(const uint16_t *X, int M, int K, const float *s, const uint16_t *down,
                      int r, int prec, uint8_t *xq, void *xscale, double *h)
{
    int G = (prec == ORACLE_INT4) ? K / 64 : K / 32;
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m) {
        float *row = (float *)malloc(sizeof(float) * (size_t)K);
        for (int k = 0; k < K; ++k)
            row[k] = (float)(bf16_val(X[(size_t)m * K + k]) * (double)s[k]);
        if (prec == ORACLE_INT4)
            quant_row(row, K, prec, xq + (size_t)m * (K / 2), (float *)xscale + (size_t)m * G);
        else
            quant_row(row, K, prec, xq + (size_t)m * (K / 2), (uint8_t *)xscale + (size_t)m * G);
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += bf16_val(X[(size_t)m * K + k]) * bf16_val(down[(size_t)j * K + k]);
            h[(size_t)m * r + j] = acc;
        }
        free(row);
    }
}

/* ----------------------------------------------------------------- output */

static double gelu_tanh(double y)
{
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * y * (1.0 + tanh(c * (y + 0.044715 * y * y * y)));
}

double oracle_gelu_tanh(double y) { return gelu_tanh(y); }

/* y for the listed rows (all rows when rows == NULL, nrows == M).
 * The 4-bit term, the low-rank term and the bias are also returned separately
 * when the matching pointer is non-NULL (each [nrows][N]). */
void oracle_linear(const uint8_t *xq, const void *xscale, const double *h,
                   const uint8_t *wq, const void *wscale, const uint16_t *up,
                   const uint16_t *bias, int M, int N, int K, int r, int prec, int gelu,
                   const int *rows, int nrows, double *y, double *y_q4, double *y_lr)
{
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nrows; ++i) {
        int m = rows ? rows[i] : i;
        const uint8_t *xr = xq + (size_t)m * (K / 2);
        for (int n = 0; n < N; ++n) {
            const uint8_t *wr = wq + (size_t)n * (K / 2);
            double q4 = 0.0;
            if (prec == ORACLE_INT4) {
                const float *sx = (const float *)xscale + (size_t)m * (K / 64);
                const float *sw = (const float *)wscale + (size_t)n * (K / 64);
                for (int g = 0; g < K / 64; ++g) {
                    long long P = 0;
                    for (int k = 64 * g; k < 64 * g + 64; ++k)
                        P += (long long)int4_of_nibble(nibble_at(xr, k)) *
                             (long long)int4_of_nibble(nibble_at(wr, k));
                    q4 += (double)sx[g] * (double)sw[g] * (double)P;
                }
            } else {
                const uint8_t *ex = (const uint8_t *)xscale + (size_t)m * (K / 32);
                const uint8_t *ew = (const uint8_t *)wscale + (size_t)n * (K / 32);
                for (int b = 0; b < K / 32; ++b) {
                    /* Every E2M1 value is a multiple of 1/2 below 6 in magnitude,
                     * so the block's dot product is the integer sum of the
                     * doubled values' products, divided by 4 (exact). */
                    long long S = 0;
                    for (int k = 32 * b; k < 32 * b + 32; ++k)
                        S += (long long)e2m1_twice(nibble_at(xr, k)) * (long long)e2m1_twice(nibble_at(wr, k));
                    const double P = (double)S / 4.0;
                    q4 += oracle_e8m0_value(ex[b]) * oracle_e8m0_value(ew[b]) * P;
                }
            }
            double lr = 0.0;
            for (int j = 0; j < r; ++j)
                lr += h[(size_t)m * r + j] * bf16_val(up[(size_t)n * r + j]);
            double v = q4 + lr + (bias ? bf16_val(bias[n]) : 0.0);
            if (gelu) v = gelu_tanh(v);
            y[(size_t)i * N + n] = v;
            if (y_q4) y_q4[(size_t)i * N + n] = q4;
            if (y_lr) y_lr[(size_t)i * N + n] = lr;
        }
    }
}

/* --------------------------------------- QKV projection + Q/K RMS-norm + RoPE */

/*
 * The fused attention-input step of the same pages ("Bringing Nunchaku 4-bit
 * Diffusion Inference to Diffusers", section "Quantizing models with
 * structural rewrites": the Nunchaku engine's fused_qkv_norm_rottary takes
 * the hidden states, the QKV projection, the Q and K norms and the rotary
 * embedding together).  Readings: the
 * projection output is the W4A4 linear's, rounded to bf16 as the linear
 * stores it; its N = 3 H 128 channels are H heads of Q, then of K, then of
 * V, each 128 wide; Q and K heads are RMS-normalized over their 128
 * channels, u_d = yb_d / sqrt(mean_d(yb_d^2) + eps) * w_d (w = the bf16 norm
 * weight of Q or K), then rotated pairwise with the token's angle table,
 * out_2p = u_2p cos_mp - u_2p+1 sin_mp, out_2p+1 = u_2p+1 cos_mp + u_2p sin_mp
 * (p < 64); V heads pass through.  fp64 throughout after the bf16 rounding.
 */
static double bf16_round(double v)
{
    /* fp64 -> fp32 (nearest) -> bf16 (nearest even on the upper 16 bits) */
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t keep = u >> 16, rem = u & 0xFFFFu;
    if (rem > 0x8000u || (rem == 0x8000u && (keep & 1u))) keep += 1u;
    return bf16_val((uint16_t)keep);
}

void oracle_qkv_norm_rope(const double *ylin, int M, int N, const uint16_t *norm_q, const uint16_t *norm_k,
                          double eps, const float *rope_cos, const float *rope_sin, double *out)
{
    const int H = N / 384;
    for (int m = 0; m < M; ++m) {
        for (int hd = 0; hd < 3 * H; ++hd) {
            const double *y = ylin + (size_t)m * N + 128 * hd;
            double *o = out + (size_t)m * N + 128 * hd;
            double yb[128];
            for (int d = 0; d < 128; ++d) yb[d] = bf16_round(y[d]);
            if (hd >= 2 * H) {                    /* V */
                for (int d = 0; d < 128; ++d) o[d] = yb[d];
                continue;
            }
            const uint16_t *w = hd < H ? norm_q : norm_k;
            double ms = 0.0;
            for (int d = 0; d < 128; ++d) ms += yb[d] * yb[d];
            ms /= 128.0;
            const double rs = 1.0 / sqrt(ms + eps);
            double u[128];
            for (int d = 0; d < 128; ++d) u[d] = yb[d] * rs * bf16_val(w[d]);
            for (int q = 0; q < 64; ++q) {
                const double c = rope_cos[(size_t)m * 64 + q], sn = rope_sin[(size_t)m * 64 + q];
                o[2 * q] = u[2 * q] * c - u[2 * q + 1] * sn;
                o[2 * q + 1] = u[2 * q + 1] * c + u[2 * q] * sn;
            }
        }
    }
}

/* ------------------------------------------------------- AWQ W4A16 (INT4) */

/*
 * Weight-only 4-bit layer of the same pages ("Bringing Nunchaku 4-bit
 * Diffusion Inference to Diffusers", section "Native loading in Diffusers":
 * the awq_w4a16 family, int4 with group size 64, used for the modulation
 * layers, which are memory-bound and precision-sensitive).  Readings (the
 * pages give only precision and group size): the group quantizer is the
 * symmetric INT4 one above, applied to fl32(W) per (n, 64-group along k);
 * the activation-aware channel scaling is a calibration step and is assumed
 * folded into W by the caller; activations stay bf16 and
 *   y_mn = sum_g sw_ng sum_{k in g} X_mk q_nk + b_n.
 *
 * Storage (K % 256 == 0): code c = q + 8 in [1, 15] (offset binary), row n
 * takes K/2 bytes.  For k = 256 C + 64 g + 32 h + 8 b + i (g < 4, h < 2,
 * b < 4, i < 8) the code sits in byte 128 C + 32 b + 4 (2 g + h) + p / 2,
 * low nibble when p is even, with p = i / 2 for even i and 4 + (i - 1) / 2
 * for odd i.
 */
static int awq_byte(int k, int *high)
{
    int C = k / 256, r = k % 256;
    int g = r / 64, h = (r % 64) / 32, b = (r % 32) / 8, i = r % 8;
    int p = (i % 2 == 0) ? i / 2 : 4 + (i - 1) / 2;
    *high = p % 2;
    return 128 * C + 32 * b + 4 * (2 * g + h) + p / 2;
}

/* q of weight (row, k) from the stored row */
int oracle_awq_code(const uint8_t *row, int k)
{
    int high;
    int byte = awq_byte(k, &high);
    int c = high ? (row[byte] >> 4) : (row[byte] & 15);
    return c - 8;
}

void oracle_awq_pack(const uint16_t *W, int N, int K, uint8_t *wq, float *wscale)
{
    float *v = (float *)malloc(sizeof(float) * 64);
    int8_t q[64];
    memset(wq, 0, (size_t)N * (K / 2));
    for (int n = 0; n < N; ++n) {
        uint8_t *row = wq + (size_t)n * (K / 2);
        for (int g = 0; g < K / 64; ++g) {
            for (int i = 0; i < 64; ++i) v[i] = (float)bf16_val(W[(size_t)n * K + 64 * g + i]);
            wscale[(size_t)n * (K / 64) + g] = oracle_quant_group_int4(v, 64, q, NULL);
            for (int i = 0; i < 64; ++i) {
                int high;
                int byte = awq_byte(64 * g + i, &high);
                int c = q[i] + 8;
                row[byte] |= (uint8_t)(high ? c << 4 : c);
            }
        }
    }
    free(v);
}

/* y [M][N] in fp64 (no bf16 rounding) */
void oracle_awq_linear(const uint16_t *X, const uint8_t *wq, const float *wscale, const uint16_t *bias,
                       int M, int N, int K, double *y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m) {
        for (int n = 0; n < N; ++n) {
            const uint8_t *row = wq + (size_t)n * (K / 2);
            double acc = 0.0;
            for (int g = 0; g < K / 64; ++g) {
                double P = 0.0;
                for (int k = 64 * g; k < 64 * g + 64; ++k)
                    P += bf16_val(X[(size_t)m * K + k]) * (double)oracle_awq_code(row, k);
                acc += (double)wscale[(size_t)n * (K / 64) + g] * P;
            }
            y[(size_t)m * N + n] = acc + (bias ? bf16_val(bias[n]) : 0.0);
        }
    }
}

int oracle_num_threads(void)
{
    int t = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        t = omp_get_num_threads();
    }
#endif
    return t;
}

/* ------------------------------------------------ NF4 W4A16 (weight-only) */

/*
 * Weight-only 4-bit comparison path of the pages ("BitsAndBytes W4
 * Quantization", vLLM-Omni docs, sections "Overview" and "Parameters":
 * BF16 weights quantized at load time to the "nf4" 4-bit data type,
 * activations kept in bf16, and with compress_statistics the block scaling
 * statistics double-quantized).  The pages name the data type only; the
 * readings below follow the published NF4 construction (quantiles of the
 * standard normal distribution normalized to [-1, 1], with an exact zero):
 *
 *   codebook   16 fp32 levels c_0 < ... < c_15: c_7 = 0; the 8 positive
 *              levels are Phi^-1(1/2 + j (1/2 - d) / 8), j = 1..8, the 7
 *              negative ones -Phi^-1(1/2 + j (1/2 - d) / 7), j = 1..7, all
 *              divided by Phi^-1(1 - d) (so c_0 = -1, c_15 = 1), with the
 *              tail probability d = (1/32 + 1/30) / 2 (halfway between the
 *              half-bin probabilities of 16 and 15 equal bins); each level
 *              rounded once to fp32
 *   block      64 consecutive weights of a row; a = max |w| (fp32)
 *   code       x = fl32(w / a); the nearest level, comparing x with the
 *              midpoints (c_i + c_i+1) / 2 exactly, a tie going to the level
 *              of smaller magnitude; a == 0 gives code 7 (zero)
 *   statistics the block absmaxes in row-major (n, block) order, in chunks
 *              of 256: s = max a over the chunk; q_b = round-half-even of
 *              the exact 255 a_b / s (0 when s == 0); the chunk stores
 *              d = fl32(s / 255)
 *   dequant    ahat_b = fl32(q_b * d);  w'_nk = bf16(fl32(c_code * ahat_b))
 *   linear     y_mn = sum_k X_mk w'_nk + b_n  (X bf16; fp64 here)
 *
 * Phi^-1 is found by bisection on Phi(x) = erfc(-x / sqrt 2) / 2 to the
 * last fp64 bit: slow and plain.
 */
static double nf4_phi(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

static double nf4_phi_inv(double p)
{
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 200; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid == lo || mid == hi) break;
        if (nf4_phi(mid) < p) lo = mid;
        else hi = mid;
    }
    return 0.5 * (lo + hi);
}

void oracle_nf4_codebook(float *c)
{
    const double d = (1.0 / 32.0 + 1.0 / 30.0) / 2.0;
    const double top = nf4_phi_inv(1.0 - d);
    c[7] = 0.0f;
    for (int j = 1; j <= 8; ++j) c[7 + j] = (float)(nf4_phi_inv(0.5 + j * (0.5 - d) / 8.0) / top);
    for (int j = 1; j <= 7; ++j) c[7 - j] = (float)(-nf4_phi_inv(0.5 + j * (0.5 - d) / 7.0) / top);
}

/* Code of one normalized weight x (|x| <= 1). */
int oracle_nf4_code(float x, const float *c)
{
    int code = 0;
    for (int i = 0; i < 15; ++i) {
        double mid = ((double)c[i] + (double)c[i + 1]) / 2.0;   /* exact in fp64 */
        if ((double)x > mid || ((double)x == mid && mid < 0.0)) code = i + 1;
    }
    return code;
}

/* Round-half-even of the exact 255 a / s, for 0 <= a <= s, s > 0. */
static int nf4_stat_code(float a, float s)
{
    double num = 255.0 * (double)a;                 /* exact */
    int k = (int)floor(num / (double)s);
    /* settle k exactly: k s <= 255 a < (k + 1) s, each product exact */
    while (k > 0 && (double)k * (double)s > num) --k;
    while ((double)(k + 1) * (double)s <= num) ++k;
    double twice = 2.0 * num, mid = (2.0 * k + 1.0) * (double)s;   /* exact */
    if (twice > mid || (twice == mid && (k & 1))) ++k;
    return k > 255 ? 255 : k;
}

/* W bf16 [N][K], K % 64 == 0 -> codes [N][K/2] (element 2i low nibble),
 * statistic codes [N*K/64], chunk scales [ceil(N*K/64 / 256)]. */
void oracle_nf4_pack(const uint16_t *W, int N, int K, uint8_t *wq, uint8_t *qabs, float *chunk)
{
    float c[16];
    oracle_nf4_codebook(c);
    const int G = K / 64;
    const int64_t nb = (int64_t)N * G;
    float *amax = (float *)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
    for (int n = 0; n < N; ++n) {
        for (int g = 0; g < G; ++g) {
            const uint16_t *w = W + (size_t)n * K + 64 * g;
            float a = 0.0f;
            for (int i = 0; i < 64; ++i) {
                float t = (float)fabs(bf16_val(w[i]));
                if (t > a) a = t;
            }
            amax[(size_t)n * G + g] = a;
            uint8_t *dst = wq + (size_t)n * (K / 2) + 32 * g;
            for (int i = 0; i < 64; i += 2) {
                int c0 = 7, c1 = 7;
                if (a > 0.0f) {
                    c0 = oracle_nf4_code((float)(bf16_val(w[i]) / (double)a), c);
                    c1 = oracle_nf4_code((float)(bf16_val(w[i + 1]) / (double)a), c);
                }
                dst[i / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
    const int64_t nchunk = (nb + 255) / 256;
    for (int64_t ch = 0; ch < nchunk; ++ch) {
        const int64_t b0 = 256 * ch, b1 = b0 + 256 < nb ? b0 + 256 : nb;
        float s = 0.0f;
        for (int64_t b = b0; b < b1; ++b)
            if (amax[b] > s) s = amax[b];
        chunk[ch] = (float)((double)s / 255.0);
        for (int64_t b = b0; b < b1; ++b) qabs[b] = (uint8_t)(s > 0.0f ? nf4_stat_code(amax[b], s) : 0);
    }
    free(amax);
}

static uint16_t bf16_bits_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(u >> 16);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Dequantized weights w' (bf16 bits) [N][K]. */
void oracle_nf4_dequant(const uint8_t *wq, const uint8_t *qabs, const float *chunk, int N, int K, uint16_t *Wd)
{
    float c[16];
    oracle_nf4_codebook(c);
    const int G = K / 64;
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k) {
            const int64_t b = (int64_t)n * G + k / 64;
            const float ahat = (float)((double)qabs[b] * (double)chunk[b / 256]);
            const uint8_t byte = wq[(size_t)n * (K / 2) + k / 2];
            const int code = (k & 1) ? byte >> 4 : byte & 15;
            Wd[(size_t)n * K + k] = bf16_bits_rne((float)((double)c[code] * (double)ahat));
        }
}

/* y = X W'^T + b in fp64 for the listed rows (rows == NULL: all M). */
void oracle_nf4_linear(const uint16_t *X, const uint8_t *wq, const uint8_t *qabs, const float *chunk,
                       const uint16_t *bias, int M, int N, int K, const int *rows, int nrows, double *out)
{
    uint16_t *Wd = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)N * (size_t)K + 2);
    oracle_nf4_dequant(wq, qabs, chunk, N, K, Wd);
    const int R = rows ? nrows : M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < R; ++i) {
        const int m = rows ? rows[i] : i;
        const uint16_t *x = X + (size_t)m * K;
        for (int n = 0; n < N; ++n) {
            const uint16_t *w = Wd + (size_t)n * K;
            double acc = 0.0;
            for (int k = 0; k < K; ++k) acc += bf16_val(x[k]) * bf16_val(w[k]);
            out[(size_t)i * N + n] = acc + (bias ? bf16_val(bias[n]) : 0.0);
        }
    }
    free(Wd);
}
