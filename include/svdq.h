/*
 * svdq.h -- C ABI of libsvdq, an MI355X (gfx950) implementation of the
 * SVDQuant W4A4 linear layer.
 *
 * The layer ("Bringing Nunchaku 4-bit Diffusion Inference to Diffusers",
 * Hugging Face blog, section "Background: SVDQuant and Nunchaku"): a
 * per-channel smoothing moves activation outliers into the weights, the
 * hardest part of each smoothed weight matrix is kept in a small 16-bit
 * low-rank branch, and the residual runs as a 4-bit-weight x 4-bit-activation
 * product.  The low-rank down projection is fused with the activation
 * quantization, and the up projection with the 4-bit product (same section,
 * figure caption).  Section "Native loading in Diffusers" fixes rank 32 and a
 * bfloat16 compute dtype.
 *
 * Notation.  X is bf16 [M][K] (M tokens), W is bf16 [N][K] (nn.Linear
 * layout, out x in), y = X W^T + b.  r = rank = 32.  The 4-bit codes come in
 * groups along K: INT4 (symmetric, 64 wide, fp32 scale) or MXFP4 (E2M1
 * elements, one E8M0 scale per 32).
 *
 * Arithmetic (every step below is what the functions compute):
 *   s_k      = fl32(1 / sqrt(max|X_k| / max_n|W_nk|)), 1 when either max is 0
 *   What_kn  = W_nk / s_k ~ U S V^T (top r)
 *   down     = bf16(s_k (U S)_kj)   stored [r][K]  (K contiguous)
 *   up       = bf16(V_nj)           stored [N][r]  (r contiguous)
 *   residual R_kn = (W_nk - sum_j down[j][k] up[n][j]) / s_k, quantized from
 *            fl32(R) per (n, group)
 *   xhat     = fl32(X_mk s_k), quantized per (m, group);  h = X down^T (fp32)
 *   y        = sum_g sx_mg sw_ng (qx . qw)_g + h up^T + b   [GELU-tanh]  -> bf16
 * INT4 group: a = max|v|, scale = fl32(a / 7) (rounded upward instead of to
 * nearest below the normal fp32 range), code = round-half-even of the exact
 * quotient v / scale (always within [-7, 7]).  MXFP4 block: X = floor(log2 a)
 * - 2 clamped to [-127, 127], E8M0 = X + 127, element = v 2^-X rounded to the
 * E2M1 grid (ties to the even index, saturating at 6, sign kept for zero).
 * Codes are nibble-packed, element 2i in the low nibble of byte i.  Both code
 * formats are sign-magnitude with the sign of the input in bit 3 (kept for
 * zero): INT4 code = sign << 3 | |q|, E2M1 code = sign << 3 | grid index.
 *
 * Layout choices (the pages fix none of them):
 *   - down is stored [r][K] and up [N][r], i.e. both factors transposed
 *     against the textbook L1 [K][r], L2 [r][N]: the activation kernel reads
 *     16 consecutive channels of all 32 ranks as 32-byte runs, and the
 *     product's epilogue reads one output channel's 32 ranks as one 64-byte
 *     line.
 *   - INT4 codes are sign-magnitude, not two's complement: a sign-magnitude
 *     code becomes the exact fp8 (E4M3) byte of q 2^-9 with bit operations
 *     only, which is how the product feeds the matrix cores.
 *   - N % 8 == 0 for the linears: every row of Y, bias and up then starts on
 *     a 16-byte boundary.
 *
 * Conventions.
 *   - Ownership: the caller allocates and frees every buffer.  No call
 *     allocates device memory or keeps a pointer after it returns.
 *   - Device calls (svdq_quantize_act, svdq_w4a4_linear,
 *     svdq_w4a4_linear_requant, svdq_w4a4_linear_splitk,
 *     svdq_w4a4_linear_qkv_norm_rope, svdq_awq_w4a16_linear) take device
 *     pointers and a hipStream_t (as void*, NULL = the null stream); they
 *     validate everything first, enqueue kernels on `stream` and return
 *     without synchronizing.  On any error nothing has been enqueued or
 *     written.  The current HIP device must be a gfx950; otherwise
 *     SVDQ_ERR_UNSUPPORTED_DEVICE is returned and nothing runs.
 *   - Host calls (svdq_pack_weights, svdq_pack_residual,
 *     svdq_awq_pack_weights) take host pointers,
 *     run synchronously on the CPU and need no GPU.
 *   - Device pointers must be 16-byte aligned (SVDQ_ERR_MISALIGNED).  A
 *     buffer whose size is zero (M == 0 or N == 0) may be NULL.
 *   - Inputs are expected finite; the device calls do not check the values
 *     of X (non-finite X gives unspecified codes).
 *   - Every function is thread-safe.  Calls that overlap on one stream are
 *     ordered by the stream; calls on different streams that share output
 *     buffers race, as with any kernel.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum svdq_status {
    SVDQ_OK = 0,
    SVDQ_ERR_INVALID_ARG = -1,        /* NULL pointer, bad enum value, negative size */
    SVDQ_ERR_SHAPE = -2,              /* a size not the multiple the call requires (K of the group, N of 8, ...),
                                         or a matrix of SVDQ_MAX_ELEMENTS elements or more */
    SVDQ_ERR_MISALIGNED = -3,         /* a device pointer not 16-byte aligned */
    SVDQ_ERR_UNSUPPORTED = -4,        /* rank other than 32, or a precision / K the call does not support */
    SVDQ_ERR_UNSUPPORTED_DEVICE = -5, /* no HIP device, or the current device is not gfx950 */
    SVDQ_ERR_NONFINITE = -6,          /* non-finite weight or calibration statistic (pack) */
    SVDQ_ERR_HIP = -7,                /* a HIP runtime or launch failure */
    SVDQ_ERR_SCRATCH = -8,            /* the allocation-free call needs more than SVDQ_NOALLOC_SCRATCH_BYTES */
    SVDQ_STATUS_INT_RANGE_ = 0x7FFFFFFF   /* not a status: makes every int a valid value of the type */
} svdq_status;

typedef enum svdq_precision {
    SVDQ_INT4 = 0,   /* symmetric INT4, 64-wide groups, fp32 scales  [rows][K/64] */
    SVDQ_MXFP4 = 1,  /* E2M1, 32-wide blocks, E8M0 scales (uint8)    [rows][K/32] */
    SVDQ_PRECISION_INT_RANGE_ = 0x7FFFFFFF   /* not a precision: every int is a valid value (calls reject it) */
} svdq_precision;

typedef enum svdq_epilogue {
    SVDQ_EPI_NONE = 0,
    SVDQ_EPI_GELU_TANH = 1, /* 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))) after the bias */
    SVDQ_EPILOGUE_INT_RANGE_ = 0x7FFFFFFF    /* not an epilogue: every int is a valid value (calls reject it) */
} svdq_epilogue;

#define SVDQ_RANK 32

/* Every matrix a call touches (M x K, N x K, M x N) must hold fewer than
 * this many elements (SVDQ_ERR_SHAPE otherwise), so that every byte offset
 * inside one buffer fits in 31 bits. */
#define SVDQ_MAX_ELEMENTS (1 << 30)

/* Human-readable text of a status code (static storage, never NULL). */
const char *svdq_status_string(svdq_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int svdq_version(void);

/* SVDQ_OK when the current HIP device is a gfx950, else
 * SVDQ_ERR_UNSUPPORTED_DEVICE.  Mirrors the capability check the pages
 * describe ("Hardware support": the quantizer validates the GPU at load time
 * and raises a clear error instead of producing incorrect outputs). */
svdq_status svdq_check_device(void);

/*
 * svdq_pack_weights -- host-side packing of one linear layer
 * ("Background: SVDQuant and Nunchaku": smoothing, low-rank branch,
 * 4-bit residual; "Native loading in Diffusers": rank 32).
 *
 *   W          [N][K] bf16 bits (nn.Linear weight, out x in), host
 *   act_absmax [K] fp32, per-channel max |X| from calibration (>= 0), host
 *   N, K       N >= 1; K >= group and K % group == 0 (group 64 INT4, 32 MXFP4)
 *   rank       must be 32
 *   prec       SVDQ_INT4 or SVDQ_MXFP4
 * Outputs (host, caller-allocated):
 *   smooth     [K] fp32                       s_k
 *   down       [rank][K] bf16 bits            bf16(s_k (U S)_kj)
 *   up         [N][rank] bf16 bits            bf16(V_nj)
 *   wq         [N][K/2] uint8                 packed residual codes
 *   wscale     INT4: [N][K/64] fp32; MXFP4: [N][K/32] uint8 (E8M0)
 * The top-r SVD is a randomized subspace iteration in fp64 with a
 * Rayleigh-Ritz step (not bit-reproducible against other SVD codes; signs:
 * the largest-|.| entry of each right singular vector is positive).  Columns
 * beyond the rank of the smoothed weight come out as zero.  Errors:
 * SVDQ_ERR_INVALID_ARG, SVDQ_ERR_SHAPE, SVDQ_ERR_UNSUPPORTED, SVDQ_ERR_NONFINITE
 * (any non-finite W, or a negative / non-finite act_absmax).  Uses all host
 * cores (std::thread); outputs are deterministic.
 */
svdq_status svdq_pack_weights(const uint16_t *W, const float *act_absmax, int N, int K, int rank,
                              svdq_precision prec, float *smooth, uint16_t *down, uint16_t *up,
                              uint8_t *wq, void *wscale);

/*
 * svdq_pack_residual -- the residual step of svdq_pack_weights alone, for
 * caller-supplied smoothing and low-rank factors (same layouts as above):
 * R_kn = (W_nk - sum_j down[j][k] up[n][j]) / smooth_k in fp64, j ascending,
 * then fl32(R) quantized per (n, group).  Host, synchronous.  Errors as for
 * svdq_pack_weights (smooth must be finite and non-zero).
 */
svdq_status svdq_pack_residual(const uint16_t *W, const float *smooth, const uint16_t *down,
                               const uint16_t *up, int N, int K, int rank, svdq_precision prec,
                               uint8_t *wq, void *wscale);

/*
 * svdq_quantize_act -- fused activation step: smoothing, per-group absmax,
 * 4-bit quantization with nibble packing, and the rank-32 down projection
 * h = X down^T in the same pass over X ("Background: SVDQuant and Nunchaku":
 * the low-rank down projection is fused with the quantization kernel).
 *
 *   X        [M][K] bf16 bits, device          M >= 0 (M == 0: no-op)
 *   smooth   [K] fp32, device
 *   down     [rank][K] bf16 bits, device
 *   xq       [M][K/2] uint8, device (out)
 *   xscale   INT4: [M][K/64] fp32; MXFP4: [M][K/32] uint8, device (out)
 *   h        [M][rank] fp32, device (out)      fp32 accumulation of bf16 products
 *   stream   hipStream_t or NULL
 * Codes and scales are bit-exact with the definition above.  One kernel
 * launch.  Errors: SVDQ_ERR_INVALID_ARG, SVDQ_ERR_SHAPE (K % group),
 * SVDQ_ERR_UNSUPPORTED (rank), SVDQ_ERR_MISALIGNED, SVDQ_ERR_UNSUPPORTED_DEVICE,
 * SVDQ_ERR_HIP.
 */
svdq_status svdq_quantize_act(const uint16_t *X, int M, int K, const float *smooth,
                              const uint16_t *down, int rank, svdq_precision prec, uint8_t *xq,
                              void *xscale, float *h, void *stream);

/*
 * svdq_w4a4_linear -- the 4-bit product with the fused low-rank up
 * projection, bias, optional GELU-tanh and bf16 store ("Background: SVDQuant
 * and Nunchaku": the up projection is fused with the 4-bit compute kernel;
 * "Introducing Nunchaku Lite": fused GELU/MLP paths).
 *
 *   xq, xscale, h   as written by svdq_quantize_act (device)
 *   wq, wscale      as written by svdq_pack_weights (device copies)
 *   up              [N][rank] bf16 bits (device)
 *   bias            [N] bf16 bits (device) or NULL
 *   M, N, K         M >= 0, N >= 0 (either 0: no-op), N % 8 == 0, K % group == 0
 *   epi             SVDQ_EPI_NONE or SVDQ_EPI_GELU_TANH
 *   Y               [M][N] bf16 bits (device, out), round-to-nearest-even
 * INT4: per 64-group exact integer partial products from the matrix
 * cores (each code enters the fp8 matrix instruction as an exact E4M3
 * value); the group scale sx * sw of each output comes from the bf16 matrix
 * instruction on high/low bf16 splits of both scales (relative error about
 * 2^-16) and multiplies the exact partial in one fp32 fma.  MXFP4: the
 * scaled f8f6f4 matrix instruction applies both E8M0 scales.  The low-rank
 * term uses h split into a bf16 high and low part and accumulates onto the
 * 4-bit term on the matrix cores; the bias enters there too, exactly, as
 * one more bf16 product (the bias row against a column of ones).  One kernel
 * launch;
 * for INT4, two when the tiles left after whole rounds of one block per CU
 * are few: those tiles are then computed in 64 x 64 pieces with K split
 * across a block's waves and the partial sums added in a fixed order (so
 * their outputs may differ in low bf16 places from what the one-launch form
 * gives for the same rows; results are deterministic for a given shape).
 * Errors as for svdq_quantize_act.
 */
svdq_status svdq_w4a4_linear(const uint8_t *xq, const void *xscale, const float *h,
                             const uint8_t *wq, const void *wscale, const uint16_t *up,
                             const uint16_t *bias, int M, int N, int K, int rank,
                             svdq_precision prec, svdq_epilogue epi, uint16_t *Y, void *stream);

/*
 * svdq_w4a4_linear_splitk_workspace_bytes -- device workspace that
 * svdq_w4a4_linear_splitk needs on the current device: S * M * N fp32
 * partial sums when the MXFP4 product is split into S slices of K (S of 2
 * to 4; every slice but the last at least 1024 channels), else 0 (INT4,
 * shapes whose 256 x 256 tiles already fill half the chip, K < 2048 or
 * K % 256 != 0, M or N <= 0, invalid arguments, or no gfx950 device).
 * It depends on the device's compute-unit count.
 */
size_t svdq_w4a4_linear_splitk_workspace_bytes(int M, int N, int K, svdq_precision prec);

/*
 * svdq_w4a4_linear_splitk -- svdq_w4a4_linear for skinny shapes (few
 * tokens, long K, such as the MLP's second linear of a 512 x 512 image:
 * 1024 x 12288 -> 3072), where the product's tiles would leave most of the
 * chip idle.  Same arguments, arithmetic and output as svdq_w4a4_linear,
 * plus:
 *   work, work_bytes  device scratch of at least
 *                     svdq_w4a4_linear_splitk_workspace_bytes(M, N, K,
 *                     prec) bytes, 16-byte aligned (may be NULL when that
 *                     is 0); overwritten, caller-owned
 * With a split, each of S work items per tile sums its K slice into the
 * workspace in fp32, and a second kernel adds the S slices in slice order
 * (so the result is deterministic) before the epilogue; slice 0 adds the
 * low-rank term with the same bf16 high/low matrix product as the unsplit
 * epilogue, and the bias is added in fp32 after the slices.  Sums in a different
 * order than svdq_w4a4_linear's, so outputs may differ from it in the last
 * bf16 place.  Without a split it is svdq_w4a4_linear.  Errors as for
 * svdq_w4a4_linear, and SVDQ_ERR_INVALID_ARG for a NULL or too small work
 * (checked after the device, whose compute units set the size).
 */
svdq_status svdq_w4a4_linear_splitk(const uint8_t *xq, const void *xscale, const float *h,
                                    const uint8_t *wq, const void *wscale, const uint16_t *up,
                                    const uint16_t *bias, int M, int N, int K, int rank,
                                    svdq_precision prec, svdq_epilogue epi, uint16_t *Y, void *work,
                                    size_t work_bytes, void *stream);

/* Size of the library's static device scratch buffer (one per GPU, held
 * until the process ends), used by svdq_w4a4_linear_splitk_noalloc. */
#define SVDQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * svdq_w4a4_linear_splitk_noalloc -- svdq_w4a4_linear_splitk for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments,
 * kernels and results, without `work`: the split-K slice sums go to a
 * static device buffer of SVDQ_NOALLOC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on.  The call itself allocates nothing (its first call
 * on a device looks up that device's buffer address once).
 *   - Shapes whose split needs more than SVDQ_NOALLOC_SCRATCH_BYTES
 *     (svdq_w4a4_linear_splitk_workspace_bytes) return SVDQ_ERR_SCRATCH and
 *     enqueue nothing.
 *   - Every call on one GPU shares that GPU's buffer: calls that overlap in
 *     time on one GPU (different streams, or different threads without
 *     ordering) race and give undefined results; calls on one stream are
 *     ordered and safe.  The buffer keeps the last call's contents; every
 *     call writes what it reads, so nothing needs clearing.
 * Errors as for svdq_w4a4_linear_splitk (without the workspace ones), plus
 * SVDQ_ERR_SCRATCH.
 */
svdq_status svdq_w4a4_linear_splitk_noalloc(const uint8_t *xq, const void *xscale, const float *h,
                                            const uint8_t *wq, const void *wscale, const uint16_t *up,
                                            const uint16_t *bias, int M, int N, int K, int rank,
                                            svdq_precision prec, svdq_epilogue epi, uint16_t *Y, void *stream);

/*
 * svdq_requant_workspace_bytes -- device workspace that
 * svdq_w4a4_linear_requant needs for M tokens and N output channels
 * (ceil(N / 256) * M * rank fp32 partial sums); 0 for M or N <= 0.
 */
size_t svdq_requant_workspace_bytes(int M, int N, int rank, svdq_precision prec);

/*
 * svdq_w4a4_linear_requant -- svdq_w4a4_linear feeding the next layer's
 * activation step directly (an MLP's fc1 -> fc2, "Introducing Nunchaku
 * Lite": fused GELU/MLP paths): Y is not stored.  Each output is rounded to
 * bf16 exactly as svdq_w4a4_linear would store it, then smoothed with the
 * next layer's `smooth2`, quantized per group of consecutive output channels
 * (64 INT4, 32 MXFP4), and multiplied into the next layer's `down2`.  The
 * results are those of svdq_quantize_act(Y, M, N, smooth2, down2, ...) on
 * that Y: codes and scales bit-exact, h2 up to the order of the fp32 sums
 * (per-tile partial sums over 256 channels, added in ascending tile order,
 * so h2 is deterministic).
 *
 *   xq ... epi   as for svdq_w4a4_linear; `prec` is that of both layers.
 *                MXFP4 needs K % 256 == 0 (SVDQ_ERR_UNSUPPORTED otherwise)
 *   N            N % 64 == 0 (the next layer's K)
 *   smooth2      [N] fp32, device                  next layer's s
 *   down2        [rank][N] bf16 bits, device       next layer's down
 *   xq2          [M][N/2] uint8, device (out)
 *   xscale2      INT4: [M][N/64] fp32; MXFP4: [M][N/32] uint8 (E8M0), device (out)
 *   h2           [M][rank] fp32, device (out)
 *   work         device scratch of at least svdq_requant_workspace_bytes(M,
 *                N, rank, prec) bytes, caller-owned; its contents on entry
 *                do not matter and are overwritten
 *   stream       hipStream_t or NULL
 * Two kernel launches on `stream` (the product with this epilogue, then the
 * fixed-order sum of the partial h2).  Errors: as for svdq_w4a4_linear;
 * SVDQ_ERR_SHAPE when N % 64 != 0; SVDQ_ERR_UNSUPPORTED for MXFP4 with
 * K % 256 != 0; SVDQ_ERR_INVALID_ARG when work_bytes is too small.
 */
svdq_status svdq_w4a4_linear_requant(const uint8_t *xq, const void *xscale, const float *h,
                                     const uint8_t *wq, const void *wscale, const uint16_t *up,
                                     const uint16_t *bias, int M, int N, int K, int rank,
                                     svdq_precision prec, svdq_epilogue epi, const float *smooth2,
                                     const uint16_t *down2, uint8_t *xq2, void *xscale2, float *h2,
                                     void *work, size_t work_bytes, void *stream);

/*
 * svdq_w4a4_linear_qkv_norm_rope -- svdq_w4a4_linear for a fused QKV
 * projection whose epilogue also applies the Q/K RMS-norm and the rotary
 * embedding ("Quantizing models with structural rewrites": the Nunchaku
 * engine's fused operator consumes the QKV projection, the Q/K normalization
 * and the rotary embeddings together).
 *
 *   xq ... bias  as for svdq_w4a4_linear; no GELU.  MXFP4 needs
 *                K % 256 == 0 (SVDQ_ERR_UNSUPPORTED otherwise)
 *   N            3 H 128 (SVDQ_ERR_SHAPE otherwise): channels [0, 128 H) are
 *                the Q heads, then H K heads, then H V heads, 128 each
 *   norm_q       [128] bf16 bits, device   RMS-norm weight of every Q head
 *   norm_k       [128] bf16 bits, device   RMS-norm weight of every K head
 *   eps          finite, >= 0 (SVDQ_ERR_INVALID_ARG otherwise)
 *   rope_cos     [M][64] fp32, device      cos of token m's angle for pair p
 *   rope_sin     [M][64] fp32, device      sin of the same angle
 *   Y            [M][N] bf16 bits, device (out)
 * With yb = the bf16 value svdq_w4a4_linear would store: V channels get yb;
 * a Q or K head gets u_d = yb_d / sqrt(mean_d(yb_d^2) + eps) * w_d (fp32),
 * then out_2p = u_2p cos_mp - u_2p+1 sin_mp, out_2p+1 = u_2p+1 cos_mp +
 * u_2p sin_mp, rounded to bf16 (round-to-nearest-even).  One kernel launch
 * (for INT4 two, with the leftover tiles in pieces, exactly when
 * svdq_w4a4_linear takes two at the same shape; yb is then that call's).
 * Errors as for svdq_w4a4_linear, plus the ones above.
 */
svdq_status svdq_w4a4_linear_qkv_norm_rope(const uint8_t *xq, const void *xscale, const float *h,
                                           const uint8_t *wq, const void *wscale, const uint16_t *up,
                                           const uint16_t *bias, int M, int N, int K, int rank,
                                           svdq_precision prec, const uint16_t *norm_q, const uint16_t *norm_k,
                                           float eps, const float *rope_cos, const float *rope_sin, uint16_t *Y,
                                           void *stream);

/*
 * svdq_awq_pack_weights -- host packing for the weight-only AWQ W4A16 layer
 * ("Native loading in Diffusers": the awq_w4a16 family, int4 with group size
 * 64, used for modulation layers, which are memory-bound and
 * precision-sensitive).  The activation-aware channel scaling of AWQ is a
 * calibration step; a caller that uses it passes the already scaled weight.
 *
 *   W        [N][K] bf16 bits, host            N >= 1, K >= 256, K % 256 == 0
 *   wq       [N][K/2] uint8, host (out)        codes q + 8, q in [-7, 7]
 *   wscale   [N][K/64] fp32, host (out)
 * q and the scale are the INT4 group quantizer of the header comment applied
 * to fl32(W) per (n, 64-group along k).  Storage order (the operand order of
 * the device kernel): in the 256-channel chunk C of a row, the 32 bytes at
 * 128 C + 32 b are 8 little-endian dwords d = 2 g + h; nibble j of dword d is
 * channel 256 C + 64 g + 32 h + 8 b + 2 j for j < 4 and + 2 (j - 4) + 1 for
 * j >= 4.  Host, synchronous, all host cores; errors SVDQ_ERR_INVALID_ARG,
 * SVDQ_ERR_SHAPE, SVDQ_ERR_NONFINITE (any non-finite W).
 */
svdq_status svdq_awq_pack_weights(const uint16_t *W, int N, int K, uint8_t *wq, float *wscale);

/*
 * svdq_awq_w4a16_linear -- y = X Wdq^T + b with Wdq_nk = wscale_ng q_nk and
 * bf16 activations (the awq_w4a16 runtime layer).
 *
 *   X        [M][K] bf16 bits, device          M >= 0 (0: no-op)
 *   wq, wscale   as written by svdq_awq_pack_weights (device copies)
 *   bias     [N] bf16 bits, device, or NULL
 *   N, K     N >= 0 (0: no-op), K >= 256, K % 256 == 0
 *   Y        [M][N] bf16 bits, device (out), round-to-nearest-even of the
 *            fp32 result
 *   stream   hipStream_t or NULL
 * Sums in fp32 on the bf16 matrix cores (each 64-channel group exactly, then
 * scaled once); the kernel streams the weights once per 16 rows of X, so it
 * is meant for the few rows of a modulation input.  One kernel launch.
 * Errors: SVDQ_ERR_INVALID_ARG, SVDQ_ERR_SHAPE (K), SVDQ_ERR_MISALIGNED,
 * SVDQ_ERR_UNSUPPORTED_DEVICE, SVDQ_ERR_HIP.
 */
svdq_status svdq_awq_w4a16_linear(const uint16_t *X, const uint8_t *wq, const float *wscale,
                                  const uint16_t *bias, int M, int N, int K, uint16_t *Y, void *stream);

/*
 * NF4 weight-only W4A16 layer -- the pages' comparison system
 * ("BitsAndBytes W4 Quantization", sections "Overview" and "Parameters":
 * BF16 weights quantized at load time to the 4-bit "nf4" data type,
 * activations kept in bf16; compress_statistics double-quantizes the block
 * scaling statistics).
 *
 * Format.  Levels: 16 fp32 quantiles of the standard normal distribution
 * normalized to [-1, 1] with an exact zero (svdq_nf4_codebook).  A block is
 * 64 consecutive weights of a row, with absmax a (fp32); a weight's code is
 * the level nearest to fl32(w / a) (a tie goes to the level of smaller
 * magnitude; a == 0 gives the zero level, code 7).  The block absmaxes, in
 * row-major (n, block) order, are double-quantized in chunks of 256: s =
 * max a over the chunk, the chunk stores d = fl32(s / 255) and block b stores
 * q_b = round-half-even of 255 a_b / s.  Dequantized weight:
 *   ahat_b = fl32(q_b * d),   w' = bf16(fl32(level[code] * ahat_b)).
 */

/* The 16 NF4 levels, ascending (level 7 is 0, levels 0 and 15 are -1 and 1);
 * host, writes 16 floats.  Error: SVDQ_ERR_INVALID_ARG for NULL. */
svdq_status svdq_nf4_codebook(float *levels);

/*
 * svdq_nf4_pack_weights -- host packing of one weight for the NF4 layer.
 *   W            [N][K] bf16 bits, host            N >= 1, K >= 64, K % 64 == 0
 *   wq           [N][K/2] uint8, host (out)        codes; in each group of 8
 *                consecutive weights of a row, byte i holds weight i (low
 *                nibble) and weight i + 4 (high nibble)
 *   qabs         [N K / 64] uint8, host (out)      statistic codes, (n, block) order
 *   chunk_scale  [ceil(N K / 64 / 256)] fp32, host (out)   d of each chunk
 * Synchronous, all host cores.  Errors: SVDQ_ERR_INVALID_ARG,
 * SVDQ_ERR_SHAPE, SVDQ_ERR_NONFINITE (any non-finite W).
 */
svdq_status svdq_nf4_pack_weights(const uint16_t *W, int N, int K, uint8_t *wq, uint8_t *qabs,
                                  float *chunk_scale);

/*
 * svdq_nf4_dequantize -- the dequantized weights w' as bf16 [N][K] (device),
 * from device copies of svdq_nf4_pack_weights' outputs.  One kernel launch
 * on `stream`.  Errors: SVDQ_ERR_INVALID_ARG, SVDQ_ERR_SHAPE (K),
 * SVDQ_ERR_MISALIGNED, SVDQ_ERR_UNSUPPORTED_DEVICE, SVDQ_ERR_HIP.
 */
svdq_status svdq_nf4_dequantize(const uint8_t *wq, const uint8_t *qabs, const float *chunk_scale, int N, int K,
                                uint16_t *Wd, void *stream);

/*
 * svdq_nf4_w4a16_linear -- y = X W'^T + b, W' dequantized inside the kernel
 * (the same w' as svdq_nf4_dequantize), sums in fp32 on the bf16 matrix
 * cores, rounded once to bf16 (round-to-nearest-even).
 *   X            [M][K] bf16 bits, device          M >= 0 (0: no-op)
 *   wq, qabs, chunk_scale   device copies of svdq_nf4_pack_weights' outputs
 *   bias         [N] bf16 bits, device, or NULL
 *   N, K         N >= 0 (0: no-op), N % 8 == 0; K >= 64, K % 64 == 0
 *   Y            [M][N] bf16 bits, device (out)
 * One kernel launch.  Errors: SVDQ_ERR_INVALID_ARG, SVDQ_ERR_SHAPE,
 * SVDQ_ERR_MISALIGNED, SVDQ_ERR_UNSUPPORTED_DEVICE, SVDQ_ERR_HIP.
 */
svdq_status svdq_nf4_w4a16_linear(const uint16_t *X, const uint8_t *wq, const uint8_t *qabs,
                                  const float *chunk_scale, const uint16_t *bias, int M, int N, int K, uint16_t *Y,
                                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
