// svdq_internal.h -- declarations shared between the C-ABI layer and the
// kernel translation units of libsvdq (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq.h"

namespace svdq {

int group_size(svdq_precision prec);

// Every matrix a call touches (M x K, N x K, M x N) must hold fewer than
// SVDQ_MAX_ELEMENTS elements, so every byte offset inside one buffer fits in
// 31 bits: the LDS-DMA loads take 32-bit lane offsets and the host loops
// index rows with int products.
inline bool elems_ok(int64_t rows, int64_t cols) { return rows * cols < (int64_t)SVDQ_MAX_ELEMENTS; }

// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count();

// Kernel launchers; arguments are already validated.  They return the HIP
// status of the launch.
hipError_t launch_quant_act(const uint16_t *X, int M, int K, const float *smooth, const uint16_t *down,
                            svdq_precision prec, uint8_t *xq, void *xscale, float *h, hipStream_t stream);

hipError_t launch_w4a4_linear(const uint8_t *xq, const void *xscale, const float *h, const uint8_t *wq,
                              const void *wscale, const uint16_t *up, const uint16_t *bias, int M, int N,
                              int K, svdq_precision prec, svdq_epilogue epi, uint16_t *Y,
                              hipStream_t stream);

// Fused requantization: the product's epilogue writes the next layer's
// codes, scales and h instead of Y.  `work` holds the per-tile partial h
// (requant_work_bytes(M, N) bytes).  MXFP4 runs on the LDS-DMA kernel only
// (requant_supported).
size_t requant_work_bytes(int M, int N);
bool requant_supported(int M, int N, int K, svdq_precision prec);
hipError_t launch_w4a4_linear_requant(const uint8_t *xq, const void *xscale, const float *h, const uint8_t *wq,
                                      const void *wscale, const uint16_t *up, const uint16_t *bias, int M, int N,
                                      int K, svdq_precision prec, svdq_epilogue epi, const float *smooth2,
                                      const uint16_t *down2, uint8_t *xq2, void *xscale2, float *h2, float *work,
                                      hipStream_t stream);

// Split K for the MXFP4 linear when its 256 x 256 tiles fill less than half
// of the chip: S slices of K (S = 1: no split; `sps` steps of 256 channels
// per slice), fp32 partial sums in `work` (splitk_work_bytes, 0 without a
// split), then a fixed-order sum with the epilogue.  Without a split the
// launch is launch_w4a4_linear's.
int splitk_slices(int M, int N, int K, svdq_precision prec, int &sps);
size_t splitk_work_bytes(int M, int N, int K, svdq_precision prec);
hipError_t launch_w4a4_linear_splitk(const uint8_t *xq, const void *xscale, const float *h, const uint8_t *wq,
                                     const void *wscale, const uint16_t *up, const uint16_t *bias, int M, int N,
                                     int K, svdq_precision prec, svdq_epilogue epi, uint16_t *Y, float *work,
                                     hipStream_t stream);

// Linear of a QKV projection (N = 3 H 128) whose epilogue RMS-normalizes the
// Q and K heads and applies the rotary embedding.  MXFP4 runs on the LDS-DMA
// kernel only (requant_supported gives its range).
hipError_t launch_w4a4_linear_qknorm(const uint8_t *xq, const void *xscale, const float *h, const uint8_t *wq,
                                     const void *wscale, const uint16_t *up, const uint16_t *bias, int M, int N,
                                     int K, svdq_precision prec, const uint16_t *norm_q, const uint16_t *norm_k,
                                     float eps, const float *rope_cos, const float *rope_sin, uint16_t *Y,
                                     hipStream_t stream);

// Weight-only AWQ W4A16 layer (K % 256 == 0).
hipError_t launch_awq_linear(const uint16_t *X, const uint8_t *wq, const float *wscale, const uint16_t *bias,
                             int M, int N, int K, uint16_t *Y, hipStream_t stream);

// Weight-only NF4 W4A16 layer: the 16 fp32 levels (computed once on the
// host), the dequantization kernel and the linear.
struct Nf4Levels {
    float c[16];
};
const float *nf4_codebook_cached();
hipError_t launch_nf4_dequant(const uint8_t *wq, const uint8_t *qabs, const float *chunk, int N, int K,
                              const Nf4Levels &lv, uint16_t *Wd, hipStream_t stream);
hipError_t launch_nf4_linear(const uint16_t *X, const uint8_t *wq, const uint8_t *qabs, const float *chunk,
                             const uint16_t *bias, int M, int N, int K, const Nf4Levels &lv, uint16_t *Y,
                             hipStream_t stream);

}  // namespace svdq
