// api.hip -- the C-ABI entry points of libsvdq that run on the GPU, plus the
// status helpers.  Each device call validates its arguments and the current
// device before enqueuing anything ("Bringing Nunchaku 4-bit Diffusion
// Inference to Diffusers", section "Hardware support": the GPU is validated
// and a clear error is raised instead of producing incorrect outputs).
#include <atomic>
#include <cstring>
#include <mutex>

#include "svdq.h"
#include "svdq_internal.h"

namespace svdq {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

svdq_status current_device_ok()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return SVDQ_ERR_UNSUPPORTED_DEVICE;
    }
    if (dev >= kMaxDevices) return SVDQ_ERR_UNSUPPORTED_DEVICE;
    int st = g_device_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return SVDQ_ERR_UNSUPPORTED_DEVICE;
        }
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_device_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED_DEVICE;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

svdq_status check_common(int M, int K, int rank, svdq_precision prec)
{
    if (prec != SVDQ_INT4 && prec != SVDQ_MXFP4) return SVDQ_ERR_INVALID_ARG;
    if (M < 0 || K < 0) return SVDQ_ERR_INVALID_ARG;
    if (rank != SVDQ_RANK) return SVDQ_ERR_UNSUPPORTED;
    const int g = group_size(prec);
    if (K < g || K % g != 0) return SVDQ_ERR_SHAPE;
    if (!elems_ok(M, K)) return SVDQ_ERR_SHAPE;
    return SVDQ_OK;
}

// the weight and output matrices of a linear
svdq_status check_linear_sizes(int M, int N, int K)
{
    return elems_ok(N, K) && elems_ok(M, N) ? SVDQ_OK : SVDQ_ERR_SHAPE;
}

}  // namespace

int device_cu_count()
{
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace svdq

using namespace svdq;

extern "C" const char *svdq_status_string(svdq_status status)
{
    switch (status) {
    case SVDQ_OK: return "ok";
    case SVDQ_ERR_INVALID_ARG: return "invalid argument (NULL pointer, bad enum or negative size)";
    case SVDQ_ERR_SHAPE:
        return "unsupported shape (a size is not the multiple the call requires: K of the group size, N of 8, ...)";
    case SVDQ_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case SVDQ_ERR_UNSUPPORTED:
        return "unsupported configuration (rank other than 32, or a precision or K the call does not support)";
    case SVDQ_ERR_UNSUPPORTED_DEVICE: return "no HIP device, or the current device is not a gfx950 (MI355X)";
    case SVDQ_ERR_NONFINITE: return "non-finite weight, calibration statistic or smoothing factor";
    case SVDQ_ERR_HIP: return "HIP runtime or kernel launch failure";
    case SVDQ_ERR_SCRATCH:
        return "the call needs more scratch memory than the library's static buffer holds (SVDQ_NOALLOC_SCRATCH_BYTES)";
    case SVDQ_STATUS_INT_RANGE_: break;    // not a status: it only sizes the enum
    }
    return "unknown status";
}

extern "C" int svdq_version(void) { return 100; }

extern "C" svdq_status svdq_check_device(void) { return current_device_ok(); }

extern "C" svdq_status svdq_quantize_act(const uint16_t *X, int M, int K, const float *smooth,
                                         const uint16_t *down, int rank, svdq_precision prec, uint8_t *xq,
                                         void *xscale, float *h, void *stream)
{
    svdq_status st = check_common(M, K, rank, prec);
    if (st != SVDQ_OK) return st;
    // buffers of zero size may be NULL (empty tensors have no storage)
    if (!smooth || !down || (M > 0 && (!X || !xq || !xscale || !h))) return SVDQ_ERR_INVALID_ARG;
    if (!aligned16(X) || !aligned16(smooth) || !aligned16(down) || !aligned16(xq) || !aligned16(xscale) ||
        !aligned16(h))
        return SVDQ_ERR_MISALIGNED;
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    hipError_t e = launch_quant_act(X, M, K, smooth, down, prec, xq, xscale, h, (hipStream_t)stream);
    return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

extern "C" svdq_status svdq_w4a4_linear(const uint8_t *xq, const void *xscale, const float *h,
                                        const uint8_t *wq, const void *wscale, const uint16_t *up,
                                        const uint16_t *bias, int M, int N, int K, int rank,
                                        svdq_precision prec, svdq_epilogue epi, uint16_t *Y, void *stream)
{
    svdq_status st = check_common(M, K, rank, prec);
    if (st != SVDQ_OK) return st;
    if (N < 0) return SVDQ_ERR_INVALID_ARG;
    if (epi != SVDQ_EPI_NONE && epi != SVDQ_EPI_GELU_TANH) return SVDQ_ERR_INVALID_ARG;
    if (N % 8 != 0) return SVDQ_ERR_SHAPE;
    if (check_linear_sizes(M, N, K) != SVDQ_OK) return SVDQ_ERR_SHAPE;
    // buffers of zero size may be NULL (empty tensors have no storage)
    if ((M > 0 && (!xq || !xscale || !h)) || (N > 0 && (!wq || !wscale || !up)) ||
        (M > 0 && N > 0 && !Y))
        return SVDQ_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(xscale) || !aligned16(h) || !aligned16(wq) || !aligned16(wscale) ||
        !aligned16(up) || !aligned16(Y) || (bias && !aligned16(bias)))
        return SVDQ_ERR_MISALIGNED;
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0 || N == 0) return SVDQ_OK;
    hipError_t e = launch_w4a4_linear(xq, xscale, h, wq, wscale, up, bias, M, N, K, prec, epi, Y,
                                      (hipStream_t)stream);
    return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

extern "C" size_t svdq_w4a4_linear_splitk_workspace_bytes(int M, int N, int K, svdq_precision prec)
{
    if (M <= 0 || N <= 0 || K <= 0 || (prec != SVDQ_INT4 && prec != SVDQ_MXFP4)) return 0;
    if (K % group_size(prec) != 0) return 0;
    if (!elems_ok(M, K) || check_linear_sizes(M, N, K) != SVDQ_OK) return 0;
    if (current_device_ok() != SVDQ_OK) return 0;       // the split depends on the device's CU count
    return splitk_work_bytes(M, N, K, prec);
}

extern "C" svdq_status svdq_w4a4_linear_splitk(const uint8_t *xq, const void *xscale, const float *h,
                                               const uint8_t *wq, const void *wscale, const uint16_t *up,
                                               const uint16_t *bias, int M, int N, int K, int rank,
                                               svdq_precision prec, svdq_epilogue epi, uint16_t *Y, void *work,
                                               size_t work_bytes, void *stream)
{
    svdq_status st = check_common(M, K, rank, prec);
    if (st != SVDQ_OK) return st;
    if (N < 0) return SVDQ_ERR_INVALID_ARG;
    if (epi != SVDQ_EPI_NONE && epi != SVDQ_EPI_GELU_TANH) return SVDQ_ERR_INVALID_ARG;
    if (N % 8 != 0) return SVDQ_ERR_SHAPE;
    if (check_linear_sizes(M, N, K) != SVDQ_OK) return SVDQ_ERR_SHAPE;
    if ((M > 0 && (!xq || !xscale || !h)) || (N > 0 && (!wq || !wscale || !up)) ||
        (M > 0 && N > 0 && !Y))
        return SVDQ_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(xscale) || !aligned16(h) || !aligned16(wq) || !aligned16(wscale) ||
        !aligned16(up) || !aligned16(Y) || (bias && !aligned16(bias)) || (work && !aligned16(work)))
        return SVDQ_ERR_MISALIGNED;
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0 || N == 0) return SVDQ_OK;
    const size_t need = splitk_work_bytes(M, N, K, prec);
    if (need > 0 && (!work || work_bytes < need)) return SVDQ_ERR_INVALID_ARG;
    hipError_t e = launch_w4a4_linear_splitk(xq, xscale, h, wq, wscale, up, bias, M, N, K, prec, epi, Y,
                                             (float *)work, (hipStream_t)stream);
    return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

extern "C" size_t svdq_requant_workspace_bytes(int M, int N, int rank, svdq_precision prec)
{
    (void)rank;
    (void)prec;
    if (M <= 0 || N <= 0) return 0;
    return requant_work_bytes(M, N);
}

extern "C" svdq_status svdq_w4a4_linear_requant(const uint8_t *xq, const void *xscale, const float *h,
                                                const uint8_t *wq, const void *wscale, const uint16_t *up,
                                                const uint16_t *bias, int M, int N, int K, int rank,
                                                svdq_precision prec, svdq_epilogue epi, const float *smooth2,
                                                const uint16_t *down2, uint8_t *xq2, void *xscale2, float *h2,
                                                void *work, size_t work_bytes, void *stream)
{
    svdq_status st = check_common(M, K, rank, prec);
    if (st != SVDQ_OK) return st;
    if (N < 0) return SVDQ_ERR_INVALID_ARG;
    if (epi != SVDQ_EPI_NONE && epi != SVDQ_EPI_GELU_TANH) return SVDQ_ERR_INVALID_ARG;
    if (N % 64 != 0) return SVDQ_ERR_SHAPE;
    if (check_linear_sizes(M, N, K) != SVDQ_OK) return SVDQ_ERR_SHAPE;
    if (!requant_supported(M, N, K, prec)) return SVDQ_ERR_UNSUPPORTED;
    // buffers of zero size may be NULL (empty tensors have no storage)
    if ((M > 0 && (!xq || !xscale || !h)) || (N > 0 && (!wq || !wscale || !up || !smooth2 || !down2)) ||
        (M > 0 && N > 0 && (!xq2 || !xscale2 || !h2 || !work)))
        return SVDQ_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && work_bytes < svdq_requant_workspace_bytes(M, N, rank, prec)) return SVDQ_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(xscale) || !aligned16(h) || !aligned16(wq) || !aligned16(wscale) ||
        !aligned16(up) || (bias && !aligned16(bias)) || !aligned16(smooth2) || !aligned16(down2) ||
        !aligned16(xq2) || !aligned16(xscale2) || !aligned16(h2) || !aligned16(work))
        return SVDQ_ERR_MISALIGNED;
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0 || N == 0) return SVDQ_OK;
    hipError_t e = launch_w4a4_linear_requant(xq, xscale, h, wq, wscale, up, bias, M, N, K, prec, epi, smooth2,
                                              down2, xq2, xscale2, h2, (float *)work, (hipStream_t)stream);
    return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

extern "C" svdq_status svdq_w4a4_linear_qkv_norm_rope(const uint8_t *xq, const void *xscale, const float *h,
                                                      const uint8_t *wq, const void *wscale, const uint16_t *up,
                                                      const uint16_t *bias, int M, int N, int K, int rank,
                                                      svdq_precision prec, const uint16_t *norm_q,
                                                      const uint16_t *norm_k, float eps, const float *rope_cos,
                                                      const float *rope_sin, uint16_t *Y, void *stream)
{
    svdq_status st = check_common(M, K, rank, prec);
    if (st != SVDQ_OK) return st;
    if (N < 0) return SVDQ_ERR_INVALID_ARG;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return SVDQ_ERR_INVALID_ARG;      // finite, non-negative
    if (N % 384 != 0) return SVDQ_ERR_SHAPE;
    if (check_linear_sizes(M, N, K) != SVDQ_OK) return SVDQ_ERR_SHAPE;
    if (!requant_supported(M, N, K, prec)) return SVDQ_ERR_UNSUPPORTED;      // MXFP4: the LDS-DMA kernel's range
    // buffers of zero size may be NULL (empty tensors have no storage)
    if ((M > 0 && (!xq || !xscale || !h || !rope_cos || !rope_sin)) ||
        (N > 0 && (!wq || !wscale || !up || !norm_q || !norm_k)) || (M > 0 && N > 0 && !Y))
        return SVDQ_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(xscale) || !aligned16(h) || !aligned16(wq) || !aligned16(wscale) ||
        !aligned16(up) || !aligned16(Y) || (bias && !aligned16(bias)) || !aligned16(norm_q) || !aligned16(norm_k) ||
        !aligned16(rope_cos) || !aligned16(rope_sin))
        return SVDQ_ERR_MISALIGNED;
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0 || N == 0) return SVDQ_OK;
    hipError_t e = launch_w4a4_linear_qknorm(xq, xscale, h, wq, wscale, up, bias, M, N, K, prec, norm_q, norm_k, eps,
                                             rope_cos, rope_sin, Y, (hipStream_t)stream);
    return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

extern "C" svdq_status svdq_awq_w4a16_linear(const uint16_t *X, const uint8_t *wq, const float *wscale,
                                             const uint16_t *bias, int M, int N, int K, uint16_t *Y,
                                             void *stream)
{
    if (M < 0 || N < 0 || K < 0) return SVDQ_ERR_INVALID_ARG;
    if (K < 256 || K % 256 != 0) return SVDQ_ERR_SHAPE;
    if (!elems_ok(M, K) || check_linear_sizes(M, N, K) != SVDQ_OK) return SVDQ_ERR_SHAPE;
    // buffers of zero size may be NULL (empty tensors have no storage)
    if ((M > 0 && !X) || (N > 0 && (!wq || !wscale)) || (M > 0 && N > 0 && !Y)) return SVDQ_ERR_INVALID_ARG;
    if (!aligned16(X) || !aligned16(wq) || !aligned16(wscale) || (bias && !aligned16(bias)) || !aligned16(Y))
        return SVDQ_ERR_MISALIGNED;
    svdq_status st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0 || N == 0) return SVDQ_OK;
    hipError_t e = launch_awq_linear(X, wq, wscale, bias, M, N, K, Y, (hipStream_t)stream);
    return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

static Nf4Levels nf4_levels_arg()
{
    Nf4Levels lv;
    std::memcpy(lv.c, nf4_codebook_cached(), sizeof(lv.c));
    return lv;
}

extern "C" svdq_status svdq_nf4_dequantize(const uint8_t *wq, const uint8_t *qabs, const float *chunk_scale, int N,
                                           int K, uint16_t *Wd, void *stream)
{
    if (N < 0 || K < 0) return SVDQ_ERR_INVALID_ARG;
    if (K < 64 || K % 64 != 0) return SVDQ_ERR_SHAPE;
    if (!elems_ok(N, K)) return SVDQ_ERR_SHAPE;
    if (N > 0 && (!wq || !qabs || !chunk_scale || !Wd)) return SVDQ_ERR_INVALID_ARG;
    if (!aligned16(wq) || !aligned16(qabs) || !aligned16(chunk_scale) || !aligned16(Wd)) return SVDQ_ERR_MISALIGNED;
    svdq_status st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (N == 0) return SVDQ_OK;
    hipError_t e = launch_nf4_dequant(wq, qabs, chunk_scale, N, K, nf4_levels_arg(), Wd, (hipStream_t)stream);
    return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

extern "C" svdq_status svdq_nf4_w4a16_linear(const uint16_t *X, const uint8_t *wq, const uint8_t *qabs,
                                             const float *chunk_scale, const uint16_t *bias, int M, int N, int K,
                                             uint16_t *Y, void *stream)
{
    if (M < 0 || N < 0 || K < 0) return SVDQ_ERR_INVALID_ARG;
    if (K < 64 || K % 64 != 0 || N % 8 != 0) return SVDQ_ERR_SHAPE;
    if (!elems_ok(M, K) || check_linear_sizes(M, N, K) != SVDQ_OK) return SVDQ_ERR_SHAPE;
    // buffers of zero size may be NULL (empty tensors have no storage)
    if ((M > 0 && !X) || (N > 0 && (!wq || !qabs || !chunk_scale)) || (M > 0 && N > 0 && !Y))
        return SVDQ_ERR_INVALID_ARG;
    if (!aligned16(X) || !aligned16(wq) || !aligned16(qabs) || !aligned16(chunk_scale) || (bias && !aligned16(bias)) ||
        !aligned16(Y))
        return SVDQ_ERR_MISALIGNED;
    svdq_status st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0 || N == 0) return SVDQ_OK;
    hipError_t e = launch_nf4_linear(X, wq, qabs, chunk_scale, bias, M, N, K, nf4_levels_arg(), Y, (hipStream_t)stream);
    return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

// ------------------------------------------------ allocation-free split K
//
// svdq_w4a4_linear_splitk_noalloc keeps the split-K slice sums in this
// file-scope device array instead of a caller workspace.  Each device holds
// its own copy at its own address; host code must use that address (from
// hipGetSymbolAddress), never the array's name.
static __device__ __align__(256) float scratch[SVDQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];     // device address of `scratch`, per device (null until looked up)

// Device address of this device's `scratch`, looked up once per device with
// that device current; null if the lookup fails.
void *scratch_address(int dev)
{
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" svdq_status svdq_w4a4_linear_splitk_noalloc(const uint8_t *xq, const void *xscale, const float *h,
                                                       const uint8_t *wq, const void *wscale, const uint16_t *up,
                                                       const uint16_t *bias, int M, int N, int K, int rank,
                                                       svdq_precision prec, svdq_epilogue epi, uint16_t *Y,
                                                       void *stream)
{
    svdq_status st = check_common(M, K, rank, prec);
    if (st != SVDQ_OK) return st;
    if (N < 0) return SVDQ_ERR_INVALID_ARG;
    if (epi != SVDQ_EPI_NONE && epi != SVDQ_EPI_GELU_TANH) return SVDQ_ERR_INVALID_ARG;
    if (N % 8 != 0) return SVDQ_ERR_SHAPE;
    if (check_linear_sizes(M, N, K) != SVDQ_OK) return SVDQ_ERR_SHAPE;
    if ((M > 0 && (!xq || !xscale || !h)) || (N > 0 && (!wq || !wscale || !up)) || (M > 0 && N > 0 && !Y))
        return SVDQ_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(xscale) || !aligned16(h) || !aligned16(wq) || !aligned16(wscale) ||
        !aligned16(up) || !aligned16(Y) || (bias && !aligned16(bias)))
        return SVDQ_ERR_MISALIGNED;
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0 || N == 0) return SVDQ_OK;
    const size_t need = splitk_work_bytes(M, N, K, prec);
    if (need > SVDQ_NOALLOC_SCRATCH_BYTES) return SVDQ_ERR_SCRATCH;
    float *work = nullptr;
    if (need > 0) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
            (void)hipGetLastError();
            return SVDQ_ERR_HIP;
        }
        work = static_cast<float *>(scratch_address(dev));
        if (!work) return SVDQ_ERR_HIP;
    }
    // every slice of every tile is written in full before the finishing
    // kernel reads it, so the scratch needs no clearing
    hipError_t e = launch_w4a4_linear_splitk(xq, xscale, h, wq, wscale, up, bias, M, N, K, prec, epi, Y, work,
                                             (hipStream_t)stream);
    return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}
