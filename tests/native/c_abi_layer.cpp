// One W4A4 layer through libsvdq's C ABI alone (no Python, no torch): pack
// the weights on the host, run the activation step and the linear on the
// GPU with plain HIP allocations, and check the results against the fp64
// oracle (liboracle, test infrastructure): codes and scales bit-exact, h
// within the blocked-summation bound, Y within 8e-3 |y| + 1e-3 rms(y).
//
// usage: c_abi_layer <int4|mxfp4>        exit status 0 when every check holds
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "svdq.h"

extern "C" {
void oracle_quant_act(const uint16_t *X, int M, int K, const float *s, const uint16_t *down, int r, int prec,
                      uint8_t *xq, void *xscale, double *h);
void oracle_linear(const uint8_t *xq, const void *xscale, const double *h, const uint8_t *wq, const void *wscale,
                   const uint16_t *up, const uint16_t *bias, int M, int N, int K, int r, int prec, int gelu,
                   const int *rows, int nrows, double *y, double *y_q4, double *y_lr);
}

namespace {

// seeded inputs: a 64-bit LCG, uniform in [-1, 1)
struct Lcg {
    uint64_t s;
    double next()
    {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return (double)(s >> 11) * (2.0 / 9007199254740992.0) - 1.0;
    }
};

uint16_t to_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

#define HIP_CHECK(x)                                                                    \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(2);                                                               \
        }                                                                               \
    } while (0)

#define SVDQ_CHECK(x)                                                                          \
    do {                                                                                       \
        svdq_status s_ = (x);                                                                  \
        if (s_ != SVDQ_OK) {                                                                   \
            std::printf("libsvdq error %s at line %d\n", svdq_status_string(s_), __LINE__);   \
            std::exit(2);                                                                      \
        }                                                                                      \
    } while (0)

template <class T>
T *to_device(const std::vector<T> &v)
{
    T *d = nullptr;
    HIP_CHECK(hipMalloc((void **)&d, v.size() * sizeof(T)));
    HIP_CHECK(hipMemcpy(d, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice));
    return d;
}

template <class T>
std::vector<T> to_host(const T *d, size_t n)
{
    std::vector<T> v(n);
    HIP_CHECK(hipMemcpy(v.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
    return v;
}

}  // namespace

int main(int argc, char **argv)
{
    if (argc != 2 || (std::strcmp(argv[1], "int4") && std::strcmp(argv[1], "mxfp4"))) {
        std::printf("usage: %s <int4|mxfp4>\n", argv[0]);
        return 2;
    }
    const svdq_precision prec = std::strcmp(argv[1], "int4") == 0 ? SVDQ_INT4 : SVDQ_MXFP4;
    const int M = 200, K = 512, N = 264, r = 32;
    const int G = prec == SVDQ_INT4 ? K / 64 : K / 32;
    const size_t sbytes = prec == SVDQ_INT4 ? 4 : 1;
    SVDQ_CHECK(svdq_check_device());
    std::printf("libsvdq %d, %s, M=%d K=%d N=%d rank=%d\n", svdq_version(), argv[1], M, K, N, r);

    // inputs: X with one outlier channel, W ~ 0.02 U(-1,1), bias ~ 0.01 U(-1,1)
    Lcg g{20261203u};
    std::vector<uint16_t> X((size_t)M * K), W((size_t)N * K), bias(N);
    for (int m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) X[(size_t)m * K + k] = to_bf16((float)(g.next() * (k == 7 ? 40.0 : 1.0)));
    for (auto &w : W) w = to_bf16((float)(0.02 * g.next()));
    for (auto &b : bias) b = to_bf16((float)(0.01 * g.next()));
    std::vector<float> act(K, 0.0f);
    for (int m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) act[k] = std::fmax(act[k], (float)std::fabs(bf16_value(X[(size_t)m * K + k])));

    // host: smoothing, low-rank factors, residual codes
    std::vector<float> smooth(K);
    std::vector<uint16_t> down((size_t)r * K), up((size_t)N * r);
    std::vector<uint8_t> wq((size_t)N * K / 2), wscale((size_t)N * G * sbytes);
    SVDQ_CHECK(svdq_pack_weights(W.data(), act.data(), N, K, r, prec, smooth.data(), down.data(), up.data(),
                                 wq.data(), wscale.data()));

    // device: the activation step and the linear
    uint16_t *dX = to_device(X), *ddown = to_device(down), *dup = to_device(up), *dbias = to_device(bias);
    float *dsmooth = to_device(smooth);
    uint8_t *dwq = to_device(wq), *dwscale = to_device(wscale);
    uint8_t *dxq = nullptr, *dxscale = nullptr;
    float *dh = nullptr;
    uint16_t *dY = nullptr;
    HIP_CHECK(hipMalloc((void **)&dxq, (size_t)M * K / 2));
    HIP_CHECK(hipMalloc((void **)&dxscale, (size_t)M * G * sbytes));
    HIP_CHECK(hipMalloc((void **)&dh, (size_t)M * r * sizeof(float)));
    HIP_CHECK(hipMalloc((void **)&dY, (size_t)M * N * sizeof(uint16_t)));
    SVDQ_CHECK(svdq_quantize_act(dX, M, K, dsmooth, ddown, r, prec, dxq, dxscale, dh, nullptr));
    SVDQ_CHECK(svdq_w4a4_linear(dxq, dxscale, dh, dwq, dwscale, dup, dbias, M, N, K, r, prec, SVDQ_EPI_GELU_TANH,
                                dY, nullptr));
    HIP_CHECK(hipDeviceSynchronize());
    const auto xq = to_host(dxq, (size_t)M * K / 2);
    const auto xscale = to_host(dxscale, (size_t)M * G * sbytes);
    const auto h = to_host(dh, (size_t)M * r);
    const auto Y = to_host(dY, (size_t)M * N);

    // the oracle on the same inputs
    std::vector<uint8_t> oxq((size_t)M * K / 2), oxscale((size_t)M * G * sbytes);
    std::vector<double> oh((size_t)M * r), y((size_t)M * N);
    oracle_quant_act(X.data(), M, K, smooth.data(), down.data(), r, (int)prec, oxq.data(), oxscale.data(), oh.data());
    int bad = 0;
    if (std::memcmp(xq.data(), oxq.data(), xq.size()) != 0) {
        std::printf("codes differ from the oracle\n");
        ++bad;
    }
    if (std::memcmp(xscale.data(), oxscale.data(), xscale.size()) != 0) {
        std::printf("scales differ from the oracle\n");
        ++bad;
    }
    // h: fp32 sums of bf16 products against the exact sum, within
    // (K/16 + 64) 2^-24 sum_k |x_k down_jk|
    for (int m = 0; m < M && bad < 10; ++m)
        for (int j = 0; j < r; ++j) {
            double a = 0.0;
            for (int k = 0; k < K; ++k)
                a += std::fabs(bf16_value(X[(size_t)m * K + k]) * bf16_value(down[(size_t)j * K + k]));
            const double err = std::fabs((double)h[(size_t)m * r + j] - oh[(size_t)m * r + j]);
            if (err > (K / 16.0 + 64.0) * std::ldexp(1.0, -24) * a) {
                std::printf("h[%d][%d] = %.9g, oracle %.9g\n", m, j, (double)h[(size_t)m * r + j],
                            oh[(size_t)m * r + j]);
                ++bad;
            }
        }
    // Y from the device codes and scales and the oracle's h
    oracle_linear(xq.data(), xscale.data(), oh.data(), wq.data(), wscale.data(), up.data(), bias.data(), M, N, K, r,
                  (int)prec, 1, nullptr, M, y.data(), nullptr, nullptr);
    double ss = 0.0;
    for (double v : y) ss += v * v;
    const double rms = std::sqrt(ss / (double)y.size());
    double worst = 0.0;
    for (size_t i = 0; i < y.size(); ++i) {
        const double err = std::fabs(bf16_value(Y[i]) - y[i]);
        const double tol = 8e-3 * std::fabs(y[i]) + 1e-3 * rms;
        worst = std::fmax(worst, err / tol);
        if (err > tol && bad < 10) {
            std::printf("Y[%zu][%zu] = %.6g, oracle %.6g\n", i / N, i % N, bf16_value(Y[i]), y[i]);
            ++bad;
        }
    }
    std::printf("worst |error| / tolerance over %zu outputs: %.3f\n", y.size(), worst);
    for (void *p : {(void *)dX, (void *)ddown, (void *)dup, (void *)dbias, (void *)dsmooth, (void *)dwq,
                    (void *)dwscale, (void *)dxq, (void *)dxscale, (void *)dh, (void *)dY})
        HIP_CHECK(hipFree(p));
    std::printf(bad ? "FAILED\n" : "c abi layer ok\n");
    return bad ? 1 : 0;
}
