// pack_host.hip -- host-side packing of one SVDQuant linear layer (CPU only).
//
// "Bringing Nunchaku 4-bit Diffusion Inference to Diffusers", section
// "Background: SVDQuant and Nunchaku": outliers move from the activations into
// the weights (per-channel smoothing), the hardest part of each smoothed
// weight matrix is kept in a small 16-bit low-rank branch, and the residual is
// quantized to 4 bits; section "Native loading in Diffusers": rank 32.
//
// Steps (fp64 throughout, compiled with -ffp-contract=off so the residual is
// evaluated exactly as written):
//   1. s_k = fl32(1 / sqrt(max|X_k| / max_n|W_nk|))   (1 when either is 0)
//   2. top-r SVD of What (K x N), What_kn = W_nk / s_k: randomized subspace
//      iteration (Gaussian start, r + 32 columns, 6 power steps with
//      re-orthonormalization), then a Rayleigh-Ritz step: the Gram matrix of
//      What^T Q is diagonalized by cyclic Jacobi.
//   3. down[j][k] = bf16(s_k U_kj sigma_j), up[n][j] = bf16(V_nj)
//   4. R_kn = (W_nk - sum_j down[j][k] up[n][j]) / s_k, then fl32, then the
//      group quantizer of svdq_quant.h per (n, group).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "svdq.h"
#include "svdq_internal.h"
#include "svdq_quant.h"

namespace svdq {
namespace {

int host_threads()
{
    unsigned n = std::thread::hardware_concurrency();
    if (n == 0) n = 1;
    if (n > 64) n = 64;
    return (int)n;
}

// Run fn(begin, end) over [0, count) split into contiguous chunks, one per thread.
void parallel_for(int64_t count, const std::function<void(int64_t, int64_t)> &fn)
{
    int nt = host_threads();
    if (count < 2 * nt || nt == 1) {
        fn(0, count);
        return;
    }
    std::vector<std::thread> th;
    int64_t chunk = (count + nt - 1) / nt;
    for (int t = 0; t < nt; ++t) {
        int64_t b = t * chunk, e = std::min<int64_t>(count, b + chunk);
        if (b >= e) break;
        th.emplace_back([&fn, b, e] { fn(b, e); });
    }
    for (auto &x : th) x.join();
}

double bf16_to_double(uint16_t b) { return (double)bits_f32((uint32_t)b << 16); }

uint16_t double_to_bf16(double v)
{
    // fp64 -> fp32 (round to nearest even) -> bf16 (round to nearest even)
    uint32_t u = f32_bits((float)v);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

bool bf16_finite(uint16_t b) { return (b & 0x7F80u) != 0x7F80u; }

// Deterministic standard normals (splitmix64 + Box-Muller).
struct Rng {
    uint64_t s;
    uint64_t next()
    {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
    double normal()
    {
        double u1 = uniform(), u2 = uniform();
        return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
    }
};

// Y[K][l] = What * Z   with What_kn = B[n][k];  Z is [N][l].
void mul_what(const double *B, int N, int K, const double *Z, int l, double *Y)
{
    parallel_for(K, [&](int64_t k0, int64_t k1) {
        std::fill(Y + k0 * l, Y + k1 * l, 0.0);
        for (int n = 0; n < N; ++n) {
            const double *b = B + (int64_t)n * K;
            const double *z = Z + (int64_t)n * l;
            for (int64_t k = k0; k < k1; ++k) {
                double v = b[k];
                if (v == 0.0) continue;
                double *y = Y + k * l;
                for (int i = 0; i < l; ++i) y[i] += v * z[i];
            }
        }
    });
}

// Z[N][l] = What^T * Q   with Q [K][l].
void mul_what_t(const double *B, int N, int K, const double *Q, int l, double *Z)
{
    parallel_for(N, [&](int64_t n0, int64_t n1) {
        std::vector<double> acc(l);
        for (int64_t n = n0; n < n1; ++n) {
            std::fill(acc.begin(), acc.end(), 0.0);
            const double *b = B + n * K;
            for (int k = 0; k < K; ++k) {
                double v = b[k];
                if (v == 0.0) continue;
                const double *q = Q + (int64_t)k * l;
                for (int i = 0; i < l; ++i) acc[i] += v * q[i];
            }
            std::memcpy(Z + n * l, acc.data(), sizeof(double) * l);
        }
    });
}

// Orthonormalize the columns of A [rows][l] (classical Gram-Schmidt, two
// passes).  Columns that vanish (rank deficiency) are set to zero.
void orthonormalize(double *A, int64_t rows, int l)
{
    std::vector<double> C((size_t)l * rows);          // column-major copy
    for (int64_t r = 0; r < rows; ++r)
        for (int i = 0; i < l; ++i) C[(size_t)i * rows + r] = A[r * l + i];
    std::vector<char> alive(l, 0);
    for (int j = 0; j < l; ++j) {
        double *cj = &C[(size_t)j * rows];
        double n0 = 0.0;
        for (int64_t r = 0; r < rows; ++r) n0 += cj[r] * cj[r];
        n0 = std::sqrt(n0);
        for (int pass = 0; pass < 2; ++pass) {
            for (int i = 0; i < j; ++i) {
                if (!alive[i]) continue;
                const double *ci = &C[(size_t)i * rows];
                double d = 0.0;
                for (int64_t r = 0; r < rows; ++r) d += ci[r] * cj[r];
                for (int64_t r = 0; r < rows; ++r) cj[r] -= d * ci[r];
            }
        }
        double nn = 0.0;
        for (int64_t r = 0; r < rows; ++r) nn += cj[r] * cj[r];
        nn = std::sqrt(nn);
        if (!(nn > 1e-10 * n0) || nn == 0.0) {
            std::fill(cj, cj + rows, 0.0);
        } else {
            alive[j] = 1;
            double inv = 1.0 / nn;
            for (int64_t r = 0; r < rows; ++r) cj[r] *= inv;
        }
    }
    for (int64_t r = 0; r < rows; ++r)
        for (int i = 0; i < l; ++i) A[r * l + i] = C[(size_t)i * rows + r];
}

// Eigen-decomposition of the symmetric l x l matrix G (cyclic Jacobi);
// on return G is (near) diagonal and V holds the eigenvectors as columns.
void jacobi_eigen(std::vector<double> &G, std::vector<double> &V, int l)
{
    V.assign((size_t)l * l, 0.0);
    for (int i = 0; i < l; ++i) V[(size_t)i * l + i] = 1.0;
    for (int sweep = 0; sweep < 60; ++sweep) {
        double off = 0.0, tot = 0.0;
        for (int i = 0; i < l; ++i)
            for (int j = 0; j < l; ++j) {
                double g = G[(size_t)i * l + j];
                tot += g * g;
                if (i != j) off += g * g;
            }
        if (off <= 1e-30 * tot || tot == 0.0) break;
        for (int p = 0; p < l - 1; ++p) {
            for (int q = p + 1; q < l; ++q) {
                double gpq = G[(size_t)p * l + q];
                if (gpq == 0.0) continue;
                double gpp = G[(size_t)p * l + p], gqq = G[(size_t)q * l + q];
                double theta = (gqq - gpp) / (2.0 * gpq);
                double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
                double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
                for (int k = 0; k < l; ++k) {          // G <- G J (columns p, q)
                    double a = G[(size_t)k * l + p], b = G[(size_t)k * l + q];
                    G[(size_t)k * l + p] = c * a - s * b;
                    G[(size_t)k * l + q] = s * a + c * b;
                }
                for (int k = 0; k < l; ++k) {          // G <- J^T G (rows p, q)
                    double a = G[(size_t)p * l + k], b = G[(size_t)q * l + k];
                    G[(size_t)p * l + k] = c * a - s * b;
                    G[(size_t)q * l + k] = s * a + c * b;
                }
                for (int k = 0; k < l; ++k) {          // V <- V J
                    double a = V[(size_t)k * l + p], b = V[(size_t)k * l + q];
                    V[(size_t)k * l + p] = c * a - s * b;
                    V[(size_t)k * l + q] = s * a + c * b;
                }
            }
        }
    }
}

// Top-r factors of What: L1 [K][r] = U S, L2t [N][r] = V (zeros past the rank).
void top_r_svd(const double *B, int N, int K, int r, std::vector<double> &L1, std::vector<double> &L2t)
{
    const int p = 32, power_steps = 6;
    int l = std::min(r + p, std::min(N, K));
    L1.assign((size_t)K * r, 0.0);
    L2t.assign((size_t)N * r, 0.0);
    std::vector<double> Om((size_t)N * l), Q((size_t)K * l), Z((size_t)N * l);
    Rng rng{0x5EED5EEDull ^ ((uint64_t)N << 32) ^ (uint64_t)K};
    for (auto &v : Om) v = rng.normal();
    mul_what(B, N, K, Om.data(), l, Q.data());
    orthonormalize(Q.data(), K, l);
    for (int it = 0; it < power_steps; ++it) {
        mul_what_t(B, N, K, Q.data(), l, Z.data());
        orthonormalize(Z.data(), N, l);
        mul_what(B, N, K, Z.data(), l, Q.data());
        orthonormalize(Q.data(), K, l);
    }
    // Rayleigh-Ritz: What ~ Q (Q^T What) = Q Z^T with Z = What^T Q (N x l).
    mul_what_t(B, N, K, Q.data(), l, Z.data());
    std::vector<double> G((size_t)l * l, 0.0), J;
    for (int i = 0; i < l; ++i)
        for (int j = i; j < l; ++j) {
            double d = 0.0;
            for (int n = 0; n < N; ++n) d += Z[(size_t)n * l + i] * Z[(size_t)n * l + j];
            G[(size_t)i * l + j] = G[(size_t)j * l + i] = d;
        }
    jacobi_eigen(G, J, l);
    // H = Z J (columns h_i = sigma_i v_i), U = Q J.
    std::vector<double> H((size_t)N * l, 0.0), U((size_t)K * l, 0.0);
    parallel_for(N, [&](int64_t n0, int64_t n1) {
        for (int64_t n = n0; n < n1; ++n)
            for (int i = 0; i < l; ++i) {
                double d = 0.0;
                for (int a = 0; a < l; ++a) d += Z[n * l + a] * J[(size_t)a * l + i];
                H[n * l + i] = d;
            }
    });
    for (int k = 0; k < K; ++k)
        for (int i = 0; i < l; ++i) {
            double d = 0.0;
            for (int a = 0; a < l; ++a) d += Q[(size_t)k * l + a] * J[(size_t)a * l + i];
            U[(size_t)k * l + i] = d;
        }
    std::vector<double> sig(l, 0.0);
    for (int i = 0; i < l; ++i) {
        double d = 0.0;
        for (int n = 0; n < N; ++n) d += H[(size_t)n * l + i] * H[(size_t)n * l + i];
        sig[i] = std::sqrt(d);
    }
    std::vector<int> order(l);
    for (int i = 0; i < l; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return sig[a] > sig[b]; });
    double smax = l ? sig[order[0]] : 0.0;
    for (int j = 0; j < std::min(r, l); ++j) {
        int i = order[j];
        double sg = sig[i];
        if (!(sg > 1e-13 * smax) || sg == 0.0) continue;   // beyond the numerical rank
        // sign: the largest-|.| entry of v_j positive
        int64_t arg = 0;
        double best = -1.0;
        for (int n = 0; n < N; ++n) {
            double a = std::fabs(H[(size_t)n * l + i]);
            if (a > best) { best = a; arg = n; }
        }
        double sgn = H[(size_t)arg * l + i] < 0 ? -1.0 : 1.0;
        for (int n = 0; n < N; ++n) L2t[(size_t)n * r + j] = sgn * H[(size_t)n * l + i] / sg;
        for (int k = 0; k < K; ++k) L1[(size_t)k * r + j] = sgn * U[(size_t)k * l + i] * sg;
    }
}

}  // namespace

int group_size(svdq_precision prec) { return prec == SVDQ_INT4 ? 64 : 32; }

// Residual codes of one row n (K values of fl32(R)).
static void quantize_row(const float *v, int K, svdq_precision prec, uint8_t *codes, void *scales)
{
    if (prec == SVDQ_INT4) {
        float *sc = (float *)scales;
        for (int g = 0; g < K / 64; ++g) {
            const float *x = v + 64 * g;
            float a = 0.0f;
            for (int i = 0; i < 64; ++i) a = std::max(a, std::fabs(x[i]));
            float scale = int4_group_scale(a);
            Int4Group G = int4_group_prepare(scale);
            for (int i = 0; i < 32; ++i)
                codes[32 * g + i] = (uint8_t)(int4_nibble(x[2 * i], G) | (int4_nibble(x[2 * i + 1], G) << 4));
            sc[g] = scale;
        }
    } else {
        uint8_t *sc = (uint8_t *)scales;
        for (int b = 0; b < K / 32; ++b) {
            const float *x = v + 32 * b;
            float a = 0.0f;
            for (int i = 0; i < 32; ++i) a = std::max(a, std::fabs(x[i]));
            uint32_t e = mx_block_e8m0(a);
            float inv = mx_inv_scale(e);
            for (int i = 0; i < 16; ++i)
                codes[16 * b + i] = (uint8_t)(e2m1_code(x[2 * i], inv) | (e2m1_code(x[2 * i + 1], inv) << 4));
            sc[b] = (uint8_t)e;
        }
    }
}

static svdq_status check_pack_args(const void *W, int N, int K, int rank, svdq_precision prec)
{
    if (!W) return SVDQ_ERR_INVALID_ARG;
    if (prec != SVDQ_INT4 && prec != SVDQ_MXFP4) return SVDQ_ERR_INVALID_ARG;
    if (N < 0 || K < 0) return SVDQ_ERR_INVALID_ARG;
    if (rank != SVDQ_RANK) return SVDQ_ERR_UNSUPPORTED;
    int g = group_size(prec);
    if (N < 1 || K < g || K % g != 0) return SVDQ_ERR_SHAPE;
    if (!elems_ok(N, K)) return SVDQ_ERR_SHAPE;
    return SVDQ_OK;
}

static svdq_status residual_impl(const uint16_t *W, const float *smooth, const uint16_t *down,
                                 const uint16_t *up, int N, int K, int r, svdq_precision prec,
                                 uint8_t *wq, void *wscale)
{
    const int G = K / group_size(prec);
    parallel_for(N, [&](int64_t n0, int64_t n1) {
        std::vector<float> row(K);
        std::vector<double> upn(r);
        for (int64_t n = n0; n < n1; ++n) {
            for (int j = 0; j < r; ++j) upn[j] = bf16_to_double(up[n * r + j]);
            for (int k = 0; k < K; ++k) {
                double acc = 0.0;
                for (int j = 0; j < r; ++j) acc += bf16_to_double(down[(int64_t)j * K + k]) * upn[j];
                double R = (bf16_to_double(W[n * K + k]) - acc) / (double)smooth[k];
                row[k] = (float)R;
            }
            void *sc = prec == SVDQ_INT4 ? (void *)((float *)wscale + n * G)
                                         : (void *)((uint8_t *)wscale + n * G);
            quantize_row(row.data(), K, prec, wq + n * (int64_t)(K / 2), sc);
        }
    });
    return SVDQ_OK;
}

}  // namespace svdq

using namespace svdq;

extern "C" svdq_status svdq_pack_residual(const uint16_t *W, const float *smooth, const uint16_t *down,
                                          const uint16_t *up, int N, int K, int rank,
                                          svdq_precision prec, uint8_t *wq, void *wscale)
{
    svdq_status st = check_pack_args(W, N, K, rank, prec);
    if (st != SVDQ_OK) return st;
    if (!smooth || !down || !up || !wq || !wscale) return SVDQ_ERR_INVALID_ARG;
    for (int64_t i = 0; i < (int64_t)N * K; ++i)
        if (!bf16_finite(W[i])) return SVDQ_ERR_NONFINITE;
    for (int k = 0; k < K; ++k)
        if (!std::isfinite(smooth[k]) || smooth[k] == 0.0f) return SVDQ_ERR_NONFINITE;
    for (int64_t i = 0; i < (int64_t)rank * K; ++i)
        if (!bf16_finite(down[i])) return SVDQ_ERR_NONFINITE;
    for (int64_t i = 0; i < (int64_t)N * rank; ++i)
        if (!bf16_finite(up[i])) return SVDQ_ERR_NONFINITE;
    return residual_impl(W, smooth, down, up, N, K, rank, prec, wq, wscale);
}

extern "C" svdq_status svdq_pack_weights(const uint16_t *W, const float *act_absmax, int N, int K,
                                         int rank, svdq_precision prec, float *smooth, uint16_t *down,
                                         uint16_t *up, uint8_t *wq, void *wscale)
{
    svdq_status st = check_pack_args(W, N, K, rank, prec);
    if (st != SVDQ_OK) return st;
    if (!act_absmax || !smooth || !down || !up || !wq || !wscale) return SVDQ_ERR_INVALID_ARG;
    for (int k = 0; k < K; ++k)
        if (!(act_absmax[k] >= 0.0f) || !std::isfinite(act_absmax[k])) return SVDQ_ERR_NONFINITE;
    bool finite = true;
    for (int64_t i = 0; i < (int64_t)N * K && finite; ++i) finite = bf16_finite(W[i]);
    if (!finite) return SVDQ_ERR_NONFINITE;

    // 1. smoothing factors
    std::vector<double> mw(K, 0.0);
    {
        int nt = host_threads();
        std::vector<std::vector<double>> part(nt, std::vector<double>(K, 0.0));
        int64_t chunk = (N + nt - 1) / nt;
        std::vector<std::thread> th;
        for (int t = 0; t < nt; ++t) {
            int64_t b = t * chunk, e = std::min<int64_t>(N, b + chunk);
            if (b >= e) break;
            th.emplace_back([&, t, b, e] {
                double *pm = part[t].data();
                for (int64_t n = b; n < e; ++n)
                    for (int k = 0; k < K; ++k) pm[k] = std::max(pm[k], std::fabs(bf16_to_double(W[n * K + k])));
            });
        }
        for (auto &x : th) x.join();
        for (auto &p : part)
            for (int k = 0; k < K; ++k) mw[k] = std::max(mw[k], p[k]);
    }
    for (int k = 0; k < K; ++k) {
        double mx = (double)act_absmax[k];
        if (mx == 0.0 || mw[k] == 0.0) {
            smooth[k] = 1.0f;
        } else {
            double lambda = std::sqrt(mx / mw[k]);
            smooth[k] = (float)(1.0 / lambda);
        }
    }

    // 2. top-r SVD of What_kn = W_nk / s_k, stored as B[n][k]
    std::vector<double> B((size_t)N * K);
    parallel_for(N, [&](int64_t n0, int64_t n1) {
        for (int64_t n = n0; n < n1; ++n)
            for (int k = 0; k < K; ++k) B[(size_t)n * K + k] = bf16_to_double(W[n * K + k]) / (double)smooth[k];
    });
    std::vector<double> L1, L2t;
    top_r_svd(B.data(), N, K, rank, L1, L2t);
    B.clear();
    B.shrink_to_fit();

    // 3. stored factors (smoothing folded into the down projection)
    for (int j = 0; j < rank; ++j)
        for (int k = 0; k < K; ++k)
            down[(size_t)j * K + k] = double_to_bf16((double)smooth[k] * L1[(size_t)k * rank + j]);
    for (int64_t n = 0; n < N; ++n)
        for (int j = 0; j < rank; ++j) up[n * rank + j] = double_to_bf16(L2t[(size_t)n * rank + j]);

    // 4. residual
    return residual_impl(W, smooth, down, up, N, K, rank, prec, wq, wscale);
}

// Weight-only AWQ W4A16 packing ("Native loading in Diffusers": awq_w4a16,
// int4, group size 64).  Codes are q + 8 (offset binary) of the symmetric
// INT4 group quantizer above, applied to fl32(W) per (n, 64-group).  Storage
// order, written byte by byte: in 256-channel chunk C of a row, the 32 bytes
// at 128 C + 32 b hold, as 8 dwords d = 2 g + h, the codes of channels
// 256 C + 64 g + 32 h + 8 b + i, where nibble j of the dword (j < 4) is
// i = 2 j and nibble j + 4 is i = 2 j + 1 -- the operand order the linear
// kernel decodes directly.
extern "C" svdq_status svdq_awq_pack_weights(const uint16_t *W, int N, int K, uint8_t *wq, float *wscale)
{
    if (!W || !wq || !wscale) return SVDQ_ERR_INVALID_ARG;
    if (N < 0 || K < 0) return SVDQ_ERR_INVALID_ARG;
    if (N < 1 || K < 256 || K % 256 != 0) return SVDQ_ERR_SHAPE;
    if (!elems_ok(N, K)) return SVDQ_ERR_SHAPE;
    for (int64_t i = 0; i < (int64_t)N * K; ++i)
        if (!bf16_finite(W[i])) return SVDQ_ERR_NONFINITE;
    const int G = K / 64;
    parallel_for(N, [&](int64_t n0, int64_t n1) {
        std::vector<uint8_t> code(K);
        for (int64_t n = n0; n < n1; ++n) {
            const uint16_t *w = W + n * K;
            for (int g = 0; g < G; ++g) {
                float a = 0.0f;
                for (int i = 0; i < 64; ++i) a = std::max(a, std::fabs(bits_f32((uint32_t)w[64 * g + i] << 16)));
                const float scale = int4_group_scale(a);
                const Int4Group Gq = int4_group_prepare(scale);
                for (int i = 0; i < 64; ++i) {
                    const float v = bits_f32((uint32_t)w[64 * g + i] << 16);
                    const int q = (int)int4_mag(std::fabs(v), Gq);
                    code[64 * g + i] = (uint8_t)((v < 0.0f ? -q : q) + 8);
                }
                wscale[n * G + g] = scale;
            }
            uint8_t *row = wq + n * (int64_t)(K / 2);
            for (int C = 0; C < K / 256; ++C)
                for (int b = 0; b < 4; ++b)
                    for (int d = 0; d < 8; ++d) {
                        const int kbase = 256 * C + 64 * (d / 2) + 32 * (d % 2) + 8 * b;
                        uint32_t dw = 0;
                        for (int j = 0; j < 4; ++j)
                            dw |= (uint32_t)code[kbase + 2 * j] << (4 * j) |
                                  (uint32_t)code[kbase + 2 * j + 1] << (4 * (j + 4));
                        uint8_t *dst = row + 128 * C + 32 * b + 4 * d;
                        for (int t = 0; t < 4; ++t) dst[t] = (uint8_t)(dw >> (8 * t));
                    }
        }
    });
    return SVDQ_OK;
}

// ------------------------------------------------------------------- NF4
//
// Weight-only NF4 packing ("BitsAndBytes W4 Quantization", sections
// "Overview" and "Parameters": weights quantized at load time to the 4-bit
// "nf4" data type, activations kept in bf16; compress_statistics
// double-quantizes the block statistics).  NF4 levels are quantiles of the
// standard normal distribution normalized to [-1, 1] with an exact zero: 8
// positive levels at probabilities 1/2 + j (1/2 - d) / 8 and 7 negative ones
// at 1/2 - j (1/2 - d) / 7, divided by Phi^-1(1 - d), d = (1/32 + 1/30) / 2.
// Phi^-1 comes from Newton's method on Phi(x) = erfc(-x / sqrt 2) / 2 started
// at 0 (Phi is concave for x > 0, so after the first step the iterates
// decrease monotonically to the root); each level is rounded once to fp32.
namespace svdq {
namespace {

double normal_quantile_upper(double p)     // p in [1/2, 1)
{
    const double inv_sqrt_2pi = 0.39894228040143267794;
    double x = 0.0;
    for (int it = 0; it < 100; ++it) {
        const double f = 0.5 * std::erfc(-x * 0.70710678118654752440) - p;
        const double step = f / (inv_sqrt_2pi * std::exp(-0.5 * x * x));
        const double nx = x - step;
        if (nx == x) break;
        if (it > 3 && std::fabs(step) <= 1e-17 * std::fabs(x)) { x = nx; break; }
        x = nx;
    }
    return x;
}

void nf4_levels(float *c)
{
    const double d = (1.0 / 32.0 + 1.0 / 30.0) / 2.0;
    const double top = normal_quantile_upper(1.0 - d);
    c[7] = 0.0f;
    for (int j = 1; j <= 8; ++j) c[7 + j] = (float)(normal_quantile_upper(0.5 + j * (0.5 - d) / 8.0) / top);
    for (int j = 1; j <= 7; ++j) c[7 - j] = (float)(-normal_quantile_upper(0.5 + j * (0.5 - d) / 7.0) / top);
    c[15] = 1.0f;      // the top quantile divided by itself
    c[0] = -1.0f;
}

}  // namespace

// The 16 levels, cached after the first call (computed once per process).
const float *nf4_codebook_cached()
{
    static float levels[16];
    static std::once_flag once;
    std::call_once(once, [] { nf4_levels(levels); });
    return levels;
}

}  // namespace svdq

extern "C" svdq_status svdq_nf4_codebook(float *levels)
{
    if (!levels) return SVDQ_ERR_INVALID_ARG;
    std::memcpy(levels, svdq::nf4_codebook_cached(), 16 * sizeof(float));
    return SVDQ_OK;
}

extern "C" svdq_status svdq_nf4_pack_weights(const uint16_t *W, int N, int K, uint8_t *wq, uint8_t *qabs,
                                             float *chunk_scale)
{
    using namespace svdq;
    if (!W || !wq || !qabs || !chunk_scale) return SVDQ_ERR_INVALID_ARG;
    if (N < 0 || K < 0) return SVDQ_ERR_INVALID_ARG;
    if (N < 1 || K < 64 || K % 64 != 0) return SVDQ_ERR_SHAPE;
    if (!elems_ok(N, K)) return SVDQ_ERR_SHAPE;
    for (int64_t i = 0; i < (int64_t)N * K; ++i)
        if (!bf16_finite(W[i])) return SVDQ_ERR_NONFINITE;
    const float *c = nf4_codebook_cached();
    double mid[15];                          // exact midpoints of neighbouring levels
    for (int i = 0; i < 15; ++i) mid[i] = 0.5 * ((double)c[i] + (double)c[i + 1]);
    const int G = K / 64;
    const int64_t nb = (int64_t)N * G;
    std::vector<float> amax((size_t)nb);
    parallel_for(N, [&](int64_t n0, int64_t n1) {
        for (int64_t n = n0; n < n1; ++n) {
            const uint16_t *w = W + n * K;
            uint8_t *row = wq + n * (int64_t)(K / 2);
            for (int g = 0; g < G; ++g) {
                float a = 0.0f;
                for (int i = 0; i < 64; ++i) a = std::max(a, std::fabs(bits_f32((uint32_t)w[64 * g + i] << 16)));
                amax[(size_t)(n * G + g)] = a;
                uint8_t code[64];
                for (int i = 0; i < 64; ++i) {
                    int q = 7;
                    if (a > 0.0f) {
                        // x = fl32(w / a): the fp64 quotient of two fp32 values rounded
                        // to fp32 is the correctly rounded fp32 quotient
                        const double x = (double)(float)((double)bits_f32((uint32_t)w[64 * g + i] << 16) / (double)a);
                        // binary search over the midpoints; a tie goes toward zero
                        int lo = 0, hi = 15;       // answer in [lo, hi]
                        while (lo < hi) {
                            const int m = (lo + hi) >> 1;       // compare with mid[m]
                            const bool above = mid[m] < 0.0 ? x >= mid[m] : x > mid[m];
                            if (above) lo = m + 1;
                            else hi = m;
                        }
                        q = lo;
                    }
                    code[i] = (uint8_t)q;
                }
                // in each group of 8 consecutive weights, byte i holds weight i
                // (low nibble) and weight i + 4 (high nibble)
                for (int e = 0; e < 8; ++e)
                    for (int i = 0; i < 4; ++i)
                        row[32 * g + 4 * e + i] = (uint8_t)(code[8 * e + i] | code[8 * e + 4 + i] << 4);
            }
        }
    });
    // statistics: chunks of 256 block absmaxes in row-major (n, block) order
    const int64_t nchunk = (nb + 255) / 256;
    for (int64_t ch = 0; ch < nchunk; ++ch) {
        const int64_t b0 = 256 * ch, b1 = std::min<int64_t>(nb, b0 + 256);
        float s = 0.0f;
        for (int64_t b = b0; b < b1; ++b) s = std::max(s, amax[(size_t)b]);
        chunk_scale[ch] = (float)((double)s / 255.0);
        for (int64_t b = b0; b < b1; ++b) {
            // round-half-even of 255 a / s: 255 a is exact in fp64; a quotient of
            // 1/2 or more that is not exactly k + 1/2 lies at least 2^-34 from it
            // (a >= s / 510, and 2 * 255 a - (2k + 1) s is a multiple of ulp(a)),
            // far beyond the fp64 rounding error of the division (< 2^-45)
            qabs[b] = (uint8_t)(s > 0.0f ? std::nearbyint(255.0 * (double)amax[(size_t)b] / (double)s) : 0.0);
        }
    }
    return SVDQ_OK;
}
