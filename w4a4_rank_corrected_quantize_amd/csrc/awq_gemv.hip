// awq_gemv.hip -- the weight-only AWQ W4A16 layer: INT4 weights in 64-wide
// groups with fp32 scales, bf16 activations ("Bringing Nunchaku 4-bit
// Diffusion Inference to Diffusers", section "Native loading in Diffusers":
// the awq_w4a16 family, int4 with group size 64, used for the modulation
// layers, which are memory-bound and precision-sensitive).
//
//   y_mn = sum_g sw_ng sum_{k in g} X_mk q_nk + b_n,   fp32 accumulation, bf16 out
//
// The layer is meant for few rows of X (a modulation input is one vector per
// image), so it is bound by the weight stream: K/2 code bytes and K/16 scale
// bytes per output channel.  Design for gfx950:
//   * a block (4 waves) owns 16 output channels; wave w takes the 256-channel
//     chunks w, w + 4, ... of K, with the loads of up to 4 of them in flight
//     before any is used, and the 4 partial results are summed in LDS in a
//     fixed order (deterministic);
//   * per chunk a lane (channel n = lane % 16, k-block b = lane / 16) reads
//     the 32 code bytes that the storage order puts together for it (one
//     coalesced 128-byte line per channel and chunk) with non-temporal loads;
//   * a code c = q + 8 becomes the bf16 number 128 + c by OR-ing it into the
//     bits of 128.0 (0x4300 | c), two codes per dword in one v_and_or: the
//     storage order makes dword d of the lane's 32 bytes the B operand of
//     product (g, h) = (d / 2, d % 2), with bf16 pair j from nibbles j and
//     j + 4;
//   * v_mfma_f32_16x16x32_bf16 with A = 16 rows of X (rows past M are zero)
//     accumulates sum X (136 + q) over a group's two 32-channel halves, then
//     the same A against the constant -136 removes the offset: every product
//     is exact in fp32 and the sum loses ~2^-24 of |X| * 143 * 64 (far below
//     the bf16 output);
//   * one fma per output and group applies sw (the lane's channel is fixed,
//     so its scale is a scalar).
// Rows of X are taken 16 at a time; more rows re-read the block's weights
// (from the L2).
#include "svdq.h"
#include "svdq_internal.h"

namespace svdq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int AWQ_WAVES = 4;
constexpr int AWQ_COLS = 16;      // output channels per block
constexpr int AWQ_BATCH = 4;      // chunks per wave whose loads are in flight together
constexpr uint32_t kBf16_128 = 0x43004300u;   // bf16 128.0 in both halves
constexpr uint32_t kBf16_m136 = 0xC308C308u;  // bf16 -136.0 in both halves

__device__ __forceinline__ uint32_t bf16_bits_rne(float f)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// B operand of one 32-channel product from one dword of 8 codes.
__device__ __forceinline__ bf16x8 awq_operand(uint32_t w)
{
    const u32x4 o = {(w & 0x000F000Fu) | kBf16_128, ((w >> 4) & 0x000F000Fu) | kBf16_128,
                     ((w >> 8) & 0x000F000Fu) | kBf16_128, ((w >> 12) & 0x000F000Fu) | kBf16_128};
    return __builtin_bit_cast(bf16x8, o);
}

__global__ __launch_bounds__(64 * AWQ_WAVES) void awq_w4a16_kernel(const uint16_t *__restrict__ X,
                                                                   const uint8_t *__restrict__ wq,
                                                                   const float *__restrict__ wscale,
                                                                   const uint16_t *__restrict__ bias, int M,
                                                                   int N, int K, uint16_t *__restrict__ Y)
{
    __shared__ f32x4 part[AWQ_WAVES][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kb = lane >> 4;
    const int n = blockIdx.x * AWQ_COLS + col;
    const int nrow = n < N ? n : N - 1;              // rows past N read the last row, never stored
    const int chunks = K >> 8;
    const int KB = K >> 1, G = K >> 6;
    const uint8_t *wrow = wq + (size_t)nrow * KB + 32 * kb;
    const float *srow = wscale + (size_t)nrow * G;
    const bf16x8 neg136 = __builtin_bit_cast(bf16x8, (u32x4){kBf16_m136, kBf16_m136, kBf16_m136, kBf16_m136});

    for (int m0 = 0; m0 < M; m0 += 16) {
        const int m = m0 + col;                      // this lane's row of the A operand
        const bool mv = m < M;
        const uint16_t *xrow = X + (size_t)(mv ? m : 0) * K + 8 * kb;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        // up to AWQ_BATCH of the wave's chunks at a time, all loads issued first
        for (int cb = wave; cb < chunks; cb += AWQ_BATCH * AWQ_WAVES) {
            u32x4 wv[AWQ_BATCH][2];
            float4 sv[AWQ_BATCH];
#pragma unroll
            for (int u = 0; u < AWQ_BATCH; ++u) {
                const int c = cb + AWQ_WAVES * u;
                if (c < chunks) {
                    wv[u][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wrow + 128 * c));
                    wv[u][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wrow + 128 * c + 16));
                    sv[u] = *reinterpret_cast<const float4 *>(srow + 4 * c);
                }
            }
#pragma unroll
            for (int u = 0; u < AWQ_BATCH; ++u) {
                const int c = cb + AWQ_WAVES * u;
                if (c >= chunks) break;
                const uint32_t wd[8] = {wv[u][0].x, wv[u][0].y, wv[u][0].z, wv[u][0].w,
                                        wv[u][1].x, wv[u][1].y, wv[u][1].z, wv[u][1].w};
                const float swv[4] = {sv[u].x, sv[u].y, sv[u].z, sv[u].w};
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    bf16x8 a[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        uint4 xv = {0u, 0u, 0u, 0u};
                        if (mv) xv = *reinterpret_cast<const uint4 *>(xrow + 256 * c + 64 * g + 32 * h);
                        a[h] = __builtin_bit_cast(bf16x8, xv);
                    }
                    f32x4 p = {0.f, 0.f, 0.f, 0.f};
                    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], awq_operand(wd[2 * g]), p, 0, 0, 0);
                    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], awq_operand(wd[2 * g + 1]), p, 0, 0, 0);
                    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], neg136, p, 0, 0, 0);
                    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], neg136, p, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(p[i], swv[g], acc[i]);
                }
            }
        }
        // the 4 waves' partial sums, added in wave order
        part[wave][lane] = acc;
        __syncthreads();
        if (wave == 0) {
            f32x4 s = part[0][lane];
#pragma unroll
            for (int w = 1; w < AWQ_WAVES; ++w) {
                const f32x4 t = part[w][lane];
                s[0] += t[0]; s[1] += t[1]; s[2] += t[2]; s[3] += t[3];
            }
            const float b = (bias && n < N) ? __builtin_bit_cast(float, (uint32_t)bias[n] << 16) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mo = m0 + 4 * kb + i;     // output row of value i (D rows = A rows)
                if (mo < M && n < N) Y[(size_t)mo * N + n] = (uint16_t)bf16_bits_rne(s[i] + b);
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_awq_linear(const uint16_t *X, const uint8_t *wq, const float *wscale, const uint16_t *bias,
                             int M, int N, int K, uint16_t *Y, hipStream_t stream)
{
    const int blocks = (N + AWQ_COLS - 1) / AWQ_COLS;
    hipLaunchKernelGGL(awq_w4a16_kernel, dim3((unsigned)blocks), dim3(64 * AWQ_WAVES), 0, stream, X, wq, wscale,
                       bias, M, N, K, Y);
    return hipGetLastError();
}

}  // namespace svdq
