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
//   * a block (4 waves) owns 16 output channels and walks K in slabs of
//     1024 channels, one 256-channel chunk per wave; the pass's rows of X
//     over the slab are staged in LDS by coalesced loads (one global read per
//     16 bytes of X instead of one per lane and product), and the next slab's
//     weights are in flight while the current one is computed; the 4 waves'
//     partial results are summed in LDS in a fixed order (deterministic);
//   * a chunk of the 16 channels' codes is 16 lines of 128 bytes; each of
//     the wave's two non-temporal loads takes 8 whole lines (8 lanes per
//     line), and the lines go through a small per-wave LDS tile, from which
//     a lane (channel n = lane % 16, k-block b = lane / 16) reads the 32 code
//     bytes that the storage order puts together for it (half-line loads
//     straight into that layout, 64 bytes of 16 lines per load, took 11-14 %
//     longer);
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

constexpr int AWQ_SLAB = 256 * AWQ_WAVES;            // channels of X staged per slab (one chunk per wave)
constexpr int AWQ_XSTRIDE = AWQ_SLAB + 8;            // bf16 per staged row (16 B pad: conflict-free rows)
constexpr int AWQ_WSTRIDE = 128 + 16;                // bytes per channel row of a wave's weight tile

__global__ __launch_bounds__(64 * AWQ_WAVES) void awq_w4a16_kernel(const uint16_t *__restrict__ X,
                                                                   const uint8_t *__restrict__ wq,
                                                                   const float *__restrict__ wscale,
                                                                   const uint16_t *__restrict__ bias, int M,
                                                                   int N, int K, uint16_t *__restrict__ Y)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // min(M, 16) rows x AWQ_XSTRIDE
    __shared__ f32x4 part[AWQ_WAVES][64];
    __shared__ __attribute__((aligned(16))) uint8_t wt[AWQ_WAVES][AWQ_COLS * AWQ_WSTRIDE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kb = lane >> 4;
    const int n = blockIdx.x * AWQ_COLS + col;
    const int nrow = n < N ? n : N - 1;              // rows past N read the last row, never stored
    const int chunks = K >> 8;
    const int slabs = (chunks + AWQ_WAVES - 1) / AWQ_WAVES;
    const int KB = K >> 1, G = K >> 6;
    // weight loads take whole 128-byte lines: 8 lanes per channel line, so
    // one load covers channels (lane / 8) and the other 8 + lane / 8
    const int l8 = lane >> 3, lp = 16 * (lane & 7);
    const int n0 = blockIdx.x * AWQ_COLS;
    const uint8_t *lrow0 = wq + (size_t)min(n0 + l8, N - 1) * KB + lp;
    const uint8_t *lrow1 = wq + (size_t)min(n0 + 8 + l8, N - 1) * KB + lp;
    uint8_t *mywt = wt[wave];
    const float *srow = wscale + (size_t)nrow * G;
    const bf16x8 neg136 = __builtin_bit_cast(bf16x8, (u32x4){kBf16_m136, kBf16_m136, kBf16_m136, kBf16_m136});

    for (int m0 = 0; m0 < M; m0 += 16) {
        const int mb = M - m0 < 16 ? M - m0 : 16;    // rows of X in this pass
        const bool mv = col < mb;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        // weights of the wave's chunk in slab 0
        u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
        float4 sw = make_float4(0.f, 0.f, 0.f, 0.f);
        if (wave < chunks) {
            w0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(lrow0 + 128 * wave));
            w1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(lrow1 + 128 * wave));
            sw = *reinterpret_cast<const float4 *>(srow + 4 * wave);
        }
        for (int s = 0; s < slabs; ++s) {
            // the pass's rows of X over the slab's channels into LDS
            const int k0 = s * AWQ_SLAB;
            for (int idx = tid; idx < mb * (AWQ_SLAB / 8); idx += 64 * AWQ_WAVES) {
                const int r = idx / (AWQ_SLAB / 8), j = idx % (AWQ_SLAB / 8);
                uint4 v = {0u, 0u, 0u, 0u};
                if (k0 + 8 * j < K) v = *reinterpret_cast<const uint4 *>(X + (size_t)(m0 + r) * K + k0 + 8 * j);
                *reinterpret_cast<uint4 *>(&xs[r * AWQ_XSTRIDE + 8 * j]) = v;
            }
            __syncthreads();
            const int c = s * AWQ_WAVES + wave;
            const u32x4 cw0 = w0, cw1 = w1;
            const float4 csw = sw;
            // next slab's weights are in flight while this one is computed
            const int cn = c + AWQ_WAVES;
            if (cn < chunks) {
                w0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(lrow0 + 128 * cn));
                w1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(lrow1 + 128 * cn));
                sw = *reinterpret_cast<const float4 *>(srow + 4 * cn);
            }
            if (c < chunks) {
                // the lines into the wave's tile, read back as the lane's 32
                // operand bytes (channel col, bytes 32 kb .. + 31)
                *reinterpret_cast<u32x4 *>(mywt + l8 * AWQ_WSTRIDE + lp) = cw0;
                *reinterpret_cast<u32x4 *>(mywt + (8 + l8) * AWQ_WSTRIDE + lp) = cw1;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const u32x4 ow0 = *reinterpret_cast<const u32x4 *>(mywt + col * AWQ_WSTRIDE + 32 * kb);
                const u32x4 ow1 = *reinterpret_cast<const u32x4 *>(mywt + col * AWQ_WSTRIDE + 32 * kb + 16);
                const uint32_t wd[8] = {ow0.x, ow0.y, ow0.z, ow0.w, ow1.x, ow1.y, ow1.z, ow1.w};
                const float swv[4] = {csw.x, csw.y, csw.z, csw.w};
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    bf16x8 a[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        uint4 xv = {0u, 0u, 0u, 0u};
                        if (mv) xv = *reinterpret_cast<const uint4 *>(&xs[col * AWQ_XSTRIDE + 256 * wave + 64 * g + 32 * h + 8 * kb]);
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
            __syncthreads();
        }
        // the 4 waves' partial sums, added in wave order
        part[wave][lane] = acc;
        __syncthreads();
        if (wave == 0) {
            f32x4 t = part[0][lane];
#pragma unroll
            for (int w = 1; w < AWQ_WAVES; ++w) {
                const f32x4 u = part[w][lane];
                t[0] += u[0]; t[1] += u[1]; t[2] += u[2]; t[3] += u[3];
            }
            const float b = (bias && n < N) ? __builtin_bit_cast(float, (uint32_t)bias[n] << 16) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mo = m0 + 4 * kb + i;     // output row of value i (D rows = A rows)
                if (mo < M && n < N) Y[(size_t)mo * N + n] = (uint16_t)bf16_bits_rne(t[i] + b);
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
    const size_t lds = (size_t)(M < 16 ? M : 16) * AWQ_XSTRIDE * sizeof(uint16_t);
    hipLaunchKernelGGL(awq_w4a16_kernel, dim3((unsigned)blocks), dim3(64 * AWQ_WAVES), lds, stream, X, wq, wscale,
                       bias, M, N, K, Y);
    return hipGetLastError();
}

}  // namespace svdq
