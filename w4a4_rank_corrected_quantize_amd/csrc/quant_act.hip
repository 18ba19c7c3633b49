// quant_act.hip -- fused activation kernel of the SVDQuant W4A4 linear
// ("Bringing Nunchaku 4-bit Diffusion Inference to Diffusers", section
// "Background: SVDQuant and Nunchaku": the low-rank down projection is fused
// with the quantization kernel, so X is read from HBM once).
//
// One pass over X computes, per row m and 64-wide group g (32-wide blocks for
// MXFP4):
//   xhat = fl32(X_mk * s_k)          (exact product, one rounding)
//   group absmax -> scale -> 4-bit codes, nibble-packed
//   h_mj = sum_k X_mk down[j][k]     (bf16 matrix cores, fp32 accumulation)
//
// Work decomposition (gfx950, wave64): a block owns 16 rows and all of K; its
// WAVES waves take the groups g = wave, wave + WAVES, ...  In a wave, lane l
// holds row l % 16 and the 16 consecutive channels 16 * (l / 16) .. + 15 of the
// group, which is exactly the operand layout of v_mfma_f32_16x16x32_bf16 (two
// instructions per group and per 16-column half of the rank).  The group
// absmax needs the four lanes l, l^16, l^32, l^48.  The per-wave partial h
// tiles are summed in a fixed order through LDS at the end (deterministic).
//
// Roofline: HBM-bound.  Algorithmic bytes per call: 2MK (X) + MK/2 (codes)
// + 4MK/64 (INT4 scales) or MK/32 (E8M0) + 4Mr (h) + 4K (s) + 2rK (down).
#include "svdq_internal.h"
#include "svdq_quant.h"

namespace svdq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int K1_ROWS = 16;
constexpr int K1_WAVES = 8;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return bits_f32(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return bits_f32(w & 0xFFFF0000u); }

// 16 consecutive channels of one row: bf16 -> fp32 and smoothing product.
__device__ __forceinline__ void smooth16(uint4 xa, uint4 xb, const float4 *s, float *v)
{
    const uint32_t w[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
    const float sv[16] = {s[0].x, s[0].y, s[0].z, s[0].w, s[1].x, s[1].y, s[1].z, s[1].w,
                          s[2].x, s[2].y, s[2].z, s[2].w, s[3].x, s[3].y, s[3].z, s[3].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf_lo(w[i]) * sv[2 * i];
        v[2 * i + 1] = bf_hi(w[i]) * sv[2 * i + 1];
    }
}

struct K1Load {
    uint4 xa, xb;          // 16 channels of X (bf16)
    uint4 d0a, d0b;        // down[rl][16 channels]
    uint4 d1a, d1b;        // down[rl + 16][16 channels]
    float4 s[4];           // smoothing factors of the 16 channels
};

template <bool MX>
__global__ __launch_bounds__(64 * K1_WAVES) void quant_act_kernel(
    const uint16_t *__restrict__ X, int M, int K, const float *__restrict__ smooth,
    const uint16_t *__restrict__ down, uint8_t *__restrict__ xq, void *__restrict__ xscale,
    float *__restrict__ h)
{
    __shared__ float red[K1_WAVES][K1_ROWS][2 * 16 + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rl = lane & 15, c = lane >> 4;
    const int row0 = blockIdx.x * K1_ROWS;
    const int row = row0 + rl;
    const bool rv = row < M;
    const int G = K >> 6;                       // INT4 groups per row
    const int steps = (K + 63) >> 6;            // 64-channel steps (MXFP4 may end on half a step)
    const size_t rowK = (size_t)(rv ? row : 0) * (size_t)K;
    const uint4 z4 = {0u, 0u, 0u, 0u};

    // Loads are unconditional (addresses clamped into the buffers) so that the
    // number of loads in flight is the same on every path and the next
    // group's loads can stay in flight while the current group is processed.
    // Rows >= M read row 0 and are never stored; channels past K (a trailing
    // half step of MXFP4) are masked out of the down projection at use.
    auto fetch = [&](int g, K1Load &L) {
        const int k0 = min(g * 64 + c * 16, K - 16);
        L.xa = *reinterpret_cast<const uint4 *>(X + rowK + k0);
        L.xb = *reinterpret_cast<const uint4 *>(X + rowK + k0 + 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) L.s[i] = *reinterpret_cast<const float4 *>(smooth + k0 + 4 * i);
        L.d0a = *reinterpret_cast<const uint4 *>(down + (size_t)rl * K + k0);
        L.d0b = *reinterpret_cast<const uint4 *>(down + (size_t)rl * K + k0 + 8);
        L.d1a = *reinterpret_cast<const uint4 *>(down + (size_t)(rl + 16) * K + k0);
        L.d1b = *reinterpret_cast<const uint4 *>(down + (size_t)(rl + 16) * K + k0 + 8);
    };

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    auto process = [&](int g, const K1Load &L) {
            const int k0 = g * 64 + c * 16;
            const bool kv = k0 < K;                 // false only in a trailing half step

            // down projection: D[m][j] += sum_k X[m][k] down[j][k]
            uint4 d0a = L.d0a, d0b = L.d0b, d1a = L.d1a, d1b = L.d1b;
            if (MX && !kv) d0a = d0b = d1a = d1b = z4;
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(L.xa), as_bf16x8(d0a), acc0, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(L.xb), as_bf16x8(d0b), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(L.xa), as_bf16x8(d1a), acc1, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(L.xb), as_bf16x8(d1b), acc1, 0, 0, 0);

            float v[16];
            smooth16(L.xa, L.xb, L.s, v);
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
            // sign bits of the 16 codes (bit 3 of each nibble), from the fp32 values
            uint32_t sg0 = 0, sg1 = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sg0 |= (f32_bits(v[i]) >> 31) << (4 * i + 3);
                sg1 |= (f32_bits(v[8 + i]) >> 31) << (4 * i + 3);
            }
            uint32_t p0 = 0, p1 = 0;
            if constexpr (!MX) {
                a = __builtin_fmaxf(a, __shfl_xor(a, 16));
                a = __builtin_fmaxf(a, __shfl_xor(a, 32));
                const float scale = int4_group_scale(a);
                const bool lifted = scale < 7.88860905e-31f;      // 2^-100: exact path only
                const float inv = scale == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(scale);
                bool near = lifted;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float t = __builtin_fabsf(v[i]) * inv;
                    const float q = __builtin_rintf(t);
                    near |= __builtin_fabsf(t - q) >= kNearTie;
                    const uint32_t m = (uint32_t)q;
                    if (i < 8) p0 |= m << (4 * i);
                    else p1 |= m << (4 * (i - 8));
                }
                if (near) {                                       // rare: exact remainder test
                    const Int4Group gq = int4_group_prepare(scale);
                    p0 = p1 = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        p0 |= int4_mag(__builtin_fabsf(v[i]), gq) << (4 * i);
                        p1 |= int4_mag(__builtin_fabsf(v[8 + i]), gq) << (4 * i);
                    }
                }
                p0 |= sg0;
                p1 |= sg1;
                if (rv && c == 0) reinterpret_cast<float *>(xscale)[(size_t)row * G + g] = scale;
            } else {
                // two 32-wide blocks per step: lanes c = 0,1 -> block 2g, c = 2,3 -> block 2g+1
                a = __builtin_fmaxf(a, __shfl_xor(a, 16));
                const uint32_t e = mx_block_e8m0(a);
                const float inv = mx_inv_scale(e);
#pragma unroll
                for (int i = 0; i < 8; ++i) p0 |= e2m1_code(v[i], inv) << (4 * i);
#pragma unroll
                for (int i = 0; i < 8; ++i) p1 |= e2m1_code(v[8 + i], inv) << (4 * i);
                if (rv && kv && (c & 1) == 0)
                    reinterpret_cast<uint8_t *>(xscale)[(size_t)row * (K >> 5) + 2 * g + (c >> 1)] = (uint8_t)e;
            }
            if (rv && kv) {
                uint2 pk = {p0, p1};
                *reinterpret_cast<uint2 *>(xq + (size_t)row * (K >> 1) + (k0 >> 1)) = pk;
            }
    };

    // ping-pong register buffers: the loads of the next group are in flight
    // while the current one is processed
    K1Load bufA, bufB;
    int g = wave;
    if (g < steps) fetch(g, bufA);
    for (; g < steps; g += 2 * K1_WAVES) {
        const int g1 = g + K1_WAVES;
        fetch(min(g1, steps - 1), bufB);
        process(g, bufA);
        if (g1 >= steps) break;
        fetch(min(g1 + K1_WAVES, steps - 1), bufA);
        process(g1, bufB);
    }

    // fixed-order reduction of the per-wave partial h tiles
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        red[wave][4 * c + i][rl] = acc0[i];
        red[wave][4 * c + i][rl + 16] = acc1[i];
    }
    __syncthreads();
    for (int t = threadIdx.x; t < K1_ROWS * 32; t += 64 * K1_WAVES) {
        const int m = t >> 5, j = t & 31;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < K1_WAVES; ++w) sum += red[w][m][j];
        if (row0 + m < M) h[(size_t)(row0 + m) * 32 + j] = sum;
    }
}

}  // namespace

hipError_t launch_quant_act(const uint16_t *X, int M, int K, const float *smooth, const uint16_t *down,
                            svdq_precision prec, uint8_t *xq, void *xscale, float *h, hipStream_t stream)
{
    const dim3 grid((unsigned)((M + K1_ROWS - 1) / K1_ROWS)), block(64 * K1_WAVES);
    if (prec == SVDQ_INT4)
        hipLaunchKernelGGL(quant_act_kernel<false>, grid, block, 0, stream, X, M, K, smooth, down, xq,
                           xscale, h);
    else
        hipLaunchKernelGGL(quant_act_kernel<true>, grid, block, 0, stream, X, M, K, smooth, down, xq,
                           xscale, h);
    return hipGetLastError();
}

}  // namespace svdq
