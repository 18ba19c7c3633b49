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
// Work decomposition (gfx950, wave64).  The kernel is HBM-bound, so every
// global access is a run of full 128-byte lines:
//   * a block owns R consecutive rows (R at most 32, chosen so that there is
//     about one block per CU) and all of K; its 8 waves (two per SIMD) take
//     the 128-channel chunks c = wave, wave + 8, ...
//   * a chunk is loaded as NL = ceil(R / 4) loads of 4 rows: each quarter of
//     the wave reads 256 contiguous bytes of one row (lane l holds channels
//     8 (l % 16) .. + 7 of row 4 i + l / 16); the next chunk's loads are in
//     flight while this one is processed;
//   * a quantization group is 8 neighbouring lanes (4 for MXFP4), so the
//     group absmax takes three DPP steps, and each lane writes its 8 codes as
//     one dword: 64 contiguous code bytes per row per load;
//   * the down projection needs X in the matrix-core operand layout (one row
//     per lane), so each wave copies its chunk into its own LDS tile and reads
//     it back transposed for v_mfma_f32_32x32x16_bf16 (A = down rows j,
//     B = X^T columns m: one 32-row tile covers the block);
//   * the chunk's slice of down (32 rows x 256 bytes) takes the same route:
//     loaded as 8 runs of 4 rows x 256 contiguous bytes (8 full lines per
//     load, where the operand layout would touch 32 lines per load) into a
//     second LDS tile of the wave, and read back as the A operands;
//   * the per-wave partial h tiles are summed in a fixed order through LDS at
//     the end (deterministic).
//
// Roofline: HBM-bound.  Algorithmic bytes per call: 2MK (X) + MK/2 (codes)
// + 4MK/64 (INT4 scales) or MK/32 (E8M0) + 4Mr (h) + 4K (s) + 2rK (down).
#include "svdq_internal.h"
#include "svdq_quant.h"

namespace svdq {
namespace {

// X is read exactly once: non-temporal loads leave the L2 to the outputs,
// which the linear kernel reads next.
__device__ __forceinline__ uint4 load_nt(const uint16_t *p)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int K1_WAVES = 8;
constexpr int K1_CH = 128;                  // channels per chunk
constexpr int K1_LPR = K1_CH / 8;           // lanes per row in a load (8 channels each)
constexpr int K1_RPL = 64 / K1_LPR;         // rows per load
constexpr int K1_RMAX = 32;                 // rows per block, at most (one 32-row product tile)
constexpr int K1_TILE_STRIDE = 2 * K1_CH + 16;   // LDS bytes per row of a wave's X tile

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return bits_f32(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return bits_f32(w & 0xFFFF0000u); }

// max over the 8 (or 4) lanes of a quantization group, via DPP
template <int LANES>
__device__ __forceinline__ float group_max(float a)
{
    a = __builtin_fmaxf(a, bits_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)f32_bits(a), 0xB1, 0xF, 0xF, false)));
    a = __builtin_fmaxf(a, bits_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)f32_bits(a), 0x4E, 0xF, 0xF, false)));
    if constexpr (LANES == 8)   // row_half_mirror: lane i <-> 7 - i within each group of 8
        a = __builtin_fmaxf(a, bits_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)f32_bits(a), 0x141, 0xF, 0xF, false)));
    return a;
}

// Sign bits of the lane's 8 values xhat, at bit 3 of each code nibble
// (element 2e -> bit 8e + 3, element 2e + 1 -> bit 8e + 7): byte 3 of each
// fp32 value carries its sign in bit 7.
__device__ __forceinline__ uint32_t sign_bits(const float *v)
{
    const uint32_t ea = __builtin_amdgcn_perm(f32_bits(v[2]), f32_bits(v[0]), 0x0c0c0703u);   // v0 v2 . .
    const uint32_t eb = __builtin_amdgcn_perm(f32_bits(v[6]), f32_bits(v[4]), 0x07030c0cu);   // . . v4 v6
    const uint32_t oa = __builtin_amdgcn_perm(f32_bits(v[3]), f32_bits(v[1]), 0x0c0c0703u);
    const uint32_t ob = __builtin_amdgcn_perm(f32_bits(v[7]), f32_bits(v[5]), 0x07030c0cu);
    return (((ea | eb) >> 4) & 0x08080808u) | ((oa | ob) & 0x80808080u);
}

template <int NL>
struct K1Chunk {
    uint4 x[NL];           // load i: lane l holds row 4 i + l / 16
    float4 s0, s1;         // smoothing factors of the lane's 8 channels
};

template <bool MX, int NL>
__global__ __launch_bounds__(64 * K1_WAVES) void quant_act_kernel(
    const uint16_t *__restrict__ X, int M, int K, int R, const float *__restrict__ smooth,
    const uint16_t *__restrict__ down, uint8_t *__restrict__ xq, void *__restrict__ xscale,
    float *__restrict__ h)
{
    // per wave: the X tile, then the down tile; the final reduction reuses
    // the space once every wave has left its loop
    constexpr int kTile = K1_RMAX * K1_TILE_STRIDE;
    __shared__ __attribute__((aligned(16))) uint8_t smem[K1_WAVES * 2 * kTile];
    static_assert(sizeof(float) * K1_WAVES * 32 * 33 <= sizeof(smem), "reduction fits in the tiles");
    float(*red)[32][33] = reinterpret_cast<float(*)[32][33]>(smem);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row0 = blockIdx.x * R;
    const int nrow = min(R, M - row0);      // 1 <= nrow <= 4 NL (the grid is sized by the host)
    const int nch = (K + K1_CH - 1) / K1_CH;
    const int rq = lane / K1_LPR;           // row within a load
    const int kl = 8 * (lane % K1_LPR);     // first channel of the lane within a chunk
    const int hk = lane >> 5;               // half of the product operand (channels 8 hk .. + 7)
    const int KB = K >> 1;                  // code bytes per row
    uint8_t *mytile = smem + wave * 2 * kTile;
    uint8_t *mydown = mytile + kTile;

    // Loads are unconditional (addresses clamped into the buffers), so the
    // number of loads in flight is the same on every path: a row past the
    // block's last row reads that last row and stores nothing; channels past
    // K read the last 8 channels and store nothing (their groups lie entirely
    // past K, since K is a multiple of the group size).
    auto fetch = [&](int c, K1Chunk<NL> &L) {
        const int k = min(c * K1_CH + kl, K - 8);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int r = min(K1_RPL * i + rq, nrow - 1);
            L.x[i] = load_nt(X + (size_t)(row0 + r) * K + k);
        }
        L.s0 = *reinterpret_cast<const float4 *>(smooth + k);
        L.s1 = *reinterpret_cast<const float4 *>(smooth + k + 4);
    };

    f32x16 acc = {};
    // Process chunk c from L while the loads of chunk cn go into Ln.  The
    // down operand of chunk c is loaded first, so waiting for it before the
    // products does not wait for chunk cn.
    auto process = [&](int c, const K1Chunk<NL> &L, int cn, K1Chunk<NL> &Ln) {
        const int kc = c * K1_CH + kl;
        const bool kv = kc < K;
        // the chunk's slice of down, row 4 t + lane / 16, channels
        // kc .. kc + 7 (clamped into the buffer; zeroed past K below)
        uint4 dn[32 / K1_RPL];
#pragma unroll
        for (int t = 0; t < 32 / K1_RPL; ++t)
            dn[t] = *reinterpret_cast<const uint4 *>(down + (size_t)(K1_RPL * t + rq) * K + min(kc, K - 8));
        fetch(cn, Ln);
        const float sv[8] = {L.s0.x, L.s0.y, L.s0.z, L.s0.w, L.s1.x, L.s1.y, L.s1.z, L.s1.w};
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const uint4 w = L.x[i];
            const int rloc = K1_RPL * i + rq;
            if (rloc < K1_RMAX) *reinterpret_cast<uint4 *>(mytile + rloc * K1_TILE_STRIDE + 2 * kl) = w;
            const bool st = kv && rloc < nrow;
            const size_t row = (size_t)(row0 + rloc);
            const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = bf_lo(wv[e]) * sv[2 * e];
                v[2 * e + 1] = bf_hi(wv[e]) * sv[2 * e + 1];
            }
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(v[e]));
            uint32_t code;
            if constexpr (!MX) {
                a = group_max<8>(a);
                const float scale = int4_group_scale(a);
                const bool lifted = scale < 7.88860905e-31f;      // 2^-100: exact path only
                const float inv = scale == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(scale);
                float q[8], dmax = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float t = __builtin_fabsf(v[e]) * inv;
                    q[e] = __builtin_rintf(t);
                    dmax = __builtin_fmaxf(dmax, __builtin_fabsf(t - q[e]));
                }
                if (lifted || dmax >= kNearTie) {                 // rare: exact remainder test
                    const Int4Group gq = int4_group_prepare(scale);
#pragma unroll
                    for (int e = 0; e < 8; ++e) q[e] = (float)int4_mag(__builtin_fabsf(v[e]), gq);
                }
                uint32_t ev = 0, od = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ev = __builtin_amdgcn_cvt_pk_u8_f32(q[2 * e], e, ev);
                    od = __builtin_amdgcn_cvt_pk_u8_f32(q[2 * e + 1], e, od);
                }
                code = (ev | (od << 4)) | sign_bits(v);
                if (st && (lane & 7) == 0) reinterpret_cast<float *>(xscale)[row * (K >> 6) + (kc >> 6)] = scale;
            } else {
                a = group_max<4>(a);
                const uint32_t e8 = mx_block_e8m0(a);
                const float inv = mx_inv_scale(e8);
                // t = xhat 2^-X is exact and below 16; the hardware E2M1
                // conversion (unit scale) rounds to the grid with ties to the
                // even index, saturates at 6 and keeps the sign of zero
                // (tests/native/e2m1_sweep.hip checks this on the GPU for every
                // fp32 t with |t| < 16, both signs)
                code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0] * inv, v[1] * inv, 1.0f, 0);
                code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(code, v[2] * inv, v[3] * inv, 1.0f, 1);
                code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(code, v[4] * inv, v[5] * inv, 1.0f, 2);
                code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(code, v[6] * inv, v[7] * inv, 1.0f, 3);
                if (st && (lane & 3) == 0) reinterpret_cast<uint8_t *>(xscale)[row * (K >> 5) + (kc >> 5)] = (uint8_t)e8;
            }
            if (st) *reinterpret_cast<uint32_t *>(xq + row * KB + (kc >> 1)) = code;
        }
        // down rows into the wave's down tile; channels past K (last, partial
        // chunk) add nothing
#pragma unroll
        for (int t = 0; t < 32 / K1_RPL; ++t)
            *reinterpret_cast<uint4 *>(mydown + (K1_RPL * t + rq) * K1_TILE_STRIDE + 2 * kl) =
                kv ? dn[t] : (uint4){0u, 0u, 0u, 0u};
        // the tile rows written above are read back by other lanes of this wave
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // h^T[j][m] += sum_k down[j][k] X[m][k] over the chunk (A: row j =
        // lane % 32, channels 16 t + 8 (lane / 32) .. + 7; B the same channels
        // of row m = lane % 32); rows m >= nrow read the last row (their
        // outputs are dropped)
        const uint8_t *src = mytile + min(lane & 31, nrow - 1) * K1_TILE_STRIDE + 16 * hk;
        const uint8_t *dsrc = mydown + (lane & 31) * K1_TILE_STRIDE + 16 * hk;
#pragma unroll
        for (int t = 0; t < K1_CH / 16; ++t) {
            const uint4 a = *reinterpret_cast<const uint4 *>(dsrc + 32 * t);
            const uint4 b = *reinterpret_cast<const uint4 *>(src + 32 * t);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
        }
        // the next chunk overwrites the tile only after every lane has read it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // ping-pong register buffers: the next chunk's loads are in flight while
    // the current one is processed
    K1Chunk<NL> bufA, bufB;
    int c = wave;
    if (c < nch) fetch(c, bufA);
    for (; c < nch; c += 2 * K1_WAVES) {
        // the prefetch is unconditional (clamped): same load count on every path
        const int c1 = c + K1_WAVES;
        process(c, bufA, min(c1, nch - 1), bufB);
        if (c1 >= nch) break;
        process(c1, bufB, min(c1 + K1_WAVES, nch - 1), bufA);
    }

    // fixed-order reduction of the per-wave partial h^T tiles; lane l holds
    // column m = l % 32 and rows j = 8 (i / 4) + 4 (l / 32) + i % 4.  The
    // partials overwrite the tiles, so every wave must be done with its own.
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave][lane & 31][8 * (i >> 2) + 4 * hk + (i & 3)] = acc[i];
    __syncthreads();
    for (int t = threadIdx.x; t < nrow * 32; t += 64 * K1_WAVES) {
        const int m = t >> 5, j = t & 31;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < K1_WAVES; ++w) sum += red[w][m][j];
        h[(size_t)(row0 + m) * 32 + j] = sum;
    }
}

}  // namespace

hipError_t launch_quant_act(const uint16_t *X, int M, int K, const float *smooth, const uint16_t *down,
                            svdq_precision prec, uint8_t *xq, void *xscale, float *h, hipStream_t stream)
{
    // rows per block: about one block per CU, at most one 32-row product tile
    const int ncu = device_cu_count();
    int R = (M + ncu - 1) / ncu;
    R = R < 1 ? 1 : (R > K1_RMAX ? K1_RMAX : R);
    const int nl = (R + K1_RPL - 1) / K1_RPL;           // loads per chunk
    const dim3 grid((unsigned)((M + R - 1) / R)), block(64 * K1_WAVES);
#define K1_LAUNCH(N)                                                                                    \
    case N:                                                                                             \
        if (prec == SVDQ_INT4)                                                                          \
            hipLaunchKernelGGL((quant_act_kernel<false, N>), grid, block, 0, stream, X, M, K, R, smooth, \
                               down, xq, xscale, h);                                                    \
        else                                                                                            \
            hipLaunchKernelGGL((quant_act_kernel<true, N>), grid, block, 0, stream, X, M, K, R, smooth,  \
                               down, xq, xscale, h);                                                    \
        break;
    switch (nl) {
        K1_LAUNCH(1)
        K1_LAUNCH(2)
        K1_LAUNCH(3)
        K1_LAUNCH(4)
        K1_LAUNCH(5)
        K1_LAUNCH(6)
        K1_LAUNCH(7)
        K1_LAUNCH(8)
    }
#undef K1_LAUNCH
    return hipGetLastError();
}

}  // namespace svdq
