// w4a4_gemm.hip -- the 4-bit x 4-bit product of the SVDQuant W4A4 linear with
// the fused low-rank up projection, bias, optional GELU-tanh and bf16 store
// ("Bringing Nunchaku 4-bit Diffusion Inference to Diffusers", section
// "Background: SVDQuant and Nunchaku": the low-rank up projection is fused
// with the 4-bit compute kernel; section "Introducing Nunchaku Lite": fused
// GELU/MLP paths).
//
//   y_mn = sum_g sx_mg sw_ng P_mng + sum_j h_mj up[n][j] + b_n   [GELU-tanh]
//
// INT4: P_mng = sum_{k in g} qx_mk qw_nk is an exact int32 from
// v_mfma_i32_16x16x64_i8 (one instruction = one 64-wide group for a 16x16
// tile).  The nibbles are widened to int8 in registers with two masks and a
// shift, which yields 16 q instead of q (no sign extension needed), so the
// instruction returns 256 P; the 2^-8 is applied once at the end (exact).  The
// rescale acc += fl(P) * (sx * sw) is fp32 VALU work (convert, multiply, fma
// per element and group), which is what bounds this kernel on gfx950.
//
// MXFP4: the E2M1 nibbles are the native fp4 operand format of
// v_mfma_scale_f32_16x16x128_f8f6f4 and the E8M0 block scales are its scale
// operands, so the matrix core applies 2^(ex + ew) itself and accumulates
// across blocks; no per-block VALU work remains.
//
// Tiling: a 256-thread block owns a BM x BN tile (m: tokens, n: output
// channels); 4 waves in a 2 x 2 arrangement each own (BM/2) x (BN/2).  Codes
// are staged through LDS, double buffered, one barrier per K step.  The matrix
// instruction's A operand is the weight tile (rows n) and B the activation tile
// (columns m), so each lane ends with 4 consecutive output channels n of one
// token m, i.e. one 8-byte bf16 store per 16x16 tile.
//
// Low-rank epilogue: h (fp32) is split into bf16 hi = bf16(h) and lo =
// bf16(h - hi); two v_mfma_f32_16x16x32_bf16 per tile with `up` as the other
// operand give h . up to ~16 bits, well inside the output tolerance.
#include "svdq_internal.h"
#include "svdq_quant.h"

namespace svdq {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 128;          // block tile (m, n)
constexpr int WM = 64, WN = 64;            // wave tile
constexpr int TM = WM / 16, TN = WN / 16;  // 16x16 tiles per wave
constexpr int NTHREADS = 256;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return bits_f32(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = f32_bits(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float gelu_tanh(float y)
{
    const float k0 = 0.7978845608028654f;   // sqrt(2/pi)
    return 0.5f * y * (1.0f + tanhf(k0 * (y + 0.044715f * y * y * y)));
}

// 16 INT4 codes (8 bytes) -> 16 int8 holding 16 q each.  Byte order inside
// the result is a fixed permutation of the k order, identical for both
// operands, so the dot products are unchanged.
__device__ __forceinline__ i32x4 widen16(uint2 p)
{
    i32x4 r;
    r[0] = (int)((p.x << 4) & 0xF0F0F0F0u);
    r[1] = (int)(p.x & 0xF0F0F0F0u);
    r[2] = (int)((p.y << 4) & 0xF0F0F0F0u);
    r[3] = (int)(p.y & 0xF0F0F0F0u);
    return r;
}

// Low-rank term + bias (+ GELU) + bf16 store for one wave's (WN x WM) tile.
// acc[tn][tm][i] holds the 4-bit product of token m = mb + tm*16 + (lane&15)
// and channel n = nb + tn*16 + 4*(lane>>4) + i.
__device__ __forceinline__ void epilogue(f32x4 (&acc)[TN][TM], float acc_scale, const float *__restrict__ h,
                                         const uint16_t *__restrict__ up, const uint16_t *__restrict__ bias,
                                         int M, int N, int gelu, uint16_t *__restrict__ Y, int mb, int nb,
                                         int lane)
{
    const int l16 = lane & 15, c = lane >> 4;
    bf16x8 hhi[TM], hlo[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int m = mb + tm * 16 + l16;
        float hv[8];
        if (m < M) {
            const float4 a = *reinterpret_cast<const float4 *>(h + (size_t)m * 32 + 8 * c);
            const float4 b = *reinterpret_cast<const float4 *>(h + (size_t)m * 32 + 8 * c + 4);
            hv[0] = a.x; hv[1] = a.y; hv[2] = a.z; hv[3] = a.w;
            hv[4] = b.x; hv[5] = b.y; hv[6] = b.z; hv[7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) hv[i] = 0.0f;
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t h0 = f32_to_bf16_rne(hv[2 * i]), h1 = f32_to_bf16_rne(hv[2 * i + 1]);
            const uint32_t l0 = f32_to_bf16_rne(hv[2 * i] - bf16_to_f32(h0));
            const uint32_t l1 = f32_to_bf16_rne(hv[2 * i + 1] - bf16_to_f32(h1));
            hi[i] = h0 | (h1 << 16);
            lo[i] = l0 | (l1 << 16);
        }
        hhi[tm] = __builtin_bit_cast(bf16x8, (uint4){hi[0], hi[1], hi[2], hi[3]});
        hlo[tm] = __builtin_bit_cast(bf16x8, (uint4){lo[0], lo[1], lo[2], lo[3]});
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const int nrow = nb + tn * 16 + l16;       // A-operand row of `up`
        uint4 uv = {0u, 0u, 0u, 0u};
        if (nrow < N) uv = *reinterpret_cast<const uint4 *>(up + (size_t)nrow * 32 + 8 * c);
        const bf16x8 ua = __builtin_bit_cast(bf16x8, uv);
        const int n = nb + tn * 16 + 4 * c;        // this lane's 4 output channels
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias && n < N) {
            const uint2 b2 = *reinterpret_cast<const uint2 *>(bias + n);
            bv[0] = bf16_to_f32(b2.x & 0xFFFFu); bv[1] = bf16_to_f32(b2.x >> 16);
            bv[2] = bf16_to_f32(b2.y & 0xFFFFu); bv[3] = bf16_to_f32(b2.y >> 16);
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            f32x4 lr = {0.f, 0.f, 0.f, 0.f};
            lr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua, hhi[tm], lr, 0, 0, 0);
            lr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua, hlo[tm], lr, 0, 0, 0);
            const int m = mb + tm * 16 + l16;
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float y = acc[tn][tm][i] * acc_scale + lr[i] + bv[i];
                if (gelu) y = gelu_tanh(y);
                o[i] = f32_to_bf16_rne(y);
            }
            if (m < M && n < N) {
                const uint2 st = {o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
                *reinterpret_cast<uint2 *>(Y + (size_t)m * N + n) = st;
            }
        }
    }
}

// ----------------------------------------------------------------- INT4

constexpr int I4_STRIDE = 48;   // LDS bytes per row: 32 code bytes + 16 pad

__global__ __launch_bounds__(NTHREADS) void w4a4_int4_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ xscale, const float *__restrict__ h,
    const uint8_t *__restrict__ wq, const float *__restrict__ wscale, const uint16_t *__restrict__ up,
    const uint16_t *__restrict__ bias, int M, int N, int K, int gelu, uint16_t *__restrict__ Y)
{
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][BN * I4_STRIDE];
    __shared__ __attribute__((aligned(16))) uint8_t sX[2][BM * I4_STRIDE];
    __shared__ float sSw[2][BN];
    __shared__ float sSx[2][BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
    const int G = K >> 6;
    const int KB = K >> 1;     // code bytes per row

    // loader: thread t moves 16 code bytes of row t/2 (both tiles) and one scale
    const int lrow = tid >> 1, lhalf = tid & 1;
    const bool wrow_ok = n0 + lrow < N, xrow_ok = m0 + lrow < M;
    const uint8_t *wsrc = wq + (size_t)(wrow_ok ? n0 + lrow : 0) * KB + lhalf * 16;
    const uint8_t *xsrc = xq + (size_t)(xrow_ok ? m0 + lrow : 0) * KB + lhalf * 16;
    const bool is_w_scale = tid < BN;
    const int srow = is_w_scale ? n0 + tid : m0 + (tid - BN);
    const bool srow_ok = is_w_scale ? srow < N : srow < M;
    const float *ssrc = (is_w_scale ? wscale : xscale) + (size_t)(srow_ok ? srow : 0) * G;
    const uint4 z4 = {0u, 0u, 0u, 0u};

    uint4 rw, rx;
    float rs;
    auto gload = [&](int g) {
        rw = wrow_ok ? *reinterpret_cast<const uint4 *>(wsrc + g * 32) : z4;
        rx = xrow_ok ? *reinterpret_cast<const uint4 *>(xsrc + g * 32) : z4;
        rs = srow_ok ? ssrc[g] : 0.0f;
    };
    auto lstore = [&](int buf) {
        *reinterpret_cast<uint4 *>(&sW[buf][lrow * I4_STRIDE + lhalf * 16]) = rw;
        *reinterpret_cast<uint4 *>(&sX[buf][lrow * I4_STRIDE + lhalf * 16]) = rx;
        if (is_w_scale) sSw[buf][tid] = rs;
        else sSx[buf][tid - BN] = rs;
    };

    f32x4 acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};

    if (G > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();
    const int l16 = lane & 15, c = lane >> 4;
    const i32x4 zi = {0, 0, 0, 0};
    for (int g = 0; g < G; ++g) {
        const int buf = g & 1;
        if (g + 1 < G) gload(g + 1);
        i32x4 aw[TN], bx[TM];
        float4 sw[TN];
        float sx[TM];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int r = wn * WN + tn * 16 + l16;
            aw[tn] = widen16(*reinterpret_cast<const uint2 *>(&sW[buf][r * I4_STRIDE + 8 * c]));
            sw[tn] = *reinterpret_cast<const float4 *>(&sSw[buf][wn * WN + tn * 16 + 4 * c]);
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int r = wm * WM + tm * 16 + l16;
            bx[tm] = widen16(*reinterpret_cast<const uint2 *>(&sX[buf][r * I4_STRIDE + 8 * c]));
            sx[tm] = sSx[buf][r];
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const i32x4 p = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[tn], bx[tm], zi, 0, 0, 0);
                acc[tn][tm][0] = __builtin_fmaf((float)p[0], sw[tn].x * sx[tm], acc[tn][tm][0]);
                acc[tn][tm][1] = __builtin_fmaf((float)p[1], sw[tn].y * sx[tm], acc[tn][tm][1]);
                acc[tn][tm][2] = __builtin_fmaf((float)p[2], sw[tn].z * sx[tm], acc[tn][tm][2]);
                acc[tn][tm][3] = __builtin_fmaf((float)p[3], sw[tn].w * sx[tm], acc[tn][tm][3]);
            }
        }
        if (g + 1 < G) lstore(buf ^ 1);
        __syncthreads();
    }
    epilogue(acc, 1.0f / 256.0f, h, up, bias, M, N, gelu, Y, m0 + wm * WM, n0 + wn * WN, lane);
}

// ---------------------------------------------------------------- MXFP4

constexpr int MX_STRIDE = 80;   // LDS bytes per row: 64 code bytes (128 fp4) + 16 pad

__global__ __launch_bounds__(NTHREADS) void w4a4_mxfp4_kernel(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ xscale, const float *__restrict__ h,
    const uint8_t *__restrict__ wq, const uint8_t *__restrict__ wscale, const uint16_t *__restrict__ up,
    const uint16_t *__restrict__ bias, int M, int N, int K, int gelu, uint16_t *__restrict__ Y)
{
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][BN * MX_STRIDE];
    __shared__ __attribute__((aligned(16))) uint8_t sX[2][BM * MX_STRIDE];
    __shared__ uint32_t sEw[2][BN];
    __shared__ uint32_t sEx[2][BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
    const int KB = K >> 1;          // code bytes per row
    const int NB = K >> 5;          // E8M0 scales per row
    const int steps = (K + 127) >> 7;

    // loader: thread t moves 2 x 16 code bytes of row t/2 for each tile, and
    // the 4 scale bytes of one row
    const int lrow = tid >> 1, lseg = (tid & 1) * 2;   // segments lseg, lseg+1 of 4
    const bool wrow_ok = n0 + lrow < N, xrow_ok = m0 + lrow < M;
    const uint8_t *wsrc = wq + (size_t)(wrow_ok ? n0 + lrow : 0) * KB;
    const uint8_t *xsrc = xq + (size_t)(xrow_ok ? m0 + lrow : 0) * KB;
    const bool is_w_scale = tid < BN;
    const int srow = is_w_scale ? n0 + tid : m0 + (tid - BN);
    const bool srow_ok = is_w_scale ? srow < N : srow < M;
    const uint8_t *ssrc = (is_w_scale ? wscale : xscale) + (size_t)(srow_ok ? srow : 0) * NB;
    const uint4 z4 = {0u, 0u, 0u, 0u};

    uint4 rw[2], rx[2];
    uint32_t rs;
    auto gload = [&](int st) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int blk = st * 4 + lseg + s;          // 32-wide block index
            const bool kv = blk < NB;
            rw[s] = (wrow_ok && kv) ? *reinterpret_cast<const uint4 *>(wsrc + blk * 16) : z4;
            rx[s] = (xrow_ok && kv) ? *reinterpret_cast<const uint4 *>(xsrc + blk * 16) : z4;
        }
        rs = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int blk = st * 4 + b;
            const uint32_t e = (srow_ok && blk < NB) ? (uint32_t)ssrc[blk] : 127u;
            rs |= e << (8 * b);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            *reinterpret_cast<uint4 *>(&sW[buf][lrow * MX_STRIDE + (lseg + s) * 16]) = rw[s];
            *reinterpret_cast<uint4 *>(&sX[buf][lrow * MX_STRIDE + (lseg + s) * 16]) = rx[s];
        }
        if (is_w_scale) sEw[buf][tid] = rs;
        else sEx[buf][tid - BN] = rs;
    };

    f32x4 acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};

    if (steps > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();
    const int l16 = lane & 15, c = lane >> 4;
    for (int st = 0; st < steps; ++st) {
        const int buf = st & 1;
        if (st + 1 < steps) gload(st + 1);
        i32x8 aw[TN], bx[TM];
        int ew[TN], ex[TM];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int r = wn * WN + tn * 16 + l16;
            const uint4 v = *reinterpret_cast<const uint4 *>(&sW[buf][r * MX_STRIDE + 16 * c]);
            aw[tn] = (i32x8){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            ew[tn] = (int)((sEw[buf][r] >> (8 * c)) & 0xFFu);
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int r = wm * WM + tm * 16 + l16;
            const uint4 v = *reinterpret_cast<const uint4 *>(&sX[buf][r * MX_STRIDE + 16 * c]);
            bx[tm] = (i32x8){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            ex[tm] = (int)((sEx[buf][r] >> (8 * c)) & 0xFFu);
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
                acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    aw[tn], bx[tm], acc[tn][tm], 4, 4, 0, ew[tn], 0, ex[tm]);
        if (st + 1 < steps) lstore(buf ^ 1);
        __syncthreads();
    }
    epilogue(acc, 1.0f, h, up, bias, M, N, gelu, Y, m0 + wm * WM, n0 + wn * WN, lane);
}

}  // namespace

hipError_t launch_w4a4_linear(const uint8_t *xq, const void *xscale, const float *h, const uint8_t *wq,
                              const void *wscale, const uint16_t *up, const uint16_t *bias, int M, int N,
                              int K, svdq_precision prec, svdq_epilogue epi, uint16_t *Y, hipStream_t stream)
{
    const dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN)), block(NTHREADS);
    const int gelu = epi == SVDQ_EPI_GELU_TANH ? 1 : 0;
    if (prec == SVDQ_INT4)
        hipLaunchKernelGGL(w4a4_int4_kernel, grid, block, 0, stream, xq, (const float *)xscale, h, wq,
                           (const float *)wscale, up, bias, M, N, K, gelu, Y);
    else
        hipLaunchKernelGGL(w4a4_mxfp4_kernel, grid, block, 0, stream, xq, (const uint8_t *)xscale, h, wq,
                           (const uint8_t *)wscale, up, bias, M, N, K, gelu, Y);
    return hipGetLastError();
}

}  // namespace svdq
