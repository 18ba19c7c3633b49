// w4a4_gemm.hip -- the 4-bit x 4-bit product of the SVDQuant W4A4 linear with
// the fused low-rank up projection, bias, optional GELU-tanh and bf16 store
// ("Bringing Nunchaku 4-bit Diffusion Inference to Diffusers", section
// "Background: SVDQuant and Nunchaku": the low-rank up projection is fused
// with the 4-bit compute kernel; section "Introducing Nunchaku Lite": fused
// GELU/MLP paths).
//
//   y_mn = sum_g sx_mg sw_ng P_mng + sum_j h_mj up[n][j] + b_n   [GELU-tanh]
//
// INT4: the codes are sign-magnitude nibbles (sign << 3 | |q|).  Widened to a
// byte as sign << 7 | |q| they are exact E4M3 values q * 2^-9 (E4M3
// subnormals), so v_mfma_f32_32x32x64_f8f6f4 in fp8 mode returns the exact
// per-group integer dot product P_mng * 2^-18 in fp32 (|P| <= 3136): one
// instruction covers exactly one 64-wide group of a 32x32 tile.  The nibbles
// are widened once per block while staging them into LDS (three bit
// operations per four codes).
//
// The per-group scale of a 32x32 tile is the outer product sx_g (x) sw_g; it
// comes from the bf16 matrix instruction as well, from hi/lo splits of both
// scales (s = hi + lo, hi = bf16(s), lo = bf16(s - hi)):
//     C_nm = sw_hi sx_hi + sw_lo sx_hi + sw_hi sx_lo      (relative error ~2^-16)
// so the fp32 VALU only runs acc = fma(P, C, acc), one instruction per
// element and group.  Both halves of the wave feed the same three terms (k =
// 0..2 and 8..10), which doubles C; that 2 and the 2^18 are folded into the
// staged sw as 2^17.
//
// MXFP4: the E2M1 nibbles are the native fp4 operand format of
// v_mfma_scale_f32_16x16x128_f8f6f4 and the E8M0 block scales are its scale
// operands, so the matrix core applies 2^(ex + ew) itself and accumulates
// across blocks; no per-block VALU work remains.
//
// Operand roles: the matrix instruction's A operand is the weight tile (rows
// n) and B the activation tile (columns m), so every lane ends up holding
// runs of 4 consecutive output channels n of one token m (8-byte bf16 stores).
//
// Low-rank epilogue: h (fp32) is split into bf16 hi = bf16(h) and lo =
// bf16(h - hi); the bf16 matrix instruction with `up` as the other operand
// gives h . up to ~16 bits, well inside the output tolerance.  It takes the
// 4-bit term as its accumulator input, and one more bf16 product (the bias
// row against a column of ones) adds the bias exactly, so the VALU only
// applies GELU and rounds.
#include "svdq_internal.h"
#include "svdq_quant.h"

namespace svdq {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return bits_f32(b << 16); }

// two fp32 -> two bf16 (round to nearest even), packed low | high << 16
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// GELU, tanh form: 0.5 y (1 + tanh(u)) = y / (1 + exp(-2u)),
// u = sqrt(2/pi) (y + 0.044715 y^3); exp via the hardware exp2.
__device__ __forceinline__ float gelu_tanh(float y)
{
    const float k1 = -2.302208198f;      // -2 sqrt(2/pi) log2(e)
    const float k3 = -0.102943836f;      // -2 sqrt(2/pi) 0.044715 log2(e)
    const float t = y * __builtin_fmaf(k3, y * y, k1);
    return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// 8 fp32 values of h -> bf16 hi and lo parts (hi = bf16(h), lo = bf16(h - hi)).
__device__ __forceinline__ void split_h(const float *hv, bf16x8 &hi8, bf16x8 &lo8)
{
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = pack_bf16x2(hv[2 * i], hv[2 * i + 1]);
        lo[i] = pack_bf16x2(hv[2 * i] - bf16_to_f32(hi[i] & 0xFFFFu), hv[2 * i + 1] - bf16_to_f32(hi[i] >> 16));
    }
    hi8 = __builtin_bit_cast(bf16x8, (uint4){hi[0], hi[1], hi[2], hi[3]});
    lo8 = __builtin_bit_cast(bf16x8, (uint4){lo[0], lo[1], lo[2], lo[3]});
}

__device__ __forceinline__ void load_h8(const float *__restrict__ h, int m, int M, int k, float *hv)
{
    if (m < M) {
        const float4 a = *reinterpret_cast<const float4 *>(h + (size_t)m * 32 + k);
        const float4 b = *reinterpret_cast<const float4 *>(h + (size_t)m * 32 + k + 4);
        hv[0] = a.x; hv[1] = a.y; hv[2] = a.z; hv[3] = a.w;
        hv[4] = b.x; hv[5] = b.y; hv[6] = b.z; hv[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = 0.0f;
    }
}

// Bias of 4 consecutive channels n..n+3 as 4 bf16 (zero when there is no
// bias or n >= N).
__device__ __forceinline__ uint2 bias4(const uint16_t *__restrict__ bias, int n, int N)
{
    if (!bias || n >= N) return make_uint2(0u, 0u);
    return *reinterpret_cast<const uint2 *>(bias + n);
}

// y (+ GELU) for 4 consecutive channels, packed as 4 bf16.
__device__ __forceinline__ uint2 finish4(const float *y, int gelu)
{
    float y0 = y[0], y1 = y[1], y2 = y[2], y3 = y[3];
    if (gelu) {
        y0 = gelu_tanh(y0); y1 = gelu_tanh(y1); y2 = gelu_tanh(y2); y3 = gelu_tanh(y3);
    }
    return make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
}

// Bias as a matrix-core operand: the A operand (rows n of a 32x32 tile) with
// the bias of the lane's row at k = 0 of lane half 0 and zeros elsewhere.
// Against kOnesB (1.0 at k = 0 of every column) the bf16 product adds b_n,
// exactly, to every output of row n.  n is the tile's first channel + l32.
__device__ __forceinline__ bf16x8 bias_operand(const uint16_t *__restrict__ bias, int n, int N, int hk)
{
    const uint32_t b = (bias && n < N && hk == 0) ? (uint32_t)bias[n] : 0u;
    return __builtin_bit_cast(bf16x8, (uint4){b, 0u, 0u, 0u});
}
__device__ __forceinline__ bf16x8 ones_operand(int hk)
{
    return __builtin_bit_cast(bf16x8, (uint4){hk == 0 ? 0x3F80u : 0u, 0u, 0u, 0u});
}

// acc + h . up^T + b for one 32x32 tile on the matrix cores: the low-rank
// term as two k steps of 16 with the hi and the lo part of h (A = up rows,
// B = h rows), then the bias product.
__device__ __forceinline__ f32x16 add_lowrank_bias(f32x16 acc, const bf16x8 (&ua)[2], const bf16x8 (&hhi)[2],
                                                   const bf16x8 (&hlo)[2], bf16x8 bq, bf16x8 ones)
{
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[s], hhi[s], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[s], hlo[s], acc, 0, 0, 0);
    }
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq, ones, acc, 0, 0, 0);
}

// Output staging: each wave writes its 64 x 64 bf16 tile into its own LDS
// area (row stride 136 bytes, conflict-free for 8-byte writes from 32 rows),
// then stores it as 64 full 128-byte row segments.
constexpr int OUT_STRIDE = 136;
constexpr int OUT_TILE_BYTES = 64 * OUT_STRIDE;

__device__ __forceinline__ void stage4(uint8_t *tile, int ml, int nl, uint2 v)
{
    *reinterpret_cast<uint2 *>(tile + ml * OUT_STRIDE + nl * 2) = v;
}

// Y is written once and not read back by this kernel: non-temporal stores
// keep it from pushing the operand tiles out of the L2.
__device__ __forceinline__ void store_nt(uint16_t *p, uint4 v)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store((u32x4){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ void flush_tile(const uint8_t *tile, uint16_t *__restrict__ Y, int mb, int nb, int M,
                                           int N, int lane)
{
    const int seg = lane & 7;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int r = (lane >> 3) + 8 * it;
        const uint4 v = *reinterpret_cast<const uint4 *>(tile + r * OUT_STRIDE + seg * 16);
        const int m = mb + r, n = nb + seg * 8;
        if (m < M && n < N) store_nt(Y + (size_t)m * N + n, v);
    }
}

// c ? v : 0, element-wise (a whole-vector select can end up in scratch memory)
__device__ __forceinline__ uint4 keep_if(bool c, uint4 v)
{
    return make_uint4(c ? v.x : 0u, c ? v.y : 0u, c ? v.z : 0u, c ? v.w : 0u);
}

// Tile order.  Consecutive workgroup ids land on different XCDs (8 on
// MI355X), each with its own L2: first give every XCD a contiguous range of
// tile indices, then walk the tiles in groups of GN weight tiles with the
// token tiles fastest, so an XCD keeps ~GN weight tiles in its L2 while it
// sweeps the activation tiles.
constexpr int TILE_GROUP_N = 6;

__device__ __forceinline__ void tile_coords(int b, int tiles_n, int tiles_m, int &tn, int &tm)
{
    const int T = tiles_n * tiles_m;
    const int t = (T % 8 == 0) ? (b & 7) * (T >> 3) + (b >> 3) : b;
    const int per_group = TILE_GROUP_N * tiles_m;
    const int first_n = (t / per_group) * TILE_GROUP_N;
    const int gsize = min(tiles_n - first_n, TILE_GROUP_N);
    const int in = t % per_group;
    tn = first_n + in % gsize;
    tm = in / gsize;
}

// ================================================================ INT4 (fp8 path)

constexpr int I4_BN = 256, I4_BM = 128;          // block tile (n, m)
constexpr int I4_WAVES_N = 4, I4_WAVES_M = 2;    // 8 waves
constexpr int I4_WN = I4_BN / I4_WAVES_N, I4_WM = I4_BM / I4_WAVES_M;   // 64 x 64
constexpr int I4_TN = I4_WN / 32, I4_TM = I4_WM / 32;                   // 2 x 2 tiles of 32x32
constexpr int I4_THREADS = 64 * I4_WAVES_N * I4_WAVES_M;
constexpr int I4_KSTEP = 128;                    // channels per pipeline step (two groups)
constexpr int I4_ROWB = I4_KSTEP + 16;           // LDS bytes per row: 128 fp8 + 16 pad
constexpr float kTwo17 = 131072.0f;

// 16 nibble bytes (32 sign-magnitude codes) -> 32 E4M3 bytes (q * 2^-9).
// Dword j of the input gives E (codes 8j, 8j+2, 8j+4, 8j+6) and O (the odd
// ones); the resulting k order is a fixed permutation, the same for both
// operands, so every dot product is unchanged.
__device__ __forceinline__ void widen_fp8(uint4 p, uint4 &lo, uint4 &hi)
{
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[2 * j] = (w[j] & 0x07070707u) | ((w[j] & 0x08080808u) << 4);
        o[2 * j + 1] = ((w[j] >> 4) & 0x07070707u) | (w[j] & 0x80808080u);
    }
    lo = (uint4){o[0], o[1], o[2], o[3]};
    hi = (uint4){o[4], o[5], o[6], o[7]};
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_offset(const void *p)
{
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_u8 *)p);
}

// One LDS-DMA load per lane: 16 (or 4) bytes from sbase + voff to LDS
// lds + 16 * lane (4 * lane).  M0 is saved and restored around it.
__device__ __forceinline__ void dma_b128(uint32_t lds, uint32_t voff, const void *sbase)
{
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(lds), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void dma_b32(uint32_t lds, uint32_t voff, const void *sbase)
{
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(lds), "v"(voff), "s"(sbase) : "memory");
}

// Scale operands of the outer-product instruction (A = weights, B = tokens):
// row n of A holds (sw_hi, sw_lo, sw_hi) at k = 0..2 and again at k = 8..10,
// column m of B holds (sx_hi, sx_hi, sx_lo) at the same k; every other k is
// zero.
__device__ __forceinline__ uint2 scale_operand_w(float s)
{
    const uint32_t hi = pack_bf16x2(s, 0.0f) & 0xFFFFu;
    const uint32_t lo = pack_bf16x2(s - bf16_to_f32(hi), 0.0f) & 0xFFFFu;
    return make_uint2(hi | lo << 16, hi);
}

__device__ __forceinline__ uint2 scale_operand_x(float s)
{
    const uint32_t hi = pack_bf16x2(s, 0.0f) & 0xFFFFu;
    const uint32_t lo = pack_bf16x2(s - bf16_to_f32(hi), 0.0f) & 0xFFFFu;
    return make_uint2(hi | hi << 16, lo);
}

struct __attribute__((aligned(16))) I4Smem {
    uint8_t w[2][I4_BN * I4_ROWB];
    uint8_t x[2][I4_BM * I4_ROWB];
    uint2 sw[2][2][I4_BN];     // [buf][group in step][n], scale_operand_w(sw * 2^17)
    uint2 sx[2][2][I4_BM];     // [buf][group in step][m], scale_operand_x(sx)
    float sp[2][(I4_BN + I4_BM) * 8];   // scale panels: 8 groups (4 steps) of the W rows, then the X rows
};

// The next layer's activation step, computed from this layer's output in the
// epilogue instead of storing Y (INT4): the bf16-rounded outputs are
// smoothed with smooth2, quantized per 64 channels (each wave tile spans one
// such group per token) and multiplied into down2 for a partial h2 over the
// block's 256 channels; the partials are summed later in a fixed order.
struct RequantArgs {
    const float *smooth2;     // [N]
    const uint16_t *down2;    // [32][N] bf16 bits
    uint8_t *xq2;             // [M][N/2]
    void *xscale2;            // INT4: fp32 [M][N/64]; MXFP4: E8M0 [M][N/32]
    float *hpart;             // [ceil(N/256)][M][32]
};

// What the INT4 kernel's epilogue does with the wave tile.
constexpr int EPI_STORE = 0;      // y -> bf16 Y
constexpr int EPI_REQUANT = 1;    // the next layer's activation step (RequantArgs)
constexpr int EPI_QKNORM = 2;     // Q/K RMS-norm + rotary embedding of a QKV projection (QKNormArgs)

// The fused attention-input step: N = 3 H 128 output channels are H heads of
// Q, then K, then V.  Q and K heads are RMS-normalized over their 128
// channels with their bf16 norm weight and then rotated pairwise by the
// token's angles; V heads are stored as the linear stores them.
struct QKNormArgs {
    const uint16_t *norm_q;   // [128] bf16 bits
    const uint16_t *norm_k;   // [128] bf16 bits
    const float *rope_cos;    // [M][64]
    const float *rope_sin;    // [M][64]
    int heads;                // H
    float eps;
};

// Q/K RMS-norm + rotary on 8 consecutive channels d0 .. d0 + 7 (d0 % 8 == 0)
// of one token's head, given as 8 bf16 in `v`: u = y rs w (the token's 1 / rms,
// the head's norm weights `wv` of those channels), then the 4 pairs rotated by
// the token's angles (`c`, `sn`: cos and sin of pairs d0 / 2 .. d0 / 2 + 3),
// rounded to bf16.
__device__ __forceinline__ uint4 qk_norm_rope8(uint4 v, float rs, uint4 wv, float4 c, float4 sn)
{
    const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
    const float cc[4] = {c.x, c.y, c.z, c.w}, ssn[4] = {sn.x, sn.y, sn.z, sn.w};
    uint32_t yd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {          // pair q: channels d0 + 2 q, + 1
        const float u0 = bf16_to_f32(yd[q] & 0xFFFFu) * rs * bf16_to_f32(wd[q] & 0xFFFFu);
        const float u1 = bf16_to_f32(yd[q] >> 16) * rs * bf16_to_f32(wd[q] >> 16);
        yd[q] = pack_bf16x2(u0 * cc[q] - u1 * ssn[q], u1 * cc[q] + u0 * ssn[q]);
    }
    return make_uint4(yd[0], yd[1], yd[2], yd[3]);
}

// Epilogue of the requantizing INT4 kernel for one wave tile (64 channels n
// of one 64-group x 64 tokens m).  Lane (l32, hk) holds, per 32-token tile
// tm, token m = mb + 32 tm + l32 and the channels nb + 32 tn + 8 j + 4 hk +
// (0..3), tn < 2, j < 4: half of the token's group, the other half being in
// lane l32 + 32 (hk = 1).  `P` is the block's LDS, free after the main loop.
__device__ __forceinline__ void requant_epilogue(const f32x16 (&acc)[I4_TN][I4_TM], const bf16x8 (&hhi)[I4_TM][2],
                                                 const bf16x8 (&hlo)[I4_TM][2], const uint16_t *__restrict__ up,
                                                 const uint16_t *__restrict__ bias, int M, int N, int gelu,
                                                 const RequantArgs &rq, int mb, int nb, int tile_n, int m0, int wn,
                                                 int wm, int tid, int lane, float *P)
{
    const int l32 = lane & 31, hk = lane >> 5;
    const bool live = nb < N;          // N % 64 == 0: a wave tile is all in or all out
    // bf16 outputs, exactly as the plain epilogue would store them
    uint2 yb[I4_TN][I4_TM][4];
#pragma unroll
    for (int tn = 0; tn < I4_TN; ++tn) {
        const int nrow = nb + tn * 32 + l32;
        bf16x8 ua[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            uint4 uv = {0u, 0u, 0u, 0u};
            if (nrow < N) uv = *reinterpret_cast<const uint4 *>(up + (size_t)nrow * 32 + 16 * s + 8 * hk);
            ua[s] = __builtin_bit_cast(bf16x8, uv);
        }
        const bf16x8 bq = bias_operand(bias, nb + tn * 32 + l32, N, hk), ones = ones_operand(hk);
#pragma unroll
        for (int tm = 0; tm < I4_TM; ++tm) {
            const f32x16 lr = add_lowrank_bias(acc[tn][tm], ua, hhi[tm], hlo[tm], bq, ones);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float y4[4] = {lr[4 * j], lr[4 * j + 1], lr[4 * j + 2], lr[4 * j + 3]};
                yb[tn][tm][j] = finish4(y4, gelu);
            }
        }
    }
    // next layer's smoothing and down projection for the lane's channels
    float4 s2[I4_TN][4];
    bf16x8 dn[4];                      // A operands: down2 rows l32, k block kb
#pragma unroll
    for (int tn = 0; tn < I4_TN; ++tn)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s2[tn][j] = live ? *reinterpret_cast<const float4 *>(rq.smooth2 + nb + tn * 32 + 8 * j + 4 * hk)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        // k block kb covers channels 16 kb .. 16 kb + 15 of the wave tile:
        // tn = kb / 2, j = 2 (kb % 2) and j + 1; lane half hk holds k = 8 hk
        // + 0..7, i.e. channels 8 j + 4 hk + 0..3 of both j
        const int c = nb + (kb >> 1) * 32 + 16 * (kb & 1) + 4 * hk;
        uint2 a = {0u, 0u}, b = {0u, 0u};
        if (live) {
            a = *reinterpret_cast<const uint2 *>(rq.down2 + (size_t)l32 * N + c);
            b = *reinterpret_cast<const uint2 *>(rq.down2 + (size_t)l32 * N + c + 8);
        }
        dn[kb] = __builtin_bit_cast(bf16x8, (uint4){a.x, a.y, b.x, b.y});
    }
    f32x16 hp[I4_TM];
#pragma unroll
    for (int tm = 0; tm < I4_TM; ++tm) {
        const int m = mb + tm * 32 + l32;
        // smoothed values and the group absmax (this lane's 32, then its partner's)
        float v[I4_TN][4][4];
        float amax = 0.0f;
#pragma unroll
        for (int tn = 0; tn < I4_TN; ++tn)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint2 y = yb[tn][tm][j];
                const float sv[4] = {s2[tn][j].x, s2[tn][j].y, s2[tn][j].z, s2[tn][j].w};
                const float yv[4] = {bf16_to_f32(y.x & 0xFFFFu), bf16_to_f32(y.x >> 16), bf16_to_f32(y.y & 0xFFFFu),
                                     bf16_to_f32(y.y >> 16)};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[tn][j][e] = yv[e] * sv[e];
                    amax = __builtin_fmaxf(amax, __builtin_fabsf(v[tn][j][e]));
                }
            }
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
        const float scale = int4_group_scale(amax);
        // magnitudes: rint(|v| rcp(scale)) unless some quotient of the lane
        // lies within 2^-19 of a half-integer (or the group needs the 2^64
        // lift); then the exact remainder test decides every code of the lane
        const bool lifted = scale < 7.88860905e-31f;
        const float inv = scale == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(scale);
        float q[I4_TN][4][4];
        float dmax = 0.0f;
#pragma unroll
        for (int tn = 0; tn < I4_TN; ++tn)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float t = __builtin_fabsf(v[tn][j][e]) * inv;
                    q[tn][j][e] = __builtin_rintf(t);
                    dmax = __builtin_fmaxf(dmax, __builtin_fabsf(t - q[tn][j][e]));
                }
        if (lifted || dmax >= kNearTie) {
            const Int4Group g = int4_group_prepare(scale);
#pragma unroll
            for (int tn = 0; tn < I4_TN; ++tn)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) q[tn][j][e] = (float)int4_mag(__builtin_fabsf(v[tn][j][e]), g);
        }
        // 4 codes (16 bits) per (tn, j): magnitudes packed as bytes, the odd
        // ones shifted into the high nibbles, sign bits from the values; lane
        // half hk keeps tn = hk and trades the other tn with its partner
        uint32_t keep[4], give[4];
#pragma unroll
        for (int tn = 0; tn < I4_TN; ++tn)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t ev = __builtin_amdgcn_cvt_pk_u8_f32(q[tn][j][2], 1,
                                                                   __builtin_amdgcn_cvt_pk_u8_f32(q[tn][j][0], 0, 0u));
                const uint32_t od = __builtin_amdgcn_cvt_pk_u8_f32(q[tn][j][3], 1,
                                                                   __builtin_amdgcn_cvt_pk_u8_f32(q[tn][j][1], 0, 0u));
                const uint32_t sg = ((f32_bits(v[tn][j][0]) >> 28) & 8u) | ((f32_bits(v[tn][j][1]) >> 24) & 0x80u) |
                                    ((f32_bits(v[tn][j][2]) >> 20) & 0x800u) | ((f32_bits(v[tn][j][3]) >> 16) & 0x8000u);
                const uint32_t piece = (ev | od << 4) | sg;
                if (tn == hk) keep[j] = piece;
                else give[j] = piece;
            }
        const uint32_t g01 = give[0] | give[1] << 16, g23 = give[2] | give[3] << 16;
        const uint32_t r01 = (uint32_t)__shfl_xor((int)g01, 32), r23 = (uint32_t)__shfl_xor((int)g23, 32);
        const uint32_t got[4] = {r01 & 0xFFFFu, r01 >> 16, r23 & 0xFFFFu, r23 >> 16};
        // bytes 16 hk .. 16 hk + 15 of the token's 32-byte group: byte 4 j +
        // 2 half holds the codes of lane half `half`
        uint4 out;
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = hk ? (got[j] | keep[j] << 16) : (keep[j] | got[j] << 16);
        out = make_uint4(o[0], o[1], o[2], o[3]);
        if (live && m < M) {
            *reinterpret_cast<uint4 *>(rq.xq2 + (size_t)m * (N / 2) + nb / 2 + 16 * hk) = out;
            if (hk == 0) static_cast<float *>(rq.xscale2)[(size_t)m * (N / 64) + nb / 64] = scale;
        }
        // partial h2 = Y down2^T over the wave tile's 64 channels
        f32x16 d = {};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int tn = kb >> 1, ja = 2 * (kb & 1);
            const uint2 y0 = yb[tn][tm][ja], y1 = yb[tn][tm][ja + 1];
            const bf16x8 bop = __builtin_bit_cast(bf16x8, live ? (uint4){y0.x, y0.y, y1.x, y1.y}
                                                               : (uint4){0u, 0u, 0u, 0u});
            d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dn[kb], bop, d, 0, 0, 0);
        }
        hp[tm] = d;
    }
    // sum the 4 channel quarters of the block in LDS (fixed order), then one
    // row of 32 partial sums per token goes to hpart
    __syncthreads();                  // every wave is done with the operand LDS
#pragma unroll
    for (int tm = 0; tm < I4_TM; ++tm) {
        const int ml = wm * I4_WM + tm * 32 + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // rows j = 8 q + 4 hk + (0..3) of the 32x32 result, column ml
            const float4 w4 = make_float4(hp[tm][4 * q], hp[tm][4 * q + 1], hp[tm][4 * q + 2], hp[tm][4 * q + 3]);
            *reinterpret_cast<float4 *>(P + ((size_t)wn * I4_BM + ml) * 32 + 8 * q + 4 * hk) = w4;
        }
    }
    __syncthreads();
    const int ml = tid >> 2, j0 = 8 * (tid & 3);
    float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
#pragma unroll
    for (int w = 0; w < I4_WAVES_N; ++w) {
        const float *src = P + ((size_t)w * I4_BM + ml) * 32 + j0;
        const float4 a = *reinterpret_cast<const float4 *>(src), b = *reinterpret_cast<const float4 *>(src + 4);
        s0.x += a.x; s0.y += a.y; s0.z += a.z; s0.w += a.w;
        s1.x += b.x; s1.y += b.y; s1.z += b.z; s1.w += b.w;
    }
    const int m = m0 + ml;
    if (m < M) {
        float *dst = rq.hpart + ((size_t)tile_n * M + m) * 32 + j0;
        *reinterpret_cast<float4 *>(dst) = s0;
        *reinterpret_cast<float4 *>(dst + 4) = s1;
    }
}

// Epilogue of the QKV kernel with Q/K RMS-norm and rotary embedding, for
// one wave tile (64 channels n x 64 tokens m).  A 128-channel head is the
// tile of this wave and of its neighbour (wn ^ 1): each lane sums the
// squares of its 32 values per token, adds its partner half (lane ^ 32), and
// the two waves exchange their sums through LDS.  Element i of tile (tn, tm)
// is channel nb + 32 tn + 8 (i / 4) + 4 hk + i % 4 of token mb + 32 tm +
// l32, so a rotation pair (2p, 2p + 1) sits in one lane.  `smem` is LDS that
// no wave reads any more.
__device__ __forceinline__ void qknorm_epilogue(const f32x16 (&acc)[I4_TN][I4_TM], const bf16x8 (&hhi)[I4_TM][2],
                                                const bf16x8 (&hlo)[I4_TM][2], const uint16_t *__restrict__ up,
                                                const uint16_t *__restrict__ bias, int M, int N,
                                                const QKNormArgs &qk, int mb, int nb, int wave, int lane,
                                                uint16_t *__restrict__ Y, uint8_t *smem)
{
    const int l32 = lane & 31, hk = lane >> 5;
    // the linear's outputs, rounded to bf16 exactly as the plain epilogue
    // stores them
    uint2 yb[I4_TN][I4_TM][4];
#pragma unroll
    for (int tn = 0; tn < I4_TN; ++tn) {
        const int nrow = nb + tn * 32 + l32;
        bf16x8 ua[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint4 uv = {0u, 0u, 0u, 0u};
            if (nrow < N) uv = *reinterpret_cast<const uint4 *>(up + (size_t)nrow * 32 + 16 * s2 + 8 * hk);
            ua[s2] = __builtin_bit_cast(bf16x8, uv);
        }
        const bf16x8 bq = bias_operand(bias, nb + tn * 32 + l32, N, hk), ones = ones_operand(hk);
#pragma unroll
        for (int tm = 0; tm < I4_TM; ++tm) {
            const f32x16 lr = add_lowrank_bias(acc[tn][tm], ua, hhi[tm], hlo[tm], bq, ones);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float y4[4] = {lr[4 * j], lr[4 * j + 1], lr[4 * j + 2], lr[4 * j + 3]};
                yb[tn][tm][j] = finish4(y4, 0);
            }
        }
    }
    const int head = nb / 128;                   // the same for this wave and its neighbour
    const bool norm = head < 2 * qk.heads;       // a Q or a K head
    float *red = reinterpret_cast<float *>(smem + 8 * OUT_TILE_BYTES);   // [8 waves][64 tokens]
    if (norm) {
#pragma unroll
        for (int tm = 0; tm < I4_TM; ++tm) {
            float ss = 0.0f;
#pragma unroll
            for (int tn = 0; tn < I4_TN; ++tn)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v0 = bf16_to_f32(yb[tn][tm][j].x & 0xFFFFu), v1 = bf16_to_f32(yb[tn][tm][j].x >> 16);
                    const float v2 = bf16_to_f32(yb[tn][tm][j].y & 0xFFFFu), v3 = bf16_to_f32(yb[tn][tm][j].y >> 16);
                    ss = __builtin_fmaf(v0, v0, ss);
                    ss = __builtin_fmaf(v1, v1, ss);
                    ss = __builtin_fmaf(v2, v2, ss);
                    ss = __builtin_fmaf(v3, v3, ss);
                }
            ss += __shfl_xor(ss, 32);
            if (hk == 0) red[wave * 64 + tm * 32 + l32] = ss;
        }
    }
    // the bf16 outputs staged as they are, the token's 1 / rms in the spare
    // bytes of its row
    uint8_t *tile = smem + wave * OUT_TILE_BYTES;
#pragma unroll
    for (int tn = 0; tn < I4_TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < I4_TM; ++tm)
#pragma unroll
            for (int j = 0; j < 4; ++j) stage4(tile, tm * 32 + l32, tn * 32 + 8 * j + 4 * hk, yb[tn][tm][j]);
    __syncthreads();
    if (norm && hk == 0) {
#pragma unroll
        for (int tm = 0; tm < I4_TM; ++tm) {
            const int ml = tm * 32 + l32;
            const float tot = red[wave * 64 + ml] + red[(wave ^ 1) * 64 + ml];
            *reinterpret_cast<float *>(tile + ml * OUT_STRIDE + 128) =
                __builtin_amdgcn_rsqf(__builtin_fmaf(tot, 1.0f / 128.0f, qk.eps));
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 8 lanes per token row, 8 channels (4 rotation pairs) each: Q and K heads
    // are normalized and rotated on the way out, with the norm weights read
    // once and the rotation tables as whole 128-byte runs per token
    const int seg = lane & 7;
    const int d0 = (nb & 127) + 8 * seg;         // the lane's first channel in the head
    uint4 wv = {0u, 0u, 0u, 0u};
    if (norm) wv = *reinterpret_cast<const uint4 *>((head < qk.heads ? qk.norm_q : qk.norm_k) + d0);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int r = (lane >> 3) + 8 * it;
        uint4 v = *reinterpret_cast<const uint4 *>(tile + r * OUT_STRIDE + seg * 16);
        const int m = mb + r, n = nb + seg * 8;
        if (norm) {
            const float rs = *reinterpret_cast<const float *>(tile + r * OUT_STRIDE + 128);
            const int mc = m < M ? m : M - 1;                     // rows past M are never stored
            v = qk_norm_rope8(v, rs, wv, *reinterpret_cast<const float4 *>(qk.rope_cos + (size_t)mc * 64 + d0 / 2),
                              *reinterpret_cast<const float4 *>(qk.rope_sin + (size_t)mc * 64 + d0 / 2));
        }
        if (m < M && n < N) store_nt(Y + (size_t)m * N + n, v);
    }
}

// Scale panels hold 8 groups of every W and X row of the block tile, a row of
// 8 floats per matrix row; group g of row r sits at position g ^ sp_swz(r), so
// that the 8-byte reads of 32 consecutive rows fall in distinct banks.
__device__ __forceinline__ int sp_swz(int r) { return 2 * ((r >> 3) & 3); }

template <int EPI>
__global__ __launch_bounds__(I4_THREADS) void w4a4_int4_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ xscale, const float *__restrict__ h,
    const uint8_t *__restrict__ wq, const float *__restrict__ wscale, const uint16_t *__restrict__ up,
    const uint16_t *__restrict__ bias, int M, int N, int K, int gelu, uint16_t *__restrict__ Y, RequantArgs rq,
    QKNormArgs qk)
{
    __shared__ I4Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % I4_WAVES_N, wm = wave / I4_WAVES_N;
    const int tiles_n = (N + I4_BN - 1) / I4_BN;
    const int tiles_m = (M + I4_BM - 1) / I4_BM;
    int tn_, tm_;
    tile_coords(blockIdx.x, tiles_n, tiles_m, tn_, tm_);
    const int n0 = tn_ * I4_BN, m0 = tm_ * I4_BM;
    const int G = K >> 6;
    const int KB = K >> 1;                  // code bytes per row
    const int steps = (G + 1) >> 1;

    // Loader: a chunk is 16 code bytes (32 codes) of one row; per step W has
    // BN*4 chunks and X BM*4.  Thread t moves W chunks t and t + 512 and X
    // chunk t (all with segment t & 3).  Loads are unconditional: rows past
    // N / M are clamped to the last row (their outputs are never stored), and
    // for an odd G the missing second group of the last step re-reads the
    // step's first group (the compute loop never reads it), so every path has
    // the same number of loads in flight and none leaves the row.
    constexpr int WCH = I4_BN * 4, XCH = I4_BM * 4;
    static_assert(WCH == 2 * I4_THREADS && XCH == I4_THREADS, "loader shape");
    const int lseg = tid & 3, lr = tid >> 2;
    const uint8_t *__restrict__ pw0 = wq + (size_t)min(n0 + lr, N - 1) * KB + lseg * 16;
    const uint8_t *__restrict__ pw1 = wq + (size_t)min(n0 + lr + I4_BN / 2, N - 1) * KB + lseg * 16;
    const uint8_t *__restrict__ px0 = xq + (size_t)min(m0 + lr, M - 1) * KB + lseg * 16;
    // Scales: threads [0, BN) turn the sw of W row t, threads [BN, BN + BM)
    // the sx of X row t - BN into the step's scale operands; the others idle.
    // The scales reach LDS as panels of 8 groups (4 steps) per row, moved by
    // LDS-DMA: 48 dword loads of 64 lanes per panel (0..31 the W rows, 32..47
    // the X rows), wave w issuing loads 6 w .. 6 w + 5.  Eight lanes cover one
    // row's 32 contiguous bytes, so a load touches 8 rows instead of the 64
    // that per-thread scale loads would.  Groups past G re-read group G - 1.
    const bool sc_w = tid < I4_BN, sc_x = tid >= I4_BN && tid < I4_BN + I4_BM;
    const uint32_t sp_lds0 = lds_offset(&sm.sp[0][0]);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);      // DMA bases and LDS offsets are uniform
    const float *__restrict__ wsb = wscale + (size_t)n0 * G;      // the tile's first rows
    const float *__restrict__ xsb = xscale + (size_t)m0 * G;
    uint32_t sp_off[6];                                          // byte offset of the lane's (row, group 0..7)
#pragma unroll
    for (int j = 0; j < 6; ++j) {
        const int i = 6 * wave + j, d = 64 * i + lane, r = d >> 3;
        const int g = (d & 7) ^ sp_swz(r);
        const int rr = r < I4_BN ? min(r, N - 1 - n0) : min(r - I4_BN, M - 1 - m0);
        sp_off[j] = (uint32_t)(rr * G + g) * 4u;
    }
    auto sp_issue = [&](int p) {
        const int g0 = 8 * p;
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            const int i = 6 * wave_u + j;
            const int d = 64 * i + lane, r = d >> 3, g = (d & 7) ^ sp_swz(r);
            // + 4 g0 bytes, or the row's last group when g0 + g is past G
            const uint32_t add = g0 + g < G ? 4u * (uint32_t)g0 : 4u * (uint32_t)(G - 1 - g);
            dma_b32(sp_lds0 + (uint32_t)(p & 1) * (uint32_t)sizeof(sm.sp[0]) + 256u * i, sp_off[j] + add,
                    i < 32 ? wsb : xsb);
        }
    };

    // Two register sets: the global loads of step st + 2 are issued at the
    // start of step st and written to LDS at the end of step st + 1.
    uint4 rgA0, rgA1, rgA2, rgB0, rgB1, rgB2;

#define I4_GLOAD(st, R)                                                                \
    do {                                                                               \
        const int koff_ = ((st) * 64 + lseg * 16 < KB) ? (st) * 64 : (st) * 64 - 32;   \
        rg##R##0 = *reinterpret_cast<const uint4 *>(pw0 + koff_);                      \
        rg##R##1 = *reinterpret_cast<const uint4 *>(pw1 + koff_);                      \
        rg##R##2 = *reinterpret_cast<const uint4 *>(px0 + koff_);                      \
    } while (0)
    // When G is odd, the second half of the last step holds codes that the
    // compute loop never reads.
#define I4_LSTORE(st, buf, R)                                                          \
    do {                                                                               \
        uint4 a_, b_;                                                                  \
        widen_fp8(rg##R##0, a_, b_);                                                   \
        uint8_t *d_ = sm.w[buf] + lr * I4_ROWB + lseg * 32;                            \
        *reinterpret_cast<uint4 *>(d_) = a_;                                           \
        *reinterpret_cast<uint4 *>(d_ + 16) = b_;                                      \
        widen_fp8(rg##R##1, a_, b_);                                                   \
        d_ = sm.w[buf] + (lr + I4_BN / 2) * I4_ROWB + lseg * 32;                       \
        *reinterpret_cast<uint4 *>(d_) = a_;                                           \
        *reinterpret_cast<uint4 *>(d_ + 16) = b_;                                      \
        widen_fp8(rg##R##2, a_, b_);                                                   \
        d_ = sm.x[buf] + lr * I4_ROWB + lseg * 32;                                     \
        *reinterpret_cast<uint4 *>(d_) = a_;                                           \
        *reinterpret_cast<uint4 *>(d_ + 16) = b_;                                      \
        if (sc_w || sc_x) {                                                            \
            const int r_ = tid, j_ = (st) & 3;                                         \
            const float2 v_ = *reinterpret_cast<const float2 *>(                       \
                &sm.sp[((st) >> 2) & 1][8 * r_ + ((2 * j_) ^ sp_swz(r_))]);            \
            if (sc_w) {                                                                \
                sm.sw[buf][0][tid] = scale_operand_w(v_.x * kTwo17);                   \
                sm.sw[buf][1][tid] = scale_operand_w(v_.y * kTwo17);                   \
            } else {                                                                   \
                sm.sx[buf][0][tid - I4_BN] = scale_operand_x(v_.x);                    \
                sm.sx[buf][1][tid - I4_BN] = scale_operand_x(v_.y);                    \
            }                                                                          \
        }                                                                              \
    } while (0)

    f32x16 acc[I4_TN][I4_TM];
#pragma unroll
    for (int a = 0; a < I4_TN; ++a)
#pragma unroll
        for (int b = 0; b < I4_TM; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    const int l32 = lane & 31, hk = lane >> 5;
    const f32x16 zero16 = {};
    // Compute of one step from LDS buffer `buf`: two groups (one for the last
    // step of an odd G), each 4 tiles of 32x32 with one fp8 product, one scale
    // outer product and 16 fmas.  (The per-group exit also keeps the compiler
    // from hoisting the second group's reads and products into the first,
    // which would run out of registers.)
    uint4 cwv[I4_TN], cxv[I4_TM];
#pragma unroll
    for (int t = 0; t < I4_TN; ++t) cwv[t] = (uint4){0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < I4_TM; ++t) cxv[t] = (uint4){0u, 0u, 0u, 0u};
    auto compute_step = [&](int st, int buf) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if (2 * st + q >= G) break;   // odd G: the last step has one group
            i32x8 aw[I4_TN], bx[I4_TM];
            bf16x8 cw[I4_TN], cx[I4_TM];
#pragma unroll
            for (int tn = 0; tn < I4_TN; ++tn) {
                const uint8_t *p = sm.w[buf] + (wn * I4_WN + tn * 32 + l32) * I4_ROWB + q * 64 + hk * 32;
                const uint4 u0 = *reinterpret_cast<const uint4 *>(p);
                const uint4 u1 = *reinterpret_cast<const uint4 *>(p + 16);
                aw[tn] = (i32x8){(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w,
                                 (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
                // scale operands: both lane halves (k = 0..7 and 8..15) carry the
                // same three terms, so the product is twice the outer product
                const uint2 v = sm.sw[buf][q][wn * I4_WN + tn * 32 + l32];
                cwv[tn].x = v.x; cwv[tn].y = v.y;
                cw[tn] = __builtin_bit_cast(bf16x8, cwv[tn]);
            }
#pragma unroll
            for (int tm = 0; tm < I4_TM; ++tm) {
                const uint8_t *p = sm.x[buf] + (wm * I4_WM + tm * 32 + l32) * I4_ROWB + q * 64 + hk * 32;
                const uint4 u0 = *reinterpret_cast<const uint4 *>(p);
                const uint4 u1 = *reinterpret_cast<const uint4 *>(p + 16);
                bx[tm] = (i32x8){(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w,
                                 (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
                const uint2 v = sm.sx[buf][q][wm * I4_WM + tm * 32 + l32];
                cxv[tm].x = v.x; cxv[tm].y = v.y;
                cx[tm] = __builtin_bit_cast(bf16x8, cxv[tm]);
            }
#pragma unroll
            for (int tn = 0; tn < I4_TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < I4_TM; ++tm) {
                    const f32x16 p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aw[tn], bx[tm], zero16, 0, 0, 0,
                                                                                     127, 0, 127);
                    const f32x16 c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cw[tn], cx[tm], zero16, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[tn][tm][i] = __builtin_fmaf(p[i], c[i], acc[tn][tm][i]);
                }
        }
    };

    if (steps > 0) {
        sp_issue(0);
        I4_GLOAD(0, A);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        I4_LSTORE(0, 0, A);
        I4_GLOAD(min(1, steps - 1), B);
    }
    __syncthreads();
    for (int st = 0; st < steps; st += 2) {
        // even step: LDS buffer 0, registers A are free for step st + 2
        I4_GLOAD(min(st + 2, steps - 1), A);     // unconditional: same load count on every path
        // the panel of steps st + 4 .. st + 7 goes to the buffer whose last reader
        // was the staging of step st - 1 (before the previous barrier)
        if ((st & 3) == 0 && st + 4 < steps) sp_issue((st >> 2) + 1);
        compute_step(st, 0);
        if (st + 1 < steps) I4_LSTORE(st + 1, 1, B);
        // a panel issued at step st - 2 is read by the staging of step st + 2:
        // every load older than the last step's register loads is done
        if ((st & 3) == 2) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
        __syncthreads();
        if (st + 1 >= steps) break;
        // odd step: LDS buffer 1, registers B are free for step st + 3
        I4_GLOAD(min(st + 3, steps - 1), B);
        compute_step(st + 1, 1);
        if (st + 2 < steps) I4_LSTORE(st + 2, 0, A);
        __syncthreads();
    }
#undef I4_GLOAD
#undef I4_LSTORE

    // epilogue: low-rank term via v_mfma_f32_32x32x16_bf16 (rank 32 = two k
    // steps of 16, each with the hi and the lo part of h), then bias, GELU, store
    const int mb = m0 + wm * I4_WM, nb = n0 + wn * I4_WN;
    bf16x8 hhi[I4_TM][2], hlo[I4_TM][2];
#pragma unroll
    for (int tm = 0; tm < I4_TM; ++tm)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float hv[8];
            load_h8(h, mb + tm * 32 + l32, M, 16 * s + 8 * hk, hv);
            split_h(hv, hhi[tm][s], hlo[tm][s]);
        }
    if constexpr (EPI == EPI_REQUANT) {
        requant_epilogue(acc, hhi, hlo, up, bias, M, N, gelu, rq, mb, nb, tn_, m0, wn, wm, tid, lane,
                         reinterpret_cast<float *>(&sm));
        return;
    }
    if constexpr (EPI == EPI_QKNORM) {
        static_assert(8 * OUT_TILE_BYTES + 8 * 64 * sizeof(float) <= sizeof(I4Smem), "staging and head sums fit");
        qknorm_epilogue(acc, hhi, hlo, up, bias, M, N, qk, mb, nb, wave, lane, Y, reinterpret_cast<uint8_t *>(&sm));
        return;
    }
    uint8_t *tile = reinterpret_cast<uint8_t *>(&sm) + wave * OUT_TILE_BYTES;
    static_assert(8 * OUT_TILE_BYTES <= sizeof(I4Smem), "output staging fits in LDS");
#pragma unroll
    for (int tn = 0; tn < I4_TN; ++tn) {
        const int nrow = nb + tn * 32 + l32;
        bf16x8 ua[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            uint4 uv = {0u, 0u, 0u, 0u};
            if (nrow < N) uv = *reinterpret_cast<const uint4 *>(up + (size_t)nrow * 32 + 16 * s + 8 * hk);
            ua[s] = __builtin_bit_cast(bf16x8, uv);
        }
        const bf16x8 bq = bias_operand(bias, nb + tn * 32 + l32, N, hk), ones = ones_operand(hk);
#pragma unroll
        for (int tm = 0; tm < I4_TM; ++tm) {
            const f32x16 lr = add_lowrank_bias(acc[tn][tm], ua, hhi[tm], hlo[tm], bq, ones);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float y4[4] = {lr[4 * j], lr[4 * j + 1], lr[4 * j + 2], lr[4 * j + 3]};
                stage4(tile, tm * 32 + l32, tn * 32 + 8 * j + 4 * hk, finish4(y4, gelu));
            }
        }
    }
    __syncthreads();
    flush_tile(tile, Y, mb, nb, M, N, lane);
}

// The last, nearly empty round of INT4 tiles.  When the tiles that remain
// after whole rounds of one block per CU are few (at 4608 x 3072 -> 9216:
// 1296 tiles, five rounds and 16 tiles), each of them is computed by several
// blocks instead of one: block b takes piece b % P (32 PTM tokens x 32 PTN
// channels) of the b / P-th remaining tile, and its 8 waves split that
// piece's K, wave w taking groups [w G / 8, (w + 1) G / 8).  A wave's
// operands come straight from global memory (the nibbles widened in
// registers, exactly as the staging of the full-size kernel writes them),
// with the same products, scale products and fma per group as there.  The 8
// partial sums are added in wave order through LDS, and wave 0 runs the
// epilogue on the sum: the plain one (pieces of 64 x 32 or 64 x 64), or the
// Q/K RMS-norm + rotary one on pieces of 32 tokens x one 128-channel head.
// Only the order of the 4-bit term's sum differs from the full-size kernel
// (partial sums over K ranges instead of one running sum), so outputs may
// differ from it in low bf16 places.
template <int PTN, int PTM>
struct I4Tail {
    static constexpr int kPieces = (I4_BM / (32 * PTM)) * (I4_BN / (32 * PTN));   // pieces per tile
    static constexpr int kAcc = 16 * PTN * PTM;                                   // accumulators per lane
};

constexpr int QKP_ROW = 264;                 // staging row of a head piece: 128 bf16 + 8 bytes

template <int PTN, int PTM, int EPI>
__global__ __launch_bounds__(I4_THREADS) void w4a4_int4_tail_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ xscale, const float *__restrict__ h,
    const uint8_t *__restrict__ wq, const float *__restrict__ wscale, const uint16_t *__restrict__ up,
    const uint16_t *__restrict__ bias, int M, int N, int K, int gelu, uint16_t *__restrict__ Y, int first,
    QKNormArgs qk)
{
    static_assert(I4_THREADS == 512, "8 waves");
    static_assert(EPI == EPI_STORE ? (PTM == 2 && PTN <= 2) : (EPI == EPI_QKNORM && PTM == 1 && PTN == 4),
                  "plain pieces of 64 x 32 / 64 x 64, head pieces of 32 x 128");
    constexpr int P = I4Tail<PTN, PTM>::kPieces, PW = 32 * PTN, PH = 32 * PTM;   // pieces per tile, width, height
    __shared__ __attribute__((aligned(16))) float red[7][I4Tail<PTN, PTM>::kAcc][64];   // waves 1-7's sums
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hk = lane >> 5;
    const int tiles_n = (N + I4_BN - 1) / I4_BN, tiles_m = (M + I4_BM - 1) / I4_BM;
    int tn_, tm_;
    tile_coords(first + (int)blockIdx.x / P, tiles_n, tiles_m, tn_, tm_);
    const int piece = (int)blockIdx.x % P;
    const int mb = tm_ * I4_BM + PH * (piece / (I4_BN / PW)), nb = tn_ * I4_BN + PW * (piece % (I4_BN / PW));
    const int G = K >> 6, KB = K >> 1;
    const int g0 = wave * G / 8, g1 = (wave + 1) * G / 8;

    // the lane's rows: weight rows nb + 32 tn + l32, token rows mb + 32 tm + l32
    // (clamped; outputs of rows past N / M are never stored)
    const uint8_t *wrow[PTN], *xrow[PTM];
    const float *wsr[PTN], *xsr[PTM];
#pragma unroll
    for (int t = 0; t < PTN; ++t) {
        const int n = min(nb + 32 * t + l32, N - 1);
        wrow[t] = wq + (size_t)n * KB + 16 * hk;
        wsr[t] = wscale + (size_t)n * G;
    }
#pragma unroll
    for (int t = 0; t < PTM; ++t) {
        const int m = min(mb + 32 * t + l32, M - 1);
        xrow[t] = xq + (size_t)m * KB + 16 * hk;
        xsr[t] = xscale + (size_t)m * G;
    }

    f32x16 acc[PTN][PTM];
#pragma unroll
    for (int a = 0; a < PTN; ++a)
#pragma unroll
        for (int b = 0; b < PTM; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
    // the lane's 32 codes of group g (bytes 32 g + 16 hk of each row) and
    // the rows' scales, loaded one group ahead
    uint4 nw[PTN], nx[PTM];
    float sw[PTN], sx[PTM];
    auto load = [&](int g) {
#pragma unroll
        for (int t = 0; t < PTN; ++t) {
            nw[t] = *reinterpret_cast<const uint4 *>(wrow[t] + 32 * g);
            sw[t] = wsr[t][g];
        }
#pragma unroll
        for (int t = 0; t < PTM; ++t) {
            nx[t] = *reinterpret_cast<const uint4 *>(xrow[t] + 32 * g);
            sx[t] = xsr[t][g];
        }
    };
    const f32x16 zero16 = {};
    if (g0 < g1) load(g0);
#pragma unroll 1
    for (int g = g0; g < g1; ++g) {
        // widened as the full-size kernel's staging does
        i32x8 aw[PTN], bx[PTM];
        bf16x8 cw[PTN], cx[PTM];
#pragma unroll
        for (int t = 0; t < PTN; ++t) {
            uint4 lo, hi;
            widen_fp8(nw[t], lo, hi);
            aw[t] = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const uint2 v = scale_operand_w(sw[t] * kTwo17);
            cw[t] = __builtin_bit_cast(bf16x8, (uint4){v.x, v.y, 0u, 0u});
        }
#pragma unroll
        for (int t = 0; t < PTM; ++t) {
            uint4 lo, hi;
            widen_fp8(nx[t], lo, hi);
            bx[t] = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const uint2 v = scale_operand_x(sx[t]);
            cx[t] = __builtin_bit_cast(bf16x8, (uint4){v.x, v.y, 0u, 0u});
        }
        if (g + 1 < g1) load(g + 1);
#pragma unroll
        for (int tn = 0; tn < PTN; ++tn)
#pragma unroll
            for (int tm = 0; tm < PTM; ++tm) {
                const f32x16 pr = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aw[tn], bx[tm], zero16, 0, 0, 0,
                                                                                  127, 0, 127);
                const f32x16 c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cw[tn], cx[tm], zero16, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[tn][tm][i] = __builtin_fmaf(pr[i], c[i], acc[tn][tm][i]);
            }
    }

    // waves 1-7 hand their sums to wave 0, which adds them in wave order
    if (wave > 0) {
#pragma unroll
        for (int tn = 0; tn < PTN; ++tn)
#pragma unroll
            for (int tm = 0; tm < PTM; ++tm)
#pragma unroll
                for (int i = 0; i < 16; ++i) red[wave - 1][16 * (PTM * tn + tm) + i][lane] = acc[tn][tm][i];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll 1
    for (int w = 0; w < 7; ++w)
#pragma unroll
        for (int tn = 0; tn < PTN; ++tn)
#pragma unroll
            for (int tm = 0; tm < PTM; ++tm)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[tn][tm][i] += red[w][16 * (PTM * tn + tm) + i][lane];

    // the full-size kernel's epilogue arithmetic for the piece (staged in the
    // first partial-sum area, which wave 0 has finished reading)
    bf16x8 hhi[PTM][2], hlo[PTM][2];
#pragma unroll
    for (int tm = 0; tm < PTM; ++tm)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            float hv[8];
            load_h8(h, mb + tm * 32 + l32, M, 16 * s2 + 8 * hk, hv);
            split_h(hv, hhi[tm][s2], hlo[tm][s2]);
        }
    // y = acc + low-rank + bias (+ GELU), rounded to bf16 as the plain
    // epilogue stores it
    uint2 yb[PTN][PTM][4];
#pragma unroll
    for (int tn = 0; tn < PTN; ++tn) {
        const int nrow = nb + tn * 32 + l32;
        bf16x8 ua[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint4 uv = {0u, 0u, 0u, 0u};
            if (nrow < N) uv = *reinterpret_cast<const uint4 *>(up + (size_t)nrow * 32 + 16 * s2 + 8 * hk);
            ua[s2] = __builtin_bit_cast(bf16x8, uv);
        }
        const bf16x8 bq = bias_operand(bias, nb + tn * 32 + l32, N, hk), ones = ones_operand(hk);
#pragma unroll
        for (int tm = 0; tm < PTM; ++tm) {
            const f32x16 lr = add_lowrank_bias(acc[tn][tm], ua, hhi[tm], hlo[tm], bq, ones);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float y4[4] = {lr[4 * j], lr[4 * j + 1], lr[4 * j + 2], lr[4 * j + 3]};
                yb[tn][tm][j] = finish4(y4, EPI == EPI_STORE ? gelu : 0);
            }
        }
    }
    uint8_t *tile = reinterpret_cast<uint8_t *>(&red[0][0][0]);
    constexpr int STRIDE = EPI == EPI_STORE ? OUT_STRIDE : QKP_ROW;
    static_assert(PH * STRIDE <= sizeof(red) && 2 * PW <= STRIDE, "the piece's staging fits");
    const int head = nb / 128;
    const bool norm = EPI == EPI_QKNORM && head < 2 * qk.heads;    // a Q or a K head
    if constexpr (EPI == EPI_QKNORM) {
        // one head, all of it in this wave: lane (l32, hk) holds 64 of token
        // mb + l32's channels, the other 64 are in lane l32 + 32 - 64 hk.  The
        // sum of squares in the full-size kernel's order: each 64-channel
        // half (a wave tile there) by fma over its channels and the two
        // lanes, then the two halves added; the token's 1 / rms goes to the
        // spare bytes of its staged row.
        if (norm) {
            float ss[2] = {0.0f, 0.0f};
#pragma unroll
            for (int tn = 0; tn < PTN; ++tn)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint2 y2 = yb[tn][0][j];
                    const float v0 = bf16_to_f32(y2.x & 0xFFFFu), v1 = bf16_to_f32(y2.x >> 16);
                    const float v2 = bf16_to_f32(y2.y & 0xFFFFu), v3 = bf16_to_f32(y2.y >> 16);
                    float &a = ss[tn >> 1];
                    a = __builtin_fmaf(v0, v0, a);
                    a = __builtin_fmaf(v1, v1, a);
                    a = __builtin_fmaf(v2, v2, a);
                    a = __builtin_fmaf(v3, v3, a);
                }
            ss[0] += __shfl_xor(ss[0], 32);
            ss[1] += __shfl_xor(ss[1], 32);
            if (hk == 0)
                *reinterpret_cast<float *>(tile + l32 * STRIDE + 256) =
                    __builtin_amdgcn_rsqf(__builtin_fmaf(ss[0] + ss[1], 1.0f / 128.0f, qk.eps));
        }
    }
#pragma unroll
    for (int tn = 0; tn < PTN; ++tn)
#pragma unroll
        for (int tm = 0; tm < PTM; ++tm)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<uint2 *>(tile + (tm * 32 + l32) * STRIDE + (tn * 32 + 8 * j + 4 * hk) * 2) =
                    yb[tn][tm][j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // PH rows x PW channels: rows of PW / 8 segments of 16 bytes; head pieces
    // are normalized and rotated on the way out (16 lanes per token, the
    // rotation tables read as whole rows)
    constexpr int SEGS = PW / 8;
    uint4 wv = {0u, 0u, 0u, 0u};
    if (norm) wv = *reinterpret_cast<const uint4 *>((head < qk.heads ? qk.norm_q : qk.norm_k) + 8 * (lane % SEGS));
#pragma unroll
    for (int it = 0; it < PH * SEGS / 64; ++it) {
        const int idx = lane + 64 * it, r = idx / SEGS, seg = idx % SEGS;
        uint4 v = *reinterpret_cast<const uint4 *>(tile + r * STRIDE + seg * 16);
        const int m = mb + r, n = nb + seg * 8;
        if (norm) {
            const float rs = *reinterpret_cast<const float *>(tile + r * STRIDE + 256);
            const int mc = m < M ? m : M - 1;                     // rows past M are never stored
            v = qk_norm_rope8(v, rs, wv, *reinterpret_cast<const float4 *>(qk.rope_cos + (size_t)mc * 64 + 4 * seg),
                              *reinterpret_cast<const float4 *>(qk.rope_sin + (size_t)mc * 64 + 4 * seg));
        }
        if (m < M && n < N) store_nt(Y + (size_t)m * N + n, v);
    }
}

// Launches the pieces of the tiles left after `full` tiles, when they fit in
// one round: plain pieces of 64 x 32 (16 per tile) or 64 x 64 (8), head
// pieces of 32 x 128 (8).
template <int EPI>
hipError_t launch_int4_tail(const uint8_t *xq, const float *xscale, const float *h, const uint8_t *wq,
                            const float *wscale, const uint16_t *up, const uint16_t *bias, int M, int N, int K,
                            int gelu, uint16_t *Y, int full, int rest, int ncu, const QKNormArgs &qk,
                            hipStream_t stream)
{
    if constexpr (EPI == EPI_QKNORM) {
        hipLaunchKernelGGL((w4a4_int4_tail_kernel<4, 1, EPI_QKNORM>), dim3((unsigned)(rest * I4Tail<4, 1>::kPieces)),
                           dim3(I4_THREADS), 0, stream, xq, xscale, h, wq, wscale, up, bias, M, N, K, 0, Y, full, qk);
    } else if (rest * I4Tail<1, 2>::kPieces <= ncu) {
        hipLaunchKernelGGL((w4a4_int4_tail_kernel<1, 2, EPI_STORE>), dim3((unsigned)(rest * I4Tail<1, 2>::kPieces)),
                           dim3(I4_THREADS), 0, stream, xq, xscale, h, wq, wscale, up, bias, M, N, K, gelu, Y, full,
                           qk);
    } else {
        hipLaunchKernelGGL((w4a4_int4_tail_kernel<2, 2, EPI_STORE>), dim3((unsigned)(rest * I4Tail<2, 2>::kPieces)),
                           dim3(I4_THREADS), 0, stream, xq, xscale, h, wq, wscale, up, bias, M, N, K, gelu, Y, full,
                           qk);
    }
    return hipGetLastError();
}

// Whole rounds of one block per CU, then the leftover tiles: the number of
// tiles the full-size kernel takes (all of them when the leftover's pieces
// would not fit in one round, which `rest` then reports as 0).
int int4_main_tiles(int tiles, int pieces_per_tile, int ncu, int &rest)
{
    const int full = (tiles / ncu) * ncu;
    rest = tiles - full;
    if (full == 0 || rest == 0 || rest * pieces_per_tile > ncu) {
        rest = 0;
        return tiles;
    }
    return full;
}

// Fixed-order sum of the per-tile partial h2: h2[m][j] = sum_t hpart[t][m][j],
// t ascending.
__global__ __launch_bounds__(256) void requant_h_reduce(const float *__restrict__ hpart, int T, int M,
                                                        float *__restrict__ h2)
{
    const int i = blockIdx.x * 256 + threadIdx.x;      // (m * 32 + j) / 4
    if (i >= M * 8) return;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    const f32x4 *p = reinterpret_cast<const f32x4 *>(hpart) + i;
    const size_t step = (size_t)M * 8;
    int t = 0;
    for (; t + 8 <= T; t += 8) {          // 8 loads in flight, added in order
        f32x4 a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] = __builtin_nontemporal_load(p + (t + u) * step);
#pragma unroll
        for (int u = 0; u < 8; ++u) s += a[u];
    }
    for (; t < T; ++t) s += __builtin_nontemporal_load(p + t * step);
    reinterpret_cast<f32x4 *>(h2)[i] = s;
}

// ===================================================================== MXFP4

// Block tile 256 (n) x 128 (m), 4 waves of 128 x 64, each 4 x 2 tiles of
// 32x32 from v_mfma_scale_f32_32x32x64_f8f6f4 (fp4 x fp4, 8 passes): per
// 128-channel step a wave issues 16 products from 12 fragment reads.
constexpr int MX_BN = 256, MX_BM = 128;        // block tile (n, m)
constexpr int MX_WN = 128, MX_WM = 64;         // wave tile
constexpr int MX_TN = MX_WN / 32, MX_TM = MX_WM / 32;
constexpr int MX_THREADS = 256;
constexpr int MX_STRIDE = 64;   // LDS bytes per row: 64 code bytes (128 fp4), segments swizzled

// 16-byte segment s of LDS row r lives at segment s ^ ((r >> 1) & 3) ^
// ((r >> 3) & 1).  A fragment read takes one segment of 32 consecutive rows;
// the LDS serves 16 lanes (256 bytes, 64 banks) per cycle, and those 16 rows
// land in 16 distinct 16-byte bank groups (as do any 8 aligned rows within
// a 128-byte window).  The loader's stores fill whole rows.
__device__ __forceinline__ int mx_seg(int r, int s) { return s ^ ((r >> 1) & 3) ^ ((r >> 3) & 1); }

struct __attribute__((aligned(16))) MXSmem {
    uint8_t w[2][MX_BN * MX_STRIDE];
    uint8_t x[2][MX_BM * MX_STRIDE];
    uint32_t ew[2][MX_BN];     // the 4 E8M0 bytes of the step's 4 blocks, per row
    uint32_t ex[2][MX_BM];
};

// Epilogue of a wave tile of TN x TM 32x32 tiles (TN even): low-rank term
// via v_mfma_f32_32x32x16_bf16 (rank 32 = two k steps of 16, each with the hi
// and the lo part of h), then bias, GELU, and the store, staged in the wave's
// own LDS area `tile` one 64 x 64 block at a time.  (mb, nb) is the wave
// tile's first token and channel.
template <int TN, int TM>
__device__ __forceinline__ void wave_epilogue(const f32x16 (&acc)[TN][TM], const float *__restrict__ h,
                                              const uint16_t *__restrict__ up, const uint16_t *__restrict__ bias,
                                              int M, int N, int gelu, uint16_t *__restrict__ Y, int mb, int nb,
                                              uint8_t *tile, int lane)
{
    static_assert(TN % 2 == 0 && TM == 2, "64 x 64 staging blocks");
    const int l32 = lane & 31, hk = lane >> 5;
    bf16x8 hhi[TM][2], hlo[TM][2];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            float hv[8];
            load_h8(h, mb + tm * 32 + l32, M, 16 * s2 + 8 * hk, hv);
            split_h(hv, hhi[tm][s2], hlo[tm][s2]);
        }
#pragma unroll
    for (int half = 0; half < TN / 2; ++half) {
#pragma unroll
        for (int th = 0; th < 2; ++th) {
            const int tn = 2 * half + th;
            const int nrow = nb + tn * 32 + l32;
            bf16x8 ua[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                uint4 uv = {0u, 0u, 0u, 0u};
                if (nrow < N) uv = *reinterpret_cast<const uint4 *>(up + (size_t)nrow * 32 + 16 * s2 + 8 * hk);
                ua[s2] = __builtin_bit_cast(bf16x8, uv);
            }
            const bf16x8 bq = bias_operand(bias, nb + tn * 32 + l32, N, hk), ones = ones_operand(hk);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const f32x16 lr = add_lowrank_bias(acc[tn][tm], ua, hhi[tm], hlo[tm], bq, ones);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float y4[4] = {lr[4 * j], lr[4 * j + 1], lr[4 * j + 2], lr[4 * j + 3]};
                    stage4(tile, tm * 32 + l32, th * 32 + 8 * j + 4 * hk, finish4(y4, gelu));
                }
            }
        }
        // the staged half is read back by other lanes of this wave
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        flush_tile(tile, Y, mb, nb + 64 * half, M, N, lane);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

__global__ __launch_bounds__(MX_THREADS) void w4a4_mxfp4_kernel(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ xscale, const float *__restrict__ h,
    const uint8_t *__restrict__ wq, const uint8_t *__restrict__ wscale, const uint16_t *__restrict__ up,
    const uint16_t *__restrict__ bias, int M, int N, int K, int gelu, uint16_t *__restrict__ Y)
{
    __shared__ MXSmem sm;
    static_assert(4 * OUT_TILE_BYTES <= sizeof(MXSmem), "output staging fits in LDS");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    int tn_, tm_;
    tile_coords(blockIdx.x, (N + MX_BN - 1) / MX_BN, (M + MX_BM - 1) / MX_BM, tn_, tm_);
    const int n0 = tn_ * MX_BN, m0 = tm_ * MX_BM;
    const int KB = K >> 1;          // code bytes per row
    const int NB = K >> 5;          // E8M0 scales per row
    const int steps = (K + 127) >> 7;

    // Loader: thread t moves segment t & 3 (32 codes, 16 bytes) of weight rows
    // t/4 + 64 i (i < 4) and token rows t/4 + 64 i (i < 2), and the E8M0
    // bytes of weight row t and (t < 128) token row t.  Loads are
    // unconditional (rows clamped, blocks past K zeroed at the LDS store), so
    // every path keeps the same number of loads in flight.
    const int lrow = tid >> 2, lseg = tid & 3;
    const uint8_t *__restrict__ wsrc = wq + (size_t)min(n0 + lrow, N - 1) * KB;
    const size_t wstep = (size_t)KB * 64;                 // 64 rows further
    const int wlast = N - 1 - n0;                        // rows past N clamp to the last row
    const uint8_t *__restrict__ xsrc0 = xq + (size_t)min(m0 + lrow, M - 1) * KB;
    const uint8_t *__restrict__ xsrc1 = xq + (size_t)min(m0 + lrow + 64, M - 1) * KB;
    const uint8_t *__restrict__ wssrc = wscale + (size_t)min(n0 + tid, N - 1) * NB;
    const uint8_t *__restrict__ xssrc = xscale + (size_t)min(m0 + (tid & 127), M - 1) * NB;
    const bool aligned_scales = (NB & 3) == 0;
    int wofs[4], xofs[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) wofs[i] = (lrow + 64 * i) * MX_STRIDE + mx_seg(lrow + 64 * i, lseg) * 16;
#pragma unroll
    for (int i = 0; i < 2; ++i) xofs[i] = (lrow + 64 * i) * MX_STRIDE + mx_seg(lrow + 64 * i, lseg) * 16;
    const uint8_t *wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wrow[i] = (lrow + 64 * i <= wlast) ? wsrc + wstep * i : wq + (size_t)(N - 1) * KB;

    uint4 rw[4], rx[2];
    uint32_t rsw, rsx;
    auto scale4 = [&](const uint8_t *src, int st) -> uint32_t {
        if (aligned_scales) return *reinterpret_cast<const uint32_t *>(src + min(st * 4, NB - 4));
        uint32_t v = 0;
        for (int q = 0; q < 4; ++q) v |= (uint32_t)src[min(st * 4 + q, NB - 1)] << (8 * q);
        return v;
    };
#define MX_GLOAD(st)                                                                       \
    do {                                                                                   \
        const int b_ = min((st) * 4 + lseg, NB - 1);                                       \
        rw[0] = *reinterpret_cast<const uint4 *>(wrow[0] + b_ * 16);                       \
        rw[1] = *reinterpret_cast<const uint4 *>(wrow[1] + b_ * 16);                       \
        rw[2] = *reinterpret_cast<const uint4 *>(wrow[2] + b_ * 16);                       \
        rw[3] = *reinterpret_cast<const uint4 *>(wrow[3] + b_ * 16);                       \
        rx[0] = *reinterpret_cast<const uint4 *>(xsrc0 + b_ * 16);                         \
        rx[1] = *reinterpret_cast<const uint4 *>(xsrc1 + b_ * 16);                         \
        rsw = scale4(wssrc, (st));                                                         \
        rsx = scale4(xssrc, (st));                                                         \
    } while (0)
#define MX_LSTORE(st, buf)                                                                 \
    do {                                                                                   \
        const bool kv_ = (st) * 4 + lseg < NB;                                             \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                   \
            *reinterpret_cast<uint4 *>(&sm.w[buf][wofs[i_]]) = keep_if(kv_, rw[i_]);       \
        _Pragma("unroll") for (int i_ = 0; i_ < 2; ++i_)                                   \
            *reinterpret_cast<uint4 *>(&sm.x[buf][xofs[i_]]) = keep_if(kv_, rx[i_]);       \
        sm.ew[buf][tid] = rsw;                                                             \
        if (tid < MX_BM) sm.ex[buf][tid] = rsx;                                            \
    } while (0)

    f32x16 acc[MX_TN][MX_TM];
#pragma unroll
    for (int a = 0; a < MX_TN; ++a)
#pragma unroll
        for (int b = 0; b < MX_TM; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    if (steps > 0) {
        MX_GLOAD(0);
        MX_LSTORE(0, 0);
        MX_GLOAD(min(1, steps - 1));
    }
    __syncthreads();
    const int l32 = lane & 31, hk = lane >> 5;
    for (int st = 0; st < steps; ++st) {
        const int buf = st & 1;
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {           // two 64-channel slices of the step
            const int seg = 2 * sl + hk;           // the lane's 32-channel block
            i32x8 aw[MX_TN], bx[MX_TM];
            int ew[MX_TN], ex[MX_TM];
#pragma unroll
            for (int tn = 0; tn < MX_TN; ++tn) {
                const int r = wn * MX_WN + tn * 32 + l32;
                const uint4 v = *reinterpret_cast<const uint4 *>(&sm.w[buf][r * MX_STRIDE + 16 * mx_seg(r, seg)]);
                aw[tn] = (i32x8){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                ew[tn] = (int)((sm.ew[buf][r] >> (8 * seg)) & 0xFFu);
            }
#pragma unroll
            for (int tm = 0; tm < MX_TM; ++tm) {
                const int r = wm * MX_WM + tm * 32 + l32;
                const uint4 v = *reinterpret_cast<const uint4 *>(&sm.x[buf][r * MX_STRIDE + 16 * mx_seg(r, seg)]);
                bx[tm] = (i32x8){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                ex[tm] = (int)((sm.ex[buf][r] >> (8 * seg)) & 0xFFu);
            }
#pragma unroll
            for (int tn = 0; tn < MX_TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < MX_TM; ++tm)
                    acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        aw[tn], bx[tm], acc[tn][tm], 4, 4, 0, ew[tn], 0, ex[tm]);
        }
        if (st + 1 < steps) {
            MX_LSTORE(st + 1, buf ^ 1);
            MX_GLOAD(min(st + 2, steps - 1));   // unconditional: same load count on every path
        }
        __syncthreads();
    }
#undef MX_GLOAD
#undef MX_LSTORE

    wave_epilogue<MX_TN, MX_TM>(acc, h, up, bias, M, N, gelu, Y, m0 + wm * MX_WM, n0 + wn * MX_WN,
                reinterpret_cast<uint8_t *>(&sm) + wave * OUT_TILE_BYTES, lane);
}

// --------------------------------------------------- MXFP4, LDS-DMA pipeline
//
// For K % 256 == 0 (every DiT shape): the operands go from HBM straight into
// LDS with global_load_lds_dwordx4 / _dword (no register staging), double
// buffered, in 256-channel steps so that every row access is a whole
// 128-byte line (the address unit handles each line once).  Block tile
// 256 (n) x 256 (m) with 8 waves (2 per SIMD) of 128 x 64, the same per-wave
// products as above.  Per step each wave moves 10 loads: 4 weight and 4 token
// blocks of 8 rows x 128 bytes, and one 32-row slice of the weight and of the
// token E8M0 bytes (two dwords per row).  An LDS-DMA load writes its 64
// lanes' 16 (or 4) bytes contiguously from the wave-uniform base in M0, so
// each lane fetches the global segment that belongs at its slot of the
// swizzled layout.  The compiler does not see these loads: completion is
// awaited by hand (vmcnt) before the barrier that publishes a stage, and M0
// is restored after each load.
constexpr int MXD_BN = 256, MXD_BM = 256;
constexpr int MXD_THREADS = 512;
constexpr int MXD_ROW = 128;        // LDS bytes per row and step: 256 fp4, 16-byte segments swizzled

// 16-byte segment s of LDS row r lives at segment s ^ (r & 7) ^ ((r >> 3) & 1).
// A fragment read takes one segment of 32 consecutive rows; the LDS serves
// 16 lanes (256 bytes, 64 banks) per cycle, and those 16 rows land in 16
// distinct 16-byte bank groups (as do any 8 aligned rows within a 128-byte
// window).  The loads write whole rows.
__device__ __forceinline__ int mxd_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int mxd_seg(int r, int s) { return s ^ mxd_swz(r); }

struct __attribute__((aligned(16))) MXDStage {
    uint8_t w[MXD_BN * MXD_ROW];
    uint8_t x[MXD_BM * MXD_ROW];
    uint32_t ew[2 * MXD_BN];         // row r, dword d (blocks 4 d .. 4 d + 3) at [64 (r / 32) + 2 (r % 32) + d]
    uint32_t ex[2 * MXD_BM];
};
static_assert(8 * OUT_TILE_BYTES <= sizeof(MXDStage), "output staging fits in one stage");

// Epilogue of the requantizing MXFP4 kernel for one wave tile (128 channels,
// four 32-channel blocks, x 64 tokens): as requant_epilogue, with E8M0 block
// scales and E2M1 codes.  Lane (l32, hk) holds, per 32-token tile tm and
// block tn, channels nb + 32 tn + 8 j + 4 hk + (0..3): half of the token's
// block.  Blocks at or past N (N % 32 == 0) are neither stored nor summed.
// `P` is LDS that no wave reads any more (the stage of the tile's last step).
__device__ __forceinline__ void requant_epilogue_mx(const f32x16 (&acc)[MX_TN][MX_TM], const float *__restrict__ h,
                                                    const uint16_t *__restrict__ up,
                                                    const uint16_t *__restrict__ bias, int M, int N, int gelu,
                                                    const RequantArgs &rq, int mb, int nb, int tile_n, int m0, int wn,
                                                    int wm, int tid, int lane, float *P)
{
    const int l32 = lane & 31, hk = lane >> 5;
    bf16x8 hhi[MX_TM][2], hlo[MX_TM][2];
#pragma unroll
    for (int tm = 0; tm < MX_TM; ++tm)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            float hv[8];
            load_h8(h, mb + tm * 32 + l32, M, 16 * s2 + 8 * hk, hv);
            split_h(hv, hhi[tm][s2], hlo[tm][s2]);
        }
    f32x16 hp[MX_TM] = {};
    uint32_t e8s[MX_TM] = {};           // E8M0 of the 4 blocks, one byte each (lanes hk = 0)
#pragma unroll
    for (int tn = 0; tn < MX_TN; ++tn) {
        const int c0 = nb + tn * 32;
        const bool live = c0 < N;
        const int nrow = c0 + l32;
        bf16x8 ua[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint4 uv = {0u, 0u, 0u, 0u};
            if (nrow < N) uv = *reinterpret_cast<const uint4 *>(up + (size_t)nrow * 32 + 16 * s2 + 8 * hk);
            ua[s2] = __builtin_bit_cast(bf16x8, uv);
        }
        const bf16x8 bq = bias_operand(bias, c0 + l32, N, hk), ones = ones_operand(hk);
        float4 s2v[4];
        bf16x8 dn[2];                    // A operands: down2 rows l32, k blocks 2 tn and 2 tn + 1
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s2v[j] = live ? *reinterpret_cast<const float4 *>(rq.smooth2 + c0 + 8 * j + 4 * hk)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const int c = c0 + 16 * kh + 4 * hk;
            uint2 a = {0u, 0u}, b = {0u, 0u};
            if (live) {
                a = *reinterpret_cast<const uint2 *>(rq.down2 + (size_t)l32 * N + c);
                b = *reinterpret_cast<const uint2 *>(rq.down2 + (size_t)l32 * N + c + 8);
            }
            dn[kh] = __builtin_bit_cast(bf16x8, (uint4){a.x, a.y, b.x, b.y});
        }
#pragma unroll
        for (int tm = 0; tm < MX_TM; ++tm) {
            const int m = mb + tm * 32 + l32;
            const f32x16 lr = add_lowrank_bias(acc[tn][tm], ua, hhi[tm], hlo[tm], bq, ones);
            uint2 yb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float y4[4] = {lr[4 * j], lr[4 * j + 1], lr[4 * j + 2], lr[4 * j + 3]};
                yb[j] = finish4(y4, gelu);
            }
            // smoothed values, block absmax over both lane halves, E8M0
            float v[4][4];
            float amax = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sv[4] = {s2v[j].x, s2v[j].y, s2v[j].z, s2v[j].w};
                const float yv[4] = {bf16_to_f32(yb[j].x & 0xFFFFu), bf16_to_f32(yb[j].x >> 16),
                                     bf16_to_f32(yb[j].y & 0xFFFFu), bf16_to_f32(yb[j].y >> 16)};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[j][e] = yv[e] * sv[e];
                    amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j][e]));
                }
            }
            amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
            const uint32_t e8 = mx_block_e8m0(amax);
            const float inv = mx_inv_scale(e8);
            // E2M1 codes (the hardware conversion at unit scale of the exactly
            // pre-scaled values): pieces j = 0, 1 in dword lo, 2, 3 in hi
            uint32_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0][0] * inv, v[0][1] * inv, 1.0f, 0);
            lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[0][2] * inv, v[0][3] * inv, 1.0f, 1);
            lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[1][0] * inv, v[1][1] * inv, 1.0f, 2);
            lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[1][2] * inv, v[1][3] * inv, 1.0f, 3);
            uint32_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[2][0] * inv, v[2][1] * inv, 1.0f, 0);
            hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[2][2] * inv, v[2][3] * inv, 1.0f, 1);
            hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[3][0] * inv, v[3][1] * inv, 1.0f, 2);
            hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[3][2] * inv, v[3][3] * inv, 1.0f, 3);
            // byte 4 j + 2 half of the block's 16 code bytes is lane half
            // `half`'s piece j: half 0 keeps j = 0, 1 and takes its partner's,
            // half 1 keeps j = 2, 3
            const uint32_t got = (uint32_t)__shfl_xor((int)(hk ? lo : hi), 32);
            const uint32_t own = hk ? hi : lo;
            uint2 out;
            if (hk == 0) out = make_uint2((own & 0xFFFFu) | got << 16, (own >> 16) | (got & 0xFFFF0000u));
            else out = make_uint2((got & 0xFFFFu) | own << 16, (got >> 16) | (own & 0xFFFF0000u));
            if (live && m < M) *reinterpret_cast<uint2 *>(rq.xq2 + (size_t)m * (N / 2) + c0 / 2 + 8 * hk) = out;
            e8s[tm] |= e8 << (8 * tn);
            // partial h2 over the block's 32 channels
            const bf16x8 b0 = __builtin_bit_cast(bf16x8, live ? (uint4){yb[0].x, yb[0].y, yb[1].x, yb[1].y}
                                                              : (uint4){0u, 0u, 0u, 0u});
            const bf16x8 b1 = __builtin_bit_cast(bf16x8, live ? (uint4){yb[2].x, yb[2].y, yb[3].x, yb[3].y}
                                                              : (uint4){0u, 0u, 0u, 0u});
            hp[tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dn[0], b0, hp[tm], 0, 0, 0);
            hp[tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dn[1], b1, hp[tm], 0, 0, 0);
        }
    }
#pragma unroll
    for (int tm = 0; tm < MX_TM; ++tm) {
        const int m = mb + tm * 32 + l32;
        if (hk == 0 && m < M) {
            uint8_t *dst = static_cast<uint8_t *>(rq.xscale2) + (size_t)m * (N / 32) + nb / 32;
#pragma unroll
            for (int tn = 0; tn < MX_TN; ++tn)
                if (nb + tn * 32 < N) dst[tn] = (uint8_t)(e8s[tm] >> (8 * tn));
        }
    }
    // the block's two channel halves summed in LDS (fixed order), one row of
    // 32 partial sums per token to hpart
    __syncthreads();
#pragma unroll
    for (int tm = 0; tm < MX_TM; ++tm) {
        const int ml = wm * MX_WM + tm * 32 + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 w4 = make_float4(hp[tm][4 * q], hp[tm][4 * q + 1], hp[tm][4 * q + 2], hp[tm][4 * q + 3]);
            *reinterpret_cast<float4 *>(P + ((size_t)wn * MXD_BM + ml) * 32 + 8 * q + 4 * hk) = w4;
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int idx = tid + MXD_THREADS * k;          // (token, 8-float slice) of the block's 256 x 32
        const int ml = idx >> 2, j0 = 8 * (idx & 3);
        const float *s0p = P + (size_t)ml * 32 + j0, *s1p = P + ((size_t)MXD_BM + ml) * 32 + j0;
        const float4 a0 = *reinterpret_cast<const float4 *>(s0p), a1 = *reinterpret_cast<const float4 *>(s0p + 4);
        const float4 b0 = *reinterpret_cast<const float4 *>(s1p), b1 = *reinterpret_cast<const float4 *>(s1p + 4);
        const int m = m0 + ml;
        if (m < M) {
            float *dst = rq.hpart + ((size_t)tile_n * M + m) * 32 + j0;
            *reinterpret_cast<float4 *>(dst) = make_float4(a0.x + b0.x, a0.y + b0.y, a0.z + b0.z, a0.w + b0.w);
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(a1.x + b1.x, a1.y + b1.y, a1.z + b1.z, a1.w + b1.w);
        }
    }
}

// Epilogue of the MXFP4 QKV kernel with Q/K RMS-norm and rotary embedding,
// for one wave tile: 4 x 2 tiles of 32 x 32 = 128 channels (one whole head,
// since nb is a multiple of 128) x 64 tokens.  Lane (l32, hk) holds, per
// token mb + 32 tm + l32, the channels 32 tn + 8 j + 4 hk + (0..3) of the head
// (64 of its 128); its partner lane (l32, hk ^ 1) holds the other 64, so the
// head's sum of squares takes one cross-half exchange.  The bf16 outputs are
// parked in the wave's own LDS area (64 tokens x 128 channels, rows of 256 +
// 8 bytes, the spare 8 holding the token's 1 / rms) while the sums are
// formed; then 16 lanes per token read the row back, 8 channels (4 rotation
// pairs) each, normalize and rotate them with the token's angles read as
// whole rows, and store the row as 256 contiguous bytes.  `area` holds
// QK_AREA_BYTES bytes per wave, used by no other wave.
constexpr int QK_ROW = 264;
constexpr int QK_AREA_BYTES = 64 * QK_ROW;

__device__ __forceinline__ void qknorm_wave_epilogue_mx(const f32x16 (&acc)[MX_TN][MX_TM], const float *__restrict__ h,
                                                        const uint16_t *__restrict__ up,
                                                        const uint16_t *__restrict__ bias, int M, int N,
                                                        const QKNormArgs &qk, uint16_t *__restrict__ Y, int mb, int nb,
                                                        uint8_t *area, int lane)
{
    const int l32 = lane & 31, hk = lane >> 5;
    bf16x8 hhi[MX_TM][2], hlo[MX_TM][2];
#pragma unroll
    for (int tm = 0; tm < MX_TM; ++tm)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            float hv[8];
            load_h8(h, mb + tm * 32 + l32, M, 16 * s2 + 8 * hk, hv);
            split_h(hv, hhi[tm][s2], hlo[tm][s2]);
        }
    const int head = nb / 128;
    const bool norm = nb < N && head < 2 * qk.heads;      // a Q or a K head
    // pass 1: the bf16 outputs, exactly as wave_epilogue stores them, into
    // the area; the sum of their squares per token
    float ss[MX_TM] = {0.0f, 0.0f};
#pragma unroll
    for (int tn = 0; tn < MX_TN; ++tn) {
        const int nrow = nb + tn * 32 + l32;
        bf16x8 ua[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint4 uv = {0u, 0u, 0u, 0u};
            if (nrow < N) uv = *reinterpret_cast<const uint4 *>(up + (size_t)nrow * 32 + 16 * s2 + 8 * hk);
            ua[s2] = __builtin_bit_cast(bf16x8, uv);
        }
        const bf16x8 bq = bias_operand(bias, nb + tn * 32 + l32, N, hk), ones = ones_operand(hk);
#pragma unroll
        for (int tm = 0; tm < MX_TM; ++tm) {
            const f32x16 lr = add_lowrank_bias(acc[tn][tm], ua, hhi[tm], hlo[tm], bq, ones);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float y4[4] = {lr[4 * j], lr[4 * j + 1], lr[4 * j + 2], lr[4 * j + 3]};
                const uint2 y = finish4(y4, 0);
                *reinterpret_cast<uint2 *>(area + (tm * 32 + l32) * QK_ROW + (tn * 32 + 8 * j + 4 * hk) * 2) = y;
                const float v0 = bf16_to_f32(y.x & 0xFFFFu), v1 = bf16_to_f32(y.x >> 16);
                const float v2 = bf16_to_f32(y.y & 0xFFFFu), v3 = bf16_to_f32(y.y >> 16);
                ss[tm] = __builtin_fmaf(v0, v0, ss[tm]);
                ss[tm] = __builtin_fmaf(v1, v1, ss[tm]);
                ss[tm] = __builtin_fmaf(v2, v2, ss[tm]);
                ss[tm] = __builtin_fmaf(v3, v3, ss[tm]);
            }
        }
    }
    // the token's 1 / rms (Q and K heads) in the 8 spare bytes of its staged row
    if (norm) {
#pragma unroll
        for (int tm = 0; tm < MX_TM; ++tm) {
            const float tot = ss[tm] + __shfl_xor(ss[tm], 32);
            const float rs = __builtin_amdgcn_rsqf(__builtin_fmaf(tot, 1.0f / 128.0f, qk.eps));
            if (hk == 0) *reinterpret_cast<float *>(area + (tm * 32 + l32) * QK_ROW + 256) = rs;
        }
    }
    // the area is read back by other lanes of this wave: whole 256-byte rows,
    // 16 lanes per row, each with 8 channels (4 rotation pairs) of its token.
    // Q and K heads are normalized and rotated on the way out, so that the
    // norm weights are read once and the rotation tables as whole rows
    // (16 lanes x 16 bytes per token).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int seg = lane & 15;
    uint4 wv = {0u, 0u, 0u, 0u};
    if (norm) wv = *reinterpret_cast<const uint4 *>((head < qk.heads ? qk.norm_q : qk.norm_k) + 8 * seg);
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int r = (lane >> 4) + 4 * it;
        uint4 v = *reinterpret_cast<const uint4 *>(area + r * QK_ROW + seg * 16);
        const int m = mb + r, n = nb + seg * 8;
        if (norm) {
            const float rs = *reinterpret_cast<const float *>(area + r * QK_ROW + 256);
            const int mc = m < M ? m : M - 1;                     // rows past M are never stored
            v = qk_norm_rope8(v, rs, wv, *reinterpret_cast<const float4 *>(qk.rope_cos + (size_t)mc * 64 + 4 * seg),
                              *reinterpret_cast<const float4 *>(qk.rope_sin + (size_t)mc * 64 + 4 * seg));
        }
        if (m < M && n < N) store_nt(Y + (size_t)m * N + n, v);
    }
}

// Persistent: block b takes the tiles b, b + gridDim.x, ...  The two stages
// alternate over the global step count, and the first step of the next tile
// is loaded into the free stage while the epilogue of the current tile runs
// (its output staging uses the other stage).
// What the LDS-DMA MXFP4 kernel does with a finished tile.
constexpr int MXE_STORE = 0;      // y -> bf16 Y
constexpr int MXE_REQUANT = 1;    // the next layer's activation step (RequantArgs)
constexpr int MXE_PARTIAL = 2;    // fp32 partial sums of one K slice (split K)
constexpr int MXE_QKNORM = 3;     // Q/K RMS-norm + rotary embedding of a QKV projection (QKNormArgs)

// Split K: work item t is tile t % tiles over K slice t / tiles, of S slices
// of `sps` 256-channel steps each (the last one may be shorter); the slice's
// fp32 sums go to part[slice][M][N].
struct SplitArgs {
    float *part;
    int S;
    int sps;
};

template <int MODE>
__global__ __launch_bounds__(MXD_THREADS) void w4a4_mxfp4_dma_kernel(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ xscale, const float *__restrict__ h,
    const uint8_t *__restrict__ wq, const uint8_t *__restrict__ wscale, const uint16_t *__restrict__ up,
    const uint16_t *__restrict__ bias, int M, int N, int K, int gelu, uint16_t *__restrict__ Y, RequantArgs rq,
    SplitArgs sk, QKNormArgs qk)
{
    __shared__ MXDStage stage[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
    const int wn = wave & 1, wm = wave >> 1;            // 2 (n) x 4 (m) waves
    const int tiles_n = (N + MXD_BN - 1) / MXD_BN, tiles_m = (M + MXD_BM - 1) / MXD_BM;
    const int tiles = tiles_n * tiles_m;
    const int KB = K >> 1;          // code bytes per row
    const int NB = K >> 5;          // E8M0 scales per row (a multiple of 8 here)
    const int steps = K >> 8;
    const int l32 = lane & 31, hk = lane >> 5;

    // Per-lane source offsets of a tile (bytes from the step's base); rows
    // past N / M read the last row (their outputs are never stored).
    uint32_t wvo[4], xvo[4], ewo, exo;
    auto set_tile = [&](int t, int &n0, int &m0) {
        int tn_, tm_;
        tile_coords(t, tiles_n, tiles_m, tn_, tm_);
        n0 = tn_ * MXD_BN;
        m0 = tm_ * MXD_BM;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 8 * (8 * i + wave) + (lane >> 3);        // block 8 i + wave
            const int seg = mxd_seg(r, lane & 7);      // LDS slot lane & 7 holds this global segment
            wvo[i] = (uint32_t)(min(n0 + r, N - 1) * KB + 16 * seg);
            xvo[i] = (uint32_t)(min(m0 + r, M - 1) * KB + 16 * seg);
        }
        ewo = (uint32_t)(min(n0 + 32 * wave + (lane >> 1), N - 1) * NB + 4 * (lane & 1));
        exo = (uint32_t)(min(m0 + 32 * wave + (lane >> 1), M - 1) * NB + 4 * (lane & 1));
    };
    auto issue = [&](int st, int sg) {
        MXDStage &S = stage[sg];
        const uint8_t *wb = wq + 128 * st, *xb = xq + 128 * st;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma_b128(lds_offset(&S.w[1024 * (8 * i + wave)]), wvo[i], wb);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma_b128(lds_offset(&S.x[1024 * (8 * i + wave)]), xvo[i], xb);
        dma_b32(lds_offset(&S.ew[64 * wave]), ewo, wscale + 8 * st);
        dma_b32(lds_offset(&S.ex[64 * wave]), exo, xscale + 8 * st);
    };

    const int items = MODE == MXE_PARTIAL ? tiles * sk.S : tiles;
    // item -> tile and its range of steps [st0, st0 + nst)
    auto item_steps = [&](int it, int &st0, int &nst) {
        if constexpr (MODE == MXE_PARTIAL) {
            st0 = (it / tiles) * sk.sps;
            nst = min(sk.sps, steps - st0);
        } else {
            st0 = 0;
            nst = steps;
        }
    };
    int t = blockIdx.x;
    if (t >= items) return;
    int n0, m0, st0, nst;
    set_tile(t % tiles, n0, m0);
    item_steps(t, st0, nst);
    int g = 0;                      // global step count: step st of the current item uses stage (g + st) & 1
    issue(st0, 0);
    while (true) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
        f32x16 acc[MX_TN][MX_TM];
#pragma unroll
        for (int a = 0; a < MX_TN; ++a)
#pragma unroll
            for (int b = 0; b < MX_TM; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
        for (int st = 0; st < nst; ++st) {
            const int sg = (g + st) & 1;
            if (st + 1 < nst) issue(st0 + st + 1, sg ^ 1);
            const MXDStage &S = stage[sg];
            // four 64-channel slices per step; the fragments of slice sl + 1
            // are read while the products of slice sl run
            // the step's E8M0 bytes of the wave's rows (8 per row: two dwords)
            uint2 esw[MX_TN], esx[MX_TM];
#pragma unroll
            for (int tn = 0; tn < MX_TN; ++tn) {
                const int r = wn * MX_WN + tn * 32 + l32;
                esw[tn] = *reinterpret_cast<const uint2 *>(&S.ew[64 * (r >> 5) + 2 * (r & 31)]);
            }
#pragma unroll
            for (int tm = 0; tm < MX_TM; ++tm) {
                const int r = wm * MX_WM + tm * 32 + l32;
                esx[tm] = *reinterpret_cast<const uint2 *>(&S.ex[64 * (r >> 5) + 2 * (r & 31)]);
            }
            // four 64-channel slices per step; the fragments of slice sl + 1
            // are read while the products of slice sl run
            struct Frag { i32x8 aw[MX_TN], bx[MX_TM]; };
            auto read_slice = [&](int sl, Frag &f) {
                const int blk = 2 * sl + hk;       // the lane's 32-channel block (segment) of the step
#pragma unroll
                for (int tn = 0; tn < MX_TN; ++tn) {
                    const int r = wn * MX_WN + tn * 32 + l32;
                    const uint4 v = *reinterpret_cast<const uint4 *>(&S.w[r * MXD_ROW + 16 * mxd_seg(r, blk)]);
                    f.aw[tn] = (i32x8){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                }
#pragma unroll
                for (int tm = 0; tm < MX_TM; ++tm) {
                    const int r = wm * MX_WM + tm * 32 + l32;
                    const uint4 v = *reinterpret_cast<const uint4 *>(&S.x[r * MXD_ROW + 16 * mxd_seg(r, blk)]);
                    f.bx[tm] = (i32x8){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                }
            };
            // E8M0 byte of block blk (= 2 sl + hk) from the row's two dwords
            auto e8 = [&](uint2 e, int sl) -> int {
                return (int)(((sl >> 1 ? e.y : e.x) >> (8 * (2 * (sl & 1) + hk))) & 0xFFu);
            };
            Frag fa, fb;
            read_slice(0, fa);
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) {
                Frag &cur = (sl & 1) ? fb : fa;
                Frag &nxt = (sl & 1) ? fa : fb;
                if (sl < 3) read_slice(sl + 1, nxt);
#pragma unroll
                for (int tn = 0; tn < MX_TN; ++tn)
#pragma unroll
                    for (int tm = 0; tm < MX_TM; ++tm)
                        acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            cur.aw[tn], cur.bx[tm], acc[tn][tm], 4, 4, 0, e8(esw[tn], sl), 0, e8(esx[tm], sl));
            }
            // issue order: the scale and first-slice reads, then per slice the
            // next slice's 6 reads ahead of its 8 products
            __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) {
                if (sl < 3) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            }
            // this wave's loads of step st + 1 have landed and its fragment
            // reads of stage sg are complete; the barrier publishes the one
            // and frees the other
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            asm volatile("s_barrier" ::: "memory");
        }
        // the last step used stage (g + nst - 1) & 1: the other one takes
        // the next item's first step while this item's epilogue runs
        const int last = (g + nst - 1) & 1;
        const int mb = m0 + wm * MX_WM, nb = n0 + wn * MX_WN;
        const int tile_n = n0 / MXD_BN, tile_m0 = m0;
        const int slice = t / tiles;
        // the QKV-norm and requantizing epilogues need the registers that the
        // next tile's prefetch would hold (the requantizing one spilled 35
        // VGPRs with it): those modes run one tile per block, and so do the
        // split-K partial sums, whose items never outnumber the CUs
        constexpr bool persistent = MODE == MXE_STORE;
        const int tnext = persistent ? t + (int)gridDim.x : items;
        const int nst_done = nst;
        if (persistent && tnext < items) {
            set_tile(tnext % tiles, n0, m0);
            item_steps(tnext, st0, nst);
            issue(st0, last ^ 1);
        }
        if constexpr (MODE == MXE_PARTIAL) {
            // lane (l32, hk) holds, per 32 x 32 tile, token mb + 32 tm + l32 and
            // channels nb + 32 tn + 8 j + 4 hk + (0..3).  Slice 0 also adds the
            // low-rank term, as the unsplit epilogue computes it.
            float *dst = sk.part + (size_t)slice * M * N;
            bf16x8 hhi[MX_TM][2], hlo[MX_TM][2];
            if (slice == 0) {
#pragma unroll
                for (int tm = 0; tm < MX_TM; ++tm)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        float hv[8];
                        load_h8(h, mb + tm * 32 + l32, M, 16 * s2 + 8 * hk, hv);
                        split_h(hv, hhi[tm][s2], hlo[tm][s2]);
                    }
            }
#pragma unroll
            for (int tn = 0; tn < MX_TN; ++tn) {
                if (slice == 0) {
                    const int nrow = nb + tn * 32 + l32;
                    bf16x8 ua[2];
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        uint4 uv = {0u, 0u, 0u, 0u};
                        if (nrow < N) uv = *reinterpret_cast<const uint4 *>(up + (size_t)nrow * 32 + 16 * s2 + 8 * hk);
                        ua[s2] = __builtin_bit_cast(bf16x8, uv);
                    }
#pragma unroll
                    for (int tm = 0; tm < MX_TM; ++tm)
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2) {
                            acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[s2], hhi[tm][s2], acc[tn][tm],
                                                                                  0, 0, 0);
                            acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[s2], hlo[tm][s2], acc[tn][tm],
                                                                                  0, 0, 0);
                        }
                }
#pragma unroll
                for (int tm = 0; tm < MX_TM; ++tm) {
                    const int m = mb + tm * 32 + l32;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int n = nb + tn * 32 + 8 * j + 4 * hk;
                        if (m < M && n < N)
                            *reinterpret_cast<float4 *>(dst + (size_t)m * N + n) =
                                make_float4(acc[tn][tm][4 * j], acc[tn][tm][4 * j + 1], acc[tn][tm][4 * j + 2],
                                            acc[tn][tm][4 * j + 3]);
                    }
                }
            }
        } else if constexpr (MODE == MXE_QKNORM) {
            // one tile per block: both stages are free for the output areas
            static_assert(8 * QK_AREA_BYTES <= 2 * sizeof(MXDStage), "the output areas fit in the two stages");
            qknorm_wave_epilogue_mx(acc, h, up, bias, M, N, qk, Y, mb, nb,
                                    reinterpret_cast<uint8_t *>(&stage[0]) + wave * QK_AREA_BYTES, lane);
        } else if constexpr (MODE == MXE_REQUANT) {
            static_assert(2 * MXD_BM * 32 * sizeof(float) <= sizeof(MXDStage), "partial sums fit in a stage");
            requant_epilogue_mx(acc, h, up, bias, M, N, gelu, rq, mb, nb, tile_n, tile_m0, wn, wm, tid, lane,
                                reinterpret_cast<float *>(&stage[last]));
        } else {
            wave_epilogue<MX_TN, MX_TM>(acc, h, up, bias, M, N, gelu, Y, mb, nb,
                                        reinterpret_cast<uint8_t *>(&stage[last]) + wave * OUT_TILE_BYTES, lane);
        }
        if (!persistent || tnext >= items) break;
        g += nst_done;
        t = tnext;
        // the staging area becomes the second stage of the next tile
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
    }
}

}  // namespace

hipError_t launch_w4a4_linear(const uint8_t *xq, const void *xscale, const float *h, const uint8_t *wq,
                              const void *wscale, const uint16_t *up, const uint16_t *bias, int M, int N,
                              int K, svdq_precision prec, svdq_epilogue epi, uint16_t *Y, hipStream_t stream)
{
    const int gelu = epi == SVDQ_EPI_GELU_TANH ? 1 : 0;
    const int64_t rows = M > N ? M : N;
    if (prec == SVDQ_INT4) {
        const int tiles = ((N + I4_BN - 1) / I4_BN) * ((M + I4_BM - 1) / I4_BM);
        // whole rounds of one block per CU, then, when the remaining tiles are
        // few enough that their pieces fill at most one round, those tiles in
        // pieces (w4a4_int4_tail_kernel)
        const int ncu = device_cu_count();
        int rest;
        const int main_tiles = int4_main_tiles(tiles, I4Tail<2, 2>::kPieces, ncu, rest);
        hipLaunchKernelGGL(w4a4_int4_kernel<EPI_STORE>, dim3((unsigned)main_tiles), dim3(I4_THREADS), 0, stream, xq,
                           (const float *)xscale, h, wq, (const float *)wscale, up, bias, M, N, K, gelu, Y,
                           RequantArgs{}, QKNormArgs{});
        if (rest > 0) {
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            return launch_int4_tail<EPI_STORE>(xq, (const float *)xscale, h, wq, (const float *)wscale, up, bias, M,
                                               N, K, gelu, Y, main_tiles, rest, ncu, QKNormArgs{}, stream);
        }
    } else {
        // the LDS-DMA kernel takes whole 256-channel steps and 32-bit offsets
        if (K % 256 == 0 && rows * (K / 2) < ((int64_t)1 << 31)) {
            const int tiles = ((N + MXD_BN - 1) / MXD_BN) * ((M + MXD_BM - 1) / MXD_BM);
            const int ncu = device_cu_count();
            const int blocks = tiles < ncu ? tiles : ncu;      // persistent: one block per CU
            hipLaunchKernelGGL(w4a4_mxfp4_dma_kernel<MXE_STORE>, dim3((unsigned)blocks), dim3(MXD_THREADS), 0, stream,
                               xq, (const uint8_t *)xscale, h, wq, (const uint8_t *)wscale, up, bias, M, N, K, gelu,
                               Y, RequantArgs{}, SplitArgs{nullptr, 1, K >> 8}, QKNormArgs{});
        } else {
            const int tiles = ((N + MX_BN - 1) / MX_BN) * ((M + MX_BM - 1) / MX_BM);
            hipLaunchKernelGGL(w4a4_mxfp4_kernel, dim3((unsigned)tiles), dim3(MX_THREADS), 0, stream, xq,
                               (const uint8_t *)xscale, h, wq, (const uint8_t *)wscale, up, bias, M, N, K, gelu, Y);
        }
    }
    return hipGetLastError();
}

size_t requant_work_bytes(int M, int N) { return (size_t)((N + I4_BN - 1) / I4_BN) * M * 32 * sizeof(float); }

bool requant_supported(int M, int N, int K, svdq_precision prec)
{
    if (prec == SVDQ_INT4) return true;
    const int64_t rows = M > N ? M : N;
    return K % 256 == 0 && rows * (K / 2) < ((int64_t)1 << 31);      // the LDS-DMA kernel's range
}

hipError_t launch_w4a4_linear_requant(const uint8_t *xq, const void *xscale, const float *h, const uint8_t *wq,
                                      const void *wscale, const uint16_t *up, const uint16_t *bias, int M, int N,
                                      int K, svdq_precision prec, svdq_epilogue epi, const float *smooth2,
                                      const uint16_t *down2, uint8_t *xq2, void *xscale2, float *h2, float *work,
                                      hipStream_t stream)
{
    const int gelu = epi == SVDQ_EPI_GELU_TANH ? 1 : 0;
    const int tiles_n = (N + I4_BN - 1) / I4_BN;       // 256-channel tiles in both kernels
    static_assert(I4_BN == MXD_BN, "one partial h row per 256 channels");
    const RequantArgs rq{smooth2, down2, xq2, xscale2, work};
    if (prec == SVDQ_INT4) {
        const int tiles = tiles_n * ((M + I4_BM - 1) / I4_BM);
        hipLaunchKernelGGL(w4a4_int4_kernel<EPI_REQUANT>, dim3((unsigned)tiles), dim3(I4_THREADS), 0, stream, xq,
                           (const float *)xscale, h, wq, (const float *)wscale, up, bias, M, N, K, gelu,
                           (uint16_t *)nullptr, rq, QKNormArgs{});
    } else {
        const int tiles = tiles_n * ((M + MXD_BM - 1) / MXD_BM);
        hipLaunchKernelGGL(w4a4_mxfp4_dma_kernel<MXE_REQUANT>, dim3((unsigned)tiles), dim3(MXD_THREADS), 0, stream,
                           xq, (const uint8_t *)xscale, h, wq, (const uint8_t *)wscale, up, bias, M, N, K, gelu,
                           (uint16_t *)nullptr, rq, SplitArgs{nullptr, 1, K >> 8}, QKNormArgs{});
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(requant_h_reduce, dim3((unsigned)((M * 8 + 255) / 256)), dim3(256), 0, stream,
                       (const float *)work, tiles_n, M, h2);
    return hipGetLastError();
}

// Split-K epilogue: y = the slices' fp32 sums added in slice order (slice 0
// carries the low-rank term) + b (+ GELU) -> bf16, 4 consecutive channels per
// thread.
__global__ __launch_bounds__(256) void splitk_finish_kernel(const float *__restrict__ part, int S,
                                                            const uint16_t *__restrict__ bias, int M, int N,
                                                            int gelu, uint16_t *__restrict__ Y)
{
    const int nq = N >> 2;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;      // (m, n / 4)
    if (i >= (int64_t)M * nq) return;
    const int m = (int)(i / nq), n = 4 * (int)(i % nq);
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < S; ++s) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(part + ((size_t)s * M + m) * N + n));
        a[0] += v.x; a[1] += v.y; a[2] += v.z; a[3] += v.w;
    }
    const uint2 b = bias4(bias, n, N);
    a[0] += bf16_to_f32(b.x & 0xFFFFu);
    a[1] += bf16_to_f32(b.x >> 16);
    a[2] += bf16_to_f32(b.y & 0xFFFFu);
    a[3] += bf16_to_f32(b.y >> 16);
    *reinterpret_cast<uint2 *>(Y + (size_t)m * N + n) = finish4(a, gelu);
}

int splitk_slices(int M, int N, int K, svdq_precision prec, int &sps)
{
    const int steps = K >> 8;
    sps = steps;
    // the LDS-DMA MXFP4 kernel only (the same range as its requantizing form)
    if (prec != SVDQ_MXFP4 || !requant_supported(M, N, K, prec) || M <= 0 || N <= 0) return 1;
    const int tiles = ((N + MXD_BN - 1) / MXD_BN) * ((M + MXD_BM - 1) / MXD_BM);
    const int ncu = device_cu_count();
    if (2 * tiles > ncu) return 1;                      // the tiles alone fill at least half the chip
    const int S = min(min(ncu / tiles, 4), steps / 4);  // at most 4 slices of at least 4 steps
    if (S < 2) return 1;
    sps = (steps + S - 1) / S;
    return (steps + sps - 1) / sps;                     // no empty slice
}

size_t splitk_work_bytes(int M, int N, int K, svdq_precision prec)
{
    int sps;
    const int S = splitk_slices(M, N, K, prec, sps);
    return S < 2 ? 0 : (size_t)S * M * N * sizeof(float);
}

hipError_t launch_w4a4_linear_splitk(const uint8_t *xq, const void *xscale, const float *h, const uint8_t *wq,
                                     const void *wscale, const uint16_t *up, const uint16_t *bias, int M, int N,
                                     int K, svdq_precision prec, svdq_epilogue epi, uint16_t *Y, float *work,
                                     hipStream_t stream)
{
    int sps;
    const int S = splitk_slices(M, N, K, prec, sps);
    if (S < 2) return launch_w4a4_linear(xq, xscale, h, wq, wscale, up, bias, M, N, K, prec, epi, Y, stream);
    const int gelu = epi == SVDQ_EPI_GELU_TANH ? 1 : 0;
    const int tiles = ((N + MXD_BN - 1) / MXD_BN) * ((M + MXD_BM - 1) / MXD_BM);
    const int items = tiles * S;                        // at most the CU count
    hipLaunchKernelGGL(w4a4_mxfp4_dma_kernel<MXE_PARTIAL>, dim3((unsigned)items), dim3(MXD_THREADS), 0, stream, xq,
                       (const uint8_t *)xscale, h, wq, (const uint8_t *)wscale, up, bias, M, N, K, gelu,
                       (uint16_t *)nullptr, RequantArgs{}, SplitArgs{work, S, sps}, QKNormArgs{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)M * (N / 4);
    hipLaunchKernelGGL(splitk_finish_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                       (const float *)work, S, bias, M, N, gelu, Y);
    return hipGetLastError();
}

hipError_t launch_w4a4_linear_qknorm(const uint8_t *xq, const void *xscale, const float *h, const uint8_t *wq,
                                     const void *wscale, const uint16_t *up, const uint16_t *bias, int M, int N,
                                     int K, svdq_precision prec, const uint16_t *norm_q, const uint16_t *norm_k,
                                     float eps, const float *rope_cos, const float *rope_sin, uint16_t *Y,
                                     hipStream_t stream)
{
    if (prec == SVDQ_MXFP4) {
        // the LDS-DMA kernel (K % 256 == 0, checked by qknorm_supported): a
        // 128-channel head is one wave's channel range
        static_assert(MX_WN == 128 && MXD_BN % 128 == 0, "a head is one wave tile");
        const QKNormArgs qk{norm_q, norm_k, rope_cos, rope_sin, N / 384, eps};
        const int tiles = ((N + MXD_BN - 1) / MXD_BN) * ((M + MXD_BM - 1) / MXD_BM);
        hipLaunchKernelGGL(w4a4_mxfp4_dma_kernel<MXE_QKNORM>, dim3((unsigned)tiles), dim3(MXD_THREADS), 0, stream, xq,
                           (const uint8_t *)xscale, h, wq, (const uint8_t *)wscale, up, bias, M, N, K, 0, Y,
                           RequantArgs{}, SplitArgs{nullptr, 1, K >> 8}, qk);
        return hipGetLastError();
    }
    const int tiles = ((N + I4_BN - 1) / I4_BN) * ((M + I4_BM - 1) / I4_BM);
    static_assert(I4_WN * 2 == 128 && I4_BN % 128 == 0, "a head is the tile of two neighbouring waves");
    const QKNormArgs qk{norm_q, norm_k, rope_cos, rope_sin, N / 384, eps};
    // whole rounds, then the leftover tiles in head pieces (as the plain linear)
    const int ncu = device_cu_count();
    int rest;
    const int main_tiles = int4_main_tiles(tiles, I4Tail<4, 1>::kPieces, ncu, rest);
    hipLaunchKernelGGL(w4a4_int4_kernel<EPI_QKNORM>, dim3((unsigned)main_tiles), dim3(I4_THREADS), 0, stream, xq,
                       (const float *)xscale, h, wq, (const float *)wscale, up, bias, M, N, K, 0, Y, RequantArgs{}, qk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || rest == 0) return e;
    return launch_int4_tail<EPI_QKNORM>(xq, (const float *)xscale, h, wq, (const float *)wscale, up, bias, M, N, K,
                                        0, Y, main_tiles, rest, ncu, qk, stream);
}

}  // namespace svdq
