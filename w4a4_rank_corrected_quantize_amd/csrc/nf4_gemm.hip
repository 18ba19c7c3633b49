// nf4_gemm.hip -- the weight-only NF4 W4A16 linear: y = X W'^T + b with bf16
// activations and 4-bit NF4 weights dequantized in the kernel
// ("BitsAndBytes W4 Quantization", sections "Overview" and "Parameters":
// weights quantized to the "nf4" data type, activations kept in bf16,
// block statistics double-quantized with compress_statistics).
//
// Dequantization of weight k of row n (block b = n K/64 + k/64):
//   ahat_b = fl32(qabs_b * chunk[b / 256]);   w' = bf16(fl32(level[code] * ahat_b))
// and y = sum_k X_mk w'_nk (fp32 accumulation on the bf16 matrix cores) + b_n,
// rounded to bf16.
//
// Decoding on gfx950.  Per 64-weight block a thread builds the block's 16
// dequantized bf16 values T[q] = bf16(level[q] * ahat) and splits them into a
// 16-byte table of low bytes and one of high bytes (4 dwords each).  A code
// dword holds 8 weights (weight i in the low nibble of byte i, weight i + 4 in
// the high nibble), so one v_perm_b32 looks up 4 bytes at once from the 8
// table bytes that the codes' low 3 bits select, a second v_perm picks, per
// byte, the half of the table that bit 3 selects, and two more interleave low
// and high bytes into bf16 pairs: about 3 VALU operations per weight.
//
// GEMM.  Block tile 256 tokens x 256 channels, 8 waves (2 per SIMD) of
// 64 tokens x 128 channels, v_mfma_f32_32x32x16_bf16 (A = weights, rows n;
// B = activations, columns m).  K advances 64 channels (one NF4 block) per
// step through two LDS stages of 64 KB (X: 256 x 128 bytes, W': 256 x 128
// bytes).  X goes from HBM to LDS by LDS-DMA (global_load_lds_dwordx4, no
// registers); the weight codes go to registers two steps ahead, and each
// thread decodes 32 weights of one row into the next stage while the current
// one is multiplied.  Every LDS row is 8 segments of 16 bytes, segment s of
// row r stored at s ^ (r & 7) ^ ((r >> 3) & 1), so the fragment reads of 32
// consecutive rows are conflict-free.
//
// Roofline: matrix-core bound (2 M N K flops on the 2.5 PFLOP/s bf16 peak);
// algorithmic bytes per launch 2MK (X) + NK/2 (codes) + NK/64 (statistic
// codes) + NK/4096 (chunk scales) + 2N (bias) + 2MN (Y).
#include "svdq_internal.h"
#include "svdq_quant.h"

namespace svdq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// two fp32 -> two bf16 (round to nearest even), packed low | high << 16
__device__ __forceinline__ uint32_t nf_pack_bf16x2(float lo, float hi)
{
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float nf_bf16_to_f32(uint32_t b) { return bits_f32(b << 16); }

// The block's decode table: L[j] holds the low bytes of T[4j .. 4j + 3], H[j]
// the high bytes.
struct Nf4Table {
    uint32_t L[4], H[4];
};

__device__ __forceinline__ Nf4Table nf4_table(const Nf4Levels &lv, float ahat)
{
    uint32_t T[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) T[i] = nf_pack_bf16x2(lv.c[2 * i] * ahat, lv.c[2 * i + 1] * ahat);
    Nf4Table t;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        t.L[j] = __builtin_amdgcn_perm(T[2 * j + 1], T[2 * j], 0x06040200u);
        t.H[j] = __builtin_amdgcn_perm(T[2 * j + 1], T[2 * j], 0x07050301u);
    }
    return t;
}

// 4 table bytes for the 4 codes whose low 3 bits are the bytes of `sel` and
// whose bit 3 (times 4, plus the byte index) is `pick`.
__device__ __forceinline__ uint32_t nf4_lookup(const uint32_t *tab, uint32_t sel, uint32_t pick)
{
    const uint32_t lo = __builtin_amdgcn_perm(tab[1], tab[0], sel);   // codes 0..7
    const uint32_t hi = __builtin_amdgcn_perm(tab[3], tab[2], sel);   // codes 8..15
    return __builtin_amdgcn_perm(hi, lo, pick);
}

// 8 weights (one code dword) -> 4 dwords of bf16 pairs in weight order.
__device__ __forceinline__ uint4 nf4_decode8(const Nf4Table &t, uint32_t w)
{
    const uint32_t se = w & 0x07070707u, so = (w >> 4) & 0x07070707u;
    const uint32_t pe = ((w >> 1) & 0x04040404u) | 0x03020100u;
    const uint32_t po = ((w >> 5) & 0x04040404u) | 0x03020100u;
    const uint32_t le = nf4_lookup(t.L, se, pe), he = nf4_lookup(t.H, se, pe);
    const uint32_t lo = nf4_lookup(t.L, so, po), ho = nf4_lookup(t.H, so, po);
    return make_uint4(__builtin_amdgcn_perm(he, le, 0x05010400u), __builtin_amdgcn_perm(he, le, 0x07030602u),
                      __builtin_amdgcn_perm(ho, lo, 0x05010400u), __builtin_amdgcn_perm(ho, lo, 0x07030602u));
}

__device__ __forceinline__ float nf4_ahat(uint32_t qabs, float chunk)
{
    return (float)qabs * chunk;      // exact conversion, one fp32 rounding
}

// ------------------------------------------------------------- dequantize

// Thread t decodes 8 consecutive weights (one code dword) of W'.
__global__ __launch_bounds__(256) void nf4_dequant_kernel(const uint32_t *__restrict__ wq,
                                                          const uint8_t *__restrict__ qabs,
                                                          const float *__restrict__ chunk, int64_t n8, Nf4Levels lv,
                                                          uint4 *__restrict__ Wd)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // weights 8 i .. 8 i + 7 (row-major)
    if (i >= n8) return;
    const int64_t b = i >> 3;                                    // 64-weight block (8 dwords each)
    const Nf4Table t = nf4_table(lv, nf4_ahat(qabs[b], chunk[b >> 8]));
    Wd[i] = nf4_decode8(t, wq[i]);
}

// ------------------------------------------------------------------- GEMM

constexpr int NF_BM = 256, NF_BN = 256;   // block tile (tokens, channels)
constexpr int NF_THREADS = 512;
constexpr int NF_ROW = 128;               // LDS bytes per row and stage: 64 bf16
constexpr int NF_WM = 64, NF_WN = 128;    // wave tile (tokens, channels)
constexpr int NF_TM = NF_WM / 32, NF_TN = NF_WN / 32;

__device__ __forceinline__ int nf_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// LDS: two stages of X (tokens) and two of W' (channels), 256 rows of 128
// bytes each.  The output staging of the epilogue reuses the X stages: 8 waves
// x 64 rows x 128 bytes, segment s of row r at s ^ (r & 7).
constexpr int NF_STAGE = NF_BM * NF_ROW;          // 32 KB
static_assert(NF_BM == NF_BN, "X and W' stages have the same size");
static_assert(8 * 64 * 128 <= 2 * NF_STAGE, "output staging fits in the X stages");

typedef __attribute__((address_space(3))) uint8_t nf_lds_u8;
__device__ __forceinline__ uint32_t nf_lds_offset(const void *p)
{
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const nf_lds_u8 *)p);
}

// One LDS-DMA load per lane: 16 bytes from sbase + voff to LDS lds + 16 lane.
// M0 is saved and restored around it.
__device__ __forceinline__ void nf_dma_b128(uint32_t lds, uint32_t voff, const void *sbase)
{
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(lds), "v"(voff), "s"(sbase) : "memory");
}

// Tile order: consecutive workgroups go to different XCDs (8 on MI355X), so
// each XCD first gets a contiguous range of tiles; within it the token tiles
// run fastest over groups of 4 channel tiles, which then stay in that XCD's L2.
__device__ __forceinline__ void nf_tile_coords(int b, int tiles_n, int tiles_m, int &tn, int &tm)
{
    const int T = tiles_n * tiles_m;
    const int t = (T % 8 == 0) ? (b & 7) * (T >> 3) + (b >> 3) : b;
    constexpr int GN = 4;
    const int per_group = GN * tiles_m;
    const int first_n = (t / per_group) * GN;
    const int gsize = min(tiles_n - first_n, GN);
    const int in = t % per_group;
    tn = first_n + in % gsize;
    tm = in / gsize;
}

__global__ __launch_bounds__(NF_THREADS) void nf4_linear_kernel(
    const uint16_t *__restrict__ X, const uint8_t *__restrict__ wq, const uint8_t *__restrict__ qabs,
    const float *__restrict__ chunk, const uint16_t *__restrict__ bias, int M, int N, int K, Nf4Levels lv,
    uint16_t *__restrict__ Y)
{
    __shared__ __attribute__((aligned(16))) uint8_t xs[2 * NF_STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t ws[2 * NF_STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1, wm = wave >> 1;              // 2 (channels) x 4 (tokens) waves
    const int l32 = lane & 31, hk = lane >> 5;
    int tn_, tm_;
    nf_tile_coords(blockIdx.x, (N + NF_BN - 1) / NF_BN, (M + NF_BM - 1) / NF_BM, tn_, tm_);
    const int n0 = tn_ * NF_BN, m0 = tm_ * NF_BM;
    const int G = K >> 6;                                 // blocks per row = steps
    const int steps = G;

    // X: per stage 32 loads of 1 KB (8 rows of 128 bytes); wave w issues
    // blocks 8 i + w.  Lane l fills slot l & 7 of row l >> 3, i.e. global
    // segment (l & 7) ^ swz(row).  Rows past M read the last row.
    uint32_t xvo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * (8 * i + wave) + (lane >> 3);
        xvo[i] = (uint32_t)(min(m0 + r, M - 1) * (2 * K) + 16 * ((lane & 7) ^ nf_swz(r)));
    }
    auto issue_x = [&](int st, int sg) {
        const uint16_t *xb = X + 64 * st;
#pragma unroll
        for (int i = 0; i < 4; ++i) nf_dma_b128(nf_lds_offset(&xs[sg * NF_STAGE + 1024 * (8 * i + wave)]), xvo[i], xb);
    };

    // W: thread t decodes weights 32 h .. 32 h + 31 (h = t & 1) of the step's
    // block of tile row r = t >> 1.  Rows past N read the last row.
    const int wr = tid >> 1, wh = tid & 1;
    const int wn_row = min(n0 + wr, N - 1);
    const uint8_t *__restrict__ wsrc = wq + (size_t)wn_row * (K / 2) + 16 * wh;
    const int64_t bbase = (int64_t)wn_row * G;
    struct Codes {
        uint4 c;
        uint32_t q;
        float s;
    };
    auto load_codes = [&](int st, Codes &R) {
        const int s = min(st, steps - 1);          // unconditional: same load count on every path
        R.c = *reinterpret_cast<const uint4 *>(wsrc + 32 * s);
        R.q = qabs[bbase + s];
        R.s = chunk[(bbase + s) >> 8];
    };
    uint8_t *const wrow = ws + wr * NF_ROW;
    const int wsw = nf_swz(wr);
    auto decode_to = [&](const Codes &R, int sg) {
        const Nf4Table t = nf4_table(lv, nf4_ahat(R.q, R.s));
        const uint32_t cw[4] = {R.c.x, R.c.y, R.c.z, R.c.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<uint4 *>(wrow + sg * NF_STAGE + 16 * ((4 * wh + j) ^ wsw)) = nf4_decode8(t, cw[j]);
    };

    f32x16 acc[NF_TN][NF_TM];
#pragma unroll
    for (int a = 0; a < NF_TN; ++a)
#pragma unroll
        for (int b = 0; b < NF_TM; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    // one step: four 16-channel slices of 8 products; the fragments of slice
    // ks + 1 are read while the products of slice ks run
    struct Frag {
        bf16x8 a[NF_TN], b[NF_TM];
    };
    // Fragment rows: weights wn 128 + 32 tn + l32, tokens wm 64 + 32 tm + l32.
    // Both are l32 plus a multiple of 16, so their swizzle is that of l32 and
    // a fragment's address is a per-lane base plus a constant.
    const int fsw = nf_swz(l32);
    const uint8_t *const fa_base = ws + (wn * NF_WN + l32) * NF_ROW;
    const uint8_t *const fb_base = xs + (wm * NF_WM + l32) * NF_ROW;
    auto read_slice = [&](int sg, int ks, Frag &f) {
        const int so = 16 * ((2 * ks + hk) ^ fsw) + sg * NF_STAGE;
#pragma unroll
        for (int tn = 0; tn < NF_TN; ++tn)
            f.a[tn] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(fa_base + so + tn * 32 * NF_ROW));
#pragma unroll
        for (int tm = 0; tm < NF_TM; ++tm)
            f.b[tm] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(fb_base + so + tm * 32 * NF_ROW));
    };
    auto compute = [&](int sg) {
        Frag fa, fb;
        read_slice(sg, 0, fa);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            Frag &cur = (ks & 1) ? fb : fa;
            Frag &nxt = (ks & 1) ? fa : fb;
            if (ks < 3) read_slice(sg, ks + 1, nxt);
#pragma unroll
            for (int tn = 0; tn < NF_TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < NF_TM; ++tm)
                    acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[tn], cur.b[tm], acc[tn][tm], 0, 0, 0);
        }
        // issue order: the first slice's 6 reads, then per slice the next
        // slice's 6 reads ahead of its 8 products
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks < 3) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
    };

    // prologue: stage 0 holds step 0, R the codes of step 1
    Codes R;
    issue_x(0, 0);
    load_codes(0, R);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    decode_to(R, 0);
    load_codes(1, R);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // step st: the other stage takes the decoded weights of step st + 1 (R,
    // loaded during step st - 1) and X of step st + 1, R takes the codes of
    // step st + 2, then the products of step st run from stage st & 1.
    // vmcnt completes in order and the compiler does not see the DMA, so
    // its waits for R must come before the DMA is issued: the decode goes
    // first, and nothing is conditional (the last step reloads its own data
    // into the free stage, which nothing reads) -- with a skipped branch the
    // compiler waited for every load where the paths merge, the DMA just
    // issued included, ahead of the products.
    for (int st = 0; st < steps; ++st) {
        const int sg = st & 1;
        decode_to(R, sg ^ 1);
        issue_x(min(st + 1, steps - 1), sg ^ 1);
        load_codes(st + 2, R);          // clamped: same load count on every path
        // the code loads stay ahead of the products (left to the scheduler,
        // they sank to the end of the step, where the wait below took their
        // whole latency)
        __builtin_amdgcn_sched_barrier(0);
        compute(sg);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // epilogue: y = acc + bias -> bf16, staged per wave as two 64 x 64 blocks
    // (row = token, 128 + 8 bytes) so that every store is a full 128-byte row
    // segment.  Lane (l32, hk) of tile (tn, tm) holds token mb + 32 tm + l32
    // and channels nb + 32 tn + 8 j + 4 hk + (0..3), j < 4.
    const int mb = m0 + wm * NF_WM, nb = n0 + wn * NF_WN;
    uint8_t *tile = xs + wave * 64 * 128;
#pragma unroll
    for (int half = 0; half < NF_TN / 2; ++half) {
#pragma unroll
        for (int th = 0; th < 2; ++th) {
            const int tn = 2 * half + th;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = nb + tn * 32 + 8 * j + 4 * hk;
                uint2 bv = make_uint2(0u, 0u);
                if (bias && n < N) bv = *reinterpret_cast<const uint2 *>(bias + n);
#pragma unroll
                for (int tm = 0; tm < NF_TM; ++tm) {
                    const float y0 = acc[tn][tm][4 * j] + nf_bf16_to_f32(bv.x & 0xFFFFu);
                    const float y1 = acc[tn][tm][4 * j + 1] + nf_bf16_to_f32(bv.x >> 16);
                    const float y2 = acc[tn][tm][4 * j + 2] + nf_bf16_to_f32(bv.y & 0xFFFFu);
                    const float y3 = acc[tn][tm][4 * j + 3] + nf_bf16_to_f32(bv.y >> 16);
                    const int r = tm * 32 + l32;        // segment 4 th + j, half hk
                    *reinterpret_cast<uint2 *>(tile + r * 128 + 16 * ((4 * th + j) ^ (r & 7)) + 8 * hk) =
                        make_uint2(nf_pack_bf16x2(y0, y1), nf_pack_bf16x2(y2, y3));
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int seg = lane & 7;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int r = (lane >> 3) + 8 * it;
            const uint4 v = *reinterpret_cast<const uint4 *>(tile + r * 128 + 16 * (seg ^ (r & 7)));
            const int m = mb + r, n = nb + 64 * half + seg * 8;
            if (m < M && n < N) {
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store((u32x4){v.x, v.y, v.z, v.w},
                                            reinterpret_cast<u32x4 *>(Y + (size_t)m * N + n));
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

}  // namespace

hipError_t launch_nf4_dequant(const uint8_t *wq, const uint8_t *qabs, const float *chunk, int N, int K,
                              const Nf4Levels &lv, uint16_t *Wd, hipStream_t stream)
{
    const int64_t n8 = (int64_t)N * K / 8;
    hipLaunchKernelGGL(nf4_dequant_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t *>(wq), qabs, chunk, n8, lv, reinterpret_cast<uint4 *>(Wd));
    return hipGetLastError();
}

hipError_t launch_nf4_linear(const uint16_t *X, const uint8_t *wq, const uint8_t *qabs, const float *chunk,
                             const uint16_t *bias, int M, int N, int K, const Nf4Levels &lv, uint16_t *Y,
                             hipStream_t stream)
{
    const int tiles = ((N + NF_BN - 1) / NF_BN) * ((M + NF_BM - 1) / NF_BM);
    hipLaunchKernelGGL(nf4_linear_kernel, dim3((unsigned)tiles), dim3(NF_THREADS), 0, stream, X, wq, qabs, chunk,
                       bias, M, N, K, lv, Y);
    return hipGetLastError();
}

}  // namespace svdq
