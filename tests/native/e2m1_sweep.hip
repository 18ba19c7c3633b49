// Exhaustive check of the gfx950 E2M1 conversion that the MXFP4 activation
// step and the fused requantizing epilogue rely on
// (v_cvt_scalef32_pk_fp4_f32 at unit scale, applied to values already scaled
// exactly by 2^-X).  For every fp32 t with |t| < 16, both signs, the
// hardware code must equal the OCP Microscaling v1.0 rule: the nearest of
// the E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even index,
// magnitudes above 6 saturating to 6, and the sign bit of t kept (also for
// zero).  The reference below takes the nearest grid value by distance in
// fp64 (exact wherever a tie is possible: near a midpoint t and the grid
// values share their exponent range).
//
// Prints "checked <n> values, mismatches <k>" and exits 0 when k == 0.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

__device__ __forceinline__ uint32_t ref_code(float t)
{
    const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    const double a = __builtin_fabs((double)t);
    uint32_t best = 0;
    double bd = a;
    for (uint32_t i = 1; i < 8; ++i) {
        const double d = __builtin_fabs(a - grid[i]);
        if (d < bd || (d == bd && (i & 1u) == 0u)) {
            bd = d;
            best = i;
        }
    }
    return ((__builtin_bit_cast(uint32_t, t) >> 28) & 8u) | best;
}

// Each thread converts the pair (t, -t) for its magnitudes u, u + stride, ...
__global__ void sweep(uint32_t n, unsigned long long *bad, unsigned int *first)
{
    const uint32_t stride = gridDim.x * blockDim.x;
    unsigned long long nb = 0;
    for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < n; u += stride) {
        const float t = __builtin_bit_cast(float, u);
        const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, t, -t, 1.0f, 0) & 0xFFu;
        const uint32_t want = ref_code(t) | (ref_code(-t) << 4);
        if (hw != want) {
            ++nb;
            atomicMin(first, u);
        }
    }
    if (nb) atomicAdd(bad, nb);
}

int main()
{
    const uint32_t n = 0x41800000u;     // every non-negative fp32 below 16 (bits of 16.0f)
    unsigned long long *bad = nullptr;
    unsigned int *first = nullptr;
    if (hipMalloc(&bad, sizeof(*bad)) != hipSuccess || hipMalloc(&first, sizeof(*first)) != hipSuccess) {
        std::printf("hipMalloc failed\n");
        return 2;
    }
    const unsigned long long zero = 0;
    const unsigned int none = 0xFFFFFFFFu;
    hipMemcpy(bad, &zero, sizeof(zero), hipMemcpyHostToDevice);
    hipMemcpy(first, &none, sizeof(none), hipMemcpyHostToDevice);
    hipLaunchKernelGGL(sweep, dim3(4096), dim3(256), 0, 0, n, bad, first);
    if (hipDeviceSynchronize() != hipSuccess) {
        std::printf("kernel failed\n");
        return 2;
    }
    unsigned long long nb = 0;
    unsigned int f = 0;
    hipMemcpy(&nb, bad, sizeof(nb), hipMemcpyDeviceToHost);
    hipMemcpy(&f, first, sizeof(f), hipMemcpyDeviceToHost);
    hipFree(bad);
    hipFree(first);
    std::printf("checked %llu values, mismatches %llu\n", 2ull * n, nb);
    if (nb) std::printf("first mismatch at |t| bits %08x\n", f);
    return nb ? 1 : 0;
}
