// Exhaustive check of the library's INT4 group scale (svdq_quant.h,
// int4_group_scale) against exact arithmetic, for every finite fp32
// absmax >= 0: scale = fl32(absmax / 7), rounded upward instead of to nearest
// when the quotient is below the smallest normal fp32.  The reference divides
// in fp64 (53 >= 2 * 24 + 2 bits, so rounding twice equals rounding once) and
// decides "upward" from the exact product scale * 7 in fp64.
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "svdq_quant.h"

static float from_bits(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

static float reference(float a)
{
    float r = (float)((double)a / 7.0);
    if (r < FLT_MIN && (double)r * 7.0 < (double)a) r = std::nextafter(r, INFINITY);
    return r;
}

int main()
{
    const int T = (int)std::max(1u, std::thread::hardware_concurrency());
    std::vector<uint64_t> bad(T, 0), first(T, ~0ull);
    std::vector<std::thread> th;
    for (int t = 0; t < T; ++t)
        th.emplace_back([&, t] {
            for (uint64_t u = (uint64_t)t; u < 0x7F800000ull; u += (uint64_t)T) {
                const float a = from_bits((uint32_t)u);
                const float got = svdq::int4_group_scale(a), want = reference(a);
                if (std::memcmp(&got, &want, 4) != 0) {
                    if (!bad[t]) first[t] = u;
                    ++bad[t];
                }
            }
        });
    for (auto &x : th) x.join();
    uint64_t nb = 0, f = ~0ull;
    for (int t = 0; t < T; ++t) { nb += bad[t]; if (first[t] < f) f = first[t]; }
    std::printf("checked %u values, mismatches %llu\n", 0x7F800000u, (unsigned long long)nb);
    if (nb) std::printf("first mismatch at bits %08llx\n", (unsigned long long)f);
    return nb ? 1 : 0;
}
