// svdq_quant.h -- the 4-bit group quantizers of libsvdq, shared by the host
// packing step and the gfx950 activation kernel (same source, so weights and
// activations are coded by one rule).
//
// INT4 (symmetric, 64 wide): a = max|v|; scale = fl32(a / 7), rounded upward
// instead of to nearest when a / 7 is below the smallest normal fp32; the code
// is the round-half-even of the exact quotient v / scale.  A reciprocal
// multiply is off by one on near-ties, so the first guess q0 = rint(v * 1/scale)
// is repaired with the exact remainder e = v - q0 * scale (one fma): the
// remainder is exactly representable (|e| <= scale/2 + ulp-level slack, and
// it is a multiple of the smaller of ulp(v) and ulp(scale)), so comparing |e|
// with scale/2 (exact) decides the correct code.  Groups with scale < 2^-100
// are first lifted by 2^64 (exact) so that 1/scale and scale/2 stay normal.
//
// MXFP4 (OCP Microscaling v1.0, 32 wide): X = floor(log2 a) - 2 read from the
// exponent bits of a, clamped to [-127, 127]; t = v * 2^-X (exact); index on
// the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6} by comparisons with the midpoints
// (strict at midpoints whose lower neighbour has the even index, inclusive
// otherwise), saturating at 6; code = sign << 3 | index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SVDQ_HD __host__ __device__ __forceinline__

namespace svdq {

SVDQ_HD uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }
SVDQ_HD float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// ------------------------------------------------------------------ INT4

// fl32(absmax / 7): the reciprocal product corrected once by its exact fma
// remainder is the correctly rounded quotient for every finite absmax >= 0
// (checked exhaustively, subnormal quotients included); below the normal
// range the result is then moved up one ulp when it lies under absmax / 7.
SVDQ_HD float int4_group_scale(float absmax)
{
    const float c = 0.142857149f;                  // fl32(1 / 7)
    float sc = absmax * c;
    sc = __builtin_fmaf(__builtin_fmaf(-sc, 7.0f, absmax), c, sc);
    if (sc < 1.17549435e-38f && __builtin_fmaf(sc, 7.0f, -absmax) < 0.0f)
        sc = bits_f32(f32_bits(sc) + 1u);          // next fp32 upward (sc >= 0)
    return sc;
}

// Working copies of the group constants: `lift` is 2^64 for tiny scales.
struct Int4Group {
    float scale;   // possibly lifted
    float inv;     // fl32(1 / scale)
    float half;    // scale / 2, exact
    float lift;    // 1 or 2^64
};

SVDQ_HD Int4Group int4_group_prepare(float scale)
{
    Int4Group g;
    g.lift = (scale < 7.88860905e-31f) ? 1.8446744073709552e19f : 1.0f;   // 2^-100, 2^64
    g.scale = scale * g.lift;
    g.inv = (scale == 0.0f) ? 0.0f : 1.0f / g.scale;
    g.half = 0.5f * g.scale;
    return g;
}

// Exact magnitude code |q| in [0, 7] for av = |v| (unlifted value).
SVDQ_HD uint32_t int4_mag(float av, const Int4Group &g)
{
    const float x = av * g.lift;
    const float q0 = __builtin_rintf(x * g.inv);
    const float e = __builtin_fmaf(-q0, g.scale, x);      // exact remainder
    const float d = __builtin_fabsf(e) - g.half;          // sign and zero are exact
    const int qi = (int)q0;
    const bool move = d > 0.0f || (d == 0.0f && (qi & 1));
    int q = qi + (move ? (e < 0.0f ? -1 : 1) : 0);
    q = q < 0 ? 0 : (q > 7 ? 7 : q);
    return (uint32_t)q;
}

// Sign-magnitude 4-bit code: bit 3 = sign of v (kept for zero), bits 0-2 = |q|.
SVDQ_HD uint32_t int4_nibble(float v, const Int4Group &g)
{
    return ((f32_bits(v) >> 28) & 8u) | int4_mag(__builtin_fabsf(v), g);
}

// Fast path used by the activation kernel: |q| = rint(|v| * inv) is exact
// unless |v|/scale lies within 2^-20 of a half-integer (the product carries a
// relative error below 2^-23 on a quotient below 7.5); such elements are
// flagged (`near`) and redone with int4_mag.  Groups that need the 2^64 lift
// are always redone.
constexpr float kNearTie = 0.49999809265136719f;          // 0.5 - 2^-19

// ----------------------------------------------------------------- MXFP4

// floor(log2 a) - 2 from the exponent field, clamped; returns the E8M0 byte.
SVDQ_HD uint32_t mx_block_e8m0(float absmax)
{
    int e = (int)((f32_bits(absmax) >> 23) & 0xFF);   // 0 for zero / subnormal
    int X = (e == 0) ? -127 : e - 127 - 2;
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
    return (uint32_t)(X + 127);
}

// 2^-X as fp32 for X = e8m0 - 127 in [-127, 125].
SVDQ_HD float mx_inv_scale(uint32_t e8m0)
{
    int X = (int)e8m0 - 127;
    return bits_f32((uint32_t)(127 - X) << 23);        // exponent field 2..254
}

SVDQ_HD uint32_t e2m1_code(float v, float inv_scale)
{
    float t = __builtin_fabsf(v * inv_scale);           // exact power-of-two scaling
    uint32_t idx = (uint32_t)(t > 0.25f) + (uint32_t)(t >= 0.75f) + (uint32_t)(t > 1.25f) +
                   (uint32_t)(t >= 1.75f) + (uint32_t)(t > 2.5f) + (uint32_t)(t >= 3.5f) +
                   (uint32_t)(t > 5.0f);
    return ((f32_bits(v) >> 28) & 8u) | idx;
}

}  // namespace svdq
