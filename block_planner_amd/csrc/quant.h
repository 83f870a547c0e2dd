// quant.h -- per-block quantisation on gfx950, shared by the planner and the
// packer kernels.  Layout of the work: one 64-entry K-block is held by 4
// consecutive lanes, lane part p owning entries [16p, 16p+16) in registers.
//
// Block rule (HyperTensor 1.0.1 page, "What it does": the format of a block
// follows from the error each format leaves; the numeric rule is the
// method's specification):
//   s = fl32(max|w| / Q), Q = 7 (INT4) or 127 (INT8), correctly rounded;
//   q = clamp(round_half_even(fl32(w / s)), -Q, Q); q = 0 if s is 0 or not
//   finite.
#pragma once
#include <float.h>

#include "ht_internal.h"

#pragma clang fp contract(off)

namespace ht {

constexpr int kLanesPerBlock = 4;
constexpr int kPerLane = 16;

// max |w| over the block, for finite entries (IEEE maxNum ignores NaN, and a
// block holding NaN or Inf is recognised separately).
__device__ __forceinline__ float block_absmax(const float (&w)[kPerLane]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kPerLane; i += 2) m = fmaxf(m, fmaxf(fabsf(w[i]), fabsf(w[i + 1])));
    m = fmaxf(m, dpp_f32<kDppXor1>(m));
    m = fmaxf(m, dpp_f32<kDppXor2>(m));
    return m;
}

// Codes of one lane's 16 entries for scale s.
//
// Fast path (s a finite normal number): t = w * rcp(s) with the hardware
// reciprocal (1 ulp).  |t - w/s| <= 1.5 * 2^-23 * |w/s| (+ tiny), with
// |w/s| < Q + 0.5: at most 2.3e-5 for Q = 127 and 1.4e-6 for Q = 7; and
// |fl32(w/s) - w/s| <= half an ulp: 2^-18 (3.8e-6) below 128, 2^-21 below 8.
// So when t lies more than band = 4e-5 (Q = 127) or 3e-6 (Q = 7) from a
// half-integer, fl32(w/s) lies strictly on the same side and rint(t) ==
// rint(fl32(w/s)).  Otherwise the entry takes the exact path: a correctly
// rounded fp32 division.  No clamp is needed on the fast path:
// s = fl32(amax/Q) >= (amax/Q)(1 - 2^-24) gives |w/s| < Q + 0.5.
//
// Subnormal s: fp32 division (correctly rounded) and the clamp, which then
// matters (amax = 10 * 2^-149 gives s = 2^-149 and w/s = 10 > 7).
//
// The exact path runs only in waves where some lane needs it (a wave vote),
// so the common case costs one multiply and one rounding per entry.
__device__ __forceinline__ void lane_codes(const float (&w)[kPerLane], float s, float Qf,
                                           float (&q)[kPerLane]) {
    const bool normal = s >= FLT_MIN && s <= FLT_MAX;
    const bool subnormal = s > 0.0f && s < FLT_MIN;
    const float rc = __builtin_amdgcn_rcpf(s);
    const float edge = Qf < 8.0f ? 0.5f - 3e-6f : 0.5f - 4e-5f;   // 0.5 - band
    // fast path: the largest distance to the rounded value decides, per
    // lane, whether any entry lies within the band (maxNum ignores NaN
    // entries, whose codes do not matter: such a block is never stored as an
    // integer format)
    float dev = 0.0f;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const float t = w[i] * rc;
        const float r = rintf(t);
        dev = fmaxf(dev, fabsf(t - r));
        q[i] = r;
    }
    const bool rare = !normal || subnormal || dev > edge;
    if (__builtin_expect(__any(rare), 0)) {
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const float t = w[i] * rc;
            const bool exact = subnormal || (normal && fabsf(t - rintf(t)) > edge);
            if (exact) q[i] = fminf(fmaxf(rintf(w[i] / s), -Qf), Qf);
            if (!normal && !subnormal) q[i] = 0.0f;   // s = 0 or not finite: all codes 0
        }
    }
}

// Balanced pairwise sum of the squares of 16 values in natural order:
// ((d0^2 + d1^2) + (d2^2 + d3^2)) + ...  Each square of an fp32 value is exact
// in fp64 (<= 48 significant bits, no overflow or underflow), so
// fma(b, b, a*a) rounds exactly like fl(a^2 + b^2).
__device__ __forceinline__ double tree16_sq(const float (&d)[kPerLane]) {
    double p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        double a = double(d[2 * j]), b = double(d[2 * j + 1]);
        p[j] = __builtin_fma(b, b, a * a);
    }
    double q0 = p[0] + p[1], q1 = p[2] + p[3], q2 = p[4] + p[5], q3 = p[6] + p[7];
    return (q0 + q1) + (q2 + q3);
}

// Complete the 64-entry tree across the block's 4 lanes:
// S[0,64) = (S[0,16) + S[16,32)) + (S[32,48) + S[48,64)).
__device__ __forceinline__ double block_tree(double v) {
    v = v + dpp_f64<kDppXor1>(v);
    v = v + dpp_f64<kDppXor2>(v);
    return v;
}

__device__ __forceinline__ uint32_t block_or(uint32_t v) {
    v |= dpp_u32<kDppXor1>(v);
    v |= dpp_u32<kDppXor2>(v);
    return v;
}

// Non-finite detection over the block's bits: bit 0 = some NaN, bit 1 = some Inf.
__device__ __forceinline__ uint32_t block_nonfinite(const float (&w)[kPerLane]) {
    uint32_t fl = 0;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        uint32_t a = __float_as_uint(w[i]) & 0x7FFFFFFFu;
        fl |= (a > 0x7F800000u ? 1u : 0u) | (a == 0x7F800000u ? 2u : 0u);
    }
    return block_or(fl);
}

// fp32 -> nearest-even binary16 -> fp32 (hardware conversion, subnormals kept,
// overflow to infinity).
__device__ __forceinline__ float round_fp16(float w) { return float(_Float16(w)); }

// fp32 -> nearest-even bfloat16 -> fp32, for finite w.
__device__ __forceinline__ float round_bf16(float w) {
    uint32_t u = __float_as_uint(w);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return __uint_as_float(u & 0xFFFF0000u);
}

}  // namespace ht
