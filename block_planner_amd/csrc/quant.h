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

// The per-block format rule (thresholds squared in fp64, preference,
// forced format), shared by the planner and the fused refresh.
struct PlanRule {
    double e2[4];        // eps^2 for INT4, INT8, BF16, FP16 (fl64(eps * eps))
    int prefer_bf16;
    int force;           // -1 or a format code
};

// Format of the block held by this quad of lanes (16 entries per lane), by
// the rule: the first admissible of INT4, INT8, the 16-bit formats in the
// preferred order, FP32.  Every lane of the wave must call it (wave votes).
//
// Screening in fp32: the sums of squares err4, err8, nrm2 to within 2^-17
// relative plus 2^-120 absolute (66 roundings of non-negative partial sums,
// underflow included).  A decision that holds for every value in those
// intervals equals the decision on the fp64 pairwise trees; only the other
// blocks (near-ties, eps = 0, zero blocks, non-finite or huge entries)
// compute the fp64 trees, in waves that vote for them.
template <bool EPS16_ZERO>
__device__ __forceinline__ int block_format(const float (&w)[kPerLane], const PlanRule &rule) {
    // amax and the two scales
    const float amax = block_absmax(w);
    const float s4 = amax / 7.0f;     // correctly rounded fp32 division
    const float s8 = amax / 127.0f;

    // codes and exact residuals d = w - q*s (exactly representable in fp32,
    // so the fused multiply-add returns it exactly)
    float q[kPerLane], d4[kPerLane], d8[kPerLane];
    lane_codes(w, s4, 7.0f, q);
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) d4[i] = __builtin_fmaf(-q[i], s4, w[i]);
    lane_codes(w, s8, 127.0f, q);
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) d8[i] = __builtin_fmaf(-q[i], s8, w[i]);

    float e4f = 0.0f, e8f = 0.0f, nf = 0.0f;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        e4f = __builtin_fmaf(d4[i], d4[i], e4f);
        e8f = __builtin_fmaf(d8[i], d8[i], e8f);
        nf = __builtin_fmaf(w[i], w[i], nf);
    }
    e4f = e4f + dpp_f32<kDppXor1>(e4f);
    e8f = e8f + dpp_f32<kDppXor1>(e8f);
    nf = nf + dpp_f32<kDppXor1>(nf);
    e4f = e4f + dpp_f32<kDppXor2>(e4f);
    e8f = e8f + dpp_f32<kDppXor2>(e8f);
    nf = nf + dpp_f32<kDppXor2>(nf);
    auto screen = [](double e2, float ef, float nfv) -> int {   // 0 no, 1 yes, 2 undecided
        if (!(e2 > 0.0)) return 2;
        const double E = ef, Nn = nfv, rel = 0x1p-17, ab = 0x1p-120;
        if (E * (1.0 - rel) - ab > e2 * (Nn * (1.0 + rel) + ab)) return 0;
        if (E * (1.0 + rel) + ab <= e2 * (Nn * (1.0 - rel) - ab)) return 1;
        return 2;
    };
    const bool in_range = nf <= 0x1p126f;   // finite, and no square near overflow
    const int dec4 = screen(rule.e2[0], e4f, nf), dec8 = screen(rule.e2[1], e8f, nf);
    const bool need = !in_range || dec4 == 2 || dec8 == 2;
    bool ok4 = dec4 == 1, ok8 = dec8 == 1, finite = true;
    if (__any(need)) {
        const double err4 = block_tree(tree16_sq(d4));
        const double err8 = block_tree(tree16_sq(d8));
        const double nrm2 = block_tree(tree16_sq(w));
        if (need) {
            ok4 = err4 <= rule.e2[0] * nrm2;
            ok8 = err8 <= rule.e2[1] * nrm2;
            finite = nrm2 <= DBL_MAX;   // false for Inf and NaN entries
        }
    }
    float (&d)[kPerLane] = d4;   // scratch for the 16-bit tests below

    // 16-bit formats
    bool okb, okh;
    if constexpr (EPS16_ZERO) {
        uint32_t orb = 0;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) orb |= __float_as_uint(w[i]);
        orb = block_or(orb);
        okb = (orb & 0xFFFFu) == 0u;
        // representable in binary16 => low 13 fraction bits are zero; only
        // then test each entry exactly (rare: the whole quad agrees on orb)
        uint32_t bad = 1u;
        if ((orb & 0x1FFFu) == 0u) {
            bad = 0u;
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) bad |= (round_fp16(w[i]) != w[i]) ? 1u : 0u;
            bad = block_or(bad);
        }
        okh = bad == 0u;
    } else {
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) d[i] = w[i] - round_bf16(w[i]);
        const double errb = block_tree(tree16_sq(d));
        // w - fp16(w) may not fit fp32 exactly only when fp16(w) overflows;
        // that difference is infinite either way
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) d[i] = w[i] - round_fp16(w[i]);
        const double errh = block_tree(tree16_sq(d));
        const double nrm2 = block_tree(tree16_sq(w));
        okb = errb <= rule.e2[2] * nrm2;
        okh = errh <= rule.e2[3] * nrm2;
    }

    const int f16a = rule.prefer_bf16 ? (okb ? 2 : (okh ? 3 : 4)) : (okh ? 3 : (okb ? 2 : 4));
    int f = ok4 ? 0 : (ok8 ? 1 : f16a);
    f = finite ? f : 4;
    return rule.force >= 0 ? rule.force : f;
}

// Where a packed buffer's regions start (byte offsets from its base).
struct RegionOffsets {
    uint64_t ids[5], scale[2], pay[5];
};

// Encode the block held by this quad of lanes as format f at position pos
// of its format's region: id (lane part 0), scale (integer formats, part 0)
// and payload (every part writes its 16 entries).  Codes and scales are
// computed exactly as the planner computes them; a forced integer format on
// a block holding NaN / Inf gets the canonical NaN / Inf scale and zero codes.
__device__ __forceinline__ void store_block(uint8_t *buf, const RegionOffsets &o, uint32_t f, uint32_t pos,
                                            uint16_t id, const float (&w)[kPerLane], int part) {
    // this format's offsets by selects (a runtime index would put the
    // offsets in scratch memory)
    uint64_t oid = o.ids[0], opay = o.pay[0], osc = o.scale[0];
#pragma unroll
    for (uint32_t k = 1; k < 5; ++k) {
        oid = f == k ? o.ids[k] : oid;
        opay = f == k ? o.pay[k] : opay;
    }
    osc = f == 1u ? o.scale[1] : osc;
    if (part == 0) *reinterpret_cast<uint16_t *>(buf + oid + 2ull * pos) = id;
    uint8_t *pay = buf + opay;
    if (f <= 1u) {
        const float Qf = f == 0u ? 7.0f : 127.0f;
        const float amax = block_absmax(w);
        float s = amax / Qf;
        float q[kPerLane];
        const uint32_t nf = block_nonfinite(w);
        if (nf) {
            s = (nf & 1u) ? __uint_as_float(0x7FC00000u) : __uint_as_float(0x7F800000u);
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) q[i] = 0.0f;
        } else {
            lane_codes(w, s, Qf, q);
        }
        if (part == 0) *reinterpret_cast<float *>(buf + osc + 4ull * pos) = s;
        uint32_t wd[4];
        if (f == 1u) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wd[j] = (uint32_t(int(q[4 * j]) & 0xFF)) | (uint32_t(int(q[4 * j + 1]) & 0xFF) << 8) |
                        (uint32_t(int(q[4 * j + 2]) & 0xFF) << 16) | (uint32_t(int(q[4 * j + 3]) & 0xFF) << 24);
            *reinterpret_cast<uint4 *>(pay + 64ull * pos + 16 * part) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        } else {
            // byte i of the 16-byte half (p/2) takes entry i of this lane in
            // its low nibble (even p) or high nibble (odd p)
            const int sh = (part & 1) * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wd[j] = ((uint32_t(int(q[4 * j]) & 0xF)) << sh) | ((uint32_t(int(q[4 * j + 1]) & 0xF)) << (8 + sh)) |
                        ((uint32_t(int(q[4 * j + 2]) & 0xF)) << (16 + sh)) |
                        ((uint32_t(int(q[4 * j + 3]) & 0xF)) << (24 + sh));
#pragma unroll
            for (int j = 0; j < 4; ++j) wd[j] |= dpp_u32<kDppXor1>(wd[j]);
            if ((part & 1) == 0)
                *reinterpret_cast<uint4 *>(pay + 32ull * pos + 16 * (part >> 1)) =
                    make_uint4(wd[0], wd[1], wd[2], wd[3]);
        }
    } else if (f == 2u || f == 3u) {
        uint32_t hv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t lo, hi;
            if (f == 2u) {
                lo = f32_to_bf16_rne(w[2 * j]);
                hi = f32_to_bf16_rne(w[2 * j + 1]);
            } else {
                lo = __builtin_bit_cast(uint16_t, _Float16(w[2 * j]));
                hi = __builtin_bit_cast(uint16_t, _Float16(w[2 * j + 1]));
            }
            hv[j] = lo | (hi << 16);
        }
        uint4 *dst = reinterpret_cast<uint4 *>(pay + 128ull * pos + 32 * part);
        dst[0] = make_uint4(hv[0], hv[1], hv[2], hv[3]);
        dst[1] = make_uint4(hv[4], hv[5], hv[6], hv[7]);
    } else {
        float4 *dst = reinterpret_cast<float4 *>(pay + 256ull * pos + 64 * part);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = make_float4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
    }
}

}  // namespace ht
