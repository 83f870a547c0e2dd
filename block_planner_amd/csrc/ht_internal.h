// ht_internal.h -- helpers shared by the gfx950 kernels and the host glue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ht.h"

namespace ht {

constexpr int kBlockK = 64;
constexpr int kNumFormats = 5;

// Bytes of one block's payload per format (INT4, INT8, BF16, FP16, FP32).
__host__ __device__ constexpr int pay_bytes(int f) {
    return f == 0 ? 32 : f == 1 ? 64 : f == 4 ? 256 : 128;
}

__host__ __device__ inline uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

// ---------------------------------------------------------------------------
// Exact unsigned 32-bit division by a run-time constant (Granlund-Montgomery
// round-up method): for d >= 1 with l = ceil(log2 d) and
// m = floor(2^32 * (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l for every
// 32-bit n.  Saves the long integer-division sequence in per-lane index math.
// ---------------------------------------------------------------------------
struct FastDiv {
    uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    f.l = l;
    f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
    return f;
}

__host__ __device__ inline uint32_t fastdiv(uint32_t n, FastDiv f) {
#ifdef __HIP_DEVICE_COMPILE__
    uint32_t t = __umulhi(n, f.m);
#else
    uint32_t t = uint32_t((uint64_t(n) * f.m) >> 32);
#endif
    return uint32_t((uint64_t(t) + n) >> f.l);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte loads: the data is read once, so hint the caches not to
// keep it (nontemporal).
__device__ __forceinline__ f32x4 ld_stream_f4(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ u32x4 ld_stream_u4(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// ---------------------------------------------------------------------------
// Cross-lane moves (DPP).  Every pattern below stays inside a row of 16 lanes
// and every source lane is active when they are used, so all lanes receive
// valid data.  Sums built from them are identical on all participating lanes
// (IEEE addition is commutative), which keeps the reductions deterministic.
// ---------------------------------------------------------------------------
enum : int {
    kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141, // lane i <- lane 7-i within each 8
    kDppMirror = 0x140,     // lane i <- lane 15-i within each 16
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    uint64_t u = uint64_t(__double_as_longlong(v));
    uint32_t lo = dpp_u32<CTRL>(uint32_t(u));
    uint32_t hi = dpp_u32<CTRL>(uint32_t(u >> 32));
    return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}

// Sum over groups of LPB consecutive lanes (LPB in 1, 2, 4, 8, 16); every lane
// of a group ends with the group's sum.
template <int LPB>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LPB >= 2) v = v + dpp_f32<kDppXor1>(v);
    if constexpr (LPB >= 4) v = v + dpp_f32<kDppXor2>(v);
    if constexpr (LPB >= 8) v = v + dpp_f32<kDppHalfMirror>(v);
    if constexpr (LPB >= 16) v = v + dpp_f32<kDppMirror>(v);
    return v;
}

// fp32 -> bfloat16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

}  // namespace ht

// Host-side launch check used by every entry point.
#define HT_LAUNCH_CHECK()                                  \
    do {                                                   \
        if (hipGetLastError() != hipSuccess) return HT_EHIP; \
    } while (0)
