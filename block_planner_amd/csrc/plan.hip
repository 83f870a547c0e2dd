// plan.hip -- the precision planner on gfx950 (HyperTensor 1.0.1 page, "What
// it does" and "Key Features": per-block format choice from measured error;
// "Convert model": zero thresholds for the 16-bit formats and bfloat16 tried
// first, by default).  For every 64-wide K-block the kernel computes the
// error each candidate format would leave and keeps the cheapest format
// whose relative error is within that format's threshold.
//
// Work layout: 4 lanes per 64-entry K-block, 16 consecutive fp32 entries per
// lane held in registers, 16 blocks per wavefront, 64 blocks per 256-thread
// workgroup.  Reductions (max, OR, and the fp64 error sums) use DPP within
// the block's quad, so the block needs no LDS.  The format pick is a chain of
// selects: no divergent branches except the rare exact-division fallback.
//
// Error sums: fp64, the balanced pairwise tree in natural order (a lane's 16
// entries as a 4-level tree, then two cross-lane levels).  The decision is
// err2 <= (eps^2) * nrm2 in fp64.  With eps_bf16 = eps_fp16 = 0 the 16-bit
// tests reduce exactly to "every entry is representable": a nonzero
// difference d has d^2 >= 2^-298 > 0 in fp64.
#include "quant.h"

#pragma clang fp contract(off)

namespace ht {

struct PlanArgs {
    const float *W;
    uint8_t *fmt;
    uint32_t n_blocks;   // N * K / 64
    uint32_t KB;         // K / 64
    FastDiv div_kb;
    int64_t ldw;
    PlanRule rule;
};

template <bool EPS16_ZERO>
__global__ __launch_bounds__(256) void plan_kernel(PlanArgs a) {
    __shared__ __align__(16) float stage[4][16 * 64];      // per wave: its 16 blocks
    const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
    const uint32_t b = tid >> 2;           // block index n * KB + kb
    const int part = int(threadIdx.x & 3);
    const bool valid = b < a.n_blocks;
    const uint32_t lane = threadIdx.x & 63u, wv = threadIdx.x >> 6;

    // The wave's 16 blocks as 4 fully coalesced 1 KiB loads (16-byte piece
    // p = 64j + lane is piece p % 16 of the wave's block p / 16), through LDS
    // to the compute layout (lane = 4 * block + part holds pieces 4*lane ..
    // 4*lane + 3).  Blocks past the end read block 0 and store nothing.
    {
        const uint32_t b0 = blockIdx.x * 64u + wv * 16u;
        f32x4 pc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t p = 64u * j + lane, bb = b0 + (p >> 4);
            const uint32_t bc = bb < a.n_blocks ? bb : 0u;
            const uint32_t n = fastdiv(bc, a.div_kb), kb = bc - n * a.KB;
            pc[j] = ld_stream_f4(a.W + int64_t(n) * a.ldw + kb * 64u + (p & 15u) * 4u);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4 *>(&stage[wv][(64u * j + lane) * 4u]) = pc[j];
    }
    __syncthreads();
    float w[kPerLane];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(&stage[wv][(4u * lane + k) * 4u]);
        w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }

    const int f = block_format<EPS16_ZERO>(w, a.rule);
    if (valid && part == 0) a.fmt[b] = uint8_t(f);
}

// Per-format block counts of a format map: one 64-bit atomic per workgroup and
// format (integer addition, so the result does not depend on the order).
__global__ __launch_bounds__(256) void zero_counts_kernel(int64_t *counts) {
    if (threadIdx.x < 5) counts[threadIdx.x] = 0;
}

__global__ __launch_bounds__(256) void count_kernel(const uint8_t *fmt, uint64_t n, int64_t *counts) {
    uint32_t c[5] = {0, 0, 0, 0, 0};
    const uint64_t stride = uint64_t(gridDim.x) * 256u * 16u;
    for (uint64_t i = (uint64_t(blockIdx.x) * 256u + threadIdx.x) * 16u; i < n; i += stride) {
        if (i + 16 <= n && (reinterpret_cast<uintptr_t>(fmt + i) & 15u) == 0) {
            uint4 v = *reinterpret_cast<const uint4 *>(fmt + i);
            uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t f = (words[j] >> (8 * k)) & 0xFFu;
#pragma unroll
                    for (int g = 0; g < 5; ++g) c[g] += (f == uint32_t(g)) ? 1u : 0u;
                }
        } else {
            for (uint64_t j = i; j < n && j < i + 16; ++j) {
                uint32_t f = fmt[j];
#pragma unroll
                for (int g = 0; g < 5; ++g) c[g] += (f == uint32_t(g)) ? 1u : 0u;
            }
        }
    }
    // wave sums, then one atomic per workgroup and format (the five counters
    // share a cache line, so fewer atomics means less serialisation)
    __shared__ uint32_t part[4][5];
#pragma unroll
    for (int g = 0; g < 5; ++g) {
        uint32_t v = c[g];
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6][g] = v;
    }
    __syncthreads();
    if (threadIdx.x < 5) {
        const uint32_t v = part[0][threadIdx.x] + part[1][threadIdx.x] + part[2][threadIdx.x] + part[3][threadIdx.x];
        if (v) atomicAdd(reinterpret_cast<unsigned long long *>(counts + threadIdx.x), (unsigned long long)v);
    }
}

}  // namespace ht

using namespace ht;

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static ht_status check_eps(double e) {
    if (!(e >= 0.0) || e > 1e150) return HT_EINVAL;   // also rejects NaN
    return HT_OK;
}

extern "C" ht_status ht_plan(const float *W, int64_t N, int64_t K, int64_t ldw,
                             const ht_plan_params *p, uint8_t *fmt_map, ht_stream stream) {
    ht_plan_params def;
    ht_plan_params_default(&def);
    if (!p) p = &def;
    if (!W || !fmt_map) return HT_EINVAL;
    if (N <= 0 || K <= 0 || K % kBlockK != 0 || ldw < K) return HT_ESHAPE;
    if ((ldw % 4) != 0) return HT_EALIGN;
    if (!aligned16(W)) return HT_EALIGN;
    const double eps[4] = {p->eps_int4, p->eps_int8, p->eps_bf16, p->eps_fp16};
    for (double e : eps)
        if (check_eps(e) != HT_OK) return HT_EINVAL;
    if (p->force_format < -1 || p->force_format > 4) return HT_EINVAL;
    const int64_t KB = K / kBlockK;
    const int64_t nb = N * KB;
    if (nb >= (int64_t(1) << 30) || KB > 0xFFFFFFFFll) return HT_ESHAPE;

    PlanArgs a;
    a.W = W;
    a.fmt = fmt_map;
    a.n_blocks = uint32_t(nb);
    a.KB = uint32_t(KB);
    a.div_kb = make_fastdiv(uint32_t(KB));
    a.ldw = ldw;
    for (int i = 0; i < 4; ++i) a.rule.e2[i] = eps[i] * eps[i];
    a.rule.prefer_bf16 = p->prefer_bf16 ? 1 : 0;
    a.rule.force = p->force_format;
    const uint32_t grid = uint32_t((nb + 63) / 64);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p->eps_bf16 == 0.0 && p->eps_fp16 == 0.0)
        hipLaunchKernelGGL(plan_kernel<true>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(plan_kernel<false>, dim3(grid), dim3(256), 0, s, a);
    HT_LAUNCH_CHECK();
    return HT_OK;
}

extern "C" ht_status ht_plan_counts(const uint8_t *fmt_map, int64_t N, int64_t K, int64_t *counts5,
                                    ht_stream stream) {
    if (!fmt_map || !counts5) return HT_EINVAL;
    if (N <= 0 || K <= 0 || K % kBlockK != 0) return HT_ESHAPE;
    if ((reinterpret_cast<uintptr_t>(counts5) & 7u) != 0) return HT_EALIGN;
    const uint64_t n = uint64_t(N) * uint64_t(K / kBlockK);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(64), 0, s, counts5);
    HT_LAUNCH_CHECK();
    uint64_t want = (n + 256 * 16 - 1) / (256 * 16);
    uint32_t grid = uint32_t(want < 1024 ? (want ? want : 1) : 1024);
    hipLaunchKernelGGL(count_kernel, dim3(grid), dim3(256), 0, s, fmt_map, n, counts5);
    HT_LAUNCH_CHECK();
    return HT_OK;
}
