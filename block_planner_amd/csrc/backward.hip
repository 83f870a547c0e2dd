// backward.hip -- the input gradient of the linear over the packed buffers:
// dX[m, k] = sum over n of dY[m, n] * w_hat[n, k]  (HyperTensor 1.0.1 page,
// "Key Features": training and inference support; "Design Philosophy":
// custom backward kernels).  Integer blocks contribute (dY * s) * q,
// float blocks dY * w; fp32 arithmetic, fixed-order sums (bitwise
// reproducible).
//
// Work split: workgroup (kg, g) owns K-blocks [4 kg, 4 kg + 4) (one per
// wavefront) and row tiles [TPG g, TPG g + TPG).  For its K-block kb a
// wavefront walks the tiles in order, one column in flight ahead of the
// arithmetic; tile t's column (t, kb) is the tile's
// 16 blocks of that K-block in the packed order (format by format, rows
// ascending), found from the kbidx entries of (t, kb) and (t, kb + 1).  Lane
// (j, q) takes the j-th block of the column and its entries [16q, 16q + 16)
// (INT4: the 16 bytes holding them, nibble q & 1), multiplies them by dY of
// that block's row and adds them to its 16 accumulators per row of dY.  At
// the end the 16 lanes of each q add their accumulators in a fixed DPP
// order and lane j keeps entry j: dX for this K-block and tile group.  With
// several tile groups the per-group sums go to the workspace and the split
// reduction kernel adds them in group order.
#include "gemv_common.h"
#include "linear_host.h"

namespace ht {

constexpr uint32_t kBwdMaxM = 4;       // rows of dY per launch (16 accumulators each per lane)
constexpr uint32_t kBwdThreads = 256;  // 4 wavefronts: one K-block each
constexpr uint32_t kBwdKPG = 4;        // K-blocks per workgroup

struct BwdArgs {
    LayerDev w;
    const float *dy;
    int64_t lddy;
    float *dx;            // [M][lddx] when G == 1, else nullptr
    int64_t lddx;
    float *partial;       // [G][M][K] when G > 1
    uint32_t M, TPG, G;
};

template <int M>
__global__ __launch_bounds__(kBwdThreads) void linear_bwd_kernel(BwdArgs a) {
    const LayerDev &w = a.w;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t j = lane & 15, q = lane >> 4;
    const uint32_t kb = blockIdx.x * kBwdKPG + wave;
    if (kb >= w.KB) return;                                // wave-uniform; no barrier below
    const uint32_t t0 = blockIdx.y * a.TPG, t1 = min(w.T, t0 + a.TPG);
    const uint8_t *base = w.base;
    const uint32_t *kbx = reinterpret_cast<const uint32_t *>(base + w.off_kbidx);

    uint32_t opay[5], oids[5];
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        opay[f] = uint32_t(w.off_pay[f]);
        oids[f] = uint32_t(w.off_ids[f]);
    }
    const uint32_t osc0 = uint32_t(w.off_scale[0]), osc1 = uint32_t(w.off_scale[1]);

    float acc[M][16];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][i] = 0.0f;

    // Column loads run one tile ahead of the arithmetic (and their kbidx
    // entries two ahead), so each wavefront keeps a column in flight.
    struct Col {
        uint32_t u[16];
        uint32_t id2, blk;
        float sc;
        int f;
        float dyv[M];   // dY[m, 16 t + j]: lane j holds row j of the tile
    };
    auto kbidx_of = [&](uint32_t t, uint32_t (&ka)[5], uint32_t (&kn)[5]) {   // wave-uniform values
        const uint64_t ci = uint64_t(min(t, t1 - 1u)) * w.KB + kb;
#pragma unroll
        for (int f = 0; f < 5; ++f) {
            ka[f] = __builtin_amdgcn_readfirstlane(kbx[uint64_t(f) * w.nk + ci]);
            kn[f] = __builtin_amdgcn_readfirstlane(kbx[uint64_t(f) * w.nk + ci + 1]);
        }
    };
    auto load = [&](const uint32_t (&ka)[5], const uint32_t (&kn)[5], uint32_t t) -> Col {
        Col c;
        // the tile's 16 rows of dY, independent of the block ids, so no wait
        // on the column's loads (rows past N read row N - 1 and are not used)
        const uint32_t nrow = min(min(t, t1 - 1u) * 16u + j, w.N - 1u);
#pragma unroll
        for (int m = 0; m < M; ++m) c.dyv[m] = a.dy[int64_t(m) * a.lddy + nrow];
        // this lane's block: slot j of the column in the packed order
        uint32_t cum = 0, blk = 0;
        int f = 5;
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            const uint32_t cnt = kn[g] - ka[g];
            if (f == 5 && j - cum < cnt) {
                f = g;
                blk = ka[g] + (j - cum);
            }
            cum += cnt;
        }
        uint32_t po = 0, io = 0, so = 0, nl = 1;
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            if (f == g) {
                po = opay[g] + blk * uint32_t(pay_bytes(g)) +
                     (g == 0 ? 16u * (q >> 1) : g == 1 ? 16u * q : g == 4 ? 64u * q : 32u * q);
                io = oids[g] + ((2u * blk) & ~3u);
                so = g == 0 ? osc0 + 4u * blk : g == 1 ? osc1 + 4u * blk : 0u;
                nl = g < 2 ? 1u : g == 4 ? 4u : 2u;
            }
        }
        // a lane without a block reads the buffer's first bytes and adds nothing
#pragma unroll
        for (uint32_t p = 0; p < 4; ++p) {
            const uint4 v = *reinterpret_cast<const uint4 *>(base + po + (p < nl ? 16u * p : 0u));
            c.u[4 * p + 0] = v.x;
            c.u[4 * p + 1] = v.y;
            c.u[4 * p + 2] = v.z;
            c.u[4 * p + 3] = v.w;
        }
        c.id2 = *reinterpret_cast<const uint32_t *>(base + io);
        c.sc = *reinterpret_cast<const float *>(base + so);
        c.blk = blk;
        c.f = f;
        return c;
    };
    auto consume = [&](const Col &c) {
        const uint32_t id = (c.blk & 1u) ? c.id2 >> 16 : c.id2 & 0xFFFFu;
        const int src = int(id & 15u) * 4;    // lane holding this block's row of dY
        const uint32_t *u = c.u;
        float e[16];
        switch (c.f) {
        case 0: {   // entry i = nibble (q & 1) of byte i of the 16 loaded bytes
            const uint32_t sh = 4u * (q & 1u);
#pragma unroll
            for (int i = 0; i < 16; ++i) e[i] = float(int32_t((u[i >> 2] >> (8 * (i & 3) + sh)) << 28) >> 28);
            break;
        }
        case 1:
#pragma unroll
            for (int i = 0; i < 16; ++i) e[i] = float(int8_t(u[i >> 2] >> (8 * (i & 3))));
            break;
        case 2:
#pragma unroll
            for (int i = 0; i < 16; ++i) e[i] = __uint_as_float((i & 1) ? (u[i >> 1] & 0xFFFF0000u) : (u[i >> 1] << 16));
            break;
        case 3:
#pragma unroll
            for (int i = 0; i < 16; ++i)
                e[i] = float(__builtin_bit_cast(_Float16, uint16_t((i & 1) ? (u[i >> 1] >> 16) : u[i >> 1])));
            break;
        case 4:
#pragma unroll
            for (int i = 0; i < 16; ++i) e[i] = __uint_as_float(u[i]);
            break;
        default:
#pragma unroll
            for (int i = 0; i < 16; ++i) e[i] = 0.0f;
            break;
        }
        // every lane takes part in the permute (the source lanes must be active)
        float dyr[M];
#pragma unroll
        for (int m = 0; m < M; ++m) dyr[m] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(c.dyv[m])));
        if (c.f < 5) {
            const float s = c.f < 2 ? c.sc : 1.0f;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float g = dyr[m] * s;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[m][i] = __builtin_fmaf(g, e[i], acc[m][i]);
            }
        }
    };

    if (t0 < t1) {
        uint32_t ka[5], kn[5], ka2[5], kn2[5];
        kbidx_of(t0, ka, kn);
        Col cur = load(ka, kn, t0);
        kbidx_of(t0 + 1, ka, kn);                             // clamped past the last tile
        for (uint32_t t = t0; t < t1; ++t) {
            kbidx_of(t + 2, ka2, kn2);
            const Col nxt = load(ka, kn, t + 1);                     // tile t + 1 (a repeat of the last tile past the end)
            consume(cur);
            cur = nxt;
#pragma unroll
            for (int f = 0; f < 5; ++f) {
                ka[f] = ka2[f];
                kn[f] = kn2[f];
            }
        }
    }

    // the 16 lanes of each q add their accumulators (fixed order); lane j
    // keeps entry j: dX[m, 64 kb + 16 q + j] of this tile group
    const uint32_t k = kb * 64u + 16u * q + j;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float mine = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float s = group_sum<16>(acc[m][i]);
            mine = j == uint32_t(i) ? s : mine;
        }
        if (uint32_t(m) < a.M) {
            if (a.partial) a.partial[(uint64_t(blockIdx.y) * a.M + m) * (uint64_t(w.KB) * 64u) + k] = mine;
            else a.dx[int64_t(m) * a.lddx + k] = mine;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

// Row tiles per workgroup: enough workgroups for the chip (about 1024 of four
// wavefronts), at least 4 tiles each, fewer groups when there are few tiles.
uint32_t bwd_tpg(const ht_packed_weight *w) {
    const uint64_t KG = uint64_t((w->K / kBlockK + kBwdKPG - 1) / kBwdKPG), T = uint64_t(w->n_tiles);
    uint64_t G = (1024 + KG - 1) / KG;
    if (G > 32) G = 32;
    if (G > (T + 3) / 4) G = (T + 3) / 4;
    if (G < 1) G = 1;
    const uint64_t tpg = (T + G - 1) / G;
    return uint32_t(tpg);
}

uint32_t bwd_groups(const ht_packed_weight *w) {
    const uint32_t tpg = bwd_tpg(w);
    return uint32_t((uint64_t(w->n_tiles) + tpg - 1) / tpg);
}

template <int M>
void launch_bwd(const BwdArgs &a, uint32_t KG, hipStream_t s) {
    hipLaunchKernelGGL(linear_bwd_kernel<M>, dim3(KG, a.G), dim3(kBwdThreads), 0, s, a);
}

}  // namespace

bool bwd_ok(const ht_packed_weight *w) { return w->row_tile == 16; }

size_t bwd_ws(const ht_packed_weight *w, int64_t M) {
    const uint32_t G = bwd_groups(w);
    const int64_t Mt = M < int64_t(kBwdMaxM) ? M : int64_t(kBwdMaxM);
    return G > 1 ? size_t(G) * size_t(Mt) * size_t(w->K) * sizeof(float) : 0;
}

ht_status run_bwd(const ht_packed_weight *w, const float *dy, int64_t M, int64_t lddy, float *dx, int64_t lddx,
                  void *ws, hipStream_t s) {
    BwdArgs a;
    a.w = layer_dev(w);
    a.lddy = lddy;
    a.lddx = lddx;
    a.TPG = bwd_tpg(w);
    a.G = bwd_groups(w);
    const uint32_t KG = (a.w.KB + kBwdKPG - 1) / kBwdKPG;
    for (int64_t m0 = 0; m0 < M; m0 += kBwdMaxM) {
        const int64_t Mt = M - m0 < int64_t(kBwdMaxM) ? M - m0 : int64_t(kBwdMaxM);
        a.M = uint32_t(Mt);
        a.dy = dy + m0 * lddy;
        a.dx = a.G > 1 ? nullptr : dx + m0 * lddx;
        a.partial = a.G > 1 ? static_cast<float *>(ws) : nullptr;
        switch (Mt) {
        case 1: launch_bwd<1>(a, KG, s); break;
        case 2: launch_bwd<2>(a, KG, s); break;
        case 3: launch_bwd<3>(a, KG, s); break;
        default: launch_bwd<4>(a, KG, s); break;
        }
        HT_LAUNCH_CHECK();
        if (a.G > 1) {
            const ht_status st = launch_split_reduce(static_cast<const float *>(ws), a.G, uint32_t(Mt),
                                                     uint32_t(w->K), dx + m0 * lddx, nullptr, lddx, HT_ACT_NONE, s);
            if (st != HT_OK) return st;
        }
    }
    return HT_OK;
}

}  // namespace ht

// ---------------------------------------------------------------------------
// Weight gradient for the fp32 master weight under the straight-through
// estimator (HyperTensor 1.0.1 page, "Design Philosophy": STE for the
// backward pass): the gradient of W_hat is passed to W unchanged, so
// dW[n, k] = sum over m of dY[m, n] * x[m, k], x being the bf16 activations
// the forward consumed.  At training batch sizes the N x K fp32 output is
// the traffic, so this is a plain coalesced kernel of one-wavefront
// workgroups (independent waves fill a compute unit's slots better than
// 4-wave groups: 31.9 against 35.0 us at 32 rows of 4096 x 4096): workgroup
// (cx, y) owns columns [256 cx, 256 cx + 256) and rows
// 16 (y >> 2) + (y & 3) + 4 r, r < kDwRpt, lane l 4 consecutive columns,
// adding the rows of dY / x in order (fixed order: bitwise reproducible).
// ---------------------------------------------------------------------------
namespace ht {

constexpr uint32_t kDwCols = 256;
constexpr int kDwRpt = 4;                        // rows per thread (one in 4: the wavefronts interleave)
constexpr uint32_t kDwRows = 4 * kDwRpt;

__global__ __launch_bounds__(64) void linear_dw_kernel(const float *dy, int64_t lddy, const uint16_t *x, int64_t ldx,
                                                        float *dw, int64_t lddw, uint32_t M, uint32_t N, uint32_t K,
                                                        int accumulate) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = blockIdx.y & 3u;                  // one wavefront per workgroup
    const uint32_t k = blockIdx.x * kDwCols + 4u * lane;
    const uint32_t n0 = (blockIdx.y >> 2) * kDwRows + wave;
    if (k >= K) return;                                     // K is a multiple of 4; no barrier below
    uint32_t nc[kDwRpt];                                    // row index clamped for the loads
    bool live[kDwRpt];
#pragma unroll
    for (int r = 0; r < kDwRpt; ++r) {
        const uint32_t n = n0 + 4u * r;
        live[r] = n < N;
        nc[r] = live[r] ? n : N - 1u;
    }
    float acc[kDwRpt][4];
#pragma unroll
    for (int r = 0; r < kDwRpt; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;
#pragma unroll 4
    for (uint32_t m = 0; m < M; ++m) {
        const uint2 xv = *reinterpret_cast<const uint2 *>(x + int64_t(m) * ldx + k);
        const float xf[4] = {__uint_as_float(xv.x << 16), __uint_as_float(xv.x & 0xFFFF0000u),
                             __uint_as_float(xv.y << 16), __uint_as_float(xv.y & 0xFFFF0000u)};
#pragma unroll
        for (int r = 0; r < kDwRpt; ++r) {
            const float g = live[r] ? dy[int64_t(m) * lddy + nc[r]] : 0.0f;   // wave-uniform
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(g, xf[c], acc[r][c]);
        }
    }
#pragma unroll
    for (int r = 0; r < kDwRpt; ++r) {
        if (!live[r]) continue;
        float4 *p = reinterpret_cast<float4 *>(dw + int64_t(n0 + 4u * r) * lddw + k);
        float4 o = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
        if (accumulate) {
            const float4 v = *p;
            o = make_float4(v.x + o.x, v.y + o.y, v.z + o.z, v.w + o.w);
        }
        *p = o;
    }
}

}  // namespace ht

extern "C" ht_status ht_linear_backward_weight(const float *dy, int64_t M, int64_t lddy, const uint16_t *x,
                                               int64_t ldx, int64_t N, int64_t K, float *dw, int64_t lddw,
                                               int32_t accumulate, ht_stream stream) {
    using namespace ht;
    auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (!dw || (M > 0 && (!dy || !x))) return HT_EINVAL;
    if (M < 0 || N <= 0 || K <= 0 || K % 4 || M > 0x7FFFFFFF || N > 0x7FFFFFFF || K > 0x7FFFFFFF) return HT_ESHAPE;
    if ((M > 0 && (lddy < N || ldx < K || ldx % 4)) || lddw < K || lddw % 4) return HT_ESHAPE;
    if (4 * ((N + kDwRows - 1) / kDwRows) > 65535) return HT_ESHAPE;
    if (!al16(dw) || (M > 0 && (!al16(dy) || !al16(x)))) return HT_EALIGN;
    if (M >= kDwGemmMinM && K < (int64_t(1) << 30))   // x rows below 2 GiB: 32-bit buffer offsets
        return run_dw_gemm(dy, M, lddy, x, ldx, N, K, dw, lddw, accumulate ? 1 : 0,
                           reinterpret_cast<hipStream_t>(stream));
    const dim3 grid(uint32_t((K + kDwCols - 1) / kDwCols), 4u * uint32_t((N + kDwRows - 1) / kDwRows));
    hipLaunchKernelGGL(linear_dw_kernel, grid, dim3(64), 0, reinterpret_cast<hipStream_t>(stream), dy, lddy, x, ldx,
                       dw, lddw, uint32_t(M), uint32_t(N), uint32_t(K), accumulate ? 1 : 0);
    HT_LAUNCH_CHECK();
    return HT_OK;
}
