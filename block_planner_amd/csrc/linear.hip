// linear.hip -- one fused mixed-format linear over the packed execution
// buffers (HyperTensor 1.0.1 page, intro: fused kernels execute the
// mixed-precision plan; "Key Features": HyperLinear, a drop-in nn.Linear).
//
// y[m, n] = sum over n's K-blocks kb of  blk(m, n, kb), where
//   INT4 / INT8:  blk = s * (sum_i q_i * x[m, 64kb+i])   (scale after the partial)
//   BF16 / FP16 / FP32:  blk = sum_i w_i * x[m, 64kb+i]
// all in fp32.  Workgroup (row tile t, K-split s) owns rows [tR, tR+R) and
// K-blocks [kb0, kb1).  Its NW wavefronts (16, or 8 when there are more
// workgroups than compute units: then two fit on a compute unit and all of
// them run at once) first issue x's loads, then one batch of 8 chunks each
// (a 16-row x 4096 tile is a single batch at 16 wavefronts), stage x in
// LDS as fp32 while the weights are in flight, and consume each chunk as soon
// as its own data has arrived.  Block partials go to an LDS table P[m][r][kb];
// each (m, r) sums its row of P in a fixed order, so the result is bitwise
// reproducible.  With several K-splits the per-split sums go to the
// workspace and a second kernel adds them in split order.
#include "gemv_common.h"
#include "layout.h"
#include "linear_host.h"

namespace ht {

struct LinArgs {
    LayerDev w;
    uint32_t S, KBs;              // K-splits and K-blocks per split
    const uint16_t *x;
    int64_t ldx;
    float *y;                     // fp32 output (S == 1) or nullptr
    uint16_t *ybf;                // bf16 output (S == 1) or nullptr
    int64_t ldy;
    float *partial;               // [S][M][N] when S > 1
    int act;
};

template <int M, int NW>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(LinArgs a) {
    constexpr uint32_t NT = 64 * NW;         // threads
    constexpr int XL = 2 * kWaves / NW;      // 16-byte x loads per thread
    extern __shared__ float lds[];
    const LayerDev &w = a.w;
    const uint32_t t = blockIdx.x, sidx = blockIdx.y;
    const uint32_t kb0 = sidx * a.KBs;
    if (kb0 >= w.KB) return;   // cannot happen: the host makes every split non-empty
    const uint32_t kb1 = min(w.KB, kb0 + a.KBs);
    const uint32_t nkb = kb1 - kb0;
    const uint32_t xstride = nkb * 64;
    const uint32_t pstride = nkb + 1;
    float *xs = lds;                       // [M][nkb*64]
    float *P = lds + M * xstride;          // [M][R][nkb+1]
    const uint32_t lane = threadIdx.x & 63;
    // wave index as a scalar: the chunk -> format decode and the per-format
    // pointers derived from it then stay in scalar registers
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // x for these K-blocks: at most XL 16-byte loads per thread (the host
    // keeps the M * nkb * 64 * 4 bytes of fp32 x within 64 KiB), issued first
    const uint32_t per_row = nkb * 8;   // 8 bf16 per 16-byte load
    uint4 xr[XL];
#pragma unroll
    for (int j = 0; j < XL; ++j) {
        const uint32_t i = threadIdx.x + j * NT;
        if (i < M * per_row) {
            const uint32_t m = i / per_row, jj = i - m * per_row;
            xr[j] = *reinterpret_cast<const uint4 *>(a.x + int64_t(m) * a.ldx + kb0 * 64 + jj * 8);
        }
    }

    // this workgroup's range of each format's blocks
    const uint32_t *kbidx = reinterpret_cast<const uint32_t *>(w.base + w.off_kbidx);
    const uint64_t col0 = uint64_t(t) * w.KB + kb0, col1 = uint64_t(t) * w.KB + kb1;
    uint32_t lo[5], hi[5];
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        hi[f] = kbidx[uint64_t(f) * w.nk + col1];
        lo[f] = kbidx[uint64_t(f) * w.nk + col0];
    }
    ChunkWalker src = chunk_src(w, lo, hi);
    walker_start(src, wave, NW);

    // first batch in flight while x goes into LDS
    Slot sl[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        sl[u].f = 5;
        if (src.f < 5) {   // wave-uniform: no loads for slots past the wave's last chunk
            sl[u] = walker_load(src, lane);
            walker_advance(src);
        }
    }

#pragma unroll
    for (int j = 0; j < XL; ++j) {
        const uint32_t i = threadIdx.x + j * NT;
        if (i < M * per_row) {
            const uint32_t m = i / per_row, jj = i - m * per_row;
            const uint4 v = xr[j];
            float4 *d = reinterpret_cast<float4 *>(xs + m * xstride + jj * 8);
            d[0] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
            d[1] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
        }
    }
    __syncthreads();

    // the first batch in straight-line code: each chunk waits for its own data
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) consume<M>(sl[u], lane, xs, xstride, P, pstride, kb0, nkb, w.R, w.lgR);
    while (src.f < 5) {   // wave-uniform: chunks left for this wave
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            sl[u].f = 5;
            if (src.f < 5) {
                sl[u] = walker_load(src, lane);
                walker_advance(src);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) consume<M>(sl[u], lane, xs, xstride, P, pstride, kb0, nkb, w.R, w.lgR);
    }
    __syncthreads();

    reduce_rows<M, NW>(P, pstride, w.R, nkb, wave, lane, [&](uint32_t m, uint32_t r, float v) {
        const uint32_t n = t * w.R + r;
        if (n >= w.N) return;
        if (a.S == 1) {
            if (a.act == HT_ACT_RELU) v = v > 0.0f ? v : 0.0f;   // +0 for zero, negative and NaN
            if (a.ybf) a.ybf[int64_t(m) * a.ldy + n] = f32_to_bf16_rne(v);
            else a.y[int64_t(m) * a.ldy + n] = v;
        } else {
            a.partial[(uint64_t(sidx) * M + m) * w.N + n] = v;
        }
    });
}

// y[m, n] = act(sum over s in order of partial[s][m][n])
// One thread per output; small workgroups so that short outputs still reach
// many compute units.  The partials are loaded 16 at a time (independent
// loads in flight) and added in split order, the same order as one load at
// a time.
constexpr uint32_t kReduceThreads = 64;

__global__ __launch_bounds__(kReduceThreads) void split_reduce_kernel(const float *partial, uint32_t S, uint32_t M,
                                                                      uint32_t N, float *y, uint16_t *ybf,
                                                                      int64_t ldy, int act) {
    const uint32_t i = blockIdx.x * kReduceThreads + threadIdx.x;
    if (i >= M * N) return;
    const uint32_t m = i / N, n = i - m * N;
    const uint64_t stride = uint64_t(M) * N;
    const float *p = partial + uint64_t(m) * N + n;
    float v = 0.0f;
    uint32_t s = 0;
    for (; s + 16 <= S; s += 16) {
        float t[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) t[u] = p[(s + u) * stride];
#pragma unroll
        for (int u = 0; u < 16; ++u) v += t[u];
    }
    for (; s < S; ++s) v += p[s * stride];
    if (act == HT_ACT_RELU) v = v > 0.0f ? v : 0.0f;
    if (ybf) ybf[int64_t(m) * ldy + n] = f32_to_bf16_rne(v);
    else y[int64_t(m) * ldy + n] = v;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

constexpr uint32_t kMaxX = 64 * 1024;     // fp32 copy of x: at most two 16-byte loads of bf16 x per thread
constexpr uint32_t kMaxLds = 96 * 1024;   // x plus the block partials (long K at M = 1 then needs no split)
constexpr int kMaxM = 8;   // rows per launch of the register path; larger M is tiled

uint32_t x_bytes(uint32_t Mt, uint32_t nkb) { return Mt * nkb * 64u * 4u; }

uint32_t lds_bytes(uint32_t Mt, uint32_t nkb, uint32_t R) { return x_bytes(Mt, nkb) + Mt * R * (nkb + 1u) * 4u; }

// Packed bytes per workgroup below which a further K-split does not pay: the
// split adds a reduction launch of a few microseconds, about what one
// workgroup needs to stream this much (measured on decode passes over
// transformer-shaped stacks, where splitting smaller layers made them slower).
constexpr uint64_t kSplitBytes = 128 * 1024;

// K-split choice: x within kMaxX and x plus partials within kMaxLds; beyond
// that, more workgroups while there are fewer than the chip's compute units
// and each still streams more than kSplitBytes; every split at least 8
// K-blocks and non-empty.
uint32_t choose_splits(const ht_packed_weight *w, uint32_t Mt) {
    const uint32_t KB = uint32_t(w->K / kBlockK), T = uint32_t(w->n_tiles), R = uint32_t(w->row_tile);
    const uint64_t per_tile = uint64_t(w->bytes) / T;
    uint32_t S = 1;
    while (S < KB && (x_bytes(Mt, (KB + S - 1) / S) > kMaxX || lds_bytes(Mt, (KB + S - 1) / S, R) > kMaxLds ||
                      (uint64_t(T) * S < 256 && per_tile / S > kSplitBytes && (KB + S) / (S + 1) >= 8)))
        ++S;
    const uint32_t KBs = (KB + S - 1) / S;
    return (KB + KBs - 1) / KBs;
}

int m_tile(int64_t M) { return int(M < kMaxM ? M : kMaxM); }

// Workgroups of 8 wavefronts when there are more of them than compute units
// and two fit on one (LDS), so that all run at once; else 16.  Both give the
// same bits (each chunk's partial lands in its own slot of P).
constexpr uint64_t kComputeUnits = 256;
constexpr uint32_t kHalfLds = 80 * 1024;

template <int M, int NW>
ht_status launch_gemv_nw(const LinArgs &a, uint32_t T, uint32_t lds, hipStream_t s) {
    // more than 64 KiB of dynamic LDS is requested explicitly
    if (lds > 64u * 1024u &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(&gemv_kernel<M, NW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxLds)) != hipSuccess)
        return HT_EHIP;
    hipLaunchKernelGGL((gemv_kernel<M, NW>), dim3(T, a.S), dim3(64 * NW), lds, s, a);
    HT_LAUNCH_CHECK();
    return HT_OK;
}

template <int M>
ht_status launch_gemv(const LinArgs &a, uint32_t T, uint32_t lds, hipStream_t s) {
    if (uint64_t(T) * a.S > kComputeUnits && lds <= kHalfLds) return launch_gemv_nw<M, kWaves / 2>(a, T, lds, s);
    return launch_gemv_nw<M, kWaves>(a, T, lds, s);
}

}  // namespace

bool desc_ok(const ht_packed_weight *w) { return w && w->base && desc_layout_ok(w); }

size_t linear_ws(const ht_packed_weight *w, int64_t M) {
    const int Mt = m_tile(M);
    const uint32_t S = choose_splits(w, uint32_t(Mt));
    return S > 1 ? size_t(S) * size_t(Mt) * size_t(w->N) * sizeof(float) : 0;
}

ht_status launch_split_reduce(const float *partial, uint32_t S, uint32_t M, uint32_t N, float *y, uint16_t *ybf,
                              int64_t ldy, int act, hipStream_t s) {
    const uint32_t tot = M * N;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((tot + kReduceThreads - 1) / kReduceThreads), dim3(kReduceThreads), 0,
                       s, partial, S, M, N, y, ybf, ldy, act);
    HT_LAUNCH_CHECK();
    return HT_OK;
}

// One linear over rows [0, M) of x; output either fp32 y or bf16 ybf.
ht_status run_linear(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y,
                     uint16_t *ybf, int64_t ldy, int act, void *ws, hipStream_t s) {
    const uint32_t KB = uint32_t(w->K / kBlockK);
    const uint32_t T = uint32_t(w->n_tiles);
    LinArgs a;
    a.w = layer_dev(w);
    a.ldx = ldx;
    a.ldy = ldy;
    a.act = act;
    for (int64_t m0 = 0; m0 < M; m0 += kMaxM) {
        const int Mt = int(M - m0 < kMaxM ? M - m0 : kMaxM);
        const uint32_t S = choose_splits(w, uint32_t(Mt));
        a.S = S;
        a.KBs = (KB + S - 1) / S;
        a.x = x + m0 * ldx;
        a.y = y ? y + m0 * ldy : nullptr;
        a.ybf = ybf ? ybf + m0 * ldy : nullptr;
        a.partial = static_cast<float *>(ws);
        const uint32_t lds = lds_bytes(uint32_t(Mt), a.KBs, a.w.R);
        LinArgs g = a;
        if (S > 1) { g.y = nullptr; g.ybf = nullptr; }
        ht_status st;
        switch (Mt) {
        case 1: st = launch_gemv<1>(g, T, lds, s); break;
        case 2: st = launch_gemv<2>(g, T, lds, s); break;
        case 3: st = launch_gemv<3>(g, T, lds, s); break;
        case 4: st = launch_gemv<4>(g, T, lds, s); break;
        case 5: st = launch_gemv<5>(g, T, lds, s); break;
        case 6: st = launch_gemv<6>(g, T, lds, s); break;
        case 7: st = launch_gemv<7>(g, T, lds, s); break;
        default: st = launch_gemv<8>(g, T, lds, s); break;
        }
        if (st != HT_OK) return st;
        if (S > 1) {
            st = launch_split_reduce(static_cast<const float *>(ws), S, uint32_t(Mt), a.w.N, a.y, a.ybf, ldy, act, s);
            if (st != HT_OK) return st;
        }
    }
    return HT_OK;
}

}  // namespace ht

using namespace ht;

static bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static bool path_ok(int32_t path) {
    return path == HT_PATH_AUTO || path == HT_PATH_GEMV || path == HT_PATH_GEMM || path == HT_PATH_GEMV_MFMA ||
           path == HT_PATH_GEMM_I8 || path == HT_PATH_W8A8;
}

static size_t path_ws(const ht_packed_weight *w, int64_t M, int32_t path) {
    return path == HT_PATH_GEMM        ? gemm_ws(w, M)
           : path == HT_PATH_GEMV_MFMA ? dec_ws(w, M)
           : path == HT_PATH_GEMM_I8   ? i8_ws(w, M)
           : path == HT_PATH_W8A8      ? i8_ws(w, M, true)
                                       : linear_ws(w, M);
}

size_t ht::linear_path_ws_min(const ht_packed_weight *w, int64_t M, int32_t path) {
    return path == HT_PATH_GEMM ? gemm_ws_min(w, M) : path_ws(w, M, path);
}

extern "C" ht_status ht_linear_workspace(const ht_packed_weight *w, int64_t M, int32_t path, size_t *bytes) {
    if (!bytes || !desc_ok(w)) return HT_EINVAL;
    if (M <= 0) return HT_ESHAPE;
    if (!path_ok(path)) return HT_EINVAL;
    if (path == HT_PATH_AUTO) path = auto_linear_path(w, M);
    if (path == HT_PATH_GEMV_MFMA && !dec_ok(w)) return HT_EINVAL;
    if ((path == HT_PATH_GEMM_I8 || path == HT_PATH_W8A8) && !i8_ok(w)) return HT_EINVAL;
    *bytes = path_ws(w, M, path);
    return HT_OK;
}

extern "C" ht_status ht_linear_forward(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx,
                                       float *y, int64_t ldy, int32_t act, int32_t path, void *ws,
                                       size_t ws_bytes, ht_stream stream) {
    if (!desc_ok(w) || !x || !y) return HT_EINVAL;
    if (act != HT_ACT_NONE && act != HT_ACT_RELU) return HT_EINVAL;
    if (!path_ok(path)) return HT_EINVAL;
    if (M <= 0 || ldx < w->K || ldy < w->N) return HT_ESHAPE;
    if (!al16(x) || !al16(y) || (ldx % 8) || !al16(w->base)) return HT_EALIGN;
    if (path == HT_PATH_AUTO) path = auto_linear_path(w, M);
    if (path == HT_PATH_GEMV_MFMA && !dec_ok(w)) return HT_EINVAL;
    if ((path == HT_PATH_GEMM_I8 || path == HT_PATH_W8A8) && !i8_ok(w)) return HT_EINVAL;
    const size_t need = linear_path_ws_min(w, M, path);
    if (need && (!ws || ws_bytes < need)) return HT_ESMALL;
    if (ws && !al16(ws)) return HT_EALIGN;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (path == HT_PATH_GEMM) return run_gemm(w, x, M, ldx, y, nullptr, ldy, act, ws, ws ? ws_bytes : 0, s);
    if (path == HT_PATH_GEMV_MFMA) return run_dec(w, x, M, ldx, y, nullptr, ldy, act, ws, s);
    if (path == HT_PATH_GEMM_I8) return run_gemm_i8(w, x, M, ldx, y, nullptr, ldy, act, ws, s);
    if (path == HT_PATH_W8A8) return run_gemm_i8(w, x, M, ldx, y, nullptr, ldy, act, ws, s, true);
    return run_linear(w, x, M, ldx, y, nullptr, ldy, act, ws, s);
}

extern "C" ht_status ht_linear_backward_workspace(const ht_packed_weight *w, int64_t M, size_t *bytes) {
    if (!bytes || !desc_ok(w)) return HT_EINVAL;
    if (M <= 0) return HT_ESHAPE;
    if (!bwd_ok(w)) return HT_EINVAL;
    *bytes = bwd_gemm_takes(w, M) ? bwd_gemm_ws(w, M) : bwd_ws(w, M);
    return HT_OK;
}

extern "C" ht_status ht_linear_backward_data(const ht_packed_weight *w, const float *dy, int64_t M, int64_t lddy,
                                             float *dx, int64_t lddx, void *ws, size_t ws_bytes, ht_stream stream) {
    if (!desc_ok(w) || !dy || !dx) return HT_EINVAL;
    if (!bwd_ok(w)) return HT_EINVAL;
    if (M <= 0 || lddy < w->N || lddx < w->K) return HT_ESHAPE;
    if (!al16(dy) || !al16(dx) || !al16(w->base)) return HT_EALIGN;
    const bool mfma = bwd_gemm_takes(w, M);
    const size_t need = mfma ? bwd_gemm_ws(w, M) : bwd_ws(w, M);
    if (need && (!ws || ws_bytes < need)) return HT_ESMALL;
    if (ws && !al16(ws)) return HT_EALIGN;
    if (mfma) return run_bwd_gemm(w, dy, M, lddy, dx, lddx, ws, reinterpret_cast<hipStream_t>(stream));
    return run_bwd(w, dy, M, lddy, dx, lddx, ws, reinterpret_cast<hipStream_t>(stream));
}
