// linear.hip -- fused mixed-format GEMV over the packed execution buffers
// (HyperTensor 1.0.1 page: "fused mixed-precision operators" run the plan;
// "Key Features": HyperLinear, a drop-in nn.Linear; "Usage Example": the
// BenchmarkMLP of HyperLinear + ReLU layers).
//
// y[m, n] = sum over n's K-blocks kb of  blk(m, n, kb), where
//   INT4 / INT8:  blk = s * (sum_i q_i * x[m, 64kb+i])   (scale after the partial)
//   BF16 / FP16 / FP32:  blk = sum_i w_i * x[m, 64kb+i]
// all in fp32.  Workgroup (row tile t, K-split s) owns rows [tR, tR+R) and
// K-blocks [kb0, kb1).  It stages x for those K-blocks in LDS as fp32, then
// its 4 wavefronts stream the tile's format segments in "chunks": 64 lanes x
// 16 bytes of one format (32 INT4 / 16 INT8 / 8 BF16 / 8 FP16 / 4 FP32
// blocks), so every chunk is one fully coalesced 1 KiB read and a wave never
// diverges on format.  Each lane dequantises its 16 bytes in registers and
// multiplies by x from LDS; the lanes of a block combine with DPP and one of
// them stores the block's partial into an LDS table P[m][r][kb].  After all
// chunks, each (m, r) sums its row of P in a fixed order (lane-strided, then
// a fixed butterfly), so the result is bitwise reproducible.  With several
// K-splits the per-split sums go to the workspace and a second kernel adds
// them in split order.
#include "ht_internal.h"

namespace ht {

struct LinArgs {
    const uint8_t *base;
    uint64_t off_kbidx, off_ids[5], off_scale[2], off_pay[5];
    uint32_t counts[5];
    uint32_t N, KB, R, lgR, nk;   // nk = T*KB + 1
    uint32_t S, KBs;              // K-splits and K-blocks per split
    const uint16_t *x;
    int64_t ldx;
    float *y;                     // fp32 output (S == 1) or nullptr
    uint16_t *ybf;                // bf16 output (S == 1) or nullptr
    int64_t ldy;
    float *partial;               // [S][M][N] when S > 1
    int act;
};

// blocks per chunk and lanes per block, by format
__host__ __device__ constexpr uint32_t bpc_of(int f) { return f == 0 ? 32u : f == 1 ? 16u : f == 4 ? 4u : 8u; }
__device__ constexpr int lpb_of(int f) { return f == 0 ? 2 : f == 1 ? 4 : f == 4 ? 16 : 8; }

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kUnroll = 8;   // chunks in flight per wave (a 16-row, 4096-wide tile is one batch)

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float fp16_lo(uint32_t v) { return float(__builtin_bit_cast(_Float16, uint16_t(v))); }
__device__ __forceinline__ float fp16_hi(uint32_t v) { return float(__builtin_bit_cast(_Float16, uint16_t(v >> 16))); }
__device__ __forceinline__ float s8(uint32_t v, int b) { return float(int8_t(v >> (8 * b))); }
// signed 4-bit field k (0..7) of v
__device__ __forceinline__ float s4(uint32_t v, int k) { return float(int32_t(v << (28 - 4 * k)) >> 28); }

template <int M>
__device__ __forceinline__ void store_partial(float *P, uint32_t pstride, uint32_t R, uint32_t r, uint32_t kbl,
                                              const float (&acc)[M], float scale, bool write) {
    if (write) {
#pragma unroll
        for (int m = 0; m < M; ++m) P[(m * R + r) * pstride + kbl] = acc[m] * scale;
    }
}

// One chunk of format F: `v` is this lane's 16 payload bytes.
template <int F, int M>
__device__ __forceinline__ void do_chunk(uint4 v, float scale, uint32_t id, bool valid, uint32_t lane,
                                         const float *xs, uint32_t xstride, float *P, uint32_t pstride,
                                         uint32_t kb0, uint32_t nkb, uint32_t R, uint32_t lgR) {
    constexpr int LPB = lpb_of(F);
    const uint32_t part = lane & (LPB - 1);
    uint32_t kbl = (id >> lgR) - kb0;
    const uint32_t r = id & (R - 1u);
    const bool ok = valid && kbl < nkb;
    kbl = ok ? kbl : 0u;
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.0f;

    if constexpr (F == 1) {          // INT8: 16 consecutive entries
        const float *xp = xs + kbl * 64 + part * 16;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float4 *x4 = reinterpret_cast<const float4 *>(xp + m * xstride);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 xv = x4[j];
                float a = acc[m];
                a = __builtin_fmaf(s8(wv[j], 0), xv.x, a);
                a = __builtin_fmaf(s8(wv[j], 1), xv.y, a);
                a = __builtin_fmaf(s8(wv[j], 2), xv.z, a);
                a = __builtin_fmaf(s8(wv[j], 3), xv.w, a);
                acc[m] = a;
            }
        }
    } else if constexpr (F == 0) {   // INT4: low nibbles entries [32p, 32p+16), high [32p+16, 32p+32)
        const float *xp = xs + kbl * 64 + part * 32;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float4 *xl = reinterpret_cast<const float4 *>(xp + m * xstride);
            const float4 *xh = reinterpret_cast<const float4 *>(xp + m * xstride + 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 a4 = xl[j], b4 = xh[j];
                float a = acc[m];
                a = __builtin_fmaf(s4(wv[j], 0), a4.x, a);
                a = __builtin_fmaf(s4(wv[j], 2), a4.y, a);
                a = __builtin_fmaf(s4(wv[j], 4), a4.z, a);
                a = __builtin_fmaf(s4(wv[j], 6), a4.w, a);
                a = __builtin_fmaf(s4(wv[j], 1), b4.x, a);
                a = __builtin_fmaf(s4(wv[j], 3), b4.y, a);
                a = __builtin_fmaf(s4(wv[j], 5), b4.z, a);
                a = __builtin_fmaf(s4(wv[j], 7), b4.w, a);
                acc[m] = a;
            }
        }
    } else if constexpr (F == 2 || F == 3) {   // BF16 / FP16: 8 consecutive entries
        const float *xp = xs + kbl * 64 + part * 8;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float4 *x4 = reinterpret_cast<const float4 *>(xp + m * xstride);
            const float4 xa = x4[0], xb = x4[1];
            const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
            float a = acc[m];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = F == 2 ? bf16_lo(wv[j]) : fp16_lo(wv[j]);
                const float hi = F == 2 ? bf16_hi(wv[j]) : fp16_hi(wv[j]);
                a = __builtin_fmaf(lo, xv[2 * j], a);
                a = __builtin_fmaf(hi, xv[2 * j + 1], a);
            }
            acc[m] = a;
        }
    } else {                          // FP32: 4 consecutive entries
        const float *xp = xs + kbl * 64 + part * 4;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float4 xv = *reinterpret_cast<const float4 *>(xp + m * xstride);
            float a = acc[m];
            a = __builtin_fmaf(__uint_as_float(wv[0]), xv.x, a);
            a = __builtin_fmaf(__uint_as_float(wv[1]), xv.y, a);
            a = __builtin_fmaf(__uint_as_float(wv[2]), xv.z, a);
            a = __builtin_fmaf(__uint_as_float(wv[3]), xv.w, a);
            acc[m] = a;
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = group_sum<LPB>(acc[m]);
    store_partial<M>(P, pstride, R, r, kbl, acc, scale, ok && part == 0);
}

template <int M>
__global__ __launch_bounds__(kThreads) void gemv_kernel(LinArgs a) {
    extern __shared__ float lds[];
    const uint32_t t = blockIdx.x, sidx = blockIdx.y;
    const uint32_t kb0 = sidx * a.KBs;
    if (kb0 >= a.KB) return;   // cannot happen: the host makes every split non-empty
    const uint32_t kb1 = min(a.KB, kb0 + a.KBs);
    const uint32_t nkb = kb1 - kb0;
    const uint32_t xstride = nkb * 64;
    const uint32_t pstride = nkb + 1;
    float *xs = lds;                       // [M][nkb*64]
    float *P = lds + M * xstride;          // [M][R][nkb+1]

    // this workgroup's range of each format's blocks (10 independent scalar
    // loads, then the per-format chunk counts)
    const uint32_t *kbidx = reinterpret_cast<const uint32_t *>(a.base + a.off_kbidx);
    const uint64_t col0 = uint64_t(t) * a.KB + kb0, col1 = uint64_t(t) * a.KB + kb1;
    uint32_t lo[5], hi[5], nch[5];
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        hi[f] = kbidx[uint64_t(f) * a.nk + col1];
        lo[f] = kbidx[uint64_t(f) * a.nk + col0];
    }
    uint32_t C = 0;
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        hi[f] = min(hi[f], a.counts[f]);
        lo[f] = min(lo[f], hi[f]);
        nch[f] = (hi[f] - lo[f] + bpc_of(f) - 1) / bpc_of(f);
        C += nch[f];
    }
    // per-format base pointers, resolved with static indices (kept in
    // scalar registers; a run-time index into the argument arrays would make
    // the compiler fetch them with vector loads and serialise every chunk)
    const uint8_t *pay_b[5];
    const uint16_t *id_b[5];
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        pay_b[f] = a.base + a.off_pay[f];
        id_b[f] = reinterpret_cast<const uint16_t *>(a.base + a.off_ids[f]);
    }
    const float *sc_b0 = reinterpret_cast<const float *>(a.base + a.off_scale[0]);
    const float *sc_b1 = reinterpret_cast<const float *>(a.base + a.off_scale[1]);

    const uint32_t lane = threadIdx.x & 63;
    // wave index as a scalar: everything derived from it (chunk -> format
    // decode, base pointers) then stays in scalar registers
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // one batch: kUnroll chunks per wave, 16 payload bytes + id + scale per lane
    uint4 pay[kUnroll];
    float sc[kUnroll];
    uint32_t ids[kUnroll];
    int fm[kUnroll];
    bool vl[kUnroll];
    // Loads are issued without branches (straight-line code lets the
    // compiler wait for the x loads alone): a slot without a chunk reads the
    // first 256 bytes of the buffer, and a lane past the end of its format's
    // range re-reads the range's last block; neither lane stores a result.
    const float *dummy_f = reinterpret_cast<const float *>(a.base);
    auto load_batch = [&](uint32_t c0) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t c = c0 + u * kWaves;
            // wave-uniform: format and chunk index within the format
            int f = 5;
            uint32_t ci = c, base_blk = 0, hb = 1, bpc = 1, pb = 0;
            const uint8_t *pp = a.base;
            const uint16_t *ip = reinterpret_cast<const uint16_t *>(a.base);
            const float *sp = dummy_f;
            int lg = 4;
#pragma unroll
            for (int g = 0; g < 5; ++g) {
                if (f == 5) {
                    if (ci < nch[g]) {
                        f = g;
                        base_blk = lo[g];
                        hb = hi[g];
                        bpc = bpc_of(g);
                        pb = uint32_t(pay_bytes(g));
                        pp = pay_b[g];
                        ip = id_b[g];
                        sp = g == 0 ? sc_b0 : g == 1 ? sc_b1 : dummy_f;
                        lg = g == 0 ? 1 : g == 1 ? 2 : g == 4 ? 4 : 3;
                    } else {
                        ci -= nch[g];
                    }
                }
            }
            uint32_t blk = base_blk + ci * bpc + (lane >> lg);
            vl[u] = f < 5 && blk < hb;
            blk = f < 5 ? min(blk, hb - 1u) : 0u;
            const uint32_t sblk = f < 2 ? blk : 0u;
            fm[u] = f;
            const u32x4 pv = ld_stream_u4(pp + uint64_t(blk) * pb + (lane & ((1u << lg) - 1u)) * 16u);
            pay[u] = make_uint4(pv.x, pv.y, pv.z, pv.w);
            ids[u] = ip[blk];
            const float sv = sp[sblk];
            sc[u] = f < 2 ? sv : 1.0f;   // float formats carry no scale
        }
    };

    // x for these K-blocks: at most two 16-byte loads per thread (the host
    // keeps M * nkb * 64 * 4 bytes of x within 64 KiB of LDS).  They are
    // issued before the weight loads, so converting them into LDS waits only
    // for themselves.
    const uint32_t per_row = nkb * 8;   // 8 bf16 per 16-byte load
    uint4 xr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t i = threadIdx.x + j * kThreads;
        if (i < M * per_row) {
            const uint32_t m = i / per_row, jj = i - m * per_row;
            xr[j] = *reinterpret_cast<const uint4 *>(a.x + int64_t(m) * a.ldx + kb0 * 64 + jj * 8);
        }
    }

    // the first batch of weights is in flight while x goes into LDS
    load_batch(wave);

#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t i = threadIdx.x + j * kThreads;
        if (i < M * per_row) {
            const uint32_t m = i / per_row, jj = i - m * per_row;
            const uint4 v = xr[j];
            float4 *d = reinterpret_cast<float4 *>(xs + m * xstride + jj * 8);
            d[0] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
            d[1] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
        }
    }
    __syncthreads();

    auto compute_batch = [&]() {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            switch (fm[u]) {
            case 0: do_chunk<0, M>(pay[u], sc[u], ids[u], vl[u], lane, xs, xstride, P, pstride, kb0, nkb, a.R, a.lgR); break;
            case 1: do_chunk<1, M>(pay[u], sc[u], ids[u], vl[u], lane, xs, xstride, P, pstride, kb0, nkb, a.R, a.lgR); break;
            case 2: do_chunk<2, M>(pay[u], sc[u], ids[u], vl[u], lane, xs, xstride, P, pstride, kb0, nkb, a.R, a.lgR); break;
            case 3: do_chunk<3, M>(pay[u], sc[u], ids[u], vl[u], lane, xs, xstride, P, pstride, kb0, nkb, a.R, a.lgR); break;
            case 4: do_chunk<4, M>(pay[u], sc[u], ids[u], vl[u], lane, xs, xstride, P, pstride, kb0, nkb, a.R, a.lgR); break;
            default: break;
            }
        }
    };
    // The first batch is consumed in straight-line code after its loads, so
    // each chunk waits only for its own data and the arithmetic on early
    // chunks overlaps the arrival of later ones.
    compute_batch();
    for (uint32_t c0 = wave + kWaves * kUnroll; c0 < C; c0 += kWaves * kUnroll) {
        load_batch(c0);
        compute_batch();
    }
    __syncthreads();

    // per (m, r): fixed-order sum of P[m][r][0 .. nkb)
    for (uint32_t pr = wave; pr < M * a.R; pr += kWaves) {
        const uint32_t m = pr / a.R, r = pr - m * a.R;
        const uint32_t n = t * a.R + r;
        float v = 0.0f;
        for (uint32_t k = lane; k < nkb; k += 64) v += P[(m * a.R + r) * pstride + k];
        v = group_sum<16>(v);
        v = v + __shfl_xor(v, 16);
        v = v + __shfl_xor(v, 32);
        if (lane == 0 && n < a.N) {
            if (a.S == 1) {
                if (a.act == HT_ACT_RELU) v = fmaxf(v, 0.0f);
                if (a.ybf) a.ybf[int64_t(m) * a.ldy + n] = f32_to_bf16_rne(v);
                else a.y[int64_t(m) * a.ldy + n] = v;
            } else {
                a.partial[(uint64_t(sidx) * M + m) * a.N + n] = v;
            }
        }
    }
}

// y[m, n] = act(sum over s in order of partial[s][m][n])
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *partial, uint32_t S, uint32_t M, uint32_t N,
                                                           float *y, uint16_t *ybf, int64_t ldy, int act) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= M * N) return;
    const uint32_t m = i / N, n = i - m * N;
    float v = 0.0f;
    for (uint32_t s = 0; s < S; ++s) v += partial[(uint64_t(s) * M + m) * N + n];
    if (act == HT_ACT_RELU) v = fmaxf(v, 0.0f);
    if (ybf) ybf[int64_t(m) * ldy + n] = f32_to_bf16_rne(v);
    else y[int64_t(m) * ldy + n] = v;
}

}  // namespace ht

using namespace ht;

namespace {

constexpr uint32_t kMaxLds = 64 * 1024;
constexpr int kMaxM = 8;   // rows per launch of the register path; larger M is tiled

uint32_t lds_bytes(uint32_t Mt, uint32_t nkb, uint32_t R) {
    return Mt * nkb * 64u * 4u + Mt * R * (nkb + 1u) * 4u;
}

// K-split choice: enough workgroups to cover the chip twice, LDS within 64 KiB.
uint32_t choose_splits(const ht_packed_weight *w, uint32_t Mt) {
    const uint32_t KB = uint32_t(w->K / kBlockK), T = uint32_t(w->n_tiles), R = uint32_t(w->row_tile);
    uint32_t S = 1;
    while (S < KB && (lds_bytes(Mt, (KB + S - 1) / S, R) > kMaxLds || (uint64_t(T) * S < 256 && (KB + S) / (S + 1) >= 8)))
        ++S;
    // every split non-empty: S = ceil(KB / KBs) with KBs = ceil(KB / S)
    const uint32_t KBs = (KB + S - 1) / S;
    return (KB + KBs - 1) / KBs;
}

bool desc_ok(const ht_packed_weight *w) {
    if (!w || !w->base || w->layout_version != HT_LAYOUT_VERSION) return false;
    if (w->N <= 0 || w->K <= 0 || w->K % kBlockK) return false;
    const int64_t R = w->row_tile;
    if (!(R == 1 || R == 2 || R == 4 || R == 8 || R == 16)) return false;
    if (w->n_tiles != (w->N + R - 1) / R) return false;
    return true;
}

int m_tile(int64_t M) { return int(M < kMaxM ? M : kMaxM); }

size_t linear_ws(const ht_packed_weight *w, int64_t M) {
    const int Mt = m_tile(M);
    const uint32_t S = choose_splits(w, uint32_t(Mt));
    return S > 1 ? size_t(S) * size_t(Mt) * size_t(w->N) * sizeof(float) : 0;
}

template <int M>
void launch_gemv(const LinArgs &a, uint32_t T, uint32_t lds, hipStream_t s) {
    hipLaunchKernelGGL(gemv_kernel<M>, dim3(T, a.S), dim3(kThreads), lds, s, a);
}

// One linear over rows [0, M) of x; out either fp32 y or bf16 ybf.
ht_status run_linear(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y,
                     uint16_t *ybf, int64_t ldy, int act, void *ws, hipStream_t s) {
    const uint32_t KB = uint32_t(w->K / kBlockK);
    const uint32_t T = uint32_t(w->n_tiles);
    LinArgs a;
    a.base = static_cast<const uint8_t *>(w->base);
    a.off_kbidx = w->off_kbidx;
    for (int f = 0; f < 5; ++f) {
        a.off_ids[f] = w->off_ids[f];
        a.off_pay[f] = w->off_payload[f];
        a.counts[f] = uint32_t(w->counts[f]);
    }
    a.off_scale[0] = w->off_scale[0];
    a.off_scale[1] = w->off_scale[1];
    a.N = uint32_t(w->N);
    a.KB = KB;
    a.R = uint32_t(w->row_tile);
    a.lgR = uint32_t(__builtin_ctzll(uint64_t(w->row_tile)));
    a.nk = T * KB + 1;
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
        const uint32_t lds = lds_bytes(uint32_t(Mt), a.KBs, a.R);
        LinArgs g = a;
        if (S > 1) { g.y = nullptr; g.ybf = nullptr; }
        switch (Mt) {
        case 1: launch_gemv<1>(g, T, lds, s); break;
        case 2: launch_gemv<2>(g, T, lds, s); break;
        case 3: launch_gemv<3>(g, T, lds, s); break;
        case 4: launch_gemv<4>(g, T, lds, s); break;
        case 5: launch_gemv<5>(g, T, lds, s); break;
        case 6: launch_gemv<6>(g, T, lds, s); break;
        case 7: launch_gemv<7>(g, T, lds, s); break;
        default: launch_gemv<8>(g, T, lds, s); break;
        }
        HT_LAUNCH_CHECK();
        if (S > 1) {
            const uint32_t tot = uint32_t(Mt) * a.N;
            hipLaunchKernelGGL(split_reduce_kernel, dim3((tot + 255) / 256), dim3(256), 0, s,
                               static_cast<const float *>(ws), S, uint32_t(Mt), a.N, a.y, a.ybf, ldy, act);
            HT_LAUNCH_CHECK();
        }
    }
    return HT_OK;
}

bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" ht_status ht_linear_workspace(const ht_packed_weight *w, int64_t M, int32_t path, size_t *bytes) {
    if (!bytes || !desc_ok(w)) return HT_EINVAL;
    if (M <= 0) return HT_ESHAPE;
    if (path != HT_PATH_AUTO && path != HT_PATH_GEMV) return HT_EINVAL;
    *bytes = linear_ws(w, M);
    return HT_OK;
}

extern "C" ht_status ht_linear_forward(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx,
                                       float *y, int64_t ldy, int32_t act, int32_t path, void *ws,
                                       size_t ws_bytes, ht_stream stream) {
    if (!desc_ok(w) || !x || !y) return HT_EINVAL;
    if (act != HT_ACT_NONE && act != HT_ACT_RELU) return HT_EINVAL;
    if (path != HT_PATH_AUTO && path != HT_PATH_GEMV) return HT_EINVAL;
    if (M <= 0 || ldx < w->K || ldy < w->N) return HT_ESHAPE;
    if (!al16(x) || !al16(y) || (ldx % 8) || !al16(w->base)) return HT_EALIGN;
    const size_t need = linear_ws(w, M);
    if (need && (!ws || ws_bytes < need)) return HT_ESMALL;
    if (ws && !al16(ws)) return HT_EALIGN;
    return run_linear(w, x, M, ldx, y, nullptr, ldy, act, ws, reinterpret_cast<hipStream_t>(stream));
}

extern "C" ht_status ht_mlp_workspace(const ht_packed_weight *const *layers, int32_t n_layers, int64_t M,
                                      size_t *bytes) {
    if (!layers || n_layers <= 0 || !bytes) return HT_EINVAL;
    if (M <= 0) return HT_ESHAPE;
    size_t part = 0, act = 0;
    for (int32_t l = 0; l < n_layers; ++l) {
        if (!desc_ok(layers[l])) return HT_EINVAL;
        if (l && layers[l]->K != layers[l - 1]->N) return HT_ESHAPE;
        size_t p = linear_ws(layers[l], M);
        part = p > part ? p : part;
        size_t h = align256(size_t(M) * size_t(layers[l]->N) * 2u);
        act = h > act ? h : act;
    }
    *bytes = align256(part) + 2 * act;
    return HT_OK;
}

extern "C" ht_status ht_mlp_forward(const ht_packed_weight *const *layers, int32_t n_layers, const uint16_t *x,
                                    int64_t M, int64_t ldx, float *y, int64_t ldy, uint16_t *act_dump, void *ws,
                                    size_t ws_bytes, ht_stream stream) {
    if (!layers || n_layers <= 0 || !x || !y) return HT_EINVAL;
    size_t need = 0;
    ht_status st = ht_mlp_workspace(layers, n_layers, M, &need);
    if (st != HT_OK) return st;
    if (ldx < layers[0]->K || ldy < layers[n_layers - 1]->N) return HT_ESHAPE;
    if (!ws || ws_bytes < need) return HT_ESMALL;
    if (!al16(x) || !al16(y) || !al16(ws) || (ldx % 8) || (act_dump && !al16(act_dump))) return HT_EALIGN;
    for (int32_t l = 0; l < n_layers; ++l)
        if (!al16(layers[l]->base)) return HT_EALIGN;
    if (act_dump)
        for (int32_t l = 0; l + 1 < n_layers; ++l)
            if ((size_t(M) * size_t(layers[l]->N) * 2u) % 16u) return HT_EALIGN;
    size_t part = 0, act = 0;
    for (int32_t l = 0; l < n_layers; ++l) {
        size_t p = linear_ws(layers[l], M);
        part = p > part ? p : part;
        size_t h = align256(size_t(M) * size_t(layers[l]->N) * 2u);
        act = h > act ? h : act;
    }
    uint8_t *wsb = static_cast<uint8_t *>(ws);
    void *partial = wsb;
    uint16_t *ping[2] = {reinterpret_cast<uint16_t *>(wsb + align256(part)),
                         reinterpret_cast<uint16_t *>(wsb + align256(part) + act)};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const uint16_t *in = x;
    int64_t ld_in = ldx;
    size_t dump_off = 0;
    for (int32_t l = 0; l < n_layers; ++l) {
        const ht_packed_weight *w = layers[l];
        if (l + 1 < n_layers) {
            uint16_t *out = act_dump ? act_dump + dump_off : ping[l & 1];
            dump_off += size_t(M) * size_t(w->N);
            st = run_linear(w, in, M, ld_in, nullptr, out, w->N, HT_ACT_RELU, partial, s);
            if (st != HT_OK) return st;
            in = out;
            ld_in = w->N;
        } else {
            st = run_linear(w, in, M, ld_in, y, nullptr, ldy, HT_ACT_RELU, partial, s);
            if (st != HT_OK) return st;
        }
    }
    return HT_OK;
}
