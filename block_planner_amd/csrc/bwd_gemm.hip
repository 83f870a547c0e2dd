// bwd_gemm.hip -- the input gradient of the linear on the matrix cores, for
// training-sized batches: dX[m, k] = sum over n of dY[m, n] * w_hat[n, k]
// (HyperTensor 1.0.1 page, "Key Features": training support; "Design
// Philosophy": custom backward kernels), read from the packed buffers.
//
// Both operands enter bf16 MFMAs (v_mfma_f32_16x16x32_bf16) as two planes,
// hi = the fp32 value with the low 16 bits cleared and lo = bf16(v - hi):
// dY as given, w_hat as s * q rounded to fp32 for integer blocks and as the
// value for float blocks.  Three products per pair of planes (hi.hi, hi.lo,
// lo.hi; lo.lo is below fp32 rounding of the sum) go straight into fp32
// accumulators, so every term carries 16 significant bits of each factor.
// A non-finite weight entry makes its lo plane NaN (Inf - Inf), so its dX
// columns are NaN; fp32-subnormal factors keep their bits down to 2^-133.
//
// A workgroup owns a BM x 128 tile of dX (BM = 128, 64 or 32 rows of dY;
// 128 columns = two K-blocks) and walks n one 64-row step (four row tiles of
// 16) at a time, over the row tiles of its split.  Per step the step's 128
// weight blocks (4 row tiles x 2 K-blocks x 16 rows) are dequantised by four
// producer waves, two threads per block, and written transposed into LDS as
// [k][n] planes (the MFMA operand holds eight consecutive n of one k); four
// MFMA waves load dY's BM x 64 fp32 tile of the next step into registers,
// split it into [m][n] planes in LDS, and multiply, each on a (BM/2) x 64
// quarter.  Two LDS stages of each; one barrier per step that waits only for
// LDS operations.  With several splits of n the per-split tiles go to the
// workspace and the split reduction adds them in split order.
#include "gemv_common.h"
#include "linear_host.h"

namespace ht {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kBgBK = 128;          // dX columns per workgroup (two K-blocks)
constexpr uint32_t kBgThreads = 512;     // 4 MFMA waves + 4 producer waves
constexpr uint32_t kBgRow = 72;          // bf16 per LDS row: 64 + 8 of padding
constexpr uint32_t kBgTilesPerStep = 4;  // row tiles of 16 per step (64 rows of W)

struct BgArgs {
    LayerDev w;
    const float *dy;
    int64_t lddy;
    float *dx;            // [M][lddx] with one split, else nullptr
    int64_t lddx;
    float *partial;       // [S][M][K] with several splits
    uint32_t M, MT, KT;   // rows of dY, row tiles of dX, column tiles of dX
    uint32_t TPS;         // row tiles of W per split (a multiple of 4)
    uint32_t vec;         // lddy % 4 == 0: dY rows read as float4
    uint32_t nbytes;      // packed buffer size (below 4 GiB: 32-bit offsets)
};

template <int MI>
struct BgStage {
    uint16_t dyh[32 * MI][kBgRow], dyl[32 * MI][kBgRow];   // [m][n]
    uint16_t wth[kBgBK][kBgRow], wtl[kBgBK][kBgRow];       // [k][n]
};

// What one producer thread loads for one step: half `h` of its block.
struct BgLoad {
    uint4 p[8];
    float sc;
    uint32_t id2, hi16;
    int f;             // 5: no block (row past N, or tile past the split)
};

__device__ __forceinline__ void bg_lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// hi / lo planes of an fp32 value: hi = upper half (truncation), lo =
// bf16_rne(v - hi); returned as the two bf16 bit patterns.
__device__ __forceinline__ void bg_split(float v, uint16_t &hi, uint16_t &lo) {
    const uint32_t u = __float_as_uint(v);
    hi = uint16_t(u >> 16);
    const float r = v - __uint_as_float(u & 0xffff0000u);
    lo = __builtin_bit_cast(uint16_t, (__bf16)r);
}

// Workgroup (mt, kt, split): rows [BM*mt, +BM) of dY, columns [128*kt, +128)
// of dX, row tiles [TPS*split, +TPS) of W.  MFMA wave c owns rows
// [16*MI*(c>>1), +16*MI) and columns [64*(c&1), +64) of the tile.
template <int MI>
__global__ __launch_bounds__(kBgThreads) void bwd_gemm_kernel(BgArgs a) {
    constexpr uint32_t BM = 32 * MI;
    __shared__ __align__(16) BgStage<MI> st0, st1;

    const LayerDev &w = a.w;
    const uint32_t tid = threadIdx.x, lane = tid & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t per_split = a.MT * a.KT;
    const uint32_t zs = blockIdx.x / per_split, rem = blockIdx.x - zs * per_split;
    const uint32_t mt = rem / a.KT, kt = rem - mt * a.KT;
    const uint32_t m0 = mt * BM, kb0 = 2 * kt;                  // first K-block of the tile
    const uint32_t t0 = zs * a.TPS, t1 = min(w.T, t0 + a.TPS);  // this split's row tiles (non-empty)
    const uint32_t nsteps = (t1 - t0 + kBgTilesPerStep - 1) / kBgTilesPerStep;

    if (wave < 4) {
        // ================= MFMA waves =================
        const uint32_t c = wave, wr = c >> 1, wc = c & 1;
        const uint32_t lr = lane & 15, lq = lane >> 4;
        f32x4 acc[MI][4];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // dY of step t: rows [m0, +BM), columns n = 16*t0 + 64 t + [0, 64),
        // zero past M and N; thread tc (0..255) reads float4 u = tc + 256 r
        // (row u / 16, columns 4 (u % 16) ..): BM / 16 of them.
        constexpr int NV = BM / 16;
        const uint32_t tc = tid;
        auto dy_load = [&](uint32_t t, float4 (&v)[NV]) {
            const uint32_t nb = 16u * t0 + 64u * t;
#pragma unroll
            for (int r = 0; r < NV; ++r) {
                const uint32_t u = tc + 256u * uint32_t(r), row = u >> 4, col = nb + 4u * (u & 15u);
                const uint32_t m = m0 + row;
                float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
                if (m < a.M && t < nsteps) {
                    const float *p = a.dy + int64_t(m) * a.lddy + col;
                    if (a.vec && col + 3u < w.N) {
                        q = *reinterpret_cast<const float4 *>(p);
                    } else {
                        q.x = col < w.N ? p[0] : 0.f;
                        q.y = col + 1u < w.N ? p[1] : 0.f;
                        q.z = col + 2u < w.N ? p[2] : 0.f;
                        q.w = col + 3u < w.N ? p[3] : 0.f;
                    }
                }
                v[r] = q;
            }
        };
        auto dy_store = [&](const float4 (&v)[NV], BgStage<MI> &s) {
#pragma unroll
            for (int r = 0; r < NV; ++r) {
                const uint32_t u = tc + 256u * uint32_t(r), row = u >> 4, c4 = 4u * (u & 15u);
                uint16_t h0, h1, h2, h3, l0, l1, l2, l3;
                bg_split(v[r].x, h0, l0);
                bg_split(v[r].y, h1, l1);
                bg_split(v[r].z, h2, l2);
                bg_split(v[r].w, h3, l3);
                *reinterpret_cast<uint2 *>(&s.dyh[row][c4]) =
                    make_uint2(uint32_t(h0) | (uint32_t(h1) << 16), uint32_t(h2) | (uint32_t(h3) << 16));
                *reinterpret_cast<uint2 *>(&s.dyl[row][c4]) =
                    make_uint2(uint32_t(l0) | (uint32_t(l1) << 16), uint32_t(l2) | (uint32_t(l3) << 16));
            }
        };
        auto mfma_step = [&](const BgStage<MI> &s) {
            bf16x8 Bh[4][2], Bl[4][2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t col = 64 * wc + 16 * j + lr;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    Bh[j][h] = *reinterpret_cast<const bf16x8 *>(&s.wth[col][32 * h + 8 * lq]);
                    Bl[j][h] = *reinterpret_cast<const bf16x8 *>(&s.wtl[col][32 * h + 8 * lq]);
                }
            }
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const uint32_t row = 16 * MI * wr + 16 * i + lr;
                bf16x8 Ah[2], Al[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    Ah[h] = *reinterpret_cast<const bf16x8 *>(&s.dyh[row][32 * h + 8 * lq]);
                    Al[h] = *reinterpret_cast<const bf16x8 *>(&s.dyl[row][32 * h + 8 * lq]);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[h], Bh[j][h], acc[i][j], 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[h], Bl[j][h], acc[i][j], 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al[h], Bh[j][h], acc[i][j], 0, 0, 0);
                }
            }
        };

        float4 v[NV];
        dy_load(0, v);
        dy_store(v, st0);
        dy_load(1, v);
        bg_lds_barrier();                                  // stage 0 (dY and W) complete
        for (uint32_t t = 0; t < nsteps; ++t) {
            BgStage<MI> &cur = (t & 1) ? st1 : st0;
            BgStage<MI> &nxt = (t & 1) ? st0 : st1;
            mfma_step(cur);
            if (t + 1 < nsteps) dy_store(v, nxt);          // step t+1's dY (loaded during step t)
            if (t + 2 < nsteps) dy_load(t + 2, v);
            bg_lds_barrier();
        }

        // ---- output: lane holds column lr, rows 4*(lane/16) + e of each 16x16 tile ----
        const uint32_t K = w.KB * 64u;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t k = 128u * kt + 64u * wc + 16u * j + lr;
                if (k >= K) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t m = m0 + 16 * MI * wr + 16 * i + 4 * lq + e;
                    if (m >= a.M) continue;
                    if (a.partial) a.partial[(uint64_t(zs) * a.M + m) * K + k] = acc[i][j][e];
                    else a.dx[int64_t(m) * a.lddx + k] = acc[i][j][e];
                }
            }
        return;
    }

    // ================= producer waves =================
    // thread pt -> half h of slot bi of (row tile t0 + 4 step + tl, K-block
    // kb0 + kbl): the bi-th block of that tile's column, in format order
    const uint32_t pt = tid - 256, h = pt & 1, slot = pt >> 1;
    const uint32_t tl = slot >> 5, kbl = (slot >> 4) & 1u, bi = slot & 15u;
    const uint32_t kb = kb0 + kbl;
    const bool kok = kb < w.KB;
    const uint8_t *base = w.base;
    uint32_t opay[5], oids[5];
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        opay[f] = uint32_t(w.off_pay[f]);
        oids[f] = uint32_t(w.off_ids[f]);
    }
    const uint32_t osc0 = uint32_t(w.off_scale[0]), osc1 = uint32_t(w.off_scale[1]);
    const uint32_t okx = uint32_t(w.off_kbidx);

    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, int(a.nbytes), 0x00020000);
    constexpr uint32_t kOut = 0xFFFFFFF0u;   // a buffer offset past the end: reads zeros
    auto load_block = [&](uint32_t t) -> BgLoad {
        BgLoad q;
        const uint32_t tile = t0 + kBgTilesPerStep * t + tl;
        const bool ok = kok && tile < t1 && t < nsteps;
        const uint32_t ix = ok ? tile * w.KB + kb : 0u;
        // the slot's format and block: c[f] <= bi < c[f+1] over the prefix
        // sums of the block counts in format order (the ten kbidx words
        // loaded at once, then compares: one round trip)
        uint32_t ka[5], kn[5];
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            const uint32_t e = uint32_t(g) * w.nk + ix;
            ka[g] = __builtin_amdgcn_raw_buffer_load_b32(rs, okx + 4u * e, 0, 0);
            kn[g] = __builtin_amdgcn_raw_buffer_load_b32(rs, okx + 4u * (e + 1u), 0, 0);
        }
        uint32_t c = 0, f = 0, cf = 0, kaf = 0;
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            const uint32_t cnt = kn[g] - ka[g];
            f += (bi >= c + cnt) ? 1u : 0u;           // the slot lies beyond format g
            cf = (f == uint32_t(g)) ? c : cf;
            kaf = (f == uint32_t(g)) ? ka[g] : kaf;
            c += cnt;
        }
        if (!ok) f = 5;
        const uint32_t blk = kaf + (bi - cf);
        uint32_t po = kOut, io = kOut, so = kOut, nl = 0;
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            if (f == uint32_t(g)) {
                po = opay[g] + blk * uint32_t(pay_bytes(g)) + h * uint32_t(pay_bytes(g) / 2);
                io = oids[g] + ((2u * blk) & ~3u);
                so = g == 0 ? osc0 + 4u * blk : g == 1 ? osc1 + 4u * blk : kOut;
                nl = uint32_t(pay_bytes(g) / 32);   // 16-byte pieces of this half
            }
        }
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, j < nl ? po + 16u * j : kOut, 0, 0);
            q.p[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
        q.id2 = __builtin_amdgcn_raw_buffer_load_b32(rs, io, 0, 0);
        q.hi16 = blk & 1u;
        q.sc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, so, 0, 0));
        q.f = int(f);
        return q;
    };

    // Dequantise the half block to fp32 (s * q for integers) and write its
    // hi / lo planes transposed: entry e of row r goes to [k][n] =
    // [64 kbl + 32 h + e][16 tl + r].  Rows without a block write zeros.
    auto store_block = [&](const BgLoad &b, BgStage<MI> &s) {
        const uint32_t id = b.hi16 ? b.id2 >> 16 : b.id2;
        const uint32_t n = 16u * tl + (b.f < 5 ? (id & 15u) : bi);
        const uint32_t u[32] = {b.p[0].x, b.p[0].y, b.p[0].z, b.p[0].w, b.p[1].x, b.p[1].y, b.p[1].z, b.p[1].w,
                                b.p[2].x, b.p[2].y, b.p[2].z, b.p[2].w, b.p[3].x, b.p[3].y, b.p[3].z, b.p[3].w,
                                b.p[4].x, b.p[4].y, b.p[4].z, b.p[4].w, b.p[5].x, b.p[5].y, b.p[5].z, b.p[5].w,
                                b.p[6].x, b.p[6].y, b.p[6].z, b.p[6].w, b.p[7].x, b.p[7].y, b.p[7].z, b.p[7].w};
        float wv[32];
        const float sc = b.sc;
        switch (b.f) {
        case 0:
            // byte i of the half's first 8 holds entries i (low nibble) and
            // 16+i (high), byte 8+i entries 8+i and 24+i (the layout's order)
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t wd = u[2 * q2 + (i >> 2)], sh = 8 * (i & 3);
                    wv[8 * q2 + i] = sc * float(int32_t(wd << (28u - sh)) >> 28);
                    wv[16 + 8 * q2 + i] = sc * float(int32_t(wd << (24u - sh)) >> 28);
                }
            break;
        case 1:
#pragma unroll
            for (int i = 0; i < 32; ++i) wv[i] = sc * float(int8_t(u[i >> 2] >> (8 * (i & 3))));
            break;
        case 2:
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                wv[2 * i] = __uint_as_float(u[i] << 16);
                wv[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
            }
            break;
        case 3:
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                wv[2 * i] = float(__builtin_bit_cast(_Float16, uint16_t(u[i])));
                wv[2 * i + 1] = float(__builtin_bit_cast(_Float16, uint16_t(u[i] >> 16)));
            }
            break;
        case 4:
#pragma unroll
            for (int i = 0; i < 32; ++i) wv[i] = __uint_as_float(u[i]);
            break;
        default:
#pragma unroll
            for (int i = 0; i < 32; ++i) wv[i] = 0.0f;
            break;
        }
        const uint32_t k0 = 64u * kbl + 32u * h;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            uint16_t hi, lo;
            bg_split(wv[e], hi, lo);
            s.wth[k0 + e][n] = hi;
            s.wtl[k0 + e][n] = lo;
        }
    };

    BgLoad QA, QB;
    QB = load_block(0);
    QA = load_block(1);
    store_block(QB, st0);
    bg_lds_barrier();
    // qc: the loads of step t+1; qn receives those of step t+2
    auto step = [&](uint32_t t, BgLoad &qc, BgLoad &qn, BgStage<MI> &dst) {
        qn = load_block(t + 2);
        if (t + 1 < nsteps) store_block(qc, dst);
        bg_lds_barrier();
    };
    for (uint32_t t = 0; t < nsteps; t += 2) {
        step(t, QA, QB, st1);
        if (t + 1 < nsteps) step(t + 1, QB, QA, st0);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

constexpr uint64_t kBgTarget = 256;   // compute units (one workgroup each)

uint32_t bg_bm(int64_t M) { return M >= 128 ? 128u : M >= 64 ? 64u : 32u; }

// Row tiles of W per split: all of them when the dX tiles fill the chip,
// else enough splits for about one workgroup per compute unit, each at least
// 8 steps (32 row tiles) long.
uint32_t bg_tps(const ht_packed_weight *w, int64_t M) {
    const uint64_t T = uint64_t(w->n_tiles);
    const uint64_t tiles = uint64_t((M + bg_bm(M) - 1) / bg_bm(M)) * uint64_t((w->K + kBgBK - 1) / kBgBK);
    uint64_t S = tiles * 4 >= kBgTarget * 3 ? 1 : (kBgTarget + tiles - 1) / tiles;
    const uint64_t smax = (T + 31) / 32;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    uint64_t tps = (T + S - 1) / S;
    tps = (tps + kBgTilesPerStep - 1) / kBgTilesPerStep * kBgTilesPerStep;
    return uint32_t(tps);
}

uint32_t bg_splits(const ht_packed_weight *w, int64_t M) {
    const uint32_t tps = bg_tps(w, M);
    return uint32_t((uint64_t(w->n_tiles) + tps - 1) / tps);
}

template <int MI>
void launch_bg(const BgArgs &a, uint32_t S, hipStream_t s) {
    hipLaunchKernelGGL(bwd_gemm_kernel<MI>, dim3(a.MT * a.KT * S), dim3(kBgThreads), 0, s, a);
}

}  // namespace

size_t bwd_gemm_ws(const ht_packed_weight *w, int64_t M) {
    const uint32_t S = bg_splits(w, M);
    return S > 1 ? size_t(S) * size_t(M) * size_t(w->K) * sizeof(float) : 0;
}

ht_status run_bwd_gemm(const ht_packed_weight *w, const float *dy, int64_t M, int64_t lddy, float *dx,
                       int64_t lddx, void *ws, hipStream_t s) {
    if (M > 0x3FFFFFFF) return HT_ESHAPE;
    BgArgs a;
    a.w = layer_dev(w);
    a.dy = dy;
    a.lddy = lddy;
    a.lddx = lddx;
    a.M = uint32_t(M);
    const uint32_t BM = bg_bm(M);
    a.MT = uint32_t((M + BM - 1) / BM);
    a.KT = uint32_t((w->K + kBgBK - 1) / kBgBK);
    a.TPS = bg_tps(w, M);
    a.vec = (lddy % 4 == 0) ? 1u : 0u;
    a.nbytes = uint32_t(w->bytes);
    const uint32_t S = bg_splits(w, M);
    a.dx = S > 1 ? nullptr : dx;
    a.partial = S > 1 ? static_cast<float *>(ws) : nullptr;
    switch (BM) {
    case 128: launch_bg<4>(a, S, s); break;
    case 64: launch_bg<2>(a, S, s); break;
    default: launch_bg<1>(a, S, s); break;
    }
    HT_LAUNCH_CHECK();
    if (S > 1)
        return launch_split_reduce(static_cast<const float *>(ws), S, uint32_t(M), uint32_t(w->K), dx, nullptr, lddx,
                                   HT_ACT_NONE, s);
    return HT_OK;
}


// ---------------------------------------------------------------------------
// The weight gradient under the straight-through estimator on the matrix
// cores, for training-sized batches: dW[n, k] = sum over m of dY[m, n] *
// x[m, k] (HyperTensor 1.0.1 page, "Design Philosophy": STE for the backward
// pass).  dY enters as hi + lo bf16 planes (16 significant bits), x as the
// bf16 it is (exact): two products per pair.  A workgroup of four waves
// owns a 128 x 128 tile of dW (wave c: rows [64 (c>>1), +64), columns
// [64 (c&1), +64)) and walks m in steps of 64 rows: the next step's dY and
// x are loaded into registers while the current step multiplies, then
// written transposed into LDS as [n][m] and [k][m] planes (the MFMA operand
// holds eight consecutive m), eight rows of one column per 16-byte write.  Fixed summation
// order: bitwise reproducible.
// ---------------------------------------------------------------------------
constexpr uint32_t kDgTile = 128;
constexpr uint32_t kDgThreads = 256;

struct DgArgs {
    const float *dy;
    int64_t lddy;
    const uint16_t *x;
    int64_t ldx;
    float *dw;
    int64_t lddw;
    uint32_t M, N, K, KT;
    uint32_t nby, kby;   // bytes of a row of dY (4 N) and of x (2 K)
    uint32_t vec;        // lddy and N even: dY read as float2 (a pair is all in or all out)
    int accumulate;
};

struct DgStage {
    uint16_t dyh[kDgTile][kBgRow], dyl[kDgTile][kBgRow];   // [n][m]
    uint16_t xt[kDgTile][kBgRow];                           // [k][m]
};

__global__ __launch_bounds__(kDgThreads) void dw_gemm_kernel(DgArgs a) {
    __shared__ __align__(16) DgStage st0, st1;
    const uint32_t tid = threadIdx.x, lane = tid & 63;
    const uint32_t c = __builtin_amdgcn_readfirstlane(tid >> 6), wr = c >> 1, wc = c & 1;
    const uint32_t nt = blockIdx.x / a.KT, kt = blockIdx.x - nt * a.KT;
    const uint32_t n0 = kDgTile * nt, k0 = kDgTile * kt;
    const uint32_t nsteps = (a.M + 63u) / 64u;
    const uint32_t lr = lane & 15, lq = lane >> 4;

    // thread -> columns 2 cp, 2 cp + 1 of the tile (cp = tid % 64; n for dY,
    // k for x) and rows [16 rg, +16) of the step (rg = the wave): 16 loads of
    // two adjacent columns each (a wave covers 512 / 256 contiguous bytes of
    // a row), written per column as two 8-row runs (16-byte LDS writes).
    // Each row is a buffer of its own (N fp32 of dY, K bf16 of x; none past
    // M), so columns and rows out of range read zeros with no branch.
    const uint32_t cp = lane, rg = c;
    struct Regs {
        float2 d[16];
        uint32_t xv[16];
    };
    auto load = [&](uint32_t t, Regs &R) {
        const uint32_t vn = 8u * cp, vk = 4u * cp;   // byte offsets of the lane's pair in its row
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t m = 64u * t + 16u * rg + uint32_t(r);
            const bool in = m < a.M;
            const int64_t mr = in ? int64_t(m) : 0;
            const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a.dy + mr * a.lddy + n0), 0, in ? int(a.nby - 4u * n0) : 0, 0x00020000);
            const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a.x + mr * a.ldx + k0), 0, in ? int(a.kby - 2u * k0) : 0, 0x00020000);
            if (a.vec) {
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rd, vn, 0, 0);
                R.d[r] = make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
            } else {
                R.d[r] = make_float2(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, vn, 0, 0)),
                                     __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, vn + 4u, 0, 0)));
            }
            R.xv[r] = __builtin_amdgcn_raw_buffer_load_b32(rx, vk, 0, 0);   // K % 4 == 0: a pair is all in or all out
        }
    };
    auto store = [&](const Regs &R, DgStage &s) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const uint32_t col = 2u * cp + uint32_t(cc);
#pragma unroll
            for (int o = 0; o < 2; ++o) {
                uint32_t hw[4], lw[4], xw[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r0 = 8 * o + 2 * q, r1 = r0 + 1;
                    uint16_t h0, l0, h1, l1;
                    bg_split(cc ? R.d[r0].y : R.d[r0].x, h0, l0);
                    bg_split(cc ? R.d[r1].y : R.d[r1].x, h1, l1);
                    hw[q] = uint32_t(h0) | (uint32_t(h1) << 16);
                    lw[q] = uint32_t(l0) | (uint32_t(l1) << 16);
                    const uint32_t a0 = cc ? R.xv[r0] >> 16 : R.xv[r0] & 0xFFFFu;
                    const uint32_t a1 = cc ? R.xv[r1] >> 16 : R.xv[r1] & 0xFFFFu;
                    xw[q] = a0 | (a1 << 16);
                }
                const uint32_t m8 = 16u * rg + 8u * uint32_t(o);
                *reinterpret_cast<uint4 *>(&s.dyh[col][m8]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                *reinterpret_cast<uint4 *>(&s.dyl[col][m8]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
                *reinterpret_cast<uint4 *>(&s.xt[col][m8]) = make_uint4(xw[0], xw[1], xw[2], xw[3]);
            }
        }
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mfma_step = [&](const DgStage &s) {
        bf16x8 Bx[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                Bx[j][h] = *reinterpret_cast<const bf16x8 *>(&s.xt[64 * wc + 16 * j + lr][32 * h + 8 * lq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t row = 64 * wr + 16 * i + lr;
            bf16x8 Ah[2], Al[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                Ah[h] = *reinterpret_cast<const bf16x8 *>(&s.dyh[row][32 * h + 8 * lq]);
                Al[h] = *reinterpret_cast<const bf16x8 *>(&s.dyl[row][32 * h + 8 * lq]);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah[h], Bx[j][h], acc[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al[h], Bx[j][h], acc[i][j], 0, 0, 0);
            }
        }
    };

    Regs R;
    load(0, R);
    store(R, st0);
    load(1, R);
    bg_lds_barrier();
    for (uint32_t t = 0; t < nsteps; ++t) {
        DgStage &cur = (t & 1) ? st1 : st0;
        DgStage &nxt = (t & 1) ? st0 : st1;
        mfma_step(cur);
        if (t + 1 < nsteps) store(R, nxt);
        if (t + 2 < nsteps) load(t + 2, R);
        bg_lds_barrier();
    }

    // ---- output: lane holds column lr (k), rows 4*(lane/16) + e (n) of each 16x16 tile ----
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t k = k0 + 64u * wc + 16u * j + lr;
            if (k >= a.K) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t n = n0 + 64u * wr + 16u * i + 4u * lq + e;
                if (n >= a.N) continue;
                float *p = a.dw + int64_t(n) * a.lddw + k;
                *p = a.accumulate ? *p + acc[i][j][e] : acc[i][j][e];
            }
        }
}

ht_status run_dw_gemm(const float *dy, int64_t M, int64_t lddy, const uint16_t *x, int64_t ldx, int64_t N,
                      int64_t K, float *dw, int64_t lddw, int accumulate, hipStream_t s) {
    DgArgs a;
    a.dy = dy;
    a.lddy = lddy;
    a.x = x;
    a.ldx = ldx;
    a.dw = dw;
    a.lddw = lddw;
    a.M = uint32_t(M);
    a.N = uint32_t(N);
    a.K = uint32_t(K);
    a.KT = uint32_t((K + kDgTile - 1) / kDgTile);
    a.nby = uint32_t(4 * N);
    a.kby = uint32_t(2 * K);
    a.vec = (lddy % 2 == 0 && N % 2 == 0) ? 1u : 0u;
    a.accumulate = accumulate;
    const uint64_t grid = uint64_t((N + kDgTile - 1) / kDgTile) * a.KT;
    if (grid > 0x7FFFFFFFull) return HT_ESHAPE;
    hipLaunchKernelGGL(dw_gemm_kernel, dim3(uint32_t(grid)), dim3(kDgThreads), 0, s, a);
    HT_LAUNCH_CHECK();
    return HT_OK;
}

}  // namespace ht
