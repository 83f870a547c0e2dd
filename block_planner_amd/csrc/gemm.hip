// gemm.hip -- the mixed-format linear for many rows of x (prefill):
// y[m, n] = sum over K-blocks kb of  blk(m, n, kb)  with fp32 accumulation,
// where an integer block contributes s * (sum_i q_i * x[m, 64kb+i]) and a
// float block sum_i w_i * x[m, 64kb+i] (HyperTensor 1.0.1 page: "fused
// mixed-precision operators" run the plan; "Key Features": HyperLinear).
//
// A workgroup owns a 32*MS x 64 tile of y and walks K one 64-wide block at a
// time.  Per step it dequantises the tile's 64 weight blocks (one per output
// column) into LDS as bfloat16:
//   INT4 / INT8   the codes themselves (|q| <= 127 is exact in bfloat16);
//                 the block's scale multiplies the 64-term partial afterwards;
//   BF16          the values;
//   FP16 / FP32   two planes, hi = w with the low 16 bits cleared and
//                 lo = bf16(w - hi) (exact for FP16; 16 significant bits for
//                 FP32), scale 1; a non-finite entry gives a NaN column.
// The partial of each step comes from bf16 MFMAs (v_mfma_f32_16x16x32_bf16)
// with a fresh accumulator; the lo plane is multiplied only for 16-column
// groups that hold an FP16 or FP32 block in that step.  Then every output
// element adds scale[n] * partial[m, n] in fp32, in K order.
//
// Pipelining: two LDS stages.  While the MFMAs run on stage kb, the loads of
// step kb+1 (x tile and packed blocks) are in flight in registers; they are
// dequantised into the other stage after the MFMAs, then one barrier.
#include "gemv_common.h"
#include "linear_host.h"

namespace ht {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kGemmBN = 64;          // output columns (weight rows) per workgroup
constexpr uint32_t kGemmThreads = 256;    // 4 waves in a 2 x 2 arrangement
constexpr uint32_t kLdsRow = 72;          // bfloat16 per LDS row: 64 + 8 of padding

struct GemmArgs {
    LayerDev w;
    const uint16_t *x;
    int64_t ldx;
    float *y;                 // fp32 output, or
    uint16_t *ybf;            // bfloat16 output (round to nearest even), or
    float *partial;           // per-split partial sums [S][M][N] (no activation)
    int64_t ldy;
    uint32_t M;
    uint32_t KBs;             // K-blocks per split (blockIdx.z)
    int act;
};

// One pipeline stage in LDS.
template <int MS>
struct GemmStage {
    uint16_t xs[32 * MS][kLdsRow];     // x tile, bfloat16
    uint16_t whi[kGemmBN][kLdsRow];    // weight planes, bfloat16, row = output column
    uint16_t wlo[kGemmBN][kLdsRow];
    float scale[kGemmBN];
    uint32_t need_lo[4];               // per 16-column group
};

template <int MS>
constexpr uint32_t gemm_lds_bytes() { return 2u * uint32_t(sizeof(GemmStage<MS>)); }

// The packed block (or its absence) one thread dequantises in a step: block
// quarter `part` (16 of the 64 entries) of output column n.
struct BlockLoad {
    uint4 p[4];        // payload bytes of this quarter (8 / 16 / 32 / 32 / 64 bytes by format)
    float sc;
    uint32_t id2;      // the 4 bytes holding the block id (kb * R + r), as loaded
    uint32_t hi16;     // which half of id2 is the id
    int f;             // format, or 5 for "no block": the column is zero in this step
};

template <int MS>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs a) {
    extern __shared__ __align__(16) unsigned char gemm_lds[];
    GemmStage<MS> *stage = reinterpret_cast<GemmStage<MS> *>(gemm_lds);
    constexpr uint32_t BM = 32 * MS;
    const LayerDev &w = a.w;
    const uint32_t tid = threadIdx.x, lane = tid & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t wm = wave >> 1, wn = wave & 1;          // wave tile: rows [wm*16*MS, +16*MS), cols [wn*32, +32)
    const uint32_t n0 = blockIdx.x * kGemmBN, m0 = blockIdx.y * BM;
    const uint32_t KB = w.KB, R = w.R;
    const uint32_t kb0 = blockIdx.z * a.KBs, kb1 = min(KB, kb0 + a.KBs);   // this split's K-blocks (non-empty)

    // ---- dequantisation role: thread -> (column block gb, quarter part) ----
    const uint32_t gb = tid >> 2, part = tid & 3;
    const uint32_t tile = n0 / R + gb / R, bi = gb % R;    // tile of the column, block slot within it
    const bool tile_ok = tile < w.T;
    const uint32_t *kbidx = reinterpret_cast<const uint32_t *>(w.base + w.off_kbidx);
    // kbidx[f][tile*KB + kb] for the step about to be loaded (ka) and the one
    // after it (kn): the index loads run two steps ahead of their use, so a
    // step's block loads need one memory round trip, not two.
    auto kbidx_at = [&](uint32_t kb, uint32_t (&v)[5]) {
#pragma unroll
        for (int f = 0; f < 5; ++f)
            v[f] = tile_ok && kb <= KB ? kbidx[uint64_t(f) * w.nk + uint64_t(tile) * KB + kb] : 0u;
    };
    uint32_t ka[5], kn[5];
    kbidx_at(kb0, ka);
    kbidx_at(kb0 + 1, kn);

    auto load_block = [&](uint32_t kb) -> BlockLoad {
        BlockLoad b;
        b.f = 5;
        b.sc = 1.0f;
        uint32_t cum = 0, blk = 0;
#pragma unroll
        for (int f = 0; f < 5; ++f) {
            const uint32_t c = kn[f] - ka[f];
            if (b.f == 5 && bi < cum + c) {
                b.f = f;
                blk = ka[f] + (bi - cum);
            }
            cum += c;
        }
#pragma unroll
        for (int f = 0; f < 5; ++f) ka[f] = kn[f];
        kbidx_at(kb + 2, kn);
        // Branch-free loads (so no load waits for another): four 16-byte loads
        // at addresses chosen per format, repeating the last one where the
        // quarter is shorter; a missing block reads the buffer's first bytes.
        // INT4's 8-byte quarter p comes with its neighbour in a 16-byte load
        // at 16 * (p / 2); the dequantisation picks its half.
        const bool has = b.f < 5;
        const int f = has ? b.f : 0;
        uint64_t po = 0, io = 0, so = 0;
        uint32_t qb = 0, nl = 1;
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            if (f == g) {
                po = w.off_pay[g] + uint64_t(blk) * uint32_t(pay_bytes(g));
                io = w.off_ids[g] + ((2ull * blk) & ~3ull);
                so = g < 2 ? w.off_scale[g] + 4ull * blk : 0ull;
                qb = g == 0 ? 16u * (part >> 1) : uint32_t(pay_bytes(g) / 4) * part;
                nl = g < 2 ? 1u : g == 4 ? 4u : 2u;
            }
        }
        if (!has) po = io = so = 0;
        const uint8_t *pq = w.base + po + qb;
#pragma unroll
        for (uint32_t j = 0; j < 4; ++j) {
            const uint32_t jj = j < nl ? j : nl - 1u;
            b.p[j] = *reinterpret_cast<const uint4 *>(pq + 16u * jj);
        }
        b.id2 = *reinterpret_cast<const uint32_t *>(w.base + io);
        b.hi16 = blk & 1u;
        b.sc = *reinterpret_cast<const float *>(w.base + so);   // meaningful for INT4 / INT8 only
        return b;
    };

    // Dequantise into stage st: entries [16*part, 16*part + 16) of column gb
    // (INT4 quarters cover two runs of 8, see the nibble order of the layout).
    // Entries are produced as packed bfloat16 pairs: integers via an exact
    // fp32 conversion whose upper half is the bfloat16 (v_perm packs two),
    // floats as hi = upper half (truncation) and lo = bf16_rne(w - hi)
    // (v_cvt_pk_bf16_f32).  A non-finite FP16/FP32 entry makes lo NaN, so its
    // output column is NaN.
    auto store_block = [&](const BlockLoad &b, GemmStage<MS> &st) {
        const uint32_t id = b.hi16 ? b.id2 >> 16 : b.id2;
        const uint32_t col = (gb / R) * R + (b.f < 5 ? (id & (R - 1u)) : bi);   // column within the workgroup's 64
        const bool flt = b.f == 3 || b.f == 4;
        const bool any_lo = __any(flt);                         // this wave's 16 columns need the lo plane
        const uint32_t u[16] = {b.p[0].x, b.p[0].y, b.p[0].z, b.p[0].w, b.p[1].x, b.p[1].y, b.p[1].z, b.p[1].w,
                                b.p[2].x, b.p[2].y, b.p[2].z, b.p[2].w, b.p[3].x, b.p[3].y, b.p[3].z, b.p[3].w};
        uint32_t hp[8], lp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) lp[i] = 0u;
        uint32_t k0 = 16 * part, k1 = k0 + 8;                  // where the two runs of 8 go
        auto nib = [](uint32_t v, uint32_t at) { return int32_t(v << (28u - at)) >> 28; };   // signed 4-bit field
        auto pair_hi = [](float f0, float f1) {                 // upper halves of two fp32 -> one word
            return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        };
        auto pair_lo = [](float f0, float f1) {                 // bf16_rne(f - trunc(f)) of two fp32
            const float r0 = f0 - __uint_as_float(__float_as_uint(f0) & 0xffff0000u);
            const float r1 = f1 - __uint_as_float(__float_as_uint(f1) & 0xffff0000u);
            const bf16x2 v = {(__bf16)r0, (__bf16)r1};
            return __builtin_bit_cast(uint32_t, v);
        };
        switch (b.f) {
        case 0:
            // bytes 8p .. 8p+7 (words 2*(p&1), +1 of the 16-byte load): low nibble
            // -> entry 32*(p/2) + 8*(p%2) + i, high nibble -> that + 16
            k0 = 32 * (part >> 1) + 8 * (part & 1);
            k1 = k0 + 16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t wd = (part & 1) ? u[2 + (i >> 1)] : u[i >> 1], sh = 16 * (i & 1);
                hp[i] = pair_hi(float(nib(wd, sh)), float(nib(wd, sh + 8)));
                hp[4 + i] = pair_hi(float(nib(wd, sh + 4)), float(nib(wd, sh + 12)));
            }
            break;
        case 1:
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t wd = u[i >> 1], sh = 16 * (i & 1);
                hp[i] = pair_hi(float(int8_t(wd >> sh)), float(int8_t(wd >> (sh + 8))));
            }
            break;
        case 2:
#pragma unroll
            for (int i = 0; i < 8; ++i) hp[i] = u[i];
            break;
        case 3:
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float f0 = float(__builtin_bit_cast(_Float16, uint16_t(u[i])));
                const float f1 = float(__builtin_bit_cast(_Float16, uint16_t(u[i] >> 16)));
                hp[i] = pair_hi(f0, f1);
                lp[i] = pair_lo(f0, f1);
            }
            break;
        case 4:
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float f0 = __uint_as_float(u[2 * i]), f1 = __uint_as_float(u[2 * i + 1]);
                hp[i] = pair_hi(f0, f1);
                lp[i] = pair_lo(f0, f1);
            }
            break;
        default:
#pragma unroll
            for (int i = 0; i < 8; ++i) hp[i] = 0u;
            break;
        }
        *reinterpret_cast<uint4 *>(&st.whi[col][k0]) = make_uint4(hp[0], hp[1], hp[2], hp[3]);
        *reinterpret_cast<uint4 *>(&st.whi[col][k1]) = make_uint4(hp[4], hp[5], hp[6], hp[7]);
        if (any_lo) {
            *reinterpret_cast<uint4 *>(&st.wlo[col][k0]) = make_uint4(lp[0], lp[1], lp[2], lp[3]);
            *reinterpret_cast<uint4 *>(&st.wlo[col][k1]) = make_uint4(lp[4], lp[5], lp[6], lp[7]);
        }
        if (part == 0) st.scale[col] = b.f < 2 ? b.sc : 1.0f;
        if (lane == 0) st.need_lo[wave] = any_lo ? 1u : 0u;
    };

    // ---- x tile: BM rows x 64 entries, 16 bytes per load ----
    constexpr uint32_t kXLoads = BM * 8 / kGemmThreads;     // = MS
    auto load_x = [&](uint32_t kb, uint4 (&xv)[kXLoads]) {
#pragma unroll
        for (uint32_t j = 0; j < kXLoads; ++j) {
            const uint32_t idx = tid + kGemmThreads * j, row = idx >> 3, seg = idx & 7;
            const uint32_t m = min(m0 + row, a.M - 1u);   // rows past M read row M-1; zeroed when stored
            xv[j] = *reinterpret_cast<const uint4 *>(a.x + int64_t(m) * a.ldx + kb * 64 + seg * 8);
        }
    };
    auto store_x = [&](const uint4 (&xv)[kXLoads], GemmStage<MS> &st) {
#pragma unroll
        for (uint32_t j = 0; j < kXLoads; ++j) {
            const uint32_t idx = tid + kGemmThreads * j, row = idx >> 3, seg = idx & 7;
            *reinterpret_cast<uint4 *>(&st.xs[row][seg * 8]) = m0 + row < a.M ? xv[j] : make_uint4(0, 0, 0, 0);
        }
    };

    f32x4 acc[MS][2];
#pragma unroll
    for (int i = 0; i < MS; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    {   // prologue: step 0 into stage 0
        uint4 xv[kXLoads];
        const BlockLoad b = load_block(kb0);
        load_x(kb0, xv);
        store_x(xv, stage[0]);
        store_block(b, stage[0]);
    }
    __syncthreads();

    const uint32_t lr = lane & 15, lk = (lane >> 4) * 8;    // MFMA operand row / first k of this lane
    for (uint32_t kb = kb0; kb < kb1; ++kb) {
        GemmStage<MS> &st = stage[(kb - kb0) & 1];
        const bool more = kb + 1 < kb1;
        uint4 xv[kXLoads];
        BlockLoad b;
        if (more) {   // block loads first: nothing in them waits, so they never wait for x's loads
            b = load_block(kb + 1);
            load_x(kb + 1, xv);
        }
        // MFMAs on this stage
        bf16x8 A[MS][2];
#pragma unroll
        for (int i = 0; i < MS; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                A[i][h] = *reinterpret_cast<const bf16x8 *>(&st.xs[wm * 16 * MS + 16 * i + lr][32 * h + lk]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t c0 = wn * 32 + 16 * j;
            const bf16x8 Bh0 = *reinterpret_cast<const bf16x8 *>(&st.whi[c0 + lr][lk]);
            const bf16x8 Bh1 = *reinterpret_cast<const bf16x8 *>(&st.whi[c0 + lr][32 + lk]);
            const float sc = st.scale[c0 + lr];
            const bool lo = __builtin_amdgcn_readfirstlane(st.need_lo[c0 >> 4]) != 0u;
            // independent MFMA chains per 16-row group, straight-line for each case
            f32x4 c[MS];
            if (lo) {
                const bf16x8 Bl0 = *reinterpret_cast<const bf16x8 *>(&st.wlo[c0 + lr][lk]);
                const bf16x8 Bl1 = *reinterpret_cast<const bf16x8 *>(&st.wlo[c0 + lr][32 + lk]);
#pragma unroll
                for (int i = 0; i < MS; ++i) {
                    c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i][0], Bh0, (f32x4{0.f, 0.f, 0.f, 0.f}), 0, 0, 0);
                    c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i][1], Bh1, c[i], 0, 0, 0);
                    c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i][0], Bl0, c[i], 0, 0, 0);
                    c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i][1], Bl1, c[i], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < MS; ++i) {
                    c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i][0], Bh0, (f32x4{0.f, 0.f, 0.f, 0.f}), 0, 0, 0);
                    c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i][1], Bh1, c[i], 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < MS; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(sc, c[i][e], acc[i][j][e]);
        }
        if (more) {
            GemmStage<MS> &nx = stage[(kb + 1 - kb0) & 1];
            store_x(xv, nx);
            store_block(b, nx);
        }
        __syncthreads();
    }

    // ---- output: lane holds column lr, rows 4*(lane/16) + e of each 16x16 tile ----
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t n = n0 + wn * 32 + 16 * j + lr;
            if (n >= w.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t m = m0 + wm * 16 * MS + 16 * i + 4 * (lane >> 4) + e;
                if (m >= a.M) continue;
                float v = acc[i][j][e];
                if (a.partial) {
                    a.partial[(uint64_t(blockIdx.z) * a.M + m) * w.N + n] = v;
                    continue;
                }
                if (a.act == HT_ACT_RELU) v = v > 0.0f ? v : 0.0f;   // +0 for zero, negative and NaN
                if (a.ybf) a.ybf[int64_t(m) * a.ldy + n] = f32_to_bf16_rne(v);
                else a.y[int64_t(m) * a.ldy + n] = v;
            }
        }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

template <int MS>
void launch_gemm(const GemmArgs &a, hipStream_t s) {
    static bool attr = false;   // dynamic LDS above 64 KiB must be allowed once per kernel
    if (!attr) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_kernel<MS>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, int(gemm_lds_bytes<MS>()));
        attr = true;
    }
    const dim3 grid((a.w.N + kGemmBN - 1) / kGemmBN, (a.M + 32 * MS - 1) / (32 * MS),
                    (a.w.KB + a.KBs - 1) / a.KBs);
    hipLaunchKernelGGL(gemm_kernel<MS>, grid, dim3(kGemmThreads), gemm_lds_bytes<MS>(), s, a);
}

}  // namespace

namespace {

constexpr int64_t kGemmChunkRows = 65535 * 32;   // rows per launch (grid y limit at 32-row tiles)
constexpr uint64_t kSplitTarget = 768;             // workgroups wanted: three per compute unit

uint32_t gemm_bm(int64_t M) { return M >= 128 ? 128u : M >= 64 ? 64u : 32u; }

// K-splits: three workgroups per compute unit (each step of a workgroup
// waits for its blocks' loads, so more of them in flight hide that), at least 4
// K-blocks per split, every split non-empty.
uint32_t gemm_splits(const ht_packed_weight *w, int64_t M) {
    const uint32_t KB = uint32_t(w->K / kBlockK);
    const uint64_t tiles = uint64_t((w->N + kGemmBN - 1) / kGemmBN) * uint64_t((M + gemm_bm(M) - 1) / gemm_bm(M));
    if (tiles >= kSplitTarget || KB < 8) return 1;
    uint32_t S = uint32_t((kSplitTarget + tiles - 1) / tiles);
    if (S > KB / 4) S = KB / 4;
    const uint32_t KBs = (KB + S - 1) / S;
    return (KB + KBs - 1) / KBs;
}

}  // namespace

size_t gemm_ws(const ht_packed_weight *w, int64_t M) {
    const int64_t Mt = M < kGemmChunkRows ? M : kGemmChunkRows;
    const uint32_t S = gemm_splits(w, Mt);
    return S > 1 ? size_t(S) * size_t(Mt) * size_t(w->N) * sizeof(float) : 0;
}

ht_status run_gemm(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y, uint16_t *ybf,
                   int64_t ldy, int act, void *ws, hipStream_t s) {
    GemmArgs a;
    a.w = layer_dev(w);
    a.ldx = ldx;
    a.ldy = ldy;
    a.act = act;
    for (int64_t m0 = 0; m0 < M; m0 += kGemmChunkRows) {
        const int64_t Mt = M - m0 < kGemmChunkRows ? M - m0 : kGemmChunkRows;
        const uint32_t S = gemm_splits(w, Mt);
        a.x = x + m0 * ldx;
        a.y = y ? y + m0 * ldy : nullptr;
        a.ybf = ybf ? ybf + m0 * ldy : nullptr;
        a.partial = S > 1 ? static_cast<float *>(ws) : nullptr;
        a.M = uint32_t(Mt);
        a.KBs = (a.w.KB + S - 1) / S;
        switch (gemm_bm(Mt)) {
        case 128: launch_gemm<4>(a, s); break;
        case 64: launch_gemm<2>(a, s); break;
        default: launch_gemm<1>(a, s); break;
        }
        HT_LAUNCH_CHECK();
        if (S > 1) {
            const ht_status st = launch_split_reduce(static_cast<const float *>(ws), S, uint32_t(Mt), a.w.N, a.y,
                                                     a.ybf, ldy, act, s);
            if (st != HT_OK) return st;
        }
    }
    return HT_OK;
}

}  // namespace ht
