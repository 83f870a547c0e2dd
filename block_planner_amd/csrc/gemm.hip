// gemm.hip -- the mixed-format linear for many rows of x (prefill):
// y[m, n] = sum over K-blocks kb of  blk(m, n, kb)  with fp32 accumulation,
// where an integer block contributes s * (sum_i q_i * x[m, 64kb+i]) and a
// float block sum_i w_i * x[m, 64kb+i] (HyperTensor 1.0.1 page, intro: fused
// kernels execute the mixed-precision plan; "Key Features": HyperLinear).
//
// A workgroup owns a BM x 128 tile of y (BM = 256, 128 or 64 rows of x) and
// walks K one 64-wide block at a time.  Per step the tile's 128 weight blocks
// (one per output column) are dequantised into LDS as bfloat16:
//   INT4 / INT8   the codes themselves (|q| <= 127 is exact in bfloat16);
//                 the block's scale multiplies the 64-term partial afterwards;
//   BF16          the values;
//   FP16 / FP32   two planes, hi = w with the low 16 bits cleared and
//                 lo = bf16(w - hi) (exact for FP16; 16 significant bits for
//                 FP32), scale 1; a non-finite entry gives a NaN column.
// The hi plane's partial of each step comes from bf16 MFMAs
// (v_mfma_f32_16x16x32_bf16) with a fresh accumulator, and every output
// element adds scale[n] * partial[m, n] in fp32, in K order.  The lo plane
// is multiplied only for 16-column groups that hold an FP16 or FP32 block in
// that step, straight into the accumulators (float blocks have scale 1, and
// integer columns hold zeros in the lo plane).
//
// Roles and pipeline (512 threads): four waves run the MFMAs, each on a
// (BM/2) x 64 quarter of the tile, and copy x tiles straight from memory into
// LDS (global_load_lds) one step ahead; four waves load the packed blocks two
// steps ahead into registers and dequantise the next step's into the other
// LDS stage, two threads per block (32 entries each).  One barrier per step;
// it waits only for LDS operations, so the producers' loads of later steps
// stay in flight across it.
#include "int8_tile.h"
#include "linear_host.h"

namespace ht {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kGemmBN = 128;         // output columns (weight rows) per workgroup: 8 groups of 16
constexpr uint32_t kGemmThreads = 512;    // 4 MFMA waves + 4 producer waves
constexpr uint32_t kLdsRow = 72;          // bfloat16 per weight row in LDS: 64 + 8 of padding

struct GemmArgs {
    LayerDev w;
    const uint16_t *x;
    int64_t ldx;
    float *y;                 // fp32 output, or
    uint16_t *ybf;            // bfloat16 output (round to nearest even), or
    float *partial;           // per-split partial sums [S][M][N] (no activation)
    int64_t ldy;
    uint32_t M;
    uint32_t KBs;             // K-blocks per split
    uint32_t MT, NT;          // row tiles of x, column tiles of the weight
    uint32_t skip_int8;       // leave all-INT8 column tiles to the int8 matrix-core kernel
    int act;
};

// The dequantised weight tile of one K-step.
struct WStage {
    uint16_t whi[kGemmBN][kLdsRow];    // bfloat16, row = output column
    uint16_t wlo[kGemmBN][kLdsRow];
    float scale[kGemmBN];
    uint32_t need_lo[kGemmBN / 16];    // per 16-column group
};

// What one producer thread loads for one K-step: half `h` of the packed block
// of its column slot (32 of the 64 entries).
struct BlockLoad {
    uint4 p[8];        // payload bytes of the half (16 / 32 / 64 / 64 / 128 bytes by format)
    float sc;
    uint32_t id2;      // the 4 bytes holding the block id (kb * R + r), as loaded
    uint32_t hi16;     // which half of id2 is the id
    int f;             // format, or 5 for "no block": the column is zero in this step
};

// Workgroup barrier that waits for this wave's LDS operations only (not for
// its outstanding global loads or copies into LDS, which are waited for
// explicitly where their data is used).
__device__ __forceinline__ void gemm_lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup (mt, nt, split) owns rows [BM*mt, +BM) of x (BM = 32*MI) and
// weight rows [128*nt, +128), over K-blocks [KBs*split, +KBs).  Consecutive
// workgroup indices go to different XCDs in turn, so the index is permuted
// (when the grid is a multiple of 8) such that each XCD gets a contiguous run
// of tiles, mostly one row tile of x, which its L2 then serves to all of them.
//
// MFMA wave c owns rows [16*MI*(c>>1), +16*MI) and columns [64*(c&1), +64) of
// the tile (MI row tiles of 16, four column groups of 16).  A workgroup's
// waves are spread over the four SIMDs in turn, so each SIMD normally runs
// one wave of each kind and its matrix core and vector ALU work at the same
// time.
template <int MI>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs a) {
    constexpr uint32_t BM = 32 * MI;
    // x tiles: row r at 128 * r bytes, 16-byte slot s holds the row's entries
    // [8 * (s ^ ((r >> 1) & 7)), +8) (a swizzle that makes the MFMA operand
    // reads conflict-free); two stages, as separate objects so that the
    // compiler sees the copies into one do not touch the other
    __shared__ __align__(16) uint16_t xs0[BM * 64], xs1[BM * 64];
    __shared__ __align__(16) WStage wt0, wt1;

    const LayerDev &w = a.w;
    const uint32_t tid = threadIdx.x, lane = tid & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    uint32_t L = blockIdx.x;
    if ((gridDim.x & 7u) == 0) L = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const uint32_t per_split = a.MT * a.NT;
    const uint32_t zs = L / per_split, rem = L - zs * per_split;
    const uint32_t mt = rem / a.NT, nt = rem - mt * a.NT;
    const uint32_t n0 = nt * kGemmBN, m0 = mt * BM;
    const uint32_t KB = w.KB, R = w.R;
    const uint32_t kb0 = zs * a.KBs, kb1 = min(KB, kb0 + a.KBs);   // this split's K-blocks (non-empty)
    const uint32_t nsteps = kb1 - kb0;
    if (a.skip_int8 && int8_tile(w, n0 / kI8TileRows, kb0, kb1)) return;   // the whole workgroup

    if (wave < 4) {
        // ================= MFMA waves =================
        const uint32_t c = wave, wr = c >> 1, wc = c & 1;
        // x copy: wave c copies rows [BM/4 * c, +BM/4) (8 * MI rows), 8 rows per instruction;
        // lane l -> row 8g + l/8, slot l%8 of 8-row group g.  Each instruction
        // takes a uniform base (the group's first row, clamped to the last row
        // of x, plus the K-step's offset) and a loop-invariant 32-bit byte
        // offset per lane (rows past M read row M-1).
        const uint32_t xr = lane >> 3, xslot = lane & 7;
        const uint16_t *xrow[MI];
        uint32_t xoff[MI];
#pragma unroll
        for (uint32_t i = 0; i < MI; ++i) {
            const uint32_t g = MI * c + i, r = 8 * g + xr;
            const uint32_t rb = min(m0 + 8 * g, a.M - 1u), rr = min(m0 + r, a.M - 1u);
            xrow[i] = a.x + int64_t(rb) * a.ldx;
            xoff[i] = uint32_t((uint64_t(rr - rb) * uint64_t(a.ldx) + 8u * (xslot ^ ((r >> 1) & 7u))) * 2u);
        }
        // Issued as inline assembly (M0 = LDS destination of the wave's 1 KiB),
        // so the compiler does not add waits for these copies before unrelated
        // LDS reads; this wave issues no other vector-memory loads, and waits
        // for its copies explicitly (vmcnt(0)) before the barrier that
        // publishes them.
        auto x_copy = [&](uint32_t kb, uint16_t *xs) {
#pragma unroll
            for (uint32_t i = 0; i < MI; ++i) {
                const uint32_t g = MI * c + i;
                const uint16_t *src = xrow[i] + kb * 64u;
                const uint32_t dst = uint32_t(uintptr_t((__attribute__((address_space(3))) uint16_t *)(xs + 8 * g * 64)));
                asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                             :
                             : "v"(xoff[i]), "s"(src), "s"(dst)
                             : "memory", "m0");
            }
        };
        const uint32_t lr = lane & 15, lq = lane >> 4;      // MFMA operand row / k-quarter of this lane
        f32x4 acc[MI][4];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // One K-step on LDS stages xs / st.  Per row tile: the hi plane's
        // 64-term partials of the four column groups (fresh accumulators),
        // added to acc times the column's scale; then the lo plane of the
        // groups that hold an FP16 / FP32 block, straight into acc.
        auto mfma_step = [&](const uint16_t *xs, const WStage &st) {
            bf16x8 Bh[4][2], Bl[4][2];
            float sc[4];
            const uint4 nlo4 = *reinterpret_cast<const uint4 *>(&st.need_lo[4 * wc]);
            const uint32_t nl[4] = {uint32_t(__builtin_amdgcn_readfirstlane(nlo4.x)),
                                    uint32_t(__builtin_amdgcn_readfirstlane(nlo4.y)),
                                    uint32_t(__builtin_amdgcn_readfirstlane(nlo4.z)),
                                    uint32_t(__builtin_amdgcn_readfirstlane(nlo4.w))};
            auto readA = [&](int i, bf16x8 (&A)[2]) {
                const uint32_t r = 16 * MI * wr + 16 * i + lr;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    A[h] = *reinterpret_cast<const bf16x8 *>(xs + r * 64 + 8 * ((lq + 4 * h) ^ ((r >> 1) & 7u)));
            };
            bf16x8 A[2];
            readA(0, A);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t col = 64 * wc + 16 * j + lr;
                Bh[j][0] = *reinterpret_cast<const bf16x8 *>(&st.whi[col][8 * lq]);
                Bh[j][1] = *reinterpret_cast<const bf16x8 *>(&st.whi[col][32 + 8 * lq]);
                sc[j] = st.scale[col];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (nl[j] != 0u) {
                    const uint32_t col = 64 * wc + 16 * j + lr;
                    Bl[j][0] = *reinterpret_cast<const bf16x8 *>(&st.wlo[col][8 * lq]);
                    Bl[j][1] = *reinterpret_cast<const bf16x8 *>(&st.wlo[col][32 + 8 * lq]);
                }
            }
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                bf16x8 An[2];
                if (i + 1 < MI) readA(i + 1, An);
                f32x4 cc[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    cc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], Bh[j][0], (f32x4{0.f, 0.f, 0.f, 0.f}), 0, 0, 0);
                    cc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], Bh[j][1], cc[j], 0, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(sc[j], cc[j][e], acc[i][j][e]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (nl[j] != 0u) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], Bl[j][0], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], Bl[j][1], acc[i][j], 0, 0, 0);
                    }
                }
                if (i + 1 < MI) {
                    A[0] = An[0];
                    A[1] = An[1];
                }
            }
        };

        // x: two LDS stages; the copy for step t+2 goes into step t's stage
        // right after the barrier that ends step t
        x_copy(kb0, xs0);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copy is in LDS
        if (nsteps > 1) x_copy(kb0 + 1, xs1);
        gemm_lds_barrier();
        auto cstep = [&](uint32_t t, uint16_t *xc) {
            mfma_step(xc, (t & 1) ? wt1 : wt0);
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the copy for step t+1 is in LDS
            gemm_lds_barrier();
            if (t + 2 < nsteps) x_copy(kb0 + t + 2, xc);
        };
        for (uint32_t t = 0; t < nsteps; t += 2) {
            cstep(t, xs0);
            if (t + 1 < nsteps) cstep(t + 1, xs1);
        }

        // ---- output: lane holds column lr, rows 4*(lane/16) + e of each 16x16 tile ----
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t n = n0 + 64 * wc + 16 * j + lr;
                if (n >= w.N) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t m = m0 + 16 * MI * wr + 16 * i + 4 * lq + e;
                    if (m >= a.M) continue;
                    float v = acc[i][j][e];
                    if (a.partial) {
                        a.partial[(uint64_t(zs) * a.M + m) * w.N + n] = v;
                        continue;
                    }
                    if (a.act == HT_ACT_RELU) v = v > 0.0f ? v : 0.0f;   // +0 for zero, negative and NaN
                    if (a.ybf) a.ybf[int64_t(m) * a.ldy + n] = f32_to_bf16_rne(v);
                    else a.y[int64_t(m) * a.ldy + n] = v;
                }
            }
        return;
    }

    // ================= producer waves =================
    // thread pt -> half h of column slot gb (the slot's block is the
    // (gb % R)-th block of its row tile in this step, in format order)
    const uint32_t pt = tid - 256, h = pt & 1, gb = pt >> 1;
    const uint8_t *base = w.base;                            // offsets below are 32-bit (buffer < 4 GiB)
    uint32_t opay[5], oids[5];
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        opay[f] = uint32_t(w.off_pay[f]);
        oids[f] = uint32_t(w.off_ids[f]);
    }
    const uint32_t osc0 = uint32_t(w.off_scale[0]), osc1 = uint32_t(w.off_scale[1]);
    const uint32_t tile = n0 / R + gb / R, bi = gb % R;     // tile of the column, block slot within it
    const bool tok = tile < w.T;
    const uint32_t kbx = uint32_t(w.off_kbidx) + 4u * (tok ? tile * KB : 0u);
    // kbidx[f][tile*KB + kb]: block index where step kb starts in format f
    // (a column past N reads tile 0's entries; load_block gives it no block)
    auto kload = [&](uint32_t kb, uint32_t (&v)[5]) {
        kb = min(kb, kb1);
#pragma unroll
        for (int f = 0; f < 5; ++f)
            v[f] = *reinterpret_cast<const uint32_t *>(base + kbx + 4u * (uint32_t(f) * w.nk + kb));
    };

    // Loads of this thread's half block in the step that starts at ka and
    // ends at kn (a step past the split's end has no blocks): eight 16-byte
    // loads at addresses chosen per format; a missing block reads the
    // buffer's first bytes.
    auto load_block = [&](const uint32_t (&ka)[5], const uint32_t (&kn)[5]) -> BlockLoad {
        BlockLoad q;
        // slot bi holds the (bi - c[f])-th block of format f, where c[] are
        // the prefix sums of the step's block counts in format order and
        // c[f] <= bi < c[f+1]; f is found by counting the boundaries c[1..5]
        // not above bi (no branches: every lane takes the same path)
        uint32_t c[6];
        c[0] = 0;
#pragma unroll
        for (int g = 0; g < 5; ++g) c[g + 1] = c[g] + (kn[g] - ka[g]);
        uint32_t f = 0;
#pragma unroll
        for (int g = 1; g <= 5; ++g) f += bi >= c[g] ? 1u : 0u;
        if (!tok) f = 5;
        uint32_t kaf = ka[0], cf = 0, op = opay[0], oi = oids[0], sh = 5, osc = osc0;
#pragma unroll
        for (int g = 1; g < 5; ++g) {
            const bool e = f == uint32_t(g);
            kaf = e ? ka[g] : kaf;
            cf = e ? c[g] : cf;
            op = e ? opay[g] : op;
            oi = e ? oids[g] : oi;
            sh = e ? uint32_t(g == 1 ? 6 : g == 4 ? 8 : 7) : sh;   // log2 of the payload bytes
            osc = e ? osc1 : osc;
        }
        const bool has = f < 5;
        const uint32_t blk = kaf + bi - cf;
        const uint32_t po = has ? op + (blk << sh) + (h << (sh - 1u)) : 0u;
        const uint32_t io = has ? oi + ((2u * blk) & ~3u) : 0u;
        const uint32_t so = has && f < 2 ? osc + 4u * blk : 0u;
        const uint32_t nl = 1u << (sh - 5u);                     // 16-byte pieces in the half
        q.f = int(f);
        // eight 16-byte loads for every lane, with no branch, so that the
        // compiler counts them exactly and waits only for the loads it uses;
        // past the half's length a lane re-reads its last 16 bytes (in cache)
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j)
            q.p[j] = *reinterpret_cast<const uint4 *>(base + (po + 16u * min(j, nl - 1u)));
        q.id2 = *reinterpret_cast<const uint32_t *>(base + io);
        q.hi16 = blk & 1u;
        q.sc = *reinterpret_cast<const float *>(base + so);   // meaningful for INT4 / INT8 only
        return q;
    };

    // Dequantise one half block into st: entries [32h, 32h + 32) of the
    // column, as packed bfloat16 pairs: integers via an exact fp32 conversion
    // whose upper half is the bfloat16 (v_perm packs two), floats as hi =
    // upper half (truncation) and lo = bf16_rne(w - hi).  A non-finite
    // FP16/FP32 entry makes lo NaN, so its output column is NaN.
    auto store_block = [&](const BlockLoad &b, WStage &st) {
        const uint32_t id = b.hi16 ? b.id2 >> 16 : b.id2;
        const uint32_t col = (gb / R) * R + (b.f < 5 ? (id & (R - 1u)) : bi);   // within the 128
        st.scale[col] = b.f < 2 ? b.sc : 1.0f;   // both halves write the same value
        const uint64_t bal = __ballot(b.f == 3 || b.f == 4);
        if ((lane & 31u) == 0) st.need_lo[gb >> 4] = ((bal >> (lane & 32u)) & 0xFFFFFFFFull) != 0 ? 1u : 0u;
        uint4 *hd = reinterpret_cast<uint4 *>(&st.whi[col][32 * h]);
        uint4 *ld = reinterpret_cast<uint4 *>(&st.wlo[col][32 * h]);
        const uint32_t u[32] = {b.p[0].x, b.p[0].y, b.p[0].z, b.p[0].w, b.p[1].x, b.p[1].y, b.p[1].z, b.p[1].w,
                                b.p[2].x, b.p[2].y, b.p[2].z, b.p[2].w, b.p[3].x, b.p[3].y, b.p[3].z, b.p[3].w,
                                b.p[4].x, b.p[4].y, b.p[4].z, b.p[4].w, b.p[5].x, b.p[5].y, b.p[5].z, b.p[5].w,
                                b.p[6].x, b.p[6].y, b.p[6].z, b.p[6].w, b.p[7].x, b.p[7].y, b.p[7].z, b.p[7].w};
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
        auto put = [](uint4 *d, const uint32_t (&v)[16]) {
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] = make_uint4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        };
        const uint4 z = make_uint4(0, 0, 0, 0);
        // Each format writes both planes itself (the integer formats and a
        // missing block write a zero lo plane), so that no value crosses the
        // end of the switch.
        switch (b.f) {
        case 0: {
            // the half's 16 bytes: byte i of the first 8 holds entries 32h+i
            // (low nibble) and 32h+16+i (high), byte 8+i entries 32h+8+i and
            // 32h+24+i (the nibble order of the layout)
            uint32_t hp[16];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t wd = u[2 * q2 + (i >> 1)];
                    const uint32_t sh = 16 * (i & 1);
                    hp[4 * q2 + i] = pair_hi(float(nib(wd, sh)), float(nib(wd, sh + 8)));
                    hp[8 + 4 * q2 + i] = pair_hi(float(nib(wd, sh + 4)), float(nib(wd, sh + 12)));
                }
            put(hd, hp);
            ld[0] = z; ld[1] = z; ld[2] = z; ld[3] = z;
            break;
        }
        case 1: {
            uint32_t hp[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t wd = u[i >> 1], sh = 16 * (i & 1);
                hp[i] = pair_hi(float(int8_t(wd >> sh)), float(int8_t(wd >> (sh + 8))));
            }
            put(hd, hp);
            ld[0] = z; ld[1] = z; ld[2] = z; ld[3] = z;
            break;
        }
        case 2:
            hd[0] = b.p[0]; hd[1] = b.p[1]; hd[2] = b.p[2]; hd[3] = b.p[3];
            ld[0] = z; ld[1] = z; ld[2] = z; ld[3] = z;
            break;
        case 3: {
            uint32_t hp[16], lp[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float f0 = float(__builtin_bit_cast(_Float16, uint16_t(u[i])));
                const float f1 = float(__builtin_bit_cast(_Float16, uint16_t(u[i] >> 16)));
                hp[i] = pair_hi(f0, f1);
                lp[i] = pair_lo(f0, f1);
            }
            put(hd, hp);
            put(ld, lp);
            break;
        }
        case 4: {
            uint32_t hp[16], lp[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float f0 = __uint_as_float(u[2 * i]), f1 = __uint_as_float(u[2 * i + 1]);
                hp[i] = pair_hi(f0, f1);
                lp[i] = pair_lo(f0, f1);
            }
            put(hd, hp);
            put(ld, lp);
            break;
        }
        default:
            hd[0] = z; hd[1] = z; hd[2] = z; hd[3] = z;
            ld[0] = z; ld[1] = z; ld[2] = z; ld[3] = z;
            break;
        }
    };

    // The kbidx entries of step k live in Ks[k % 4]: those of step t+5 are
    // loaded in step t, two steps before their first use (by the loads of
    // step t+4, issued in step t+2); the block loads of step t+2 are issued
    // in step t and dequantised in step t+1.  The loop is unrolled four
    // times, so that a register just loaded is never copied (a copy would
    // wait for the load).
    uint32_t Ks[4][5];
    BlockLoad QA, QB;
    kload(kb0, Ks[0]);
    kload(kb0 + 1, Ks[1]);
    kload(kb0 + 2, Ks[2]);
    kload(kb0 + 3, Ks[3]);
    QB = load_block(Ks[0], Ks[1]);
    QA = load_block(Ks[1], Ks[2]);
    kload(kb0 + 4, Ks[0]);
    store_block(QB, wt0);
    gemm_lds_barrier();
    // step t (t % 4 == S): qc holds the loads of step t+1, qn receives those
    // of step t+2; the entries of step t+5 replace those of step t+1 (last
    // used in step t-1)
    auto step = [&](uint32_t t, auto S, BlockLoad &qc, BlockLoad &qn, WStage &dst) {
        constexpr int s = decltype(S)::value;
        qn = load_block(Ks[(s + 2) & 3], Ks[(s + 3) & 3]);
        kload(kb0 + t + 5, Ks[(s + 1) & 3]);
        if (t + 1 < nsteps) store_block(qc, dst);
        gemm_lds_barrier();
    };
    for (uint32_t t = 0; t < nsteps; t += 4) {
        step(t, std::integral_constant<int, 0>{}, QA, QB, wt1);
        if (t + 1 < nsteps) step(t + 1, std::integral_constant<int, 1>{}, QB, QA, wt0);
        if (t + 2 < nsteps) step(t + 2, std::integral_constant<int, 2>{}, QA, QB, wt1);
        if (t + 3 < nsteps) step(t + 3, std::integral_constant<int, 3>{}, QB, QA, wt0);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

template <int MI>
void launch_gemm(const GemmArgs &a, uint32_t S, hipStream_t s) {
    const uint32_t grid = a.MT * a.NT * S;
    hipLaunchKernelGGL(gemm_kernel<MI>, dim3(grid), dim3(kGemmThreads), 0, s, a);
}

constexpr int64_t kGemmChunkRows = int64_t(1) << 20;   // rows per launch
constexpr int64_t kGemmMaxLdx = int64_t(1) << 28;       // x row stride limit (elements)
constexpr uint64_t kSplitTarget = 256;                   // compute units (one workgroup each)

uint32_t gemm_bm(int64_t M) { return M >= 256 ? 256u : M >= 128 ? 128u : 64u; }

// K-splits when there are fewer tiles than compute units: at least 8
// K-blocks per split, every split non-empty.
uint32_t gemm_splits(const ht_packed_weight *w, int64_t M) {
    const uint32_t KB = uint32_t(w->K / kBlockK);
    const uint64_t tiles = uint64_t((w->N + kGemmBN - 1) / kGemmBN) * uint64_t((M + gemm_bm(M) - 1) / gemm_bm(M));
    const uint64_t target = kSplitTarget;
    if (tiles * 4 >= target * 3 || KB < 16) return 1;
    uint32_t S = uint32_t((target + tiles - 1) / tiles);
    if (S > KB / 8) S = KB / 8;
    const uint32_t KBs = (KB + S - 1) / S;
    return (KB + KBs - 1) / KBs;
}

}  // namespace

uint32_t gemm_split_count(const ht_packed_weight *w, int64_t Mt) { return gemm_splits(w, Mt); }

ht_status gemm_tiles(const ht_packed_weight *w, const uint16_t *x, int64_t Mt, int64_t ldx, float *y, uint16_t *ybf,
                     int64_t ldy, int act, float *partial, uint32_t S, bool skip_int8, hipStream_t s) {
    if (ldx >= kGemmMaxLdx) return HT_ESHAPE;   // the x copies take 32-bit offsets of up to 7 rows
    GemmArgs a;
    a.w = layer_dev(w);
    a.x = x;
    a.ldx = ldx;
    a.y = S > 1 ? nullptr : y;
    a.ybf = S > 1 ? nullptr : ybf;
    a.partial = S > 1 ? partial : nullptr;
    a.ldy = ldy;
    a.act = act;
    a.M = uint32_t(Mt);
    a.KBs = (a.w.KB + S - 1) / S;
    const uint32_t BM = gemm_bm(Mt);
    a.MT = uint32_t((Mt + BM - 1) / BM);
    a.NT = uint32_t((a.w.N + kGemmBN - 1) / kGemmBN);
    a.skip_int8 = skip_int8 ? 1u : 0u;
    switch (BM) {
    case 256: launch_gemm<8>(a, S, s); break;
    case 128: launch_gemm<4>(a, S, s); break;
    default: launch_gemm<2>(a, S, s); break;
    }
    HT_LAUNCH_CHECK();
    return HT_OK;
}

size_t gemm_ws_min(const ht_packed_weight *w, int64_t M) {
    const int64_t Mt = M < kGemmChunkRows ? M : kGemmChunkRows;
    const uint32_t S = gemm_splits(w, Mt);
    return S > 1 ? size_t(S) * size_t(Mt) * size_t(w->N) * sizeof(float) : 0;
}

size_t gemm_ws(const ht_packed_weight *w, int64_t M) {
    const size_t m = gemm_ws_min(w, M);
    return xw_takes(w, M) && xw_ws(w, M) > m ? xw_ws(w, M) : m;
}

ht_status run_gemm(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y, uint16_t *ybf,
                   int64_t ldy, int act, void *ws, size_t ws_bytes, hipStream_t s) {
    if (xw_takes(w, M) && ws && ws_bytes >= xw_ws(w, M)) return run_gemm_xw(w, x, M, ldx, y, ybf, ldy, act, ws, s);
    for (int64_t m0 = 0; m0 < M; m0 += kGemmChunkRows) {
        const int64_t Mt = M - m0 < kGemmChunkRows ? M - m0 : kGemmChunkRows;
        const uint32_t S = gemm_splits(w, Mt);
        float *yc = y ? y + m0 * ldy : nullptr;
        uint16_t *ybc = ybf ? ybf + m0 * ldy : nullptr;
        ht_status st = gemm_tiles(w, x + m0 * ldx, Mt, ldx, yc, ybc, ldy, act, static_cast<float *>(ws), S, false, s);
        if (st != HT_OK) return st;
        if (S > 1) {
            st = launch_split_reduce(static_cast<const float *>(ws), S, uint32_t(Mt), uint32_t(w->N), yc, ybc, ldy,
                                     act, s);
            if (st != HT_OK) return st;
        }
    }
    return HT_OK;
}

}  // namespace ht
