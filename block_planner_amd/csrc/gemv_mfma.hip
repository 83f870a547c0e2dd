// gemv_mfma.hip -- the mixed-format linear for a few rows of x (decode at
// batch 1 to 32 per launch) with the dot products on the matrix cores
// (HyperTensor 1.0.1 page, intro: fused kernels execute the mixed-precision
// plan; "Key Features": HyperLinear).  Same sums as the MFMA prefill path:
//   y[m, n] = sum over K-blocks kb of  blk(m, n, kb),
//   INT4 / INT8   blk = s * (sum_i q_i * x[m, 64kb+i]),
//   BF16          blk = sum_i w_i * x[m, 64kb+i],
//   FP16 / FP32   the same with w = hi + lo, two bfloat16 planes
//                 (hi = w with the low 16 bits cleared, lo = bf16(w - hi)),
// with bf16 MFMA products and fp32 accumulation.
//
// No LDS staging of weights: a wavefront takes one 16-row tile (row tile 16)
// and a few K-blocks at a time; for each K-block ("column") lane (j, q) =
// (lane % 16, lane / 16) dequantises entries [16q, 16q + 16) of the column's
// j-th block in the packed order (format by format, rows ascending) straight
// into the B operand of v_mfma_f32_16x16x32_bf16; the A operand is x rows
// 16g + j at the same entries, from LDS.  The K index inside an MFMA is a
// permutation of the block's entries, the same for A and B, so the products
// are the block's dot products.  The MFMA result's column j then belongs to
// the row named by that block's id; a forward lane permute moves it (and the
// block's scale) to the lane that owns the row before acc += scale * partial.
//
// A workgroup (16 wavefronts) owns one K range and one to four row tiles
// (tiles blockIdx.x + i * gridDim.x; several only when there are more tiles
// than compute units), walked in rounds of 64 / MG K-blocks: the round's x
// rows are staged in LDS once for all of its tiles, and for each tile every
// wavefront has the loads of all of its columns of the round (four, or two
// at MG = 2) in flight, so a tile costs about one memory round trip per
// round.  The workgroup then adds each tile's 16 wavefront sums in wavefront
// order through LDS and writes y (or, with several K ranges, the range's
// partial sums, which a second kernel adds in range order).
#include "gemv_common.h"
#include "linear_host.h"

namespace ht {

typedef __bf16 dbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 dbf16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kDecWaves = 16;
constexpr uint32_t kDecThreads = 64 * kDecWaves;

struct DecArgs {
    LayerDev w;
    const uint16_t *x;
    int64_t ldx;
    float *y;                 // fp32 output, or
    uint16_t *ybf;            // bfloat16 output, or
    float *partial;           // per-split partial sums [S][M][N] (no activation)
    int64_t ldy;
    uint32_t M;
    uint32_t KBs;             // K-blocks per split
    uint32_t TPW;             // row tiles per workgroup (tiles blockIdx.x + i * gridDim.x, i < TPW)
    uint32_t nbytes;          // packed buffer size (below 4 GiB)
    int act;
};

// What one lane loads for one column: its quarter of the block in slot j.
struct DecLoad {
    uint4 p[4];               // payload: 16 (INT4, INT8), 32 (BF16, FP16) or 64 (FP32) bytes
    uint32_t id2;             // the 4 bytes holding the block id
    float sc;
    uint32_t hi16;
    int f;                    // format, or 5: no block in this slot
};

// x staging: a chunk of kDecChunk / MG K-blocks of x rows [0, 16 MG) per
// round, row stride padded by 16 bytes so that the 16 rows an MFMA operand
// read touches fall in distinct banks.
constexpr uint32_t kDecChunk = 64;                    // K-blocks per round at MG = 1
constexpr uint32_t kDecMaxTPW = 4;                    // row tiles per workgroup at most
template <int MG> constexpr uint32_t dec_row() { return (kDecChunk / MG) * 64u + 8u; }   // bfloat16 entries

// ROLL: the workgroup has more than one (round, tile) step, so columns are
// refilled as they are consumed; without it each wavefront loads its columns
// once.  BUF: the layer has many blocks wider than 16 bytes per lane (BF16,
// FP16, FP32), so every column issues the same six loads with the unneeded
// pieces masked per lane (buffer loads past the buffer's end read zeros
// without a memory access); without it the pieces past the column's widest
// format are skipped and lanes that need fewer re-read their first piece.
template <int MG, bool ROLL, bool BUF>
__global__ __launch_bounds__(kDecThreads) void gemv_mfma_kernel(DecArgs a) {
    constexpr uint32_t CK = kDecChunk / MG;           // K-blocks per round
    constexpr uint32_t CW = CK / kDecWaves;           // K-blocks per wavefront per round (4 or 2)
    constexpr uint32_t XR = dec_row<MG>();
    constexpr uint32_t NT = ROLL ? kDecMaxTPW : 1u;   // row tiles a workgroup can hold
    __shared__ __align__(16) uint16_t xs[16 * MG * XR];
    float *red = reinterpret_cast<float *>(xs);       // [wave][MG * 4][64] after the last round
    const LayerDev &w = a.w;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t j = lane & 15, q = lane >> 4;
    const uint32_t kbs0 = blockIdx.y * a.KBs;
    const uint32_t kbs1 = min(w.KB, kbs0 + a.KBs);
    const uint8_t *base = w.base;                          // offsets below are 32-bit (buffer < 4 GiB)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, int(a.nbytes), 0x00020000);
    constexpr uint32_t kOut = 0xFFFFFFF0u;                 // an offset past the buffer (nbytes < kOut)
    const uint32_t *kbx = reinterpret_cast<const uint32_t *>(base + w.off_kbidx);

    uint32_t opay[5], oids[5];
#pragma unroll
    for (int f = 0; f < 5; ++f) {
        opay[f] = uint32_t(w.off_pay[f]);
        oids[f] = uint32_t(w.off_ids[f]);
    }
    const uint32_t osc0 = uint32_t(w.off_scale[0]), osc1 = uint32_t(w.off_scale[1]);

    // kbidx[f][t*KB + kb0 + c] for c = 0..15 of the wavefront's columns of
    // row tile t in a round starting at kc: lane i holds format i / 16
    // (formats 0-3) and, in kv4, format 4, at column i % 16
    auto kbidx_window = [&](uint32_t t, uint32_t kc, uint32_t &v, uint32_t &v4) {
        const uint32_t ci = t * w.KB + min(kc + wave * CW + j, w.KB);
        v = kbx[q * w.nk + ci];
        v4 = kbx[4u * w.nk + ci];
    };
    auto kbidx_at = [&](uint32_t kv, uint32_t kv4, uint32_t c, uint32_t (&v)[5]) {   // wave-uniform
#pragma unroll
        for (int f = 0; f < 4; ++f) v[f] = __builtin_amdgcn_readlane(kv, 16 * f + c);
        v[4] = __builtin_amdgcn_readlane(kv4, c);
    };

    // Loads of column c of the window: the lane's block is slot j of the
    // column in the packed order; a missing block (slot past the tile's rows,
    // or a column past the range) reads the buffer's first bytes, or with
    // BUF nothing.
    auto load_col = [&](uint32_t kv, uint32_t kv4, uint32_t c) -> DecLoad {
        DecLoad d;
        uint32_t ka[5], kn[5];
        kbidx_at(kv, kv4, c, ka);
        kbidx_at(kv, kv4, c + 1, kn);
        uint32_t cum = 0, blk = 0;
        int f = 5;
        uint32_t nlw = 1;                                  // 16-byte pieces some lane needs (uniform)
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            const uint32_t cnt = kn[g] - ka[g];
            if (f == 5 && j - cum < cnt) {
                f = g;
                blk = ka[g] + (j - cum);
            }
            cum += cnt;
            if (cnt) nlw = g == 4 ? 4u : (g >= 2 && nlw < 2u) ? 2u : nlw;
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
        d.f = f;
        d.hi16 = blk & 1u;
        if (BUF) {
            // a fixed count of loads per column, so that the wait before a
            // column's arithmetic counts exactly the later columns' loads
            const bool has = f < 5;
#pragma unroll
            for (uint32_t i = 0; i < 4; ++i) {
                const u32x4 pv = __builtin_amdgcn_raw_buffer_load_b128(rs, has && i < nl ? po + 16u * i : kOut, 0, 0);
                d.p[i] = make_uint4(pv.x, pv.y, pv.z, pv.w);
            }
            d.id2 = __builtin_amdgcn_raw_buffer_load_b32(rs, has ? io : kOut, 0, 0);
            d.sc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, f < 2 ? so : kOut, 0, 0));
            return d;
        }
        const u32x4 p0 = ld_stream_u4(base + po);
        d.p[0] = make_uint4(p0.x, p0.y, p0.z, p0.w);
        // further pieces only when some lane of the column needs them; a lane
        // that needs fewer re-reads its first piece (same cache line)
#pragma unroll
        for (uint32_t i = 1; i < 4; ++i) {
            d.p[i] = make_uint4(0u, 0u, 0u, 0u);
            if (i < nlw) {
                const u32x4 pi = ld_stream_u4(base + po + (i < nl ? 16u * i : 0u));
                d.p[i] = make_uint4(pi.x, pi.y, pi.z, pi.w);
            }
        }
        d.id2 = *reinterpret_cast<const uint32_t *>(base + io);
        d.sc = *reinterpret_cast<const float *>(base + so);
        return d;
    };

    f32x4 acc[NT][MG];
#pragma unroll
    for (int i = 0; i < int(NT); ++i)
#pragma unroll
        for (int g = 0; g < MG; ++g) acc[i][g] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto pair_hi = [](float f0, float f1) {   // upper halves of two fp32 -> one word
        return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    };
    auto pair_lo = [](float f0, float f1) {   // bf16_rne(f - trunc(f)) of two fp32
        const float r0 = f0 - __uint_as_float(__float_as_uint(f0) & 0xffff0000u);
        const float r1 = f1 - __uint_as_float(__float_as_uint(f1) & 0xffff0000u);
        const dbf16x2 v = {(__bf16)r0, (__bf16)r1};
        return __builtin_bit_cast(uint32_t, v);
    };

    // Multiply one loaded column (K-block kl of the round) into acc[i].
    auto compute = [&](const DecLoad &d, uint32_t kl, f32x4 (&acc)[MG]) {
        const uint32_t u[16] = {d.p[0].x, d.p[0].y, d.p[0].z, d.p[0].w, d.p[1].x, d.p[1].y, d.p[1].z, d.p[1].w,
                                d.p[2].x, d.p[2].y, d.p[2].z, d.p[2].w, d.p[3].x, d.p[3].y, d.p[3].z, d.p[3].w};
        uint32_t hp[8], lp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) lp[i] = 0u;
        switch (d.f) {
        case 0: {
            // entry i of the quarter = nibble (q & 1) of byte i of the 16 bytes
            const uint32_t sh = 4u * (q & 1u);
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t wd = u[p >> 1] >> sh;
                const uint32_t b = 16u * (p & 1);
                hp[p] = pair_hi(float(int32_t(wd << (28u - b)) >> 28), float(int32_t(wd << (20u - b)) >> 28));
            }
            break;
        }
        case 1:
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t wd = u[p >> 1], b = 16u * (p & 1);
                hp[p] = pair_hi(float(int8_t(wd >> b)), float(int8_t(wd >> (b + 8))));
            }
            break;
        case 2:
#pragma unroll
            for (int p = 0; p < 8; ++p) hp[p] = u[p];
            break;
        case 3:
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const float f0 = float(__builtin_bit_cast(_Float16, uint16_t(u[p])));
                const float f1 = float(__builtin_bit_cast(_Float16, uint16_t(u[p] >> 16)));
                hp[p] = pair_hi(f0, f1);
                lp[p] = pair_lo(f0, f1);
            }
            break;
        case 4:
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const float f0 = __uint_as_float(u[2 * p]), f1 = __uint_as_float(u[2 * p + 1]);
                hp[p] = pair_hi(f0, f1);
                lp[p] = pair_lo(f0, f1);
            }
            break;
        default:
#pragma unroll
            for (int p = 0; p < 8; ++p) hp[p] = 0u;
            break;
        }
        const dbf16x8 bh0 = __builtin_bit_cast(dbf16x8, make_uint4(hp[0], hp[1], hp[2], hp[3]));
        const dbf16x8 bh1 = __builtin_bit_cast(dbf16x8, make_uint4(hp[4], hp[5], hp[6], hp[7]));
        const dbf16x8 bl0 = __builtin_bit_cast(dbf16x8, make_uint4(lp[0], lp[1], lp[2], lp[3]));
        const dbf16x8 bl1 = __builtin_bit_cast(dbf16x8, make_uint4(lp[4], lp[5], lp[6], lp[7]));
        const bool any_lo = __any(d.f == 3 || d.f == 4);
        // column j of the product is the block of row (id & 15) (a missing
        // block: row j, which then has no block either, so the map is a
        // permutation of the 16 rows); it moves, with the scale, to the lane
        // of that row
        const uint32_t id = d.hi16 ? d.id2 >> 16 : d.id2 & 0xFFFFu;
        const uint32_t r = d.f < 5 ? (id & 15u) : j;
        const float sc = d.f < 2 ? d.sc : d.f < 5 ? 1.0f : 0.0f;
        const int dst = int(4u * (r + 16u * q));
        const float scr = __int_as_float(__builtin_amdgcn_ds_permute(dst, __float_as_int(sc)));
#pragma unroll
        for (int g = 0; g < MG; ++g) {
            // A operand: x row 16g + j, entries [16q, 16q + 16) of the K-block
            const uint16_t *xp = xs + (16u * g + j) * XR + kl * 64u + 16u * q;
            const dbf16x8 a0 = *reinterpret_cast<const dbf16x8 *>(xp);
            const dbf16x8 a1 = *reinterpret_cast<const dbf16x8 *>(xp + 8);
            f32x4 cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bh0, (f32x4{0.f, 0.f, 0.f, 0.f}), 0, 0, 0);
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bh1, cc, 0, 0, 0);
            if (any_lo) {
                cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bl0, cc, 0, 0, 0);
                cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bl1, cc, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = __int_as_float(__builtin_amdgcn_ds_permute(dst, __float_as_int(cc[e])));
                acc[g][e] = __builtin_fmaf(scr, v, acc[g][e]);
            }
        }
    };

    // Rounds of CK K-blocks.  The round's x rows [0, 16 MG) are copied
    // straight from memory into LDS (global_load_lds, issued as inline
    // assembly with M0 = the LDS destination of a wavefront's 1 KiB piece;
    // rows past M repeat row M - 1 and entries past the range repeat its last
    // piece, so no copy is masked): the first round's before the first
    // K-block index window is loaded, so the two trips overlap, each later
    // round's right after the previous round's MFMAs.  In a round each
    // wavefront issues the loads of all CW of its columns, then one wait for
    // everything, one barrier, the MFMAs, and a barrier before the next
    // round's copies overwrite x.
    constexpr uint32_t PPR = CK / 8;                      // 1 KiB pieces per x row
    auto stage_x = [&](uint32_t kc) {                     // 16 MG * PPR = 128 pieces, 8 per wavefront
        const uint32_t nkc = min(CK, kbs1 - kc);
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i) {
            const uint32_t P = wave + kDecWaves * i;
            const uint32_t row = P / PPR, pc = P % PPR;
            const uint32_t cu = min(pc * 64u + lane, 8u * nkc - 1u);
            const uint16_t *src = a.x + int64_t(min(row, a.M - 1u)) * a.ldx + kc * 64u + 8u * cu;
            const uint32_t dst =
                uint32_t(uintptr_t((__attribute__((address_space(3))) uint16_t *)(xs + row * XR + pc * 512u)));
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                         :
                         : "v"(src), "s"(dst)
                         : "memory", "m0");
        }
    };
    // Rounds over K outside, the workgroup's row tiles inside: the round's x
    // is copied once for all of them.  The column registers roll: as soon as
    // column c of the current (round, tile) has been multiplied, they are
    // reloaded with column c of the next (round, tile), whose kbidx window is
    // already in registers (the window after that is then requested), so the
    // next tile's loads overlap this tile's arithmetic.  Windows past the end
    // of K are clamped to it: their loads find no block.
    const uint32_t tpw = a.TPW;
    auto tile_ok = [&](uint32_t i) { return i < tpw && blockIdx.x + i * gridDim.x < w.T; };
    uint32_t pk = kbs0, pi = 0;                           // (round, tile) whose window is in kv
    auto advance = [&]() {                                // to the next (round, tile)
        if (tile_ok(pi + 1)) {
            ++pi;
        } else {
            pi = 0;
            pk += CK;
        }
    };
    auto window = [&](uint32_t &kv, uint32_t &kv4) {
        kbidx_window(blockIdx.x + pi * gridDim.x, pk < kbs1 ? pk : w.KB, kv, kv4);
    };
    uint32_t kv, kv4;
    stage_x(kbs0);                                        // in flight together with the first window
    window(kv, kv4);
    DecLoad d[CW];
    if (ROLL) {
#pragma unroll
        for (uint32_t c = 0; c < CW; ++c) d[c] = load_col(kv, kv4, c);
        advance();
        if (MG == 1 || pk < kbs1) window(kv, kv4);
    }
    for (uint32_t kc = kbs0; kc < kbs1; kc += CK) {
        const uint32_t nkc = min(CK, kbs1 - kc);
        const uint32_t nc = min(nkc, wave * CW + CW) - min(nkc, wave * CW);   // columns of this wavefront
#pragma unroll
        for (uint32_t i = 0; i < NT; ++i) {
            if (!tile_ok(i)) continue;                    // workgroup-uniform
            if (i == 0) {
                __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0): this wavefront's x pieces are in LDS
                __syncthreads();
            }
            if (!ROLL) {
                // one tile: load its columns now, after the barrier, so that
                // each column's arithmetic waits only for its own loads
#pragma unroll
                for (uint32_t c = 0; c < CW; ++c) d[c] = load_col(kv, kv4, c);
                if (kc + CK < kbs1) kbidx_window(blockIdx.x, kc + CK, kv, kv4);   // the next round's window
            }
            // after the workgroup's last tile of its last round there is
            // nothing to refill; at MG = 2 the loads are skipped then, at
            // MG = 1 they stay unconditional (clamped windows, no block
            // found), which keeps the register allocation free of spills
            const bool more = MG == 1 || pk < kbs1;       // workgroup-uniform
#pragma unroll
            for (uint32_t c = 0; c < CW; ++c) {
                if (c < nc) compute(d[c], wave * CW + c, acc[i]);
                if (ROLL && more) d[c] = load_col(kv, kv4, c);
            }
            if (ROLL) {
                advance();
                if (MG == 1 || pk < kbs1) window(kv, kv4);
            }
        }
        __syncthreads();
        if (kc + CK < kbs1) stage_x(kc + CK);
    }

    // Per tile: lane (r, q) holds rows m = 16g + 4q + e of output row
    // t*16 + r; the 16 wavefronts' sums are added in wavefront order.
#pragma unroll
    for (uint32_t i = 0; i < NT; ++i) {
        if (!tile_ok(i)) continue;                        // workgroup-uniform
        const uint32_t t = blockIdx.x + i * gridDim.x;
        if (i) __syncthreads();                           // the previous tile's sums are read
#pragma unroll
        for (int g = 0; g < MG; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[(wave * (MG * 4) + g * 4 + e) * 64 + lane] = acc[i][g][e];
        __syncthreads();
        const uint32_t o = threadIdx.x;
        if (o < 256u * MG) {
            const uint32_t m = o >> 4, r = o & 15u;
            const uint32_t g = m >> 4, qq = (m >> 2) & 3u, e = m & 3u;
            float v = 0.0f;
#pragma unroll
            for (uint32_t k = 0; k < kDecWaves; ++k) v += red[(k * (MG * 4) + g * 4 + e) * 64 + r + 16u * qq];
            const uint32_t n = t * 16u + r;
            if (m < a.M && n < w.N) {
                if (a.partial) {
                    a.partial[(uint64_t(blockIdx.y) * a.M + m) * w.N + n] = v;
                } else {
                    if (a.act == HT_ACT_RELU) v = v > 0.0f ? v : 0.0f;
                    if (a.ybf) a.ybf[int64_t(m) * a.ldy + n] = f32_to_bf16_rne(v);
                    else a.y[int64_t(m) * a.ldy + n] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

constexpr uint32_t kDecMinGrid = 192;   // workgroups before K is split further
constexpr int64_t kDecMaxM = 32;        // rows of x per launch (two MFMA row groups)

struct DecShape {
    uint32_t S, KBs;
};

// K-splits only to cover the chip when there are few row tiles (at least 16
// K-blocks per split, every split non-empty).
DecShape dec_shape(const ht_packed_weight *w) {
    const uint32_t KB = uint32_t(w->K / kBlockK), T = uint32_t(w->n_tiles);
    uint32_t S = 1;
    while (uint64_t(T) * S < kDecMinGrid && KB / (S + 1) >= kDecWaves) ++S;
    DecShape d;
    d.KBs = (KB + S - 1) / S;
    d.S = (KB + d.KBs - 1) / d.KBs;
    return d;
}

// Row tiles per workgroup: one while the tiles fit one workgroup per compute
// unit (the LDS of a workgroup allows one per compute unit), else up to
// kDecMaxTPW, so that x is copied once for several tiles instead of the
// launch running in several waves of workgroups.
uint32_t dec_tpw(uint32_t T) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (T <= uint32_t(cus)) return 1;
    const uint32_t tpw = (T + uint32_t(cus) - 1) / uint32_t(cus);
    return tpw < kDecMaxTPW ? tpw : kDecMaxTPW;
}

template <int MG, bool ROLL>
void launch_dec(const DecArgs &a, uint32_t G, uint32_t S, bool buf, hipStream_t s) {
    if (buf) hipLaunchKernelGGL((gemv_mfma_kernel<MG, ROLL, true>), dim3(G, S), dim3(kDecThreads), 0, s, a);
    else hipLaunchKernelGGL((gemv_mfma_kernel<MG, ROLL, false>), dim3(G, S), dim3(kDecThreads), 0, s, a);
}

template <int MG>
void launch_dec(const DecArgs &a, uint32_t G, uint32_t S, bool roll, bool buf, hipStream_t s) {
    if (roll) launch_dec<MG, true>(a, G, S, buf, s);
    else launch_dec<MG, false>(a, G, S, buf, s);
}

// Masked fixed-count loads pay when most columns hold a block wider than 16
// bytes per lane: with a share p of such blocks a 16-block column has one
// with probability 1 - (1 - p)^16, one half at p = 4.2%.
bool dec_buf(const ht_packed_weight *w) {
    const int64_t wide = w->counts[2] + w->counts[3] + w->counts[4];
    const int64_t all = wide + w->counts[0] + w->counts[1];
    return wide * 24 >= all;
}

}  // namespace

bool dec_ok(const ht_packed_weight *w) { return w->row_tile == 16 && w->bytes < 0xFFFFFF00ull; }

size_t dec_ws(const ht_packed_weight *w, int64_t M) {
    const int64_t Mt = M < kDecMaxM ? M : kDecMaxM;
    const DecShape d = dec_shape(w);
    return d.S > 1 ? size_t(d.S) * size_t(Mt) * size_t(w->N) * sizeof(float) : 0;
}

ht_status run_dec(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y, uint16_t *ybf,
                  int64_t ldy, int act, void *ws, hipStream_t s) {
    const DecShape d = dec_shape(w);
    DecArgs a;
    a.w = layer_dev(w);
    a.ldx = ldx;
    a.ldy = ldy;
    a.act = act;
    a.KBs = d.KBs;
    const uint32_t T = uint32_t(w->n_tiles);
    a.TPW = dec_tpw(T);
    a.nbytes = uint32_t(w->bytes);
    const bool buf = dec_buf(w);
    const uint32_t G = (T + a.TPW - 1) / a.TPW;
    for (int64_t m0 = 0; m0 < M; m0 += kDecMaxM) {
        const int64_t Mt = M - m0 < kDecMaxM ? M - m0 : kDecMaxM;
        a.x = x + m0 * ldx;
        a.M = uint32_t(Mt);
        a.y = nullptr;
        a.ybf = nullptr;
        a.partial = nullptr;
        float *yo = y ? y + m0 * ldy : nullptr;
        uint16_t *yb = ybf ? ybf + m0 * ldy : nullptr;
        if (d.S > 1) {
            a.partial = static_cast<float *>(ws);
        } else {
            a.y = yo;
            a.ybf = yb;
        }
        // more than one (round, tile) step per workgroup: several tiles, or
        // a K range longer than one round (64 K-blocks at MG = 1, 32 at 2)
        const uint32_t ck = Mt <= 16 ? kDecChunk : kDecChunk / 2;
        const bool roll = a.TPW > 1 || d.KBs > ck;
        if (Mt <= 16) launch_dec<1>(a, G, d.S, roll, buf, s);
        else launch_dec<2>(a, G, d.S, roll, buf, s);
        HT_LAUNCH_CHECK();
        if (d.S > 1) {
            const ht_status st = launch_split_reduce(static_cast<const float *>(ws), d.S, uint32_t(Mt), a.w.N, yo,
                                                     yb, ldy, act, s);
            if (st != HT_OK) return st;
        }
    }
    return HT_OK;
}

}  // namespace ht
