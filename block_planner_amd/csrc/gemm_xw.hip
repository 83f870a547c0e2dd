// gemm_xw.hip -- the mixed-format linear for many rows of x (prefill) in two
// passes (HyperTensor 1.0.1 page, intro: fused kernels execute the
// mixed-precision plan; "Key Features": HyperLinear).
//
// Pass 1 (xw_expand_kernel) turns each 128-column x 64-K weight tile of the
// packed layout, once, into a record in the workspace: the bfloat16 hi and
// lo planes and the per-column scales that the fused prefill kernel
// (gemm.hip) builds in LDS, with the same arithmetic:
//   INT4 / INT8   hi = the codes (exact in bfloat16), lo = 0, scale s;
//   BF16          hi = the values, lo = 0, scale 1;
//   FP16 / FP32   hi = w with the low 16 bits cleared, lo = bf16(w - hi),
//                 scale 1; a non-finite entry gives a NaN lo.
// Pass 2 (gemm_xw_kernel) multiplies x by those records on the matrix cores
// (v_mfma_f32_16x16x32_bf16) in the fused kernel's order: per 64-K step the
// hi partial from a fresh accumulator, added to the output times the column's
// scale; the lo plane's products for 16-column groups that hold an FP16 or
// FP32 block go to accumulators of their own, added once at the end (the
// fused kernel adds them per step), so the two differ by fp32 rounding only.
//
// Why two passes: at M rows the fused kernel dequantises every weight tile
// once per 256-row tile of x (8 times at M = 2048) on dedicated waves.  Here
// one expansion serves all of them, and every wave of the GEMM runs MFMAs and
// copies its share of the x tile and of the record straight into LDS
// (global_load_lds), with no per-step dequantisation.  The price is the
// workspace (33 KiB per tile, 4.1 bytes per weight) and one extra pass that
// streams it (about 8 bytes per weight of HBM traffic).
#include "gemv_common.h"
#include "linear_host.h"

namespace ht {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kXwBN = 128;                       // weight rows (output columns) per tile
constexpr uint32_t kXwBM = 256;                       // rows of x per workgroup
constexpr uint32_t kXwThreads = 512;                  // eight waves, all on the matrix cores
constexpr uint32_t kXwPlane = kXwBN * 64 * 2;         // one bfloat16 plane of a tile: 16 KiB
constexpr uint32_t kXwMeta = 1024;                    // 128 fp32 scales, 8 group flags, padding
constexpr uint32_t kXwRec = 2 * kXwPlane + kXwMeta;   // hi plane, lo plane, meta: 33 KiB
constexpr uint32_t kXwX = kXwBM * 64 * 2;             // x tile of a step: 32 KiB
constexpr uint32_t kXwExpandKb = 1;                   // K-blocks per expansion workgroup

// Byte offset of entries [8q, 8q+8) of column c in a 128 x 64 bfloat16
// plane: column c at 128*c, its 16-byte slots permuted by ((c >> 1) & 7) so
// that the MFMA operand reads of 16 columns are free of bank conflicts.
__device__ __forceinline__ uint32_t xw_off(uint32_t c, uint32_t q) { return 128u * c + 16u * (q ^ ((c >> 1) & 7u)); }

struct XwExpandArgs {
    LayerDev w;
    uint8_t *rec;    // [NT][KB] records
    uint32_t NT;
    uint32_t nbytes; // packed buffer size (below 4 GiB: 32-bit offsets)
};

// One workgroup per (column tile nt, run of kXwExpandKb K-blocks); thread
// (slot gb = tid/2, half h = tid%2) decodes 32 entries of the gb-th block of
// its row tile in format order (the packed layout's order within a step).
__global__ __launch_bounds__(256) void xw_expand_kernel(XwExpandArgs a) {
    __shared__ __align__(16) uint8_t srec[kXwRec];
    const LayerDev &w = a.w;
    const uint32_t tid = threadIdx.x, lane = tid & 63, h = tid & 1, gb = tid >> 1;
    const uint32_t nt = blockIdx.x % a.NT, kbr = blockIdx.x / a.NT;
    const uint32_t kb0 = kbr * kXwExpandKb, kb1 = min(w.KB, kb0 + kXwExpandKb);
    const uint32_t R = w.R, tile = nt * (kXwBN / R) + gb / R, bi = gb % R;
    const bool tok = tile < w.T;
    const uint32_t *kbidx = reinterpret_cast<const uint32_t *>(w.base + w.off_kbidx);
    auto nib = [](uint32_t v, uint32_t at) { return int32_t(v << (28u - at)) >> 28; };   // signed 4-bit field
    auto pair_hi = [](float f0, float f1) {   // upper halves of two fp32 -> one word
        return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    };
    auto pair_lo = [](float f0, float f1) {   // bf16_rne(f - trunc(f)) of two fp32
        const float r0 = f0 - __uint_as_float(__float_as_uint(f0) & 0xffff0000u);
        const float r1 = f1 - __uint_as_float(__float_as_uint(f1) & 0xffff0000u);
        const bf16x2 v = {(__bf16)r0, (__bf16)r1};
        return __builtin_bit_cast(uint32_t, v);
    };
    // per-format offsets as scalars (selected below by compares, not by
    // indexing the argument block); buffer loads past the buffer read zeros
    uint32_t opay[5], oids[5];
#pragma unroll
    for (int g = 0; g < 5; ++g) {
        opay[g] = uint32_t(w.off_pay[g]);
        oids[g] = uint32_t(w.off_ids[g]);
    }
    const uint32_t osc0 = uint32_t(w.off_scale[0]), osc1 = uint32_t(w.off_scale[1]);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)w.base, 0, int(a.nbytes), 0x00020000);
    constexpr uint32_t kOut = 0xFFFFFFF0u;
    for (uint32_t kb = kb0; kb < kb1; ++kb) {
        // the slot's format f and block index: c[f] <= bi < c[f+1] over the
        // prefix sums of the step's block counts in format order (all ten
        // kbidx words loaded at once, then compares: one round trip)
        uint32_t ka[5], kn[5];
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            const uint32_t e = uint32_t(g) * w.nk + (tok ? tile : 0u) * w.KB + kb;
            ka[g] = __builtin_amdgcn_raw_buffer_load_b32(rs, uint32_t(w.off_kbidx) + 4u * e, 0, 0);
            kn[g] = __builtin_amdgcn_raw_buffer_load_b32(rs, uint32_t(w.off_kbidx) + 4u * (e + 1u), 0, 0);
        }
        uint32_t c = 0, f = 0, cf = 0, kaf = 0;
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            const uint32_t cnt = kn[g] - ka[g];
            const bool past = bi >= c + cnt;          // the slot lies beyond format g
            f += past ? 1u : 0u;
            cf = (f == uint32_t(g)) ? c : cf;         // set while f == g: the start of the slot's format
            kaf = (f == uint32_t(g)) ? ka[g] : kaf;
            c += cnt;
        }
        if (!tok) f = 5;
        const uint32_t blk = kaf + (bi - cf);
        uint32_t po = kOut, io = kOut, so = kOut, np = 0, pb = 0;
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            if (f == uint32_t(g)) {
                pb = uint32_t(pay_bytes(g));
                po = opay[g] + blk * pb + h * (pb / 2);
                io = oids[g] + 2u * blk;
                so = g == 0 ? osc0 + 4u * blk : g == 1 ? osc1 + 4u * blk : kOut;
                np = pb / 32;   // 16-byte pieces of this half
            }
        }
        // eight 16-byte pieces, those past this half's bytes masked
        uint32_t u[32];
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, j < np ? po + 16u * j : kOut, 0, 0);
            u[4 * j] = v.x;
            u[4 * j + 1] = v.y;
            u[4 * j + 2] = v.z;
            u[4 * j + 3] = v.w;
        }
        const uint32_t idv = __builtin_amdgcn_raw_buffer_load_b32(rs, io & ~3u, 0, 0);
        const float scv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, so, 0, 0));
        uint32_t hp[16], lp[16];
        const uint32_t id = f < 5 ? ((io & 2u) ? idv >> 16 : idv & 0xFFFFu) : gb;
        const float sc = f < 2 ? scv : 1.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) hp[i] = lp[i] = 0u;
        switch (f) {
        case 0:
            // byte i of the half's first 8 holds entries 32h+i (low nibble)
            // and 32h+16+i (high), byte 8+i entries 32h+8+i and 32h+24+i
            for (int q2 = 0; q2 < 2; ++q2)
                for (int i = 0; i < 4; ++i) {
                    const uint32_t wd = u[2 * q2 + (i >> 1)], sh = 16 * (i & 1);
                    hp[4 * q2 + i] = pair_hi(float(nib(wd, sh)), float(nib(wd, sh + 8)));
                    hp[8 + 4 * q2 + i] = pair_hi(float(nib(wd, sh + 4)), float(nib(wd, sh + 12)));
                }
            break;
        case 1:
            for (int i = 0; i < 16; ++i) {
                const uint32_t wd = u[i >> 1], sh = 16 * (i & 1);
                hp[i] = pair_hi(float(int8_t(wd >> sh)), float(int8_t(wd >> (sh + 8))));
            }
            break;
        case 2:
            for (int i = 0; i < 16; ++i) hp[i] = u[i];
            break;
        case 3:
            for (int i = 0; i < 16; ++i) {
                const float f0 = float(__builtin_bit_cast(_Float16, uint16_t(u[i])));
                const float f1 = float(__builtin_bit_cast(_Float16, uint16_t(u[i] >> 16)));
                hp[i] = pair_hi(f0, f1);
                lp[i] = pair_lo(f0, f1);
            }
            break;
        case 4:
            for (int i = 0; i < 16; ++i) {
                const float f0 = __uint_as_float(u[2 * i]), f1 = __uint_as_float(u[2 * i + 1]);
                hp[i] = pair_hi(f0, f1);
                lp[i] = pair_lo(f0, f1);
            }
            break;
        default:
            break;
        }
        // column within the tile: the block's row (a missing block keeps its
        // slot, which is then a row past the weight's last); the record is
        // assembled in LDS, then written out in contiguous 16-byte pieces
        const uint32_t col = f < 5 ? (gb / R) * R + (id & (R - 1u)) : gb;
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint4 *>(srec + xw_off(col, 4 * h + i)) =
                make_uint4(hp[4 * i], hp[4 * i + 1], hp[4 * i + 2], hp[4 * i + 3]);
            *reinterpret_cast<uint4 *>(srec + kXwPlane + xw_off(col, 4 * h + i)) =
                make_uint4(lp[4 * i], lp[4 * i + 1], lp[4 * i + 2], lp[4 * i + 3]);
        }
        float *meta = reinterpret_cast<float *>(srec + 2 * kXwPlane);
        if (h == 0) meta[col] = sc;
        // group flag: any FP16 / FP32 block among the 16 columns of this half-wave
        const uint64_t bal = __ballot(f == 3 || f == 4);
        if ((lane & 31u) == 0)
            reinterpret_cast<uint32_t *>(meta + kXwBN)[gb >> 4] = ((bal >> (lane & 32u)) & 0xFFFFFFFFull) != 0 ? 1u : 0u;
        __syncthreads();
        // the lo plane of a 16-column group without FP16 / FP32 blocks is
        // all zeros and never read: it is not written
        uint4 *dst = reinterpret_cast<uint4 *>(a.rec + uint64_t(nt * w.KB + kb) * kXwRec);
        const uint4 *src = reinterpret_cast<const uint4 *>(srec);
        const uint32_t *flags = reinterpret_cast<const uint32_t *>(meta + kXwBN);
        for (uint32_t o = tid; o < kXwRec / 16; o += 256) {
            const bool lo = o >= kXwPlane / 16 && o < 2 * kXwPlane / 16;
            if (!lo || flags[(o - kXwPlane / 16) >> 7] != 0u) dst[o] = src[o];   // 128 pieces per group
        }
        __syncthreads();
    }
}

struct XwGemmArgs {
    const uint8_t *rec;      // [NT][KB] records
    const uint16_t *x;
    int64_t ldx;
    float *y;                // fp32 output, or
    uint16_t *ybf;           // bfloat16 output (round to nearest even)
    int64_t ldy;
    uint32_t M, N, KB, MT, NT;
    int act;
    // tiles [full, MT*NT) run as two workgroups each, K-blocks [0, KBh) and
    // [KBh, KB), dispatched after the others; they write fp32 partial sums
    // part[half][tile - full][256][128] that xw_tail_kernel adds
    uint32_t full, KBh;
    float *part;
};

// Workgroup barrier that waits for this wave's LDS operations only.
__device__ __forceinline__ void xw_lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup (mt, nt) owns rows [256*mt, +256) of x and columns [128*nt, +128)
// of y over all of K.  Workgroup indices are spread so that each XCD gets a
// contiguous run, ordered column tile first: the XCD's L2 then serves one
// record to the row tiles that share it.  Wave w runs MFMAs on rows
// [128*(w>>2), +128) (eight row tiles of 16) and columns [32*(w&3), +32)
// (two groups of 16), and copies 4 of the x tile's 32 KiB and 4 or 5 of the
// record's 33 KiB into the other LDS stage for the step after next.
__global__ __launch_bounds__(kXwThreads) void gemm_xw_kernel(XwGemmArgs a) {
    __shared__ __align__(16) uint8_t lds0[kXwX + kXwRec], lds1[kXwX + kXwRec];

    const uint32_t tid = threadIdx.x, lane = tid & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroup -> tile: the whole-K tiles first, then the split tiles' halves
    // (so that those short workgroups fill the last round); each range
    // spread over the XCDs in contiguous runs.
    uint32_t L, kb0 = 0, kb1 = a.KB, half = 2u;
    if (blockIdx.x < a.full) {
        L = blockIdx.x;
        if ((a.full & 7u) == 0) L = (L & 7u) * (a.full >> 3) + (L >> 3);
    } else {
        const uint32_t n = gridDim.x - a.full;
        uint32_t j = blockIdx.x - a.full;
        if ((n & 7u) == 0) j = (j & 7u) * (n >> 3) + (j >> 3);
        L = a.full + (j >> 1);
        half = j & 1u;
        kb0 = half ? a.KBh : 0u;
        kb1 = half ? a.KB : a.KBh;
    }
    const uint32_t nt = L / a.MT, mt = L - nt * a.MT;
    const uint32_t n0 = nt * kXwBN, m0 = mt * kXwBM;
    const uint32_t KB = kb1 - kb0;
    const uint32_t wr = wave >> 2, wc = wave & 3;

    // x copy: instruction g (of 32) moves rows [8g, +8): lane l -> row
    // 8g + l/8, 16-byte slot l%8, which holds entries [8*(slot ^ ((row >> 1) & 7)), +8);
    // a uniform base per instruction (the group's first row, clamped to the
    // last row of x) and a 32-bit offset per lane (rows past M read row M-1)
    const uint32_t xr = lane >> 3, xslot = lane & 7;
    const uint16_t *xrow[4];
    uint32_t xoff[4];
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
        const uint32_t g = 4 * wave + i, r = 8 * g + xr;
        const uint32_t rb = min(m0 + 8 * g, a.M - 1u), rr = min(m0 + r, a.M - 1u);
        xrow[i] = a.x + int64_t(rb) * a.ldx;
        xoff[i] = uint32_t((uint64_t(rr - rb) * uint64_t(a.ldx) + 8u * (xslot ^ ((r >> 1) & 7u))) * 2u);
    }
    const uint8_t *recs = a.rec + (uint64_t(nt) * a.KB + kb0) * kXwRec;
    // Issued as inline assembly (M0 = LDS destination of the instruction's
    // 1 KiB), so the compiler adds no waits for them before unrelated LDS
    // reads; each wave waits for its own copies (vmcnt(0)) before the barrier
    // that publishes them.
    auto copy = [&](uint32_t kb, uint8_t *st) {
        const uint32_t base = uint32_t(uintptr_t((__attribute__((address_space(3))) uint8_t *)st));
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i) {
            const uint16_t *src = xrow[i] + (kb0 + kb) * 64u;
            const uint32_t dst = base + 1024u * (4 * wave + i);
            asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                         :
                         : "v"(xoff[i]), "s"(src), "s"(dst)
                         : "memory", "m0");
        }
        const uint8_t *rsrc = recs + uint64_t(kb) * kXwRec;
#pragma unroll
        for (uint32_t i = 0; i < 5; ++i) {
            const uint32_t j = wave + 8 * i;   // 1 KiB piece of the record
            if (i < 4 || j < kXwRec / 1024) {
                const uint32_t off = 1024u * j + 16u * lane;
                const uint32_t dst = base + kXwX + 1024u * j;
                asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                             :
                             : "v"(off), "s"(rsrc), "s"(dst)
                             : "memory", "m0");
            }
        }
    };

    const uint32_t lr = lane & 15, lq = lane >> 4;   // MFMA operand row / k-quarter of this lane
    // acc: the scaled hi partials; alo: the lo plane's products, which are
    // non-zero only in FP16 / FP32 columns (scale 1) and join acc at the end
    f32x4 acc[8][2], alo[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = alo[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One K-step.  Per row tile: the hi partials of the wave's two column
    // groups (fresh accumulators), added to acc times the column's scale two
    // row tiles later (so the FMAs read finished results), and the lo plane
    // into alo for a group that holds an FP16 / FP32 block in this step (the
    // record's group flag; other groups' lo planes are not even written).
    // A operands are read two row tiles ahead; one scheduling region per row
    // tile keeps that order.
    auto mfma_step = [&](const uint8_t *st, auto &&mid) {
        const uint16_t *xs = reinterpret_cast<const uint16_t *>(st);
        const uint8_t *rec = st + kXwX;
        bf16x8 Bh[2][2], Bl[2][2];
        float sc[2];
        const uint2 nl2 = *reinterpret_cast<const uint2 *>(rec + 2 * kXwPlane + 4 * kXwBN + 8 * wc);
        const uint32_t nl[2] = {uint32_t(__builtin_amdgcn_readfirstlane(nl2.x)),
                                uint32_t(__builtin_amdgcn_readfirstlane(nl2.y))};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t col = 32 * wc + 16 * j + lr;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                Bh[j][q] = *reinterpret_cast<const bf16x8 *>(rec + xw_off(col, lq + 4 * q));
                Bl[j][q] = *reinterpret_cast<const bf16x8 *>(rec + kXwPlane + xw_off(col, lq + 4 * q));
            }
            sc[j] = reinterpret_cast<const float *>(rec + 2 * kXwPlane)[col];
        }
        auto readA = [&](int i, bf16x8 (&A)[2]) {
            const uint32_t r = 128 * wr + 16 * i + lr;
#pragma unroll
            for (int q = 0; q < 2; ++q)
                A[q] = *reinterpret_cast<const bf16x8 *>(xs + r * 64 + 8 * ((lq + 4 * q) ^ ((r >> 1) & 7u)));
        };
        bf16x8 Ar[3][2];
        readA(0, Ar[0]);
        readA(1, Ar[1]);
        f32x4 cp[2][2];
        auto scale_add = [&](int i, const f32x4 (&c)[2]) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(sc[j], c[j][e], acc[i][j][e]);
                asm volatile("" : "+v"(acc[i][j]));   // keeps the update in this row tile's slot
            }
        };
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i + 2 < 8) readA(i + 2, Ar[(i + 2) % 3]);
            const bf16x8 (&A)[2] = Ar[i % 3];
            f32x4 cc[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                cc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], Bh[j][0], (f32x4{0.f, 0.f, 0.f, 0.f}), 0, 0, 0);
                cc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], Bh[j][1], cc[j], 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (nl[j] != 0u) {
                    alo[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], Bl[j][0], alo[i][j], 0, 0, 0);
                    alo[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], Bl[j][1], alo[i][j], 0, 0, 0);
                }
            }
            if (i > 1) scale_add(i - 2, cp[i % 2]);
            if (i == 1) mid();   // the next copies, once this step's first operands are in registers
            cp[i % 2][0] = cc[0];
            cp[i % 2][1] = cc[1];
            __builtin_amdgcn_sched_barrier(0);
        }
        scale_add(6, cp[0]);
        scale_add(7, cp[1]);
    };

    // two LDS stages; the copy for step t+2 goes into step t's stage during
    // step t+1 (after the barrier that ends step t), issued once step t+1's
    // first operands have been read, so that they do not queue behind it
    copy(0, lds0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies are in LDS
    if (KB > 1) copy(1, lds1);
    xw_lds_barrier();
    auto step = [&](uint32_t t, const uint8_t *st, uint8_t *prev) {
        mfma_step(st, [&]() {
            if (t >= 1 && t + 1 < KB) copy(t + 1, prev);
        });
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the copies for step t+1 are in LDS
        xw_lds_barrier();
    };
    for (uint32_t t = 0; t < KB; t += 2) {
        step(t, lds0, lds1);
        if (t + 1 < KB) step(t + 1, lds1, lds0);
    }

    // ---- output: lane holds column lr, rows 4*(lane/16) + e of each 16x16 tile ----
    if (half < 2u) {   // a split tile: this half's partial sums, whole tile, no activation
        float *p = a.part + (uint64_t(half) * (a.MT * a.NT - a.full) + (L - a.full)) * (kXwBM * kXwBN);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p[(128 * wr + 16 * i + 4 * lq + e) * kXwBN + 32 * wc + 16 * j + lr] = acc[i][j][e] + alo[i][j][e];
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t n = n0 + 32 * wc + 16 * j + lr;
            if (n >= a.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t m = m0 + 128 * wr + 16 * i + 4 * lq + e;
                if (m >= a.M) continue;
                float v = acc[i][j][e] + alo[i][j][e];
                if (a.act == HT_ACT_RELU) v = v > 0.0f ? v : 0.0f;   // +0 for zero, negative and NaN
                if (a.ybf) a.ybf[int64_t(m) * a.ldy + n] = f32_to_bf16_rne(v);
                else a.y[int64_t(m) * a.ldy + n] = v;
            }
        }
}

// The split tiles: y = act(part[0] + part[1]) (the first K half's sum plus
// the second's, always in that order), four outputs per thread.
__global__ __launch_bounds__(256) void xw_tail_kernel(XwGemmArgs a) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;     // [tile][row][column / 4]
    const uint32_t tail = a.MT * a.NT - a.full;
    if (i >= tail * (kXwBM * kXwBN / 4)) return;
    const uint32_t tl = i / (kXwBM * kXwBN / 4), rem = i - tl * (kXwBM * kXwBN / 4);
    const uint32_t r = rem / (kXwBN / 4), c4 = rem - r * (kXwBN / 4);
    const uint32_t L = a.full + tl, nt = L / a.MT, mt = L - nt * a.MT;
    const uint32_t m = mt * kXwBM + r;
    if (m >= a.M) return;
    const uint64_t off = uint64_t(tl) * (kXwBM * kXwBN) + r * kXwBN + 4 * c4;
    const float4 p0 = *reinterpret_cast<const float4 *>(a.part + off);
    const float4 p1 = *reinterpret_cast<const float4 *>(a.part + uint64_t(tail) * (kXwBM * kXwBN) + off);
    const float v[4] = {p0.x + p1.x, p0.y + p1.y, p0.z + p1.z, p0.w + p1.w};
#pragma unroll
    for (uint32_t e = 0; e < 4; ++e) {
        const uint32_t n = nt * kXwBN + 4 * c4 + e;
        if (n >= a.N) continue;
        float o = v[e];
        if (a.act == HT_ACT_RELU) o = o > 0.0f ? o : 0.0f;
        if (a.ybf) a.ybf[int64_t(m) * a.ldy + n] = f32_to_bf16_rne(o);
        else a.y[int64_t(m) * a.ldy + n] = o;
    }
}

constexpr int64_t kXwChunkRows = int64_t(1) << 20;   // rows per GEMM launch
constexpr int64_t kXwMaxLdx = int64_t(1) << 28;      // x row stride limit (elements)

}  // namespace

bool xw_takes(const ht_packed_weight *w, int64_t M) {
    const int64_t NT = (w->N + kXwBN - 1) / kXwBN;
    const int64_t Mt = M < kXwChunkRows ? M : kXwChunkRows;
    // several row tiles share each expansion, and the tiles fill the chip;
    // the expansion reads the packed buffer with 32-bit offsets
    return M >= kXwMinM && NT * ((Mt + kXwBM - 1) / kXwBM) >= 192 && w->bytes < 0xFFFFFF00ull;
}

// Compute units (one GEMM workgroup each: its LDS allows one).
uint32_t xw_units() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return uint32_t(cus);
}

// Tiles of one launch run with K split in two: the last round's, when it
// would fill at most half of the compute units (then its halves fill it, in
// about half the time), and only when K has two K-blocks or more.
uint32_t xw_split_tiles(uint32_t tiles, uint32_t KB, uint32_t units) {
    const uint32_t tail = tiles % units;
    return tiles > units && tail > 0 && 2 * tail <= units && KB >= 2 ? tail : 0u;
}

size_t xw_records(const ht_packed_weight *w) {
    const uint64_t NT = uint64_t((w->N + kXwBN - 1) / kXwBN), KB = uint64_t(w->K / kBlockK);
    return size_t(NT * KB * kXwRec);
}

size_t xw_ws(const ht_packed_weight *w, int64_t M) {
    const uint64_t NT = uint64_t((w->N + kXwBN - 1) / kXwBN);
    const int64_t Mt = M < kXwChunkRows ? M : kXwChunkRows;
    const uint64_t tiles = NT * uint64_t((Mt + kXwBM - 1) / kXwBM);
    const uint32_t split = xw_split_tiles(uint32_t(tiles), uint32_t(w->K / kBlockK), xw_units());
    return xw_records(w) + size_t(split) * 2u * kXwBM * kXwBN * sizeof(float);
}

ht_status run_gemm_xw(const ht_packed_weight *w, const uint16_t *x, int64_t M, int64_t ldx, float *y, uint16_t *ybf,
                      int64_t ldy, int act, void *ws, hipStream_t s) {
    if (ldx >= kXwMaxLdx) return HT_ESHAPE;   // the x copies take 32-bit offsets of up to 7 rows
    XwExpandArgs e;
    e.w = layer_dev(w);
    e.rec = static_cast<uint8_t *>(ws);
    e.NT = uint32_t((w->N + kXwBN - 1) / kXwBN);
    e.nbytes = uint32_t(w->bytes);
    const uint32_t kbr = (e.w.KB + kXwExpandKb - 1) / kXwExpandKb;
    hipLaunchKernelGGL(xw_expand_kernel, dim3(e.NT * kbr), dim3(256), 0, s, e);
    HT_LAUNCH_CHECK();
    for (int64_t r0 = 0; r0 < M; r0 += kXwChunkRows) {
        const int64_t Mt = M - r0 < kXwChunkRows ? M - r0 : kXwChunkRows;
        XwGemmArgs a;
        a.rec = e.rec;
        a.x = x + r0 * ldx;
        a.ldx = ldx;
        a.y = y ? y + r0 * ldy : nullptr;
        a.ybf = ybf ? ybf + r0 * ldy : nullptr;
        a.ldy = ldy;
        a.M = uint32_t(Mt);
        a.N = uint32_t(w->N);
        a.KB = e.w.KB;
        a.MT = uint32_t((Mt + kXwBM - 1) / kXwBM);
        a.NT = e.NT;
        a.act = act;
        const uint32_t tiles = a.MT * a.NT, split = xw_split_tiles(tiles, a.KB, xw_units());
        a.full = tiles - split;
        a.KBh = a.KB / 2;
        a.part = reinterpret_cast<float *>(e.rec + xw_records(w));
        hipLaunchKernelGGL(gemm_xw_kernel, dim3(a.full + 2 * split), dim3(kXwThreads), 0, s, a);
        HT_LAUNCH_CHECK();
        if (split) {
            hipLaunchKernelGGL(xw_tail_kernel, dim3(split * (kXwBM * kXwBN / 4) / 256), dim3(256), 0, s, a);
            HT_LAUNCH_CHECK();
        }
    }
    return HT_OK;
}

}  // namespace ht
